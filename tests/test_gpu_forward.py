"""GPU forward (y and the saved fp32 statistics) against the fp64 oracle.

The forward computes, per row, LayerNorm mean / biased variance / rstd and
y = gamma * (x - mean) * rstd + beta, or RMSNorm rstd = 1/sqrt(mean(x^2) + eps)
and y = gamma * x * rstd ("05: Layer norm", the Phobos tutorial's forward;
"Norm backward in Triton", "The gradients"). Small sizes are compared element
by element, full sizes on sampled rows (every output is row-local). The round
trip runs the GPU backward on the statistics the GPU forward saved.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import parity
from rmsnorm_backward_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nb():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import rmsnorm_backward_amd as nbmod
    nbmod.load_library()
    return nbmod


def _beta(w, inp):
    if w.kind != "layernorm":
        return None
    if "beta" in inp:
        return inp["beta"]
    g = torch.Generator().manual_seed(w.seed + 17)
    return torch.rand(w.N, generator=g).to(w.io_dtype)


def gpu_forward(nb, w, x, gamma, beta, **kw):
    if w.kind == "layernorm":
        y, mean, rstd = nb.norm_fwd_layernorm(x.cuda(), gamma.cuda(),
                                              None if beta is None else beta.cuda(), w.eps, **kw)
    else:
        y, rstd = nb.norm_fwd_rmsnorm(x.cuda(), gamma.cuda(), w.eps, **kw)
        mean = None
    torch.cuda.synchronize()
    return (y.cpu(), None if mean is None else mean.cpu(), None if rstd is None else rstd.cpu())


def check(w, x, gamma, beta, got):
    ry, rm, rr = oracle.fwd(w.kind, x, gamma, beta, w.eps)
    return parity.check_forward(w.io_dtype, w.kind, x, gamma, beta, got[0], got[1], got[2],
                                ry, rm, rr)


SMALL = [
    W.LN_F32_128x512,
    W.RMS_F32_128x512,
    W.LN_F16_1151x8192,
    W.scaled(W.RMS_BF16_16384x4096, M=2003),
    W.scaled(W.LN_BF16_65536x8192, M=777),
    W.scaled(W.RMS_BF16_262144x768, M=5001),
    W.scaled(W.RMS_BF16_262144x768, M=3001, name="rmsnorm_bf16_3001x768_entry_outliers",
             outlier_mode="entries"),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_forward_parity(nb, w):
    inp = W.make_inputs(w)
    beta = _beta(w, inp)
    got = gpu_forward(nb, w, inp["x"], inp["gamma"], beta)
    print(w.name, check(w, inp["x"], inp["gamma"], beta, got))
    if w.kind == "layernorm":       # beta = NULL is y = gamma * xhat
        got0 = gpu_forward(nb, w, inp["x"], inp["gamma"], None)
        check(w, inp["x"], inp["gamma"], None, got0)
        assert torch.equal(got0[1], got[1]) and torch.equal(got0[2], got[2])


def test_phobos_forward_distribution(nb):
    """The Phobos tutorial's inputs: x = -2.3 + 0.5*N(0,1), gamma, beta ~ U(0,1),
    fp16, 1151 x 8192, eps 1e-5 ("05: Layer norm", its check)."""
    g = torch.Generator().manual_seed(0)
    M, N = 1151, 8192
    gamma = torch.rand(N, generator=g).half()
    beta = torch.rand(N, generator=g).half()
    x = (-2.3 + 0.5 * torch.randn(M, N, generator=g)).half()
    w = W.scaled(W.LN_F16_1151x8192, name="phobos_forward")
    got = gpu_forward(nb, w, x, gamma, beta)
    check(w, x, gamma, beta, got)


FWD_N = {
    torch.float32: [1, 3, 8, 63, 64, 65, 257, 1000, 4100, 8191, 16384],
    torch.float16: [1, 2, 63, 64, 65, 513, 768, 4100, 8192, 16384, 32768],
    torch.bfloat16: [1, 7, 16, 65, 520, 2048, 4096, 6144, 8192, 20000, 32768],
}
FWD_M = [1, 2, 3, 511, 513]


def _fwd_edges():
    out = []
    for dt, ns in FWD_N.items():
        for i, n in enumerate(ns):
            for kind in ("layernorm", "rmsnorm"):
                m = FWD_M[(i + (kind == "rmsnorm")) % len(FWD_M)]
                if n >= 16384:
                    m = min(m, 64)
                out.append((kind, dt, m, n))
    return out


@pytest.mark.parametrize("kind,dt,M,N", _fwd_edges(), ids=lambda v: str(v).replace("torch.", ""))
def test_forward_edge_shapes(nb, kind, dt, M, N):
    base = W.LN_F32_128x512 if kind == "layernorm" else W.RMS_F32_128x512
    w = W.scaled(base, M=M, N=N, io_dtype=dt, seed=300 + M + N)
    inp = W.make_inputs(w)
    beta = _beta(w, inp)
    got = gpu_forward(nb, w, inp["x"], inp["gamma"], beta)
    check(w, inp["x"], inp["gamma"], beta, got)


WIDE_FWD = [(kind, dt, M, N)
            for kind in ("layernorm", "rmsnorm")
            for dt, M, N in ((torch.float32, 3, 16385), (torch.float32, 7, 40000),
                             (torch.bfloat16, 5, 32776), (torch.float16, 2, 100003),
                             (torch.bfloat16, 300, 65536), (torch.float16, 11, 9001))]


@pytest.mark.parametrize("kind,dt,M,N", WIDE_FWD, ids=lambda v: str(v).replace("torch.", ""))
def test_forward_wide_rows(nb, kind, dt, M, N):
    """Rows wider than the fused forward holds (or unaligned beyond 8192) take
    the wide-row forward: held in registers when they fit (32776 and 65536
    16-bit, 40000 fp32 hold their row; LayerNorm with beta at 8 chunks and
    100003 stream it), streamed by the row loop otherwise. Same results to
    the same tolerance."""
    base = W.LN_F32_128x512 if kind == "layernorm" else W.RMS_F32_128x512
    w = W.scaled(base, M=M, N=N, io_dtype=dt, seed=40 + M + N)
    inp = W.make_inputs(w)
    beta = _beta(w, inp)
    got = gpu_forward(nb, w, inp["x"], inp["gamma"], beta)
    check(w, inp["x"], inp["gamma"], beta, got)
    if kind == "layernorm":
        got0 = gpu_forward(nb, w, inp["x"], inp["gamma"], None)
        check(w, inp["x"], inp["gamma"], None, got0)


def test_forward_constant_rows_and_zero_rows(nb):
    """Degenerate rows: a constant row has variance 0 (xhat = 0, rstd =
    1/sqrt(eps), y = beta); an all-zero row gives RMSNorm rstd = 1/sqrt(eps)
    and y = 0."""
    N = 1024
    x = torch.zeros(4, N)
    x[1] = 3.25
    x[2] = -7.5
    x[3, ::2] = 1.0
    gamma = torch.linspace(0.5, 1.5, N)
    beta = torch.linspace(-1, 1, N)
    for dt in (torch.float32, torch.bfloat16):
        xs, gs, bs = x.to(dt), gamma.to(dt), beta.to(dt)
        w = W.scaled(W.LN_F32_128x512, M=4, N=N, io_dtype=dt)
        y, mean, rstd = gpu_forward(nb, w, xs, gs, bs)
        check(w, xs, gs, bs, (y, mean, rstd))
        assert torch.equal(y[:3], bs.expand(3, N))
        assert torch.allclose(rstd[:3], torch.full((3,), w.eps).rsqrt(), rtol=2 ** -20)
        wr = W.scaled(W.RMS_F32_128x512, M=4, N=N, io_dtype=dt)
        y, _, rstd = gpu_forward(nb, wr, xs, gs, None)
        check(wr, xs, gs, None, (y, None, rstd))
        assert torch.all(y[0] == 0)


@pytest.mark.parametrize("w", [W.RMS_BF16_16384x4096, W.LN_BF16_65536x8192,
                               W.RMS_BF16_262144x768], ids=lambda w: w.name)
def test_forward_full_size_sampled(nb, w):
    print(f"[gen] {w.name}", flush=True)
    inp = W.make_inputs(w)
    beta = _beta(w, inp)
    print(f"[run] {w.name}", flush=True)
    y, mean, rstd = gpu_forward(nb, w, inp["x"], inp["gamma"], beta)
    rows = W.sample_rows(w.M, 64, seed=w.seed + 5,
                         extra=[511, 512, 1023, 1024, 2047, 2048, w.M // 2, w.M - 2])
    got = (y[rows], None if mean is None else mean[rows], rstd[rows])
    check(w, inp["x"][rows], inp["gamma"], beta, got)
    assert torch.isfinite(rstd).all() and (rstd > 0).all()


def test_forward_statistics_optional_and_deterministic(nb):
    w = W.scaled(W.LN_BF16_65536x8192, M=300, N=3000)
    inp = W.make_inputs(w)
    x, g, b = inp["x"].cuda(), inp["gamma"].cuda(), _beta(w, inp).cuda()
    y1, m1, r1 = nb.norm_fwd_layernorm(x, g, b, w.eps)
    y2, m2, r2 = nb.norm_fwd_layernorm(x, g, b, w.eps, want_stats=False)
    assert m2 is None and r2 is None
    y3, m3, r3 = nb.norm_fwd_layernorm(x, g, b, w.eps)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(y1, y3)
    assert torch.equal(m1, m3) and torch.equal(r1, r3)
    # caller-provided outputs are written in place
    y = torch.full_like(x, float("nan"))
    r = torch.full((w.M,), float("nan"), device="cuda")
    nb.norm_fwd_rmsnorm(x, g, 1e-6, y=y, rstd=r)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all() and torch.isfinite(r).all()


@pytest.mark.parametrize("kind,dt,M,m,N", [
    ("layernorm", torch.bfloat16, 4096, 600, 8192),    # 1 -> 2 rows in flight
    ("rmsnorm", torch.bfloat16, 8192, 1000, 4096),     # 2 -> 4
    ("rmsnorm", torch.float32, 4096, 300, 4096),       # 1 -> 2
    ("layernorm", torch.float16, 1151, 500, 8192),     # too few rows: stays at 1
])
def test_forward_rows_do_not_depend_on_the_launch(nb, kind, dt, M, m, N):
    """The forward doubles its rows in flight only where each row-lane keeps
    at least 4 rows, so a large batch and its first m rows launch with
    different geometry; every output row is the same bit for bit, and both
    match the oracle."""
    base = W.LN_BF16_65536x8192 if kind == "layernorm" else W.RMS_BF16_16384x4096
    w = W.scaled(base, M=M, N=N, io_dtype=dt)
    inp = W.make_inputs(w)
    x, g = inp["x"].cuda(), inp["gamma"].cuda()
    if kind == "layernorm":
        b = _beta(w, inp).cuda()
        big = nb.norm_fwd_layernorm(x, g, b, w.eps)
        small = nb.norm_fwd_layernorm(x[:m].contiguous(), g, b, w.eps)
    else:
        big = nb.norm_fwd_rmsnorm(x, g, w.eps)
        small = nb.norm_fwd_rmsnorm(x[:m].contiguous(), g, w.eps)
    torch.cuda.synchronize()
    for t_big, t_small in zip(big, small):
        assert torch.equal(t_big[:m], t_small)
    rows = slice(0, 64)
    beta = _beta(w, inp) if kind == "layernorm" else None
    if kind == "layernorm":
        got = (big[0][rows].cpu(), big[1][rows].cpu(), big[2][rows].cpu())
    else:
        got = (big[0][rows].cpu(), None, big[1][rows].cpu())
    check(W.scaled(w, M=64), inp["x"][rows], inp["gamma"], beta, got)


@pytest.mark.parametrize("kind,dt,M,N", [
    ("rmsnorm", torch.bfloat16, 700, 5120), ("layernorm", torch.bfloat16, 300, 7168),
    ("layernorm", torch.float16, 513, 3072), ("rmsnorm", torch.float32, 333, 1536),
    ("layernorm", torch.bfloat16, 4100, 5120),       # 1024 threads of rows in flight
    ("rmsnorm", torch.bfloat16, 2001, 1536), ("layernorm", torch.bfloat16, 777, 2560),
    ("rmsnorm", torch.float16, 5000, 3584)])          # 16-byte lanes
def test_forward_exact_non_power_of_two_waves(nb, kind, dt, M, N):
    """The forward on the widths whose rows take 3, 5 or 7 waves."""
    base = W.LN_BF16_65536x8192 if kind == "layernorm" else W.RMS_BF16_16384x4096
    w = W.scaled(base, M=M, N=N, io_dtype=dt)
    inp = W.make_inputs(w)
    x, g = inp["x"].cuda(), inp["gamma"].cuda()
    beta = _beta(w, inp)
    if kind == "layernorm":
        got = nb.norm_fwd_layernorm(x, g, beta.cuda(), w.eps)
    else:
        y, r = nb.norm_fwd_rmsnorm(x, g, w.eps)
        got = (y, None, r)
    torch.cuda.synchronize()
    check(w, inp["x"], inp["gamma"], beta, tuple(None if t is None else t.cpu() for t in got))


@pytest.mark.parametrize("kind,dt,M,m,N", [
    ("rmsnorm", torch.bfloat16, 1, 1, 768), ("layernorm", torch.bfloat16, 2, 1, 768),
    ("layernorm", torch.float16, 3, 2, 256), ("rmsnorm", torch.float16, 8193, 77, 256),
    ("layernorm", torch.float32, 515, 3, 384), ("rmsnorm", torch.float32, 1000, 999, 128),
    # sweeps of complete pairs (the steady-state loop), then a last pair of one row
    ("layernorm", torch.bfloat16, 45001, 1001, 768),
    ("rmsnorm", torch.bfloat16, 65536, 4097, 256)])
def test_forward_two_rows_per_wave(nb, kind, dt, M, m, N):
    """Rows that 32 lanes of 16-byte vectors cover exactly (N = 32 * vec *
    1 or 3) run two rows per wave. Every row matches the oracle, and a
    row's outputs do not depend on which pair or sweep it fell in: the
    first m rows alone (another grid, another pairing of the last row)
    give the same bits."""
    base = W.LN_BF16_65536x8192 if kind == "layernorm" else W.RMS_BF16_16384x4096
    w = W.scaled(base, M=M, N=N, io_dtype=dt, seed=900 + M + N)
    inp = W.make_inputs(w)
    x, g = inp["x"].cuda(), inp["gamma"].cuda()
    beta = _beta(w, inp)

    def fwd(xx):
        if kind == "layernorm":
            return nb.norm_fwd_layernorm(xx, g, beta.cuda(), w.eps)
        y, r = nb.norm_fwd_rmsnorm(xx, g, w.eps)
        return (y, None, r)

    big, small = fwd(x), fwd(x[:m].contiguous())
    torch.cuda.synchronize()
    for t_big, t_small in zip(big, small):
        if t_big is not None:
            assert torch.equal(t_big[:m], t_small)
    check(w, inp["x"], inp["gamma"], beta, tuple(None if t is None else t.cpu() for t in big))


def test_forward_misaligned_rows_take_the_scalar_path(nb):
    w = W.scaled(W.RMS_BF16_16384x4096, M=37, N=1000)
    inp = W.make_inputs(w)
    buf = torch.zeros(w.M * w.N + 1, dtype=w.io_dtype, device="cuda")
    x = buf[1:].view(w.M, w.N)
    x.copy_(inp["x"].cuda())
    y, rstd = nb.norm_fwd_rmsnorm(x, inp["gamma"].cuda(), w.eps)
    torch.cuda.synchronize()
    check(w, inp["x"], inp["gamma"], None, (y.cpu(), None, rstd.cpu()))


def test_forward_empty(nb):
    x = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    g = torch.ones(64, dtype=torch.bfloat16, device="cuda")
    y, m, r = nb.norm_fwd_layernorm(x, g, None)
    assert y.shape == (0, 64) and m.shape == (0,) and r.shape == (0,)
    x0 = torch.empty(3, 0, dtype=torch.bfloat16, device="cuda")
    y, r = nb.norm_fwd_rmsnorm(x0, torch.empty(0, dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    assert y.shape == (3, 0)


@pytest.mark.parametrize("w", [W.scaled(W.RMS_BF16_16384x4096, M=1500),
                               W.scaled(W.LN_BF16_65536x8192, M=300),
                               W.LN_F32_128x512], ids=lambda w: w.name)
def test_forward_then_backward(nb, w):
    """Training-step composition: the GPU backward reads the statistics the GPU
    forward saved. The saved statistics match the oracle's forward, and the
    backward matches the oracle's backward on those same fp32 statistics."""
    inp = W.make_inputs(w)
    beta = _beta(w, inp)
    x, dy, g = inp["x"].cuda(), inp["dy"].cuda(), inp["gamma"].cuda()
    if w.kind == "layernorm":
        y, mean, rstd = nb.norm_fwd_layernorm(x, g, beta.cuda(), w.eps)
        dx, dg, db = nb.norm_bwd_layernorm(x, dy, g, mean, rstd, w.eps,
                                           wgrad_dtype=w.wgrad_dtype)
    else:
        y, rstd = nb.norm_fwd_rmsnorm(x, g, w.eps)
        mean = None
        dx, dg, db = nb.norm_bwd_rmsnorm(x, dy, g, rstd, w.eps, wgrad_dtype=w.wgrad_dtype)
    torch.cuda.synchronize()
    mean_c = None if mean is None else mean.cpu()
    rstd_c = rstd.cpu()
    check(w, inp["x"], inp["gamma"], beta, (y.cpu(), mean_c, rstd_c))
    rdx, rdg, rdb = oracle.bwd(w.kind, inp["x"], inp["dy"], inp["gamma"], mean_c, rstd_c)
    scale = parity.dx_term_scale(w.kind, inp["x"], inp["dy"], inp["gamma"], mean_c, rstd_c)
    parity.check_dx(w.io_dtype, dx.cpu(), rdx, scale=scale)
    bg, bb = parity.wgrad_bounds(w.kind, inp["x"], inp["dy"], mean_c, rstd_c,
                                 parity.depth_path(w.M, w.N, w.io_dtype, db is not None))
    parity.check_wgrad(w.io_dtype, dg.cpu(), rdg, **bg)
    if db is not None:
        parity.check_wgrad(w.io_dtype, db.cpu(), rdb, "dbeta", **bb)
    assert np.isfinite(rdx).all()
