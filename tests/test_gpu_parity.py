"""GPU path against the fp64 oracle, through the C ABI (needs a gfx950 GPU).

Inputs come from the seeded generator; both sides read the same bits. Every
case here is compared element by element; the three large workloads at their
full size are in test_gpu_full_size.py.
"""

from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
import parity
from inputs import backward_inputs, oracle_stats
from rmsnorm_backward_amd import workloads as W

pytestmark = pytest.mark.gpu
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def nb():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import rmsnorm_backward_amd as nbmod
    nbmod.load_library()
    return nbmod


def to_gpu(inp):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) and k != "outliers" else v)
            for k, v in inp.items()}


def run(nb, w, g, *, dbeta=None, groups=0, wgrad=None, stream=None, plan=None):
    """Run the library on GPU tensors g; returns CPU (dx, dgamma, dbeta)."""
    with_db = (w.kind == "layernorm") if dbeta is None else dbeta
    wg = wgrad or w.wgrad_dtype
    if plan is None and groups:
        plan = nb.norm_bwd_make_plan(w.kind, w.M, w.N, w.io_dtype, with_db, groups)
    if plan is not None:
        out = nb.norm_bwd_execute(plan, g["x"], g["dy"], g["gamma"], g.get("mean"), g["rstd"],
                                  wgrad_dtype=wg, stream=stream)
    elif w.kind == "layernorm":
        out = nb.norm_bwd_layernorm(g["x"], g["dy"], g["gamma"], g["mean"], g["rstd"], w.eps,
                                    wgrad_dtype=wg, with_dbeta=with_db, stream=stream)
    else:
        out = nb.norm_bwd_rmsnorm(g["x"], g["dy"], g["gamma"], g["rstd"], w.eps,
                                  wgrad_dtype=wg, with_dbeta=with_db, stream=stream)
    torch.cuda.synchronize()
    return tuple(None if t is None else t.cpu() for t in out)


def compare_full(w, inp, out, with_db, groups=None, aligned=True, coef32=0.0):
    """Every element of dx, dgamma (and dbeta) against the oracle. `groups`
    and `aligned` describe the run (for the weight gradients' summation
    depth); `coef32` is passed only for a named ill-conditioned fp32 case."""
    dx, dg, db = out
    rdx, rdg, rdb = oracle.bwd(w.kind, inp["x"], inp["dy"], inp["gamma"], inp.get("mean"),
                               inp["rstd"], want_dbeta=True)
    scale = parity.dx_term_scale(w.kind, inp["x"], inp["dy"], inp["gamma"], inp.get("mean"),
                                 inp["rstd"])
    depth = parity.depth_path(w.M, w.N, w.io_dtype, with_db, groups, aligned)
    bg, bb = parity.wgrad_bounds(w.kind, inp["x"], inp["dy"], inp.get("mean"), inp["rstd"],
                                 depth)
    stats = {"dx": parity.check_dx(w.io_dtype, dx, rdx, scale=scale, coef32=coef32),
             "dgamma": parity.check_wgrad(w.io_dtype, dg, rdg, **bg)}
    if with_db:
        stats["dbeta"] = parity.check_wgrad(w.io_dtype, db, rdb, "dbeta", **bb)
    return stats


# ----------------------------------------------------------------------------
# The five workloads at sizes the oracle finishes in seconds, spanning many
# row groups and a ragged last group (and the first two at their full size).
SMALL = [
    W.LN_F32_128x512,
    W.RMS_F32_128x512,
    W.LN_F16_1151x8192,
    W.scaled(W.RMS_BF16_16384x4096, M=2003),
    W.scaled(W.LN_BF16_65536x8192, M=777),
    W.scaled(W.RMS_BF16_262144x768, M=5001),
    W.scaled(W.RMS_BF16_262144x768, M=3001, name="rmsnorm_bf16_3001x768_entry_outliers",
             outlier_mode="entries"),
    W.scaled(W.LN_F16_1151x8192, M=257, N=8192, name="layernorm_f16_phobos_like",
             x_dist="normal"),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_workload_parity(nb, w):
    inp = backward_inputs(w)
    with_db = w.kind == "layernorm"
    out = run(nb, w, to_gpu(inp))
    s = compare_full(w, inp, out, with_db)
    print(w.name, s)


def test_phobos_check_distribution(nb):
    """The Phobos tutorial's own inputs: x = -2.3 + 0.5*N(0,1), dy = 0.1*N(0,1),
    gamma, beta ~ U(0,1), fp16, 1151 x 8192 ("05: Layer norm", its check)."""
    g = torch.Generator().manual_seed(0)
    M, N, eps = 1151, 8192, 1e-5
    gamma = torch.rand(N, generator=g).half()
    x = (-2.3 + 0.5 * torch.randn(M, N, generator=g)).half()
    dy = (0.1 * torch.randn(M, N, generator=g)).half()
    mean, rstd = oracle_stats(x, "layernorm", eps)
    inp = {"x": x, "dy": dy, "gamma": gamma, "mean": mean, "rstd": rstd}
    w = W.scaled(W.LN_F16_1151x8192, name="phobos_check")
    out = run(nb, w, to_gpu(inp))
    compare_full(w, inp, out, True)


# ----------------------------------------------------------------------------
# Edge shapes: ragged N (vector and scalar paths), tiny and maximal rows.
EDGE_N = {
    torch.float32: [1, 3, 4, 8, 63, 64, 65, 255, 256, 257, 1000, 1024, 4100, 8191, 16384],
    torch.float16: [1, 2, 8, 63, 64, 65, 512, 513, 768, 1000, 4096, 4100, 8191, 8192, 32768],
    torch.bfloat16: [1, 7, 8, 16, 63, 64, 65, 520, 768, 2048, 4096, 6144, 8192, 16384, 32768],
}
EDGE_M = [1, 2, 3, 511, 513]


def _edge_cases():
    out = []
    for dt, ns in EDGE_N.items():
        for i, n in enumerate(ns):
            for kind in ("layernorm", "rmsnorm"):
                m = EDGE_M[(i + (kind == "rmsnorm")) % len(EDGE_M)]
                if n >= 16384:
                    m = min(m, 64)
                out.append((kind, dt, m, n))
    return out


@pytest.mark.parametrize("kind,dt,M,N", _edge_cases(),
                         ids=lambda v: str(v).replace("torch.", ""))
def test_edge_shapes(nb, kind, dt, M, N):
    base = W.LN_F32_128x512 if kind == "layernorm" else W.RMS_F32_128x512
    w = W.scaled(base, M=M, N=N, io_dtype=dt, wgrad_dtype=torch.float32, seed=99 + M + N)
    inp = backward_inputs(w)
    # N = 1: RMSNorm dx = eps * rstd^3 * dyhat is what is left of two terms
    # that cancel, and LayerNorm dx = 0 is formed as the difference of two
    # rounded products; fp32 then needs the arithmetic term (parity.py).
    coef32 = 2.0 ** -18 if N == 1 else 0.0
    for with_db in (True, False):
        # half rows wider than 16384 with dbeta take the wide-row path
        out = run(nb, w, to_gpu(inp), dbeta=with_db)
        compare_full(w, inp, out, with_db, coef32=coef32)
        if not with_db:
            assert out[2] is None


@pytest.mark.parametrize("groups", [1, 2, 7, 100, 999, 1000])
def test_explicit_groups(nb, groups):
    w = W.scaled(W.LN_BF16_65536x8192, M=1000, N=1536)
    inp = backward_inputs(w)
    out = run(nb, w, to_gpu(inp), groups=groups)
    compare_full(w, inp, out, True, groups=groups)


@pytest.mark.parametrize("kind,dt,M,N,groups", [
    ("layernorm", torch.bfloat16, 777, 8192, 2),     # both gradients, 8 waves a row
    ("rmsnorm", torch.bfloat16, 2003, 4096, 3),      # ragged last group
    ("layernorm", torch.float16, 600, 4096, 1),
    ("rmsnorm", torch.float32, 515, 2048, 1),
])
def test_general_loop_two_rows_in_flight(nb, kind, dt, M, N, groups):
    """Groups that sweep more than 2 MiB of each operand run kernel A's general
    loop with two rows in flight, combined one accumulator at a time."""
    base = W.LN_BF16_65536x8192 if kind == "layernorm" else W.RMS_BF16_16384x4096
    w = W.scaled(base, M=M, N=N, io_dtype=dt)
    with_db = kind == "layernorm"
    p = nb.norm_bwd_make_plan(kind, M, N, dt, with_db, groups)
    eb = torch.tensor([], dtype=dt).element_size()
    # one row in flight by the row-size rule; two for the group size
    assert p.rows_in_flight == 2 and 2 * N * eb >= 16384 and p.rows_per_group * N * eb > 2 << 20
    inp = backward_inputs(w)
    g = to_gpu(inp)
    out = run(nb, w, g, plan=p)
    compare_full(w, inp, out, with_db, groups=groups)
    # one row in flight: each row's sums keep their order, so dx is the same
    # bit for bit; only the order of the group sums (dgamma, dbeta) changes
    q = p.copy()
    q.rows_in_flight, q.threads, q.lds_bytes = 1, 64 * p.waves_per_row, 0
    one = run(nb, w, g, plan=q)
    assert torch.equal(one[0], out[0])
    compare_full(w, inp, one, with_db, groups=groups)


@pytest.mark.parametrize("kind,dt,M,N,groups", [
    ("rmsnorm", torch.bfloat16, 1001, 5120, 0),
    ("layernorm", torch.bfloat16, 777, 5120, 0),
    ("rmsnorm", torch.float16, 513, 3072, 0),
    ("layernorm", torch.bfloat16, 300, 7168, 0),
    ("rmsnorm", torch.bfloat16, 257, 12288, 0),
    ("layernorm", torch.float32, 301, 5120, 0),
    ("rmsnorm", torch.float32, 333, 1536, 0),
    ("layernorm", torch.float16, 1000, 6144, 0),
    ("layernorm", torch.bfloat16, 601, 5120, 2),   # general loop, two rows in flight
    # 16-byte lanes, one chunk: 3, 5, 7, 9 waves per row
    ("rmsnorm", torch.bfloat16, 2001, 1536, 0),
    ("rmsnorm", torch.float16, 1001, 2560, 0),
    ("layernorm", torch.bfloat16, 777, 2560, 0),
    ("rmsnorm", torch.bfloat16, 1001, 3584, 0),
    ("layernorm", torch.float16, 513, 3584, 0),
    ("rmsnorm", torch.bfloat16, 300, 4608, 0),
    ("layernorm", torch.float32, 701, 1280, 0),
    ("rmsnorm", torch.bfloat16, 1201, 3584, 2),    # general loop, two rows in flight
])
def test_exact_non_power_of_two_waves(nb, kind, dt, M, N, groups):
    """Widths that waves of 32-byte (or, failing that, 16-byte) lanes cover
    exactly run 3 to 12 waves per row: the row exchange sums that many wave
    partials in order, and the results match the oracle."""
    base = W.LN_BF16_65536x8192 if kind == "layernorm" else W.RMS_BF16_16384x4096
    w = W.scaled(base, M=M, N=N, io_dtype=dt)
    with_db = kind == "layernorm"
    p = nb.norm_bwd_make_plan(kind, M, N, dt, with_db, groups)
    S = p.waves_per_row
    assert S & (S - 1) != 0 and S * 64 * p.vec * p.chunks == N
    inp = backward_inputs(w)
    out = run(nb, w, to_gpu(inp), plan=p if groups else None)
    compare_full(w, inp, out, with_db, groups=groups or None)


@pytest.mark.parametrize("kind", ["layernorm", "rmsnorm"])
@pytest.mark.parametrize("dt", [torch.float16, torch.bfloat16])
def test_wgrad_in_io_dtype(nb, kind, dt):
    base = W.LN_F16_1151x8192 if kind == "layernorm" else W.RMS_BF16_16384x4096
    w = W.scaled(base, M=300, N=2048, io_dtype=dt, wgrad_dtype=dt)
    inp = backward_inputs(w)
    out = run(nb, w, to_gpu(inp), dbeta=True)
    assert out[1].dtype == dt and out[2].dtype == dt
    compare_full(w, inp, out, True)


def test_geometry_variants_agree(nb):
    """Edited plans (waves per row, rows in flight, chunks) stay in tolerance,
    and dgamma bits do not depend on the lane layout when the row grouping is
    unchanged (only the in-row sums, i.e. dx, may differ in the last bit)."""
    w = W.scaled(W.RMS_BF16_16384x4096, M=1500, N=4096)
    inp = backward_inputs(w)
    g = to_gpu(inp)
    base = nb.norm_bwd_make_plan("rmsnorm", w.M, w.N, torch.bfloat16, False)
    ref = None
    for S, C, P in ((1, 8, 4), (1, 8, 2), (2, 4, 2), (2, 4, 4), (4, 2, 1), (4, 2, 2), (8, 1, 1),
                    (2, 4, 8), (4, 2, 4)):
        p = base.copy()
        p.waves_per_row, p.chunks, p.rows_in_flight = S, C, P
        p.threads = 64 * S * P
        p.lds_bytes = S * C * 64 * p.vec * 4 if P > 1 else 0
        if p.threads > (512 if p.vec * C > 16 else 1024):
            continue
        out = run(nb, w, g, plan=p)
        compare_full(w, inp, out, False)
        if P == base.rows_in_flight:
            if ref is None:
                ref = out[1]
            assert torch.equal(out[1], ref), (S, C, P)


def test_streamed_and_cached_partials_agree(nb):
    """Workspaces of 12 MiB and more are written and read back with
    non-temporal accesses, smaller ones with cached accesses; the values are
    the same. 1151x8192 LayerNorm at 256 groups has 16 MiB of partials with
    dbeta (streamed) and 8 MiB without (cached): dx and dgamma are bitwise
    equal, and both runs stay within tolerance of the oracle."""
    w = W.LN_F16_1151x8192
    inp = backward_inputs(w)
    g = to_gpu(inp)
    with_db = run(nb, w, g, dbeta=True, groups=256)
    without = run(nb, w, g, dbeta=False, groups=256)
    assert nb.norm_bwd_make_plan(w.kind, w.M, w.N, w.io_dtype, True, 256).workspace_bytes == 16 << 20
    assert nb.norm_bwd_make_plan(w.kind, w.M, w.N, w.io_dtype, False, 256).workspace_bytes == 8 << 20
    assert torch.equal(with_db[0], without[0])
    assert torch.equal(with_db[1], without[1])
    compare_full(w, inp, with_db, True, groups=256)
    compare_full(w, inp, without, False, groups=256)


def test_determinism_repeats_and_perturbation(nb):
    w = W.scaled(W.LN_BF16_65536x8192, M=4099, N=4096)
    g = to_gpu(backward_inputs(w))
    first = run(nb, w, g)
    side = torch.cuda.Stream()
    junk = torch.randn(4096, 4096, device="cuda")
    for i in range(20):
        if i % 2:
            with torch.cuda.stream(side):     # concurrent work perturbs scheduling
                junk = junk @ junk
                junk = junk / junk.abs().max()
        out = run(nb, w, g)
        for a, b, name in zip(out, first, ("dx", "dgamma", "dbeta")):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), \
                f"{name} changed on repeat {i}"
    torch.cuda.synchronize()


def test_nan_poisoned_outputs_and_workspace(nb):
    """Prior contents of dx, dgamma, dbeta and the workspace are never read."""
    w = W.scaled(W.LN_BF16_65536x8192, M=999, N=768)
    inp = backward_inputs(w)
    g = to_gpu(inp)
    clean = run(nb, w, g)
    need = nb.norm_bwd_workspace_bytes("layernorm", w.M, w.N, w.io_dtype, True)
    ws = torch.full((need // 4,), float("nan"), device="cuda")
    dx = torch.full((w.M, w.N), float("nan"), dtype=w.io_dtype, device="cuda")
    dg = torch.full((w.N,), float("nan"), device="cuda")
    db = torch.full((w.N,), float("nan"), device="cuda")
    nb.norm_bwd_layernorm(g["x"], g["dy"], g["gamma"], g["mean"], g["rstd"], w.eps,
                          dx=dx, dgamma=dg, dbeta=db, workspace=ws)
    torch.cuda.synchronize()
    for a, b in zip((dx.cpu(), dg.cpu(), db.cpu()), clean):
        assert torch.equal(a, b)


def test_guard_bands_untouched(nb):
    """Outputs and workspace carved out of larger buffers: the bytes around
    them keep their canary values (no out-of-bounds writes)."""
    w = W.scaled(W.RMS_BF16_262144x768, M=1031, N=1000)   # ragged N, vector path
    inp = backward_inputs(w)
    g = to_gpu(inp)
    pad = 4096
    canary = -1536.0   # exact in bf16, fp16 and fp32
    n_dx = w.M * w.N
    dx_buf = torch.full((n_dx + 2 * pad,), canary, dtype=w.io_dtype, device="cuda")
    dg_buf = torch.full((w.N + 2 * pad,), canary, device="cuda")
    db_buf = torch.full((w.N + 2 * pad,), canary, device="cuda")
    need = nb.norm_bwd_workspace_bytes("rmsnorm", w.M, w.N, w.io_dtype, True)
    ws_buf = torch.full((need // 4 + 2 * pad,), canary, device="cuda")
    dx = dx_buf[pad:pad + n_dx].view(w.M, w.N)
    dg, db = dg_buf[pad:pad + w.N], db_buf[pad:pad + w.N]
    ws = ws_buf[pad:pad + need // 4]
    nb.norm_bwd_rmsnorm(g["x"], g["dy"], g["gamma"], g["rstd"], w.eps, dx=dx, dgamma=dg,
                        dbeta=db, workspace=ws)
    torch.cuda.synchronize()
    for buf, n in ((dx_buf, n_dx), (dg_buf, w.N), (db_buf, w.N), (ws_buf, need // 4)):
        c = buf.float().cpu()
        assert torch.all(c[:pad] == canary) and torch.all(c[pad + n:] == canary)
    compare_full(w, inp, (dx.cpu(), dg.cpu(), db.cpu()), True)


def test_misaligned_rows_take_the_scalar_path(nb):
    """Tensors offset by one element (not 16-byte aligned) still give the
    right answer (the automatic plan falls back to one element per lane)."""
    w = W.scaled(W.RMS_BF16_16384x4096, M=130, N=1024)
    inp = backward_inputs(w)
    def off(t):
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device="cuda")
        v = buf[1:].view(t.shape)
        v.copy_(t.cuda())
        return v
    g = {"x": off(inp["x"]), "dy": off(inp["dy"]), "gamma": off(inp["gamma"]),
         "rstd": inp["rstd"].cuda()}
    out = run(nb, w, g)
    compare_full(w, inp, out, False, aligned=False)


def test_stream_semantics(nb):
    w = W.scaled(W.RMS_BF16_16384x4096, M=512, N=4096)
    inp = backward_inputs(w)
    g = to_gpu(inp)
    ref = run(nb, w, g)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out = nb.norm_bwd_rmsnorm(g["x"], g["dy"], g["gamma"], g["rstd"], w.eps)
        ev = torch.cuda.Event()
        ev.record(s)
    ev.synchronize()
    for a, b in zip(out, ref):
        if b is not None:
            assert torch.equal(a.cpu(), b)


def test_concurrent_streams_do_not_interfere(nb):
    """Calls on separate streams, each with its own outputs and workspace,
    may run at the same time: four different problems issued back to back on
    four streams (default priority), several times over, give bitwise the
    results each gives alone."""
    cases = [W.scaled(W.RMS_BF16_16384x4096, M=2000, N=4096),
             W.scaled(W.LN_F16_1151x8192, M=700),
             W.scaled(W.LN_BF16_65536x8192, M=300, N=24576),      # wide rows
             W.scaled(W.RMS_F32_128x512, M=3000, N=768)]
    prepared = []
    for w in cases:
        inp = backward_inputs(w)
        g = to_gpu(inp)
        prepared.append((w, g, run(nb, w, g)))
    streams = [torch.cuda.Stream() for _ in cases]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = []
    for rep in range(3):
        for (w, g, _), s in zip(prepared, streams):
            with torch.cuda.stream(s):
                if w.kind == "layernorm":
                    o = nb.norm_bwd_layernorm(g["x"], g["dy"], g["gamma"], g["mean"], g["rstd"],
                                              w.eps, wgrad_dtype=w.wgrad_dtype)
                else:
                    o = nb.norm_bwd_rmsnorm(g["x"], g["dy"], g["gamma"], g["rstd"], w.eps,
                                            wgrad_dtype=w.wgrad_dtype)
                outs.append((rep, w, o))
    torch.cuda.synchronize()
    for rep, w, o in outs:
        ref = next(r for (ww, _, r) in prepared if ww is w)
        for a, b in zip(o, ref):
            if b is not None:
                assert torch.equal(a.cpu(), b), (w.name, rep)


def test_two_phase_api_matches_full_call(nb):
    w = W.scaled(W.LN_BF16_65536x8192, M=2048, N=2048)
    g = to_gpu(backward_inputs(w))
    full = run(nb, w, g)
    plan = nb.norm_bwd_make_plan("layernorm", w.M, w.N, w.io_dtype, True)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
    dx = torch.empty_like(g["x"])
    nb.norm_bwd_execute_partials(plan, g["x"], g["dy"], g["gamma"], g["mean"], g["rstd"], dx, ws)
    dg = torch.empty(w.N, device="cuda")
    db = torch.empty(w.N, device="cuda")
    nb.norm_bwd_reduce_partials(plan.groups, w.N, ws, dg, db)
    torch.cuda.synchronize()
    assert torch.equal(dx.cpu(), full[0])
    assert torch.equal(dg.cpu(), full[1]) and torch.equal(db.cpu(), full[2])


@pytest.mark.parametrize("wdt", [torch.float16, torch.bfloat16, torch.float32])
def test_two_phase_reduce_output_dtypes(nb, wdt):
    """Kernel B alone rounds the same fp32 sums to any output type."""
    w = W.scaled(W.LN_F16_1151x8192, M=333, N=1000)
    g = to_gpu(backward_inputs(w))
    plan = nb.norm_bwd_make_plan("layernorm", w.M, w.N, w.io_dtype, True)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
    dx = torch.empty_like(g["x"])
    nb.norm_bwd_execute_partials(plan, g["x"], g["dy"], g["gamma"], g["mean"], g["rstd"], dx, ws)
    ref_g = torch.empty(w.N, device="cuda")
    ref_b = torch.empty(w.N, device="cuda")
    nb.norm_bwd_reduce_partials(plan.groups, w.N, ws, ref_g, ref_b)
    dg = torch.empty(w.N, dtype=wdt, device="cuda")
    db = torch.empty(w.N, dtype=wdt, device="cuda")
    nb.norm_bwd_reduce_partials(plan.groups, w.N, ws, dg, db)
    torch.cuda.synchronize()
    assert torch.equal(dg.cpu(), ref_g.cpu().to(wdt)) and torch.equal(db.cpu(), ref_b.cpu().to(wdt))


def test_empty_problems(nb):
    for kind in ("layernorm", "rmsnorm"):
        x = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
        st = torch.empty(0, device="cuda")
        dg = torch.full((64,), float("nan"), device="cuda")
        db = torch.full((64,), float("nan"), device="cuda")
        gam = torch.ones(64, dtype=torch.bfloat16, device="cuda")
        if kind == "layernorm":
            nb.norm_bwd_layernorm(x, x, gam, st, st, dgamma=dg, dbeta=db)
        else:
            nb.norm_bwd_rmsnorm(x, x, gam, st, dgamma=dg, dbeta=db)
        torch.cuda.synchronize()
        assert torch.all(dg == 0) and torch.all(db == 0)      # the empty sum
        x0 = torch.empty(5, 0, dtype=torch.bfloat16, device="cuda")
        st5 = torch.ones(5, device="cuda")
        g0 = torch.empty(0, dtype=torch.bfloat16, device="cuda")
        if kind == "layernorm":
            out = nb.norm_bwd_layernorm(x0, x0, g0, st5, st5)
        else:
            out = nb.norm_bwd_rmsnorm(x0, x0, g0, st5)
        torch.cuda.synchronize()
        assert out[0].shape == (5, 0) and out[1].shape == (0,)


def test_rejects_bad_tensors_before_launch(nb):
    w = W.scaled(W.RMS_BF16_16384x4096, M=64, N=256)
    g = to_gpu(backward_inputs(w))
    small_ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(nb.NormBwdError) as e:
        nb.norm_bwd_rmsnorm(g["x"], g["dy"], g["gamma"], g["rstd"], workspace=small_ws)
    assert e.value.status == nb.ERR_WORKSPACE
    with pytest.raises(nb.NormBwdError) as e:
        nb.norm_bwd_rmsnorm(g["x"], g["dy"], g["gamma"], g["rstd"], dx=g["x"])
    assert e.value.status == nb.ERR_INVALID_ARG
    with pytest.raises(nb.NormBwdError) as e:
        nb.norm_bwd_rmsnorm(g["x"], g["dy"], g["gamma"], g["rstd"], eps=-1.0)
    assert e.value.status == nb.ERR_INVALID_ARG
    with pytest.raises(ValueError):
        nb.norm_bwd_rmsnorm(g["x"], g["dy"].float(), g["gamma"], g["rstd"])


@pytest.mark.parametrize("n16,grid,unroll", [(1 << 16, 0, 4), (1 << 16, 7, 8), (12345, 3, 2),
                                              (1000, 1, 1), (257, 0, 8), (4097, 2, 4)])
def test_triad_probe(nb, n16, grid, unroll):
    """The streaming-ceiling probe computes c = a + b on 32-bit words over
    exactly n16 16-byte vectors, for any grid and unroll (ragged tails
    included), and writes nothing past c's end."""
    g = torch.Generator(device="cuda").manual_seed(n16)
    a = torch.randint(0, 1 << 30, (4 * n16,), dtype=torch.int32, device="cuda", generator=g)
    b = torch.randint(0, 1 << 30, (4 * n16,), dtype=torch.int32, device="cuda", generator=g)
    cbuf = torch.full((4 * n16 + 64,), -7, dtype=torch.int32, device="cuda")
    c = cbuf[:4 * n16]
    nb.norm_bwd_probe_triad(a, b, c, grid, unroll)
    torch.cuda.synchronize()
    assert torch.equal(c, a + b)
    assert torch.all(cbuf[4 * n16:] == -7)


@pytest.mark.parametrize("unroll", [1, 2, 4])
def test_triad_policy_probe(nb, unroll):
    """The cache-policy triad computes c = a + b on 32-bit words under every
    load and store policy, and writes nothing past c's end."""
    n = 4096 * unroll * 5 // 4          # 32-bit words: 5 workgroups
    g = torch.Generator(device="cuda").manual_seed(unroll)
    a = torch.randint(0, 1 << 30, (n,), dtype=torch.int32, device="cuda", generator=g)
    b = torch.randint(0, 1 << 30, (n,), dtype=torch.int32, device="cuda", generator=g)
    for lp in nb.POLICIES:
        for sp in nb.POLICIES:
            cbuf = torch.full((n + 1024,), -7, dtype=torch.int32, device="cuda")
            nb.norm_bwd_probe_triad_policy(a, b, cbuf[:n], unroll, lp, sp)
            torch.cuda.synchronize()
            assert torch.equal(cbuf[:n], a + b), (lp, sp)
            assert torch.all(cbuf[n:] == -7), (lp, sp)


def test_copy_probe(nb):
    src = torch.randint(0, 1 << 30, (1 << 20,), dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    nb.norm_bwd_probe_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def test_offsets_beyond_2gib(nb):
    """x, dy and dx of 2^20 + 3 rows x 1024 bf16 (just over 2 GiB each): rows
    near the end sit past byte offset 2^31, so every kernel's address
    arithmetic must be 64-bit. Inputs are drawn on the GPU from a seeded
    generator; sampled rows and columns go to the oracle."""
    M, N, eps = (1 << 20) + 3, 1024, 1e-6
    gen = torch.Generator(device="cuda").manual_seed(2024)
    x = torch.randn(M, N, generator=gen, device="cuda").to(torch.bfloat16)
    dy = (torch.randn(M, N, generator=gen, device="cuda") * 1e-2).to(torch.bfloat16)
    gamma = (torch.rand(N, generator=gen, device="cuda") + 0.5).to(torch.bfloat16)
    assert (M - 1) * N * 2 > (1 << 31)
    y, rstd = nb.norm_fwd_rmsnorm(x, gamma, eps)
    dx, dg, _ = nb.norm_bwd_rmsnorm(x, dy, gamma, rstd, eps)
    cg, _ = nb.norm_bwd_wgrad("rmsnorm", x, dy, None, rstd)
    torch.cuda.synchronize()
    rows = torch.tensor([0, 1, M // 2, (1 << 20) - 1, 1 << 20, M - 2, M - 1])
    xr, dyr, gc = x[rows].cpu(), dy[rows].cpu(), gamma.cpu()
    ry, _, rr = oracle.fwd("rmsnorm", xr, gc, None, eps)
    parity.check_forward(torch.bfloat16, "rmsnorm", xr, gc, None, y[rows].cpu(), None,
                         rstd[rows].cpu(), ry, None, rr)
    rs = rstd[rows].cpu()
    rdx = oracle.bwd_dx("rmsnorm", xr, dyr, gc, None, rs)
    parity.check_dx(torch.bfloat16, dx[rows].cpu(),
                    rdx, scale=parity.dx_term_scale("rmsnorm", xr, dyr, gc, None, rs))
    cols = torch.tensor([0, 5, 511, 1023])
    xc, dyc = x[:, cols].cpu(), dy[:, cols].cpu()
    rdg, _ = oracle.bwd_wgrad("rmsnorm", xc, dyc, None, rstd.cpu(), want_dbeta=False)
    ag, _ = parity.abs_terms("rmsnorm", xc, dyc, None, rstd.cpu())
    parity.check_wgrad(torch.bfloat16, dg[cols].cpu(), rdg, absum=ag,
                       depth=parity.depth_fused(M))
    parity.check_wgrad(torch.bfloat16, cg[cols].cpu(), rdg, absum=ag,
                       depth=parity.depth_colwalk(M))
    del x, dy, dx, y
    torch.cuda.empty_cache()
