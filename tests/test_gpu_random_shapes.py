"""Seeded sweeps of random problem shapes against the oracle: the backward,
the forward and the column walk.

The targeted parity tests pick their shapes; this sweep draws them: kind,
I/O dtype, N (biased towards widths around vector, chunk and path limits,
but also arbitrary), M (including 1 and a few rows), dbeta on or off, saved
or recomputed statistics, contiguous or row-strided storage, and the
weight-gradient dtype; strided cases also draw accumulation into existing
fp32 weight gradients and explicit group counts. Every case runs through the
public entry points (norm_bwd_layernorm / norm_bwd_rmsnorm, or norm_bwd_ex
for strides) and is
compared with the fp64 oracle under the same tolerances as the other parity
tests. The draw is fixed, so a failure names a reproducible case. The forward
(beta on or off, statistics requested or not) and norm_bwd_wgrad
(accumulating or not) get sweeps of their own, and the widths of the
two-rows-per-wave layout a backward and a forward sweep of their own.
"""

from __future__ import annotations

import random

import pytest
import torch

import oracle
import parity
from inputs import backward_inputs
from rmsnorm_backward_amd import workloads as W

pytestmark = pytest.mark.gpu

DTYPES = (torch.float32, torch.float16, torch.bfloat16)
EDGE_N = [1, 2, 3, 7, 8, 9, 15, 16, 17, 63, 64, 65, 255, 256, 257, 511, 512, 768, 1000, 1023,
          1024, 1025, 2047, 2048, 4095, 4096, 4097, 8191, 8192, 8193, 16383, 16384, 16385,
          20000, 32767, 32768, 32769]


def _cases(n=200, seed=20261202):
    rng = random.Random(seed)
    out = []
    for i in range(n):
        kind = rng.choice(("layernorm", "rmsnorm"))
        dt = rng.choice(DTYPES)
        N = rng.choice(EDGE_N) if rng.random() < 0.7 else rng.randint(1, 40000)
        if dt == torch.float32:
            N = min(N, 24000)
        M = rng.choice((1, 2, 3, 5, 17)) if rng.random() < 0.3 else rng.randint(1, 300)
        M = max(1, min(M, 2_000_000 // max(N, 1)))     # keep the fp64 oracle quick
        with_db = kind == "layernorm" if rng.random() < 0.6 else rng.random() < 0.5
        recompute = rng.random() < 0.3
        pad = rng.choice((0, 0, 0, 8, 24, 5))        # row padding in elements (0 = contiguous)
        wg = torch.float32 if rng.random() < 0.75 else dt
        # norm_bwd_ex only (pad > 0): accumulate into fp32 buffers, groups
        acc = pad > 0 and rng.random() < 0.3
        groups = rng.choice((1, 2, 7, 64, 300, 1000)) if pad > 0 and rng.random() < 0.3 else 0
        out.append((i, kind, dt, M, N, with_db, recompute, pad, wg, acc, groups))
    return out


def _long_group_cases(n=40, seed=20261203):
    """Explicit group counts (1 to 3) with enough rows that every group
    sweeps more than 2 MiB of each operand: kernel A's general loop, where
    the planner keeps two rows in flight; the last group is ragged."""
    rng = random.Random(seed)
    out = []
    for i in range(n):
        kind = rng.choice(("layernorm", "rmsnorm"))
        dt = rng.choice(DTYPES)
        eb = 4 if dt == torch.float32 else 2
        N = rng.choice((512, 768, 1000, 1024, 2048, 3000, 4096, 4100, 8192))
        groups = rng.choice((1, 1, 2, 3))
        need = (2 << 20) // (N * eb) + 1              # rows per group beyond 2 MiB
        M = groups * need + rng.randint(0, need - 1)
        with_db = kind == "layernorm" if rng.random() < 0.6 else rng.random() < 0.5
        recompute = rng.random() < 0.25
        pad = rng.choice((0, 0, 8, 24, 5))
        wg = torch.float32 if rng.random() < 0.75 else dt
        acc = rng.random() < 0.2
        out.append((1000 + i, kind, dt, M, N, with_db, recompute, pad, wg, acc, groups))
    return out


def _two_row_cases(n=48, seed=20261204):
    """Widths of the two-rows-per-wave layout (32 lanes of 16-byte vectors:
    256 or 768 16-bit elements, 128 or 384 fp32), saved or recomputed
    statistics, odd and even M up to sizes where groups run the steady-state
    loop, strides and explicit groups."""
    rng = random.Random(seed)
    out = []
    for i in range(n):
        kind = rng.choice(("layernorm", "rmsnorm"))
        dt = rng.choice(DTYPES)
        N = rng.choice((128, 384) if dt == torch.float32 else (256, 768))
        M = rng.choice((1, 2, 3, 511, 513)) if rng.random() < 0.3 else rng.randint(1, 12000)
        with_db = kind == "layernorm" if rng.random() < 0.6 else rng.random() < 0.5
        recompute = rng.random() < 0.5
        pad = rng.choice((0, 0, 0, 8, 24))
        wg = torch.float32 if rng.random() < 0.75 else dt
        acc = pad > 0 and rng.random() < 0.3
        groups = rng.choice((1, 3, 64, 1000)) if pad > 0 and rng.random() < 0.4 else 0
        out.append((2000 + i, kind, dt, M, N, with_db, recompute, pad, wg, acc, groups))
    return out


def _strided(t, pad):
    M, N = t.shape
    buf = torch.zeros(M * (N + pad), dtype=t.dtype, device="cuda")
    v = buf.view(M, N + pad)[:, :N]
    v.copy_(t.cuda())
    return v


@pytest.fixture(scope="module")
def nb():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import rmsnorm_backward_amd as nbmod
    nbmod.load_library()
    return nbmod


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "-".join(str(v).replace("torch.", "")
                                                                   for v in c))
def test_random_shape(nb, case):
    _run_backward_case(nb, case)


@pytest.mark.parametrize("case", _long_group_cases(),
                         ids=lambda c: "-".join(str(v).replace("torch.", "") for v in c))
def test_random_long_groups(nb, case):
    _run_backward_case(nb, case)


@pytest.mark.parametrize("case", _two_row_cases(),
                         ids=lambda c: "-".join(str(v).replace("torch.", "") for v in c))
def test_random_two_row_widths(nb, case):
    _run_backward_case(nb, case)


def _run_backward_case(nb, case):
    """One drawn case through the public entry points (norm_bwd_ex when rows
    are strided or groups are explicit), compared with the oracle."""
    i, kind, dt, M, N, with_db, recompute, pad, wg, acc, groups = case
    if acc:
        wg = torch.float32
    if N > 8192:
        # explicit groups are for rows the fused path holds at any row
        # alignment (NORM_BWD_MAX_N_UNALIGNED); wider ones are UNSUPPORTED
        groups = 0
    base = W.LN_F32_128x512 if kind == "layernorm" else W.RMS_F32_128x512
    w = W.scaled(base, M=M, N=N, io_dtype=dt, wgrad_dtype=wg, seed=9000 + i)
    inp = backward_inputs(w)
    use_ex = pad > 0 or groups > 0 or acc
    x = _strided(inp["x"], pad) if use_ex else inp["x"].cuda()
    dy = _strided(inp["dy"], pad) if use_ex else inp["dy"].cuda()
    g = inp["gamma"].cuda()
    mean = None if (recompute or kind == "rmsnorm") else inp["mean"].cuda()
    rstd = None if recompute else inp["rstd"].cuda()
    old = torch.randn(N, generator=torch.Generator().manual_seed(i)) if acc else None
    if use_ex:
        dg0 = old.clone().cuda() if acc else None
        db0 = old.clone().cuda() if (acc and with_db) else None
        dx, dg, db = nb.norm_bwd_ex(kind, x, dy, g, mean, rstd, w.eps, wgrad_dtype=wg,
                                    with_dbeta=with_db, dgamma=dg0, dbeta=db0,
                                    accumulate=acc, groups=groups)
    elif kind == "layernorm":
        dx, dg, db = nb.norm_bwd_layernorm(x, dy, g, mean, rstd, w.eps, wgrad_dtype=wg,
                                           with_dbeta=with_db)
    else:
        dx, dg, db = nb.norm_bwd_rmsnorm(x, dy, g, rstd, w.eps, wgrad_dtype=wg,
                                         with_dbeta=with_db)
    torch.cuda.synchronize()
    dx, dg = dx.cpu(), dg.cpu()
    assert (db is not None) == with_db
    if recompute:
        m64, r64 = oracle.fwd_stats(kind, inp["x"], w.eps)          # fp64, not rounded
        rdx = oracle.bwd_dx(kind, inp["x"], inp["dy"], inp["gamma"], m64, r64)
        t_dx, t_dg = parity.recompute_terms(kind, inp["x"], inp["dy"], inp["gamma"], m64, r64)
        parity.check_dx(dt, dx, rdx, scale=t_dx, coef32=2.0 ** -16)
        rdg, rdb = oracle.bwd_wgrad(kind, inp["x"], inp["dy"], m64, r64)
        extra = 2.0 ** -16 * t_dg
    else:
        rdx, rdg, rdb = oracle.bwd(kind, inp["x"], inp["dy"], inp["gamma"], inp.get("mean"),
                                   inp["rstd"])
        scale = parity.dx_term_scale(kind, inp["x"], inp["dy"], inp["gamma"], inp.get("mean"),
                                     inp["rstd"])
        # N = 1, and LayerNorm N = 2 (xhat = +-1, so dx is 0 in exact
        # arithmetic): the named ill-conditioned fp32 cases (parity.py)
        ill = N == 1 or (kind == "layernorm" and N == 2)
        parity.check_dx(dt, dx, rdx, scale=scale, coef32=2.0 ** -18 if ill else 0.0)
        extra = None
    # passed in their own dtype, the weight gradients' output rounding is
    # part of the bound; accumulated ones are compared as (new - old), with
    # the fp32 rounding of old + sum
    assert dg.dtype == wg
    # summation depth: the fused kernels' (explicit or automatic groups), or
    # the column walk's for rows wider than every fused limit may be
    depth = parity.depth_fused(M, groups or None)
    if N > 8192:
        depth = max(depth, parity.depth_colwalk(M))
    if recompute:
        bg, bb = parity.wgrad_bounds(kind, inp["x"], inp["dy"], m64, r64, depth)
    else:
        bg, bb = parity.wgrad_bounds(kind, inp["x"], inp["dy"], inp.get("mean"), inp["rstd"],
                                     depth)
    # the named long-sum case for fp32 (parity.fp32_long_sum_extra)
    long_g = parity.fp32_long_sum_extra(dt, bg, rdg)
    long_b = parity.fp32_long_sum_extra(dt, bb, rdb)
    if acc:
        old64 = old.double().abs().numpy()
        a_extra = 2.0 ** -24 * (old64 + abs(parity.f64(rdg)))
        parity.check_wgrad(dt, dg - old, rdg, extra=parity.add_extra(a_extra, extra, long_g),
                           **bg)
        if with_db:
            b_extra = 2.0 ** -24 * (old64 + abs(parity.f64(rdb)))
            parity.check_wgrad(dt, db.cpu() - old, rdb, "dbeta",
                               extra=parity.add_extra(b_extra, long_b), **bb)
    else:
        parity.check_wgrad(dt, dg, rdg, extra=parity.add_extra(extra, long_g), **bg)
        if with_db:
            parity.check_wgrad(dt, db.cpu(), rdb, "dbeta", extra=long_b, **bb)


def _fwd_cases(n=80, seed=1202):
    rng = random.Random(seed)
    out = []
    for i in range(n):
        kind = rng.choice(("layernorm", "rmsnorm"))
        dt = rng.choice(DTYPES)
        N = rng.choice(EDGE_N + [40000, 65536, 65537]) if rng.random() < 0.7 \
            else rng.randint(1, 70000)
        M = rng.choice((1, 2, 3, 7)) if rng.random() < 0.3 else rng.randint(1, 300)
        M = max(1, min(M, 2_000_000 // max(N, 1)))
        beta = kind == "layernorm" and rng.random() < 0.6
        stats = rng.random() < 0.8
        out.append((i, kind, dt, M, N, beta, stats))
    return out


def _fwd_two_row_cases(n=24, seed=1203):
    rng = random.Random(seed)
    out = []
    for i in range(n):
        kind = rng.choice(("layernorm", "rmsnorm"))
        dt = rng.choice(DTYPES)
        N = rng.choice((128, 384) if dt == torch.float32 else (256, 768))
        M = rng.choice((1, 2, 3, 4097)) if rng.random() < 0.3 else rng.randint(1, 20000)
        beta = kind == "layernorm" and rng.random() < 0.6
        stats = rng.random() < 0.8
        out.append((100 + i, kind, dt, M, N, beta, stats))
    return out


@pytest.mark.parametrize("case", _fwd_cases() + _fwd_two_row_cases(), ids=lambda c: "-".join(
    str(v).replace("torch.", "") for v in c))
def test_random_forward(nb, case):
    """y and the statistics of the forward (fused, register-held or streamed
    wide rows) against the oracle's forward."""
    i, kind, dt, M, N, with_beta, stats = case
    base = W.LN_F32_128x512 if kind == "layernorm" else W.RMS_F32_128x512
    w = W.scaled(base, M=M, N=N, io_dtype=dt, seed=7000 + i)
    inp = W.make_inputs(w)
    x, gamma = inp["x"], inp["gamma"]
    beta = None
    if with_beta:
        beta = torch.rand(N, generator=torch.Generator().manual_seed(i)).to(dt)
    if kind == "layernorm":
        y, mean, rstd = nb.norm_fwd_layernorm(x.cuda(), gamma.cuda(),
                                              None if beta is None else beta.cuda(), w.eps,
                                              want_stats=stats)
    else:
        y, rstd = nb.norm_fwd_rmsnorm(x.cuda(), gamma.cuda(), w.eps, want_stats=stats)
        mean = None
    torch.cuda.synchronize()
    ry, rm, rr = oracle.fwd(kind, x, gamma, beta, w.eps)
    if stats:
        parity.check_forward(dt, kind, x, gamma, beta, y.cpu(),
                             None if mean is None else mean.cpu(), rstd.cpu(), ry, rm, rr)
    else:
        assert rstd is None and mean is None
        parity.check_forward(dt, kind, x, gamma, beta, y.cpu(), None, None, ry, rm, rr)


def _wgrad_cases(n=60, seed=2026):
    rng = random.Random(seed)
    out = []
    for i in range(n):
        kind = rng.choice(("layernorm", "rmsnorm"))
        dt = rng.choice(DTYPES)
        N = rng.choice(EDGE_N + [40000, 65537]) if rng.random() < 0.7 else rng.randint(1, 70000)
        M = rng.choice((1, 2, 5)) if rng.random() < 0.3 else rng.randint(1, 400)
        M = max(1, min(M, 2_000_000 // max(N, 1)))
        with_db = rng.random() < 0.5
        acc = rng.random() < 0.3
        wg = torch.float32 if rng.random() < 0.75 else dt
        out.append((i, kind, dt, M, N, with_db, acc, wg))
    return out


@pytest.mark.parametrize("case", _wgrad_cases(), ids=lambda c: "-".join(
    str(v).replace("torch.", "") for v in c))
def test_random_wgrad(nb, case):
    """dgamma/dbeta by the column walk (norm_bwd_wgrad), plain or accumulated
    into an existing fp32 buffer, against the oracle."""
    i, kind, dt, M, N, with_db, acc, wg = case
    if acc:
        wg = torch.float32
    base = W.LN_F32_128x512 if kind == "layernorm" else W.RMS_F32_128x512
    w = W.scaled(base, M=M, N=N, io_dtype=dt, wgrad_dtype=wg, seed=8000 + i)
    inp = backward_inputs(w)
    mean = inp["mean"].cuda() if kind == "layernorm" else None
    old = torch.randn(N, generator=torch.Generator().manual_seed(i)) if acc else None
    dg = old.clone().cuda() if acc else None
    db = old.clone().cuda() if (acc and with_db) else None
    dg, db = nb.norm_bwd_wgrad(kind, inp["x"].cuda(), inp["dy"].cuda(), mean,
                               inp["rstd"].cuda(), wgrad_dtype=wg, dgamma=dg, dbeta=db,
                               with_dbeta=with_db, accumulate=acc)
    torch.cuda.synchronize()
    rdg, rdb = oracle.bwd_wgrad(kind, inp["x"], inp["dy"], inp.get("mean"), inp["rstd"])
    got_g = dg.cpu() - old if acc else dg.cpu()
    extra = 2.0 ** -24 * old.abs() if acc else None
    bg, bb = parity.wgrad_bounds(kind, inp["x"], inp["dy"], inp.get("mean"), inp["rstd"],
                                 parity.depth_colwalk(M))
    parity.check_wgrad(dt, got_g, rdg, extra=extra, **bg)
    assert (db is not None) == with_db
    if with_db:
        got_b = db.cpu() - old if acc else db.cpu()
        parity.check_wgrad(dt, got_b, rdb, "dbeta", extra=extra, **bb)
