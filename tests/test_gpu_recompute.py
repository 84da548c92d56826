"""Recompute mode of the GPU backward (mean/rstd = NULL) against the oracle.

In this mode kernel A computes each row's statistics from x with eps before
the gradient (recomputing sigma on chip instead of reading it: "Norm &
activation backward", "Half one"). The reference is the oracle's backward on
the oracle's fp64 forward statistics of the same x and eps; the tolerance adds
the first-order effect of fp32 statistics (parity.recompute_terms).
"""

from __future__ import annotations

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


def run_recompute(nb, w, x, dy, gamma, with_db, eps=None):
    eps = w.eps if eps is None else eps
    x, dy, gamma = x.cuda(), dy.cuda(), gamma.cuda()
    if w.kind == "layernorm":
        out = nb.norm_bwd_layernorm(x, dy, gamma, None, None, eps, wgrad_dtype=w.wgrad_dtype,
                                    with_dbeta=with_db)
    else:
        out = nb.norm_bwd_rmsnorm(x, dy, gamma, None, eps, wgrad_dtype=w.wgrad_dtype,
                                  with_dbeta=with_db)
    torch.cuda.synchronize()
    return tuple(None if t is None else t.cpu() for t in out)


def compare(w, x, dy, gamma, out, with_db, eps=None, rows=None, cols=None):
    """Check dx on `rows` (all by default) and dgamma/dbeta on `cols`."""
    eps = w.eps if eps is None else eps
    dx, dg, db = out
    mean, rstd = oracle.fwd_stats(w.kind, x, eps)          # fp64, not rounded
    xs, dys = (x, dy) if rows is None else (x[rows], dy[rows])
    ms = None if mean is None else (mean if rows is None else mean[rows.numpy()])
    rs = rstd if rows is None else rstd[rows.numpy()]
    rdx = oracle.bwd_dx(w.kind, xs, dys, gamma, ms, rs)
    t_dx, _ = parity.recompute_terms(w.kind, xs, dys, gamma, ms, rs)
    parity.check_dx(w.io_dtype, dx if rows is None else dx[rows], rdx, scale=t_dx,
                    coef32=2.0 ** -16)
    xc, dyc = (x, dy) if cols is None else (x[:, cols], dy[:, cols])
    rdg, rdb = oracle.bwd_wgrad(w.kind, xc, dyc, mean, rstd, want_dbeta=True)
    _, t_dg = parity.recompute_terms(w.kind, xc, dyc, gamma if cols is None else gamma[cols],
                                     mean, rstd)
    bg, bb = parity.wgrad_bounds(w.kind, xc, dyc, mean, rstd,
                                 parity.depth_path(x.shape[0], x.shape[1], w.io_dtype, with_db))
    parity.check_wgrad(w.io_dtype, dg if cols is None else dg[cols], rdg,
                       extra=2.0 ** -16 * t_dg, **bg)
    if with_db:
        parity.check_wgrad(w.io_dtype, db if cols is None else db[cols], rdb, "dbeta", **bb)


SMALL = [
    W.LN_F32_128x512,
    W.RMS_F32_128x512,
    W.LN_F16_1151x8192,
    W.scaled(W.RMS_BF16_16384x4096, M=2003),
    W.scaled(W.LN_BF16_65536x8192, M=777),
    W.scaled(W.RMS_BF16_262144x768, M=5001),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_recompute_parity(nb, w):
    inp = W.make_inputs(w)
    for with_db in (w.kind == "layernorm", w.kind != "layernorm"):
        out = run_recompute(nb, w, inp["x"], inp["dy"], inp["gamma"], with_db)
        compare(w, inp["x"], inp["dy"], inp["gamma"], out, with_db)


@pytest.mark.parametrize("eps", [0.0, 1e-3, 1.0, 100.0])
@pytest.mark.parametrize("kind", ["layernorm", "rmsnorm"])
def test_recompute_uses_eps(nb, kind, eps):
    """eps enters rstd = 1/sqrt(var + eps); a large eps changes dx a lot, so
    a kernel that dropped or misplaced it fails here."""
    base = W.LN_F32_128x512 if kind == "layernorm" else W.RMS_F32_128x512
    w = W.scaled(base, M=64, N=1024, io_dtype=torch.float32)
    inp = W.make_inputs(w)
    out = run_recompute(nb, w, inp["x"], inp["dy"], inp["gamma"], True, eps=eps)
    compare(w, inp["x"], inp["dy"], inp["gamma"], out, True, eps=eps)


REC_EDGES = [(kind, dt, m, n)
             for kind in ("layernorm", "rmsnorm")
             for dt, ns in ((torch.float32, [1, 3, 65, 1000, 16384]),
                            (torch.float16, [2, 63, 513, 4100, 32768]),
                            (torch.bfloat16, [7, 64, 768, 6144, 20000]))
             for m, n in zip([1, 3, 511, 2, 64], ns)]


@pytest.mark.parametrize("kind,dt,M,N", REC_EDGES, ids=lambda v: str(v).replace("torch.", ""))
def test_recompute_edge_shapes(nb, kind, dt, M, N):
    base = W.LN_F32_128x512 if kind == "layernorm" else W.RMS_F32_128x512
    w = W.scaled(base, M=M, N=N, io_dtype=dt, wgrad_dtype=torch.float32, seed=500 + M + N)
    inp = W.make_inputs(w)
    with_db = not (dt != torch.float32 and N > 16384)
    out = run_recompute(nb, w, inp["x"], inp["dy"], inp["gamma"], with_db)
    compare(w, inp["x"], inp["dy"], inp["gamma"], out, with_db)


@pytest.mark.parametrize("kind,dt,M,N", [
    ("rmsnorm", torch.bfloat16, 700, 5120), ("layernorm", torch.bfloat16, 300, 7168),
    ("layernorm", torch.float16, 513, 3072), ("rmsnorm", torch.float32, 333, 1536),
    ("rmsnorm", torch.bfloat16, 1001, 1536), ("layernorm", torch.bfloat16, 300, 2560),
    ("rmsnorm", torch.float16, 600, 3584)])
def test_recompute_exact_non_power_of_two_waves(nb, kind, dt, M, N):
    base = W.LN_F32_128x512 if kind == "layernorm" else W.RMS_F32_128x512
    w = W.scaled(base, M=M, N=N, io_dtype=dt, wgrad_dtype=torch.float32, seed=700 + N)
    inp = W.make_inputs(w)
    with_db = kind == "layernorm"
    out = run_recompute(nb, w, inp["x"], inp["dy"], inp["gamma"], with_db)
    compare(w, inp["x"], inp["dy"], inp["gamma"], out, with_db)


@pytest.mark.parametrize("kind,dt,M,N", [
    ("rmsnorm", torch.bfloat16, 1, 768), ("layernorm", torch.bfloat16, 3, 256),
    ("rmsnorm", torch.float32, 999, 128), ("layernorm", torch.float16, 4097, 768),
    # groups of at least 20 complete pairs: the steady-state loop
    ("layernorm", torch.bfloat16, 20001, 768), ("rmsnorm", torch.float16, 30000, 256),
    ("layernorm", torch.float32, 12001, 384), ("rmsnorm", torch.bfloat16, 24576, 768)])
def test_recompute_two_rows_per_wave(nb, kind, dt, M, N):
    """Recompute mode on the two-rows-per-wave layout (each 32-lane half forms
    its row's statistics), both gradients."""
    base = W.LN_F32_128x512 if kind == "layernorm" else W.RMS_F32_128x512
    w = W.scaled(base, M=M, N=N, io_dtype=dt, wgrad_dtype=torch.float32, seed=800 + N)
    inp = W.make_inputs(w)
    out = run_recompute(nb, w, inp["x"], inp["dy"], inp["gamma"], True)
    compare(w, inp["x"], inp["dy"], inp["gamma"], out, True)


def test_recompute_constant_rows(nb):
    """A constant LayerNorm row has var = 0: rstd = 1/sqrt(eps), xhat = 0, so
    dx = rstd * (dyhat - mean(dyhat)) and its dgamma terms vanish."""
    w = W.scaled(W.LN_F32_128x512, M=6, N=512)
    inp = W.make_inputs(w)
    x = inp["x"].clone()
    x[1] = 2.5
    x[4] = -0.75
    out = run_recompute(nb, w, x, inp["dy"], inp["gamma"], True)
    compare(w, x, inp["dy"], inp["gamma"], out, True)


@pytest.mark.parametrize("w", [W.RMS_BF16_16384x4096, W.LN_BF16_65536x8192,
                               W.RMS_BF16_262144x768], ids=lambda w: w.name)
def test_recompute_full_size_sampled(nb, w):
    print(f"[gen] {w.name}", flush=True)
    inp = W.make_inputs(w)
    with_db = w.kind == "layernorm"
    print(f"[run] {w.name}", flush=True)
    out = run_recompute(nb, w, inp["x"], inp["dy"], inp["gamma"], with_db)
    rows = W.sample_rows(w.M, 48, seed=w.seed + 9)
    cols = W.sample_rows(w.N, 32, seed=w.seed + 10)
    if "outliers" in inp and inp["outliers"].dim() == 1:
        cols = torch.unique(torch.cat([cols, inp["outliers"]]))
    compare(w, inp["x"], inp["dy"], inp["gamma"], out, with_db, rows=rows, cols=cols)


def recompute_plan(nb, kind, M, N, dt, db):
    """The plan recompute mode runs, as a saved-statistics plan. Rows on the
    two-rows-per-wave layout take the saved-statistics plan with 16 KiB of x
    and dy in flight in both kinds. RMSNorm recompute otherwise takes the
    saved-statistics plan itself. LayerNorm recompute
    keeps the lane layout but fills 512 threads with rows (one when the
    combine buffer would not fit in LDS), with its own group count (about
    4096 waves in flight, counted on the dbeta-less layout; at least 4 rows
    per group; above 256 a multiple of 256)."""
    def rows(S, C, vec):
        P = max(1, 512 // (64 * S))
        while P > 1 and S * P * 64 > (512 if vec * C > 16 else 1024):
            P //= 2
        # the combine buffer: one plane of per-lane partials
        return 1 if P > 1 and S * C * 64 * vec * 4 > 65536 - 1024 else P

    base = nb.norm_bwd_make_plan(kind, M, N, dt, db)
    if base.rows_per_wave == 2:
        # RMSNorm recompute aims at LayerNorm's 16 KiB of x and dy in flight
        P = 2
        while P * 32 < 512 and P * 2 * N * dt.itemsize < 16384:
            P *= 2
        p = base.copy()
        p.rows_in_flight, p.threads = P, 32 * P
        p.lds_bytes = (2 if db else 1) * base.chunks * 32 * base.vec * 4 if P > 2 else 0
        return p
    if kind == "rmsnorm":
        # the saved-statistics rules, except that rows on 16-byte lanes with
        # an odd wave count aim at 16 KiB of x and dy in flight, not 12 KiB
        S, C, vec, eb = base.waves_per_row, base.chunks, base.vec, dt.itemsize
        if base.rows_per_wave == 1 and C == 1 and S > 1 and S % 2 and S * 64 * vec == N:
            P = 1
            while P < 16 and P * 2 * N * eb < 16384:
                P *= 2
            while P > 1 and (S * P > 16 or S * P * 64 > 1024):
                P //= 2
            p = base.copy()
            p.rows_in_flight, p.threads = P, 64 * S * P
            p.lds_bytes = S * C * 64 * vec * 4 if P > 1 else 0
            return p
        return base
    S, C, vec = base.waves_per_row, base.chunks, base.vec
    G = min(4096 // (S * rows(S, C, vec)), -(-M // 4))
    G = max(1, G - G % 256 if G > 256 else G)
    p = nb.norm_bwd_make_plan(kind, M, N, dt, db, G)
    P = rows(S, C, vec)
    p.rows_in_flight, p.threads = P, 64 * S * P
    p.lds_bytes = S * C * 64 * vec * 4 if P > 1 else 0
    return p


@pytest.mark.parametrize("w", [W.scaled(W.RMS_BF16_16384x4096, M=1024),
                               W.scaled(W.LN_BF16_65536x8192, M=600),
                               W.scaled(W.LN_F32_128x512, M=300, N=1000),
                               # LayerNorm's exchanges pipelined across rows,
                               # groups ending on inactive rows
                               W.scaled(W.LN_BF16_65536x8192, M=2001, N=4096),
                               # the fp16 kernel that keeps the two-exchange order
                               W.LN_F16_1151x8192,
                               # 5 and 3 waves per row
                               W.scaled(W.RMS_BF16_16384x4096, M=700, N=5120),
                               W.scaled(W.LN_BF16_65536x8192, M=500, N=3072),
                               # 7 waves of 16-byte lanes
                               W.scaled(W.RMS_BF16_16384x4096, M=900, N=3584),
                               W.scaled(W.LN_BF16_65536x8192, M=400, N=3584),
                               # two rows per wave (odd M: a last pair of one row)
                               W.scaled(W.RMS_BF16_262144x768, M=3001),
                               W.scaled(W.LN_BF16_65536x8192, M=2001, N=768),
                               W.scaled(W.RMS_BF16_16384x4096, M=999, N=256),
                               W.scaled(W.LN_BF16_65536x8192, M=20000, N=256),
                               W.scaled(W.LN_F32_128x512, M=515, N=384),
                               W.scaled(W.RMS_F32_128x512, M=77, N=128)],
                         ids=lambda w: w.name)
def test_recompute_matches_forward_statistics_bitwise(nb, w):
    """The forward and recompute mode share the lane layout, so the
    recomputed statistics are summed in the forward's order: recompute mode
    equals the saved-statistics path fed by the GPU forward bit for bit when
    that path runs recompute mode's plan (the automatic saved-statistics
    plan may keep fewer rows in flight, another dgamma order)."""
    with_db = w.kind == "layernorm"
    plan = recompute_plan(nb, w.kind, w.M, w.N, w.io_dtype, with_db)
    inp = W.make_inputs(w)
    x, dy, g = inp["x"].cuda(), inp["dy"].cuda(), inp["gamma"].cuda()
    if w.kind == "layernorm":
        _, mean, rstd = nb.norm_fwd_layernorm(x, g, None, w.eps)
        a = nb.norm_bwd_execute(plan, x, dy, g, mean, rstd, wgrad_dtype=w.wgrad_dtype)
        b = nb.norm_bwd_layernorm(x, dy, g, None, None, w.eps, wgrad_dtype=w.wgrad_dtype)
    else:
        _, rstd = nb.norm_fwd_rmsnorm(x, g, w.eps)
        a = nb.norm_bwd_execute(plan, x, dy, g, None, rstd, wgrad_dtype=w.wgrad_dtype)
        b = nb.norm_bwd_rmsnorm(x, dy, g, None, w.eps, wgrad_dtype=w.wgrad_dtype)
    torch.cuda.synchronize()
    for ta, tb in zip(a, b):
        if ta is not None:
            assert torch.equal(ta, tb)


def test_recompute_is_deterministic(nb):
    w = W.scaled(W.LN_BF16_65536x8192, M=1000, N=2048)
    inp = W.make_inputs(w)
    outs = [run_recompute(nb, w, inp["x"], inp["dy"], inp["gamma"], True) for _ in range(5)]
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert torch.equal(a, b)


def test_recompute_workspace_rule(nb):
    """LayerNorm in recompute mode plans twice the row groups (4096 waves);
    norm_bwd_workspace_bytes covers it, the saved-statistics plan's size does
    not, and a short workspace is refused before any launch."""
    w = W.scaled(W.LN_BF16_65536x8192, M=4096, N=1024)
    inp = W.make_inputs(w)
    x, dy, g = inp["x"].cuda(), inp["dy"].cuda(), inp["gamma"].cuda()
    saved = nb.norm_bwd_make_plan("layernorm", w.M, w.N, w.io_dtype, True).workspace_bytes
    need = nb.norm_bwd_workspace_bytes("layernorm", w.M, w.N, w.io_dtype, True)
    assert need == 2 * saved
    short = torch.empty(saved, dtype=torch.uint8, device="cuda")
    with pytest.raises(nb.NormBwdError) as e:
        nb.norm_bwd_layernorm(x, dy, g, None, None, w.eps, workspace=short)
    assert e.value.status == nb.ERR_WORKSPACE
    full = torch.empty(need, dtype=torch.uint8, device="cuda")
    out = nb.norm_bwd_layernorm(x, dy, g, None, None, w.eps, workspace=full)
    torch.cuda.synchronize()
    compare(w, inp["x"], inp["dy"], inp["gamma"], tuple(t.cpu() for t in out), True)


def test_recompute_argument_rules(nb):
    w = W.scaled(W.LN_F32_128x512, M=8, N=64)
    inp = W.make_inputs(w)
    x, dy, g = inp["x"].cuda(), inp["dy"].cuda(), inp["gamma"].cuda()
    rstd = torch.ones(8, device="cuda")
    with pytest.raises(ValueError):
        nb.norm_bwd_layernorm(x, dy, g, None, rstd)
    plan = nb.norm_bwd_make_plan("layernorm", 8, 64, torch.float32, True)
    with pytest.raises(ValueError):
        nb.norm_bwd_execute(plan, x, dy, g, None, None)
    # an empty problem in recompute mode still writes the empty sums
    x0 = torch.empty(0, 64, device="cuda")
    dg = torch.full((64,), float("nan"), device="cuda")
    nb.norm_bwd_rmsnorm(x0, x0, g, None, dgamma=dg)
    torch.cuda.synchronize()
    assert torch.all(dg == 0)
