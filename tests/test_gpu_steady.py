"""The steady-state row loop of kernel A and of the forward against the fp64
oracle (needs a gfx950 GPU).

When the lanes cover a row exactly and a workgroup has at least 2D - 1 full
iterations ahead (D, the register ring's depth: 3 here, 4 for the LayerNorm
forward), kernel A and the forward run those iterations through a loop with
no per-lane or per-row conditions and then hand the ring to the general loop
for the rest. These cases put few groups (or forward sweeps) over many rows so
that the loop runs, with group lengths just below and at the threshold, tails
of every length after it, and one, two, four and eight rows in flight per
workgroup, for both kinds, all three element types, saved statistics and
recompute mode. Every output is compared element by element with the oracle.
"""

from __future__ import annotations

import pytest
import torch

import oracle
import parity
from inputs import backward_inputs
from rmsnorm_backward_amd import workloads as W

pytestmark = pytest.mark.gpu

BASE = {"layernorm": W.LN_F16_1151x8192, "rmsnorm": W.RMS_BF16_16384x4096}


@pytest.fixture(scope="module")
def nb():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import rmsnorm_backward_amd as nbmod
    nbmod.load_library()
    return nbmod


def workload(kind, dt, M, N):
    w = BASE[kind]
    wg = w.wgrad_dtype if dt == w.io_dtype else torch.float32
    return W.scaled(w, M=M, N=N, io_dtype=dt, wgrad_dtype=wg,
                    name=f"{kind}_{W._dt(dt)}_{M}x{N}")


def compare(w, inp, out, mean, rstd, with_db, groups):
    dx, dg, db = (None if t is None else t.cpu() for t in out)
    rdx, rdg, rdb = oracle.bwd(w.kind, inp["x"], inp["dy"], inp["gamma"], mean, rstd,
                               want_dbeta=True)
    scale = parity.dx_term_scale(w.kind, inp["x"], inp["dy"], inp["gamma"], mean, rstd)
    parity.check_dx(w.io_dtype, dx, rdx, scale=scale)
    bg, bb = parity.wgrad_bounds(w.kind, inp["x"], inp["dy"], mean, rstd,
                                 parity.depth_fused(w.M, groups))
    parity.check_wgrad(w.io_dtype, dg, rdg, **bg)
    if with_db:
        parity.check_wgrad(w.io_dtype, db, rdb, "dbeta", **bb)


# (kind, dtype, N, groups, row counts): N is covered exactly by the lanes;
# the rows per workgroup in flight (P) follow from N; group lengths around
# 5 * P rows (the threshold for D = 3) and tails of 0 .. D - 1 iterations
# and 0 .. P - 1 rows after the last full pass.
SAVED = [
    ("rmsnorm", torch.bfloat16, 4096, 3, (12, 15, 19, 26, 50)),       # P = 1
    ("layernorm", torch.bfloat16, 8192, 2, (8, 10, 15, 23)),          # P = 1, both gradients
    ("layernorm", torch.bfloat16, 2048, 2, (18, 20, 23, 42, 61)),     # P = 2, both gradients
    ("rmsnorm", torch.bfloat16, 1024, 2, (38, 40, 47, 83, 126)),      # P = 4
    ("layernorm", torch.float32, 512, 2, (40, 45, 90, 133)),          # P = 4, both gradients
    ("rmsnorm", torch.bfloat16, 512, 2, (78, 80, 95, 161, 250)),      # P = 8
    ("rmsnorm", torch.float16, 2048, 1, (9, 10, 11, 12, 29)),         # one group: P = 2
    # fp16 with both gradients: groups of 11 rows and more (5 * P + 1) take
    # the 512-thread-bound kernel and its steady-state loop, shorter ones the
    # 1024-thread-bound kernel without it
    ("layernorm", torch.float16, 2048, 2, (18, 20, 22, 23, 61)),      # P = 2
]


def _saved_cases():
    for kind, dt, N, G, Ms in SAVED:
        for M in Ms:
            yield kind, dt, N, G, M


@pytest.mark.parametrize("kind,dt,N,G,M", list(_saved_cases()),
                         ids=lambda v: str(v).replace("torch.", ""))
def test_steady_loop_saved_statistics(nb, kind, dt, N, G, M):
    w = workload(kind, dt, M, N)
    with_db = kind == "layernorm"
    inp = backward_inputs(w)
    plan = nb.norm_bwd_make_plan(kind, M, N, dt, with_db, G)
    assert plan.waves_per_row * 64 * plan.vec * plan.chunks == N   # lanes cover the row
    g = {k: v.cuda() for k, v in inp.items() if isinstance(v, torch.Tensor) and k != "outliers"}
    print(f"[run] {w.name} groups={G} P={plan.rows_in_flight}", flush=True)
    out = nb.norm_bwd_execute(plan, g["x"], g["dy"], g["gamma"], g.get("mean"), g["rstd"],
                              wgrad_dtype=w.wgrad_dtype)
    torch.cuda.synchronize()
    compare(w, inp, out, inp.get("mean"), inp["rstd"], with_db, G)


# Recompute mode runs the steady-state loop where a lane holds one 16-byte
# vector per operand (RMSNorm, and LayerNorm's pipelined loop), and two under
# the 512-thread launch bound that workgroups of up to 512 threads take when
# their groups hold at least 5 * P + 1 rows (the fp16 LayerNorm kernel with
# both gradients there keeps its two exchanges per row).
RECOMPUTE = [
    ("rmsnorm", torch.bfloat16, 512, 2, (78, 80, 95, 250)),           # P = 8
    ("layernorm", torch.bfloat16, 512, 2, (78, 80, 95, 250)),         # P = 8, pipelined
    ("layernorm", torch.float32, 256, 1, (39, 40, 41, 77)),           # P = 8, pipelined
    ("layernorm", torch.float16, 2048, 2, (38, 40, 47, 126)),         # P = 4, two exchanges
    # P = 1, 512-thread bound; M = 16 gives groups of 6, 5 and 5 rows, the
    # narrow kernel at its threshold (5 * P rows) with every group
    ("rmsnorm", torch.bfloat16, 4096, 3, (12, 15, 16, 19, 77)),
]


def _recompute_cases():
    for kind, dt, N, G, Ms in RECOMPUTE:
        for M in Ms:
            yield kind, dt, N, G, M


@pytest.mark.parametrize("kind,dt,N,G,M", list(_recompute_cases()),
                         ids=lambda v: str(v).replace("torch.", ""))
def test_steady_loop_recompute(nb, kind, dt, N, G, M):
    recompute_and_compare(nb, kind, dt, N, G, M)


def recompute_and_compare(nb, kind, dt, N, G, M):
    w = workload(kind, dt, M, N)
    with_db = kind == "layernorm"
    inp = W.make_inputs(w)
    print(f"[run] recompute {w.name} groups={G}", flush=True)
    out = nb.norm_bwd_ex(kind, inp["x"].cuda(), inp["dy"].cuda(), inp["gamma"].cuda(), None, None,
                         w.eps, wgrad_dtype=w.wgrad_dtype, with_dbeta=with_db, groups=G)
    torch.cuda.synchronize()
    # the reference: the oracle's backward on the oracle's unrounded fp64
    # statistics; the tolerance adds the first-order effect of the kernel's
    # own fp32 statistics (parity.recompute_terms)
    x, dy, gamma = inp["x"], inp["dy"], inp["gamma"]
    dx, dg, db = (None if t is None else t.cpu() for t in out)
    mean, rstd = oracle.fwd_stats(kind, x, w.eps)
    rdx = oracle.bwd_dx(kind, x, dy, gamma, mean, rstd)
    t_dx, t_dg = parity.recompute_terms(kind, x, dy, gamma, mean, rstd)
    parity.check_dx(w.io_dtype, dx, rdx, scale=t_dx, coef32=2.0 ** -16)
    rdg, rdb = oracle.bwd_wgrad(kind, x, dy, mean, rstd, want_dbeta=True)
    bg, bb = parity.wgrad_bounds(kind, x, dy, mean, rstd, parity.depth_fused(M, G))
    parity.check_wgrad(w.io_dtype, dg, rdg, extra=2.0 ** -16 * t_dg, **bg)
    if with_db:
        parity.check_wgrad(w.io_dtype, db, rdb, "dbeta", **bb)


# The forward: a sweep of rows_per_sweep = grid * P rows (4096 / S for
# these N), so the steady-state loop needs at least 5 sweeps (7 for the
# LayerNorm forward, whose ring is one row deeper).
FORWARD = [
    ("rmsnorm", torch.bfloat16, 512, (4096 * 5 - 1, 4096 * 5 + 1000, 4096 * 9 + 17)),
    ("layernorm", torch.bfloat16, 512, (4096 * 7 - 3, 4096 * 7 + 5, 4096 * 11 + 300)),
    ("rmsnorm", torch.float32, 1024, (2048 * 5 + 7, 2048 * 8 + 2047)),
]


def _forward_cases():
    for kind, dt, N, Ms in FORWARD:
        for M in Ms:
            yield kind, dt, N, M


@pytest.mark.parametrize("kind,dt,N,M", list(_forward_cases()),
                         ids=lambda v: str(v).replace("torch.", ""))
def test_steady_loop_forward(nb, kind, dt, N, M):
    w = workload(kind, dt, M, N)
    inp = W.make_inputs(w)
    x, g = inp["x"], inp["gamma"]
    print(f"[run] forward {w.name}", flush=True)
    if kind == "layernorm":
        y, mean, rstd = nb.norm_fwd_layernorm(x.cuda(), g.cuda(), None, w.eps)
    else:
        y, rstd = nb.norm_fwd_rmsnorm(x.cuda(), g.cuda(), w.eps)
        mean = None
    torch.cuda.synchronize()
    ry, rm, rr = oracle.fwd(kind, x, g, None, w.eps)
    parity.check_forward(w.io_dtype, kind, x, g, None, y.cpu(),
                         None if mean is None else mean.cpu(), rstd.cpu(), ry, rm, rr)


# The two-rows-per-wave kernel (rows that 32 lanes of 16-byte vectors cover
# exactly: N = 32 * VEC * 1 or 3). Its steady-state loop needs 2 * D - 1
# complete iterations, that is (2 * D - 1) * P rows per group (P = rows in
# flight, two per wave), with a ring of D row pairs: 3 for RMSNorm with saved
# statistics (5 * P rows), 2 for LayerNorm with saved statistics (3 * P
# rows). Row counts around that threshold and with every kind of tail.
TWO_ROW = [
    ("rmsnorm", torch.bfloat16, 768, 2),      # P = 8 (4 waves)
    ("layernorm", torch.bfloat16, 768, 2),    # both gradients
    ("layernorm", torch.float16, 256, 3),     # one chunk, P = 16
    ("rmsnorm", torch.float16, 768, 1),       # one group
    ("rmsnorm", torch.float32, 384, 2),       # fp32, three chunks of 4
    ("layernorm", torch.float32, 128, 1),     # fp32, one chunk
]


def _two_row_cases():
    for kind, dt, N, G in TWO_ROW:
        eb = torch.tensor([], dtype=dt).element_size()
        P = 2
        while P < 16 and P * 2 * N * eb < (16384 if kind == "layernorm" else 8192):
            P *= 2
        T = 3 if kind == "layernorm" else 5          # 2 * D - 1 iterations
        for M in (G * T * P - 1, G * T * P, G * T * P + 1, G * ((T + 1) * P + 3) + 1,
                  G * ((T + 3) * P - 1), 3):
            yield kind, dt, N, G, M


@pytest.mark.parametrize("kind,dt,N,G,M", list(_two_row_cases()),
                         ids=lambda v: str(v).replace("torch.", ""))
def test_two_row_kernel(nb, kind, dt, N, G, M):
    w = workload(kind, dt, M, N)
    with_db = kind == "layernorm"
    inp = backward_inputs(w)
    plan = nb.norm_bwd_make_plan(kind, M, N, dt, with_db, G)
    assert plan.rows_per_wave == 2 and plan.waves_per_row == 1
    g = {k: v.cuda() for k, v in inp.items() if isinstance(v, torch.Tensor) and k != "outliers"}
    print(f"[run] two-row {w.name} groups={G} P={plan.rows_in_flight}", flush=True)
    out = nb.norm_bwd_execute(plan, g["x"], g["dy"], g["gamma"], g.get("mean"), g["rstd"],
                              wgrad_dtype=w.wgrad_dtype)
    torch.cuda.synchronize()
    compare(w, inp, out, inp.get("mean"), inp["rstd"], with_db, G)


@pytest.mark.parametrize("P", [2, 4, 16])
def test_two_row_rows_in_flight(nb, P):
    """Edited plans with other rows in flight (1, 2 or 8 waves) stay within
    tolerance; 90 rows in 3 groups leave every kind of tail."""
    w = workload("layernorm", torch.bfloat16, 5 * 16 * 3 + 90, 768)
    inp = backward_inputs(w)
    plan = nb.norm_bwd_make_plan("layernorm", w.M, w.N, w.io_dtype, True, 3)
    plan.rows_per_wave, plan.chunks, plan.waves_per_row = 2, 3, 1
    plan.rows_in_flight, plan.threads = P, 32 * P
    pairs = -(-w.M // 2)                   # groups of adjacent row pairs
    plan.rows_per_group = 2 * -(-pairs // 3)
    plan.lds_bytes = 2 * plan.chunks * 32 * plan.vec * 4 if P > 2 else 0
    g = {k: v.cuda() for k, v in inp.items() if isinstance(v, torch.Tensor) and k != "outliers"}
    out = nb.norm_bwd_execute(plan, g["x"], g["dy"], g["gamma"], g["mean"], g["rstd"])
    torch.cuda.synchronize()
    compare(w, inp, out, inp["mean"], inp["rstd"], True, 3)


# Recompute mode on the two-rows-per-wave layout: 16 KiB of x and dy in
# flight in both kinds, a ring of 2 row pairs for RMSNorm rows of three chunks
# (3 * P rows per group for the steady-state loop), 3 otherwise (5 * P).
TWO_ROW_RECOMPUTE = [
    ("rmsnorm", torch.bfloat16, 768, 2),      # P = 8, ring of 2
    ("rmsnorm", torch.float32, 384, 1),       # P = 8, ring of 2, one group
    ("rmsnorm", torch.float16, 256, 2),       # P = 16, ring of 3
    ("layernorm", torch.bfloat16, 768, 2),    # P = 8, ring of 3, both gradients
    ("layernorm", torch.float32, 128, 3),     # P = 16, ring of 3
]


def _two_row_recompute_cases():
    for kind, dt, N, G in TWO_ROW_RECOMPUTE:
        eb = torch.tensor([], dtype=dt).element_size()
        P = 2
        while P < 16 and P * 2 * N * eb < 16384:
            P *= 2
        T = 3 if (kind == "rmsnorm" and N * eb == 3 * 512) else 5
        for M in (G * T * P - 1, G * T * P, G * T * P + 1, G * ((T + 2) * P + 1) + 3):
            yield kind, dt, N, G, M


@pytest.mark.parametrize("kind,dt,N,G,M", list(_two_row_recompute_cases()),
                         ids=lambda v: str(v).replace("torch.", ""))
def test_two_row_recompute_steady(nb, kind, dt, N, G, M):
    recompute_and_compare(nb, kind, dt, N, G, M)


# The two-row forward: 8 waves a workgroup and up to 256 workgroups, so a
# sweep covers 4096 rows; the steady-state loop needs 2 * D - 1 sweeps of
# complete pairs, with a ring of D = 2 for rows of three chunks (12288 rows)
# and D = 3 for rows of one (20480).
FORWARD_TWO_ROW = [
    ("rmsnorm", torch.bfloat16, 768, (12287, 12288, 12289, 4096 * 5 - 1)),
    ("layernorm", torch.float32, 384, (12287, 12289)),
    ("layernorm", torch.float16, 256, (20479, 20480, 20481, 4096 * 7 + 3)),
    ("rmsnorm", torch.float32, 128, (20479, 20481)),
]


@pytest.mark.parametrize("kind,dt,N,M", [(k, d, n, m) for k, d, n, Ms in FORWARD_TWO_ROW
                                         for m in Ms],
                         ids=lambda v: str(v).replace("torch.", ""))
def test_two_row_forward_steady(nb, kind, dt, N, M):
    test_steady_loop_forward(nb, kind, dt, N, M)


def test_two_row_strided_rows_are_bit_identical(nb):
    """Row strides (16-byte aligned) give the bits of contiguous rows on the
    two-row layout."""
    w = workload("rmsnorm", torch.bfloat16, 1000, 768)
    inp = backward_inputs(w)
    x, dy, gam, rs = (inp[k].cuda() for k in ("x", "dy", "gamma", "rstd"))

    def strided(t, ld):
        buf = torch.zeros(t.shape[0] * ld, dtype=t.dtype, device="cuda")
        v = buf.view(t.shape[0], ld)[:, :t.shape[1]]
        v.copy_(t)
        return v

    ref = nb.norm_bwd_ex("rmsnorm", x, dy, gam, None, rs, w.eps)
    got = nb.norm_bwd_ex("rmsnorm", strided(x, 768 + 8), strided(dy, 768 + 64), gam, None, rs,
                         w.eps, dx=strided(torch.zeros_like(x), 768 + 24))
    torch.cuda.synchronize()
    assert torch.equal(got[0].cpu(), ref[0].cpu()) and torch.equal(got[1].cpu(), ref[1].cpu())


# Seeded random cases aimed at the steady-state loops: few groups over many
# rows (so the loops run), saved statistics through an explicit plan, recompute
# mode, and norm_bwd_ex with row strides accumulating onto zeros. Widths cover
# the exact-cover layouts (including the two-rows-per-wave ones) and some
# ragged ones.
_COVER_N = {torch.float32: [128, 256, 384, 512, 1024, 2048, 4096, 8192],
            torch.float16: [256, 512, 768, 1024, 2048, 4096, 8192, 16384],
            torch.bfloat16: [256, 512, 768, 1024, 2048, 4096, 8192, 16384]}


def _random_steady_cases(n=120, seed=3141):
    import random
    rng = random.Random(seed)
    out = []
    for i in range(n):
        kind = rng.choice(("layernorm", "rmsnorm"))
        dt = rng.choice((torch.float32, torch.float16, torch.bfloat16))
        N = rng.choice(_COVER_N[dt]) if rng.random() < 0.8 else rng.choice((1000, 3000, 6144))
        G = rng.choice((1, 2, 3, 5))
        rows = rng.randint(1, 90)
        M = max(1, min(G * rows + rng.randint(0, G - 1), 2_000_000 // N))
        mode = rng.choice(("saved", "saved", "recompute", "ex"))
        pad = rng.choice((8, 64, 128))
        out.append((i, mode, kind, dt, M, N, G, pad))
    return out


@pytest.mark.parametrize("case", _random_steady_cases(),
                         ids=lambda c: "-".join(str(v).replace("torch.", "") for v in c))
def test_steady_random(nb, case):
    i, mode, kind, dt, M, N, G, pad = case
    w = workload(kind, dt, M, N)
    with_db = kind == "layernorm"
    print(f"[run] {mode} {w.name} groups={G}", flush=True)
    if mode == "recompute":
        inp = W.make_inputs(w)
        out = nb.norm_bwd_ex(kind, inp["x"].cuda(), inp["dy"].cuda(), inp["gamma"].cuda(), None,
                             None, w.eps, wgrad_dtype=w.wgrad_dtype, with_dbeta=with_db,
                             groups=G)
        torch.cuda.synchronize()
        x, dy, gamma = inp["x"], inp["dy"], inp["gamma"]
        dx, dg, db = (None if t is None else t.cpu() for t in out)
        mean, rstd = oracle.fwd_stats(kind, x, w.eps)
        rdx = oracle.bwd_dx(kind, x, dy, gamma, mean, rstd)
        t_dx, t_dg = parity.recompute_terms(kind, x, dy, gamma, mean, rstd)
        parity.check_dx(w.io_dtype, dx, rdx, scale=t_dx, coef32=2.0 ** -16)
        rdg, rdb = oracle.bwd_wgrad(kind, x, dy, mean, rstd, want_dbeta=True)
        bg, bb = parity.wgrad_bounds(kind, x, dy, mean, rstd, parity.depth_fused(M, G))
        parity.check_wgrad(w.io_dtype, dg, rdg, extra=2.0 ** -16 * t_dg, **bg)
        if with_db:
            parity.check_wgrad(w.io_dtype, db, rdb, "dbeta", **bb)
        return
    inp = backward_inputs(w)
    g = {k: v.cuda() for k, v in inp.items() if isinstance(v, torch.Tensor) and k != "outliers"}
    if mode == "saved":
        plan = nb.norm_bwd_make_plan(kind, M, N, dt, with_db, G)
        out = nb.norm_bwd_execute(plan, g["x"], g["dy"], g["gamma"], g.get("mean"), g["rstd"],
                                  wgrad_dtype=w.wgrad_dtype)
    else:  # row-strided views, accumulating onto zeros
        xs = torch.zeros(M, N + pad, dtype=dt, device="cuda")
        ys = torch.zeros(M, N + pad, dtype=dt, device="cuda")
        dxs = torch.zeros(M, N + pad, dtype=dt, device="cuda")
        xs[:, :N] = g["x"]
        ys[:, :N] = g["dy"]
        dg0 = torch.zeros(N, dtype=w.wgrad_dtype, device="cuda")
        db0 = torch.zeros(N, dtype=w.wgrad_dtype, device="cuda") if with_db else None
        out = nb.norm_bwd_ex(kind, xs[:, :N], ys[:, :N], g["gamma"], g.get("mean"), g["rstd"],
                             w.eps, dx=dxs[:, :N], dgamma=dg0, dbeta=db0, accumulate=True,
                             groups=G)
    torch.cuda.synchronize()
    compare(w, inp, out, inp.get("mean"), inp["rstd"], with_db, G)


def _random_forward_cases(n=24, seed=2718):
    import random
    rng = random.Random(seed)
    out = []
    for i in range(n):
        kind = rng.choice(("layernorm", "rmsnorm"))
        dt = rng.choice((torch.float32, torch.float16, torch.bfloat16))
        N = rng.choice((256, 512, 768, 1024, 2048)) if dt != torch.float32 else \
            rng.choice((256, 512, 1024))
        M = min(rng.randint(16000, 40000), 20_000_000 // N)
        beta = kind == "layernorm" and rng.random() < 0.5
        out.append((i, kind, dt, M, N, beta))
    return out


@pytest.mark.parametrize("case", _random_forward_cases(),
                         ids=lambda c: "-".join(str(v).replace("torch.", "") for v in c))
def test_forward_steady_random(nb, case):
    """Seeded forward cases long enough for the forward's steady-state loop."""
    i, kind, dt, M, N, with_beta = case
    w = workload(kind, dt, M, N)
    inp = W.make_inputs(w)
    x, gm = inp["x"], inp["gamma"]
    beta = torch.rand(N, generator=torch.Generator().manual_seed(i)).to(dt) if with_beta else None
    print(f"[run] forward {w.name} beta={with_beta}", flush=True)
    if kind == "layernorm":
        y, mean, rstd = nb.norm_fwd_layernorm(x.cuda(), gm.cuda(),
                                              None if beta is None else beta.cuda(), w.eps)
    else:
        y, rstd = nb.norm_fwd_rmsnorm(x.cuda(), gm.cuda(), w.eps)
        mean = None
    torch.cuda.synchronize()
    ry, rm, rr = oracle.fwd(kind, x, gm, beta, w.eps)
    parity.check_forward(w.io_dtype, kind, x, gm, beta, y.cpu(),
                         None if mean is None else mean.cpu(), rstd.cpu(), ry, rm, rr)
