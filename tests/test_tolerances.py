"""The parity tolerances themselves (CPU only): an fp32 evaluation of the
gradient formulas, in the order the fused kernels use, passes them without
any widening; a plausible mistake fails them.

The formulas are those of "Norm backward in Triton -- the dγ/dβ reduction",
"The gradients". The fp32 evaluation here is NumPy float32 arithmetic,
written for this test: it shares nothing with the HIP kernels except the
order of the sums it imitates (row r in group r mod G, a group's rows in
ascending order, then 16 contiguous slices of groups added in slice order).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import parity
from inputs import backward_inputs
from rmsnorm_backward_amd import workloads as W

F = np.float32


def fp32_dx(kind, x, dy, gamma, mean, rstd, drop_m1=False):
    """dx = dyhat * rstd + xc * c2 + c1 evaluated in float32."""
    xc = (x - mean[:, None]).astype(F) if kind == "layernorm" else x.astype(F)
    dyh = (dy * gamma).astype(F)
    n = F(1.0 / x.shape[1])
    s1 = dyh.sum(1, dtype=F) if kind == "layernorm" and not drop_m1 else np.zeros(len(x), F)
    s2 = (dyh * xc).sum(1, dtype=F)
    m2 = (s2 * n * rstd).astype(F)
    c2 = (-(rstd * rstd) * m2).astype(F)
    c1 = (-rstd * (s1 * n)).astype(F)
    return (dyh * rstd[:, None] + (xc * c2[:, None] + c1[:, None])).astype(F)


def fp32_wgrad(kind, x, dy, mean, rstd, groups):
    """dgamma (and dbeta) summed in float32: per-group partials in ascending
    row order, then 16 slices of groups, then the slices in order."""
    xc = (x - mean[:, None]).astype(F) if kind == "layernorm" else x.astype(F)
    out = []
    for t in ((dy * xc).astype(F) * rstd[:, None], dy.astype(F)):
        t = t.astype(F)
        part = np.zeros((groups, x.shape[1]), F)
        for r in range(len(x)):
            part[r % groups] += t[r]
        total = None
        for q in range(16):
            s = np.zeros(x.shape[1], F)
            for g in range(groups * q // 16, groups * (q + 1) // 16):
                s += part[g]
            total = s if total is None else (total + s).astype(F)
        out.append(total)
    return out


def _np(inp, k):
    v = inp.get(k)
    return None if v is None else v.float().numpy()


@pytest.mark.parametrize("w", [W.LN_F32_128x512, W.RMS_F32_128x512], ids=lambda w: w.name)
def test_fp32_evaluation_meets_the_plain_bound(w):
    inp = backward_inputs(w)
    x, dy, g, rs = (_np(inp, k) for k in ("x", "dy", "gamma", "rstd"))
    mu = _np(inp, "mean") if w.kind == "layernorm" else np.zeros(w.M, F)
    rdx, rdg, rdb = oracle.bwd(w.kind, inp["x"], inp["dy"], inp["gamma"], inp.get("mean"),
                               inp["rstd"])
    s = parity.check_dx(torch.float32, torch.from_numpy(fp32_dx(w.kind, x, dy, g, mu, rs)), rdx)
    assert s["max_err_over_bound"] < 0.1
    dg, db = fp32_wgrad(w.kind, x, dy, mu, rs, groups=32)
    parity.check_wgrad(torch.float32, torch.from_numpy(dg), rdg)
    parity.check_wgrad(torch.float32, torch.from_numpy(db), rdb, "dbeta")
    if w.kind == "layernorm":
        # a dropped mean_j(dyhat) term fails the plain bound
        with pytest.raises(parity.Mismatch):
            parity.check_dx(torch.float32,
                            torch.from_numpy(fp32_dx(w.kind, x, dy, g, mu, rs, drop_m1=True)), rdx)


def test_half_weight_gradients_bound():
    """bf16 inputs of the 16384 x 4096 workload's distributions at 2048 x 256:
    the float32 two-pass sum with 256 groups passes with depth_fused; a
    column whose terms do not cancel is held to about 1e-3 relative."""
    w = W.scaled(W.RMS_BF16_16384x4096, M=2048, N=256)
    inp = backward_inputs(w)
    # column 0: every term positive (no cancellation)
    inp["x"][:, 0] = inp["x"][:, 0].abs() + 0.5
    inp["dy"][:, 0] = inp["dy"][:, 0].abs() + 1e-3
    x, dy, rs = (_np(inp, k) for k in ("x", "dy", "rstd"))
    mu = np.zeros(w.M, F)
    rdg, rdb = oracle.bwd_wgrad(w.kind, inp["x"], inp["dy"], None, inp["rstd"])
    dg, _ = fp32_wgrad(w.kind, x, dy, mu, rs, groups=256)
    bg, _ = parity.wgrad_bounds(w.kind, inp["x"], inp["dy"], None, inp["rstd"],
                                parity.depth_fused(w.M, 256))
    s = parity.check_wgrad(torch.bfloat16, torch.from_numpy(dg), rdg, **bg)
    assert s["max_err_over_bound"] < 0.5
    # the bound on the non-cancelling column is 1e-3 relative to within 1e-4
    lim0 = 1e-3 * abs(rdg[0]) + bg["depth"] * 2.0 ** -24 * bg["absum"][0]
    assert lim0 < 1.1e-3 * abs(rdg[0])
    bad = dg.copy()
    bad[0] = rdg[0] * (1 + 1.5e-3)
    with pytest.raises(parity.Mismatch):
        parity.check_wgrad(torch.bfloat16, torch.from_numpy(bad), rdg, **bg)
    # half-precision weight gradients cannot be checked without the bound's terms
    with pytest.raises(TypeError):
        parity.check_wgrad(torch.bfloat16, torch.from_numpy(dg), rdg)


def test_fp32_long_sums_need_the_summation_bound():
    """The named long-sum case: float32 column sums that cancel far below
    their partial sums. Evaluated in float32 in the kernels' order, 1327 rows
    in one or two groups (a deep chain) and 8192 rows in 256 groups (many
    rows, depth 84) miss the plain 1e-5 bound on such columns; every column
    that misses it is in the case, where the fp32 summation term meets it,
    and the case takes few columns (at most 1/8 of them in 256 groups, 1/4
    in the deep chains; the plain bound holds on the rest). The
    same 1327 rows in 256 groups meet the plain bound (the case, a bound on
    what fp32 may cost, still takes a few of their columns); the 128 x 512
    workloads have no column in it. Half precision never is."""
    def check(w, groups, plain_fails, most_named=8):
        inp = backward_inputs(w)
        x, dy, rs, mu = (_np(inp, k) for k in ("x", "dy", "rstd", "mean"))
        if mu is None:
            mu = np.zeros(w.M, F)
        rdg, _ = oracle.bwd_wgrad(w.kind, inp["x"], inp["dy"], inp.get("mean"), inp["rstd"])
        dg, _ = fp32_wgrad(w.kind, x, dy, mu, rs, groups=groups)
        bg, _ = parity.wgrad_bounds(w.kind, inp["x"], inp["dy"], inp.get("mean"), inp["rstd"],
                                    parity.depth_fused(w.M, groups))
        extra = parity.fp32_long_sum_extra(torch.float32, bg, rdg)
        err = np.abs(dg.astype(np.float64) - rdg)
        over = err > 1e-5 + 1e-5 * np.abs(rdg)
        if plain_fails:
            assert over.any() and extra is not None and np.all(extra[over] > 0)
            with pytest.raises(parity.Mismatch):
                parity.check_wgrad(torch.float32, torch.from_numpy(dg), rdg)
            parity.check_wgrad(torch.float32, torch.from_numpy(dg), rdg, extra=extra)
            named = extra > 0
            assert np.max(err[named] / extra[named]) < 0.05     # far inside the added term
            assert np.count_nonzero(named) <= w.N // most_named
        else:
            parity.check_wgrad(torch.float32, torch.from_numpy(dg), rdg)
            assert extra is None or np.count_nonzero(extra) <= w.N // most_named
        return bg, rdg, extra

    deep = W.scaled(W.LN_F32_128x512, M=1327, N=1000, seed=10000)
    for groups in (1, 2):                 # a chain of 664 to 1327 rows: more columns
        check(deep, groups, True, most_named=4)
    check(deep, 256, False)
    bg, rdg, _ = check(W.scaled(W.LN_F32_128x512, M=8192, N=256, seed=10001), 256, True)
    assert bg["depth"] <= 128
    for w in (W.LN_F32_128x512, W.RMS_F32_128x512):
        assert check(w, 32, False)[2] is None
    assert parity.fp32_long_sum_extra(torch.bfloat16, bg, rdg) is None


def test_summation_depths():
    # the fused path: a group's rows, 16 row-lanes, a slice of groups, 16 slices
    assert parity.depth_fused(16384, 256) == 64 + 16 + 16 + 16 + 4
    assert parity.depth_fused(16384) >= parity.depth_fused(16384, 256)
    assert parity.depth_fused(1151) >= parity.depth_fused(1151, 256)
    # the column walk: a lane's rows, a 64-slot butterfly, 16 waves
    assert parity.depth_colwalk(1600) == 100 + 6 + 16 + 4
    # rows wider than the fused limits are summed by the column walk
    assert parity.depth_path(64, 40000, torch.bfloat16, True) == parity.depth_colwalk(64)
    assert parity.depth_path(64, 32768, torch.bfloat16, False) == parity.depth_fused(64)
    assert parity.depth_path(64, 32768, torch.bfloat16, True) == parity.depth_colwalk(64)
    assert parity.depth_path(64, 8193, torch.float32, True, aligned=False) == \
        parity.depth_colwalk(64)
