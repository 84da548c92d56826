"""Comparison of the GPU path against the fp64 oracle, with the tolerances.

Tolerances (all comparisons in fp64, oracle unrounded):

* fp32 I/O: every element of dx, dgamma, dbeta within 1e-5 + 1e-5*|ref|,
  the stated rel/abs bound, with nothing added. Only a test that names an
  ill-conditioned case passes ``coef32`` to check_dx, which then adds
  coef32 * T_j (T_j below) for dx: the fp32 arithmetic bound (2^-18 with at
  most 16 elements per lane), which matters only where the terms of dx_j
  cancel. The named cases are N = 1 (RMSNorm dx = eps*rstd^3*dyhat is what is
  left of two terms that cancel; LayerNorm dx is exactly 0, formed as a
  difference of two rounded products) and rows whose variance is far below
  eps (constant or near-constant rows, where xhat*m2 and dyhat nearly cancel).
  Recompute mode passes 2^-16 with its own scale (below): the kernel's fp32
  statistics stand in for the exact ones.
* fp16/bf16 I/O, dx:
  - |got - ref| <= 2e-2 + u * |ref| for every element, u = 2^-8 (bf16) or
    2^-11 (fp16) the rounding of the stored value to nearest even: the 2e-2
    bounds the computation, on top of that rounding (as for stored fp16/bf16
    weight gradients below). A bf16 value of magnitude 8 or more is stored
    with spacing 2^-4, so no stored value could be within 2e-2 of every exact
    result there; where |dx| < 0.1, as in every workload here, the added term
    is below 4e-4. And
  - per row, max_j |got - ref| <= tau * max_j |ref| + 2^-16 * max_j T_j with
    tau = 2^-7 (bf16) or 2^-10 (fp16). Rounding fp32 to bf16 (fp16) to nearest
    even moves a value by at most 2^-8 (2^-11) of itself, so tau is twice the
    output-rounding bound relative to the row's largest element. The absolute
    bound alone would be loose when dy is small (|dx| ~ 0.05 for
    dy ~ N(0, 1e-2)).
  - T_j = rstd * (|dyhat_j| + mean_k|dyhat_k| + |xhat_j| * mean_k|dyhat_k xhat_k|)
    is the size of the terms dx_j is assembled from. The kernel's fp32
    arithmetic (products, and in-row sums of at most 64 per-lane terms, a
    6-step wave tree and 16 slice partials) is accurate to about 90 fp32 ulps
    of that size, i.e. < 2^-16 * T_j. This term matters only where the terms
    cancel, e.g. N = 1 RMSNorm, where dx = rstd*dyhat*(1 - xhat^2) and
    1 - xhat^2 = eps*rstd^2 is tiny; elsewhere it is far below the first.
* fp16/bf16 I/O, dgamma/dbeta: every element within
  1e-3*|ref| + d * 2^-24 * A_j, where A_j = sum_r |dy_rj * xhat_rj| (dbeta:
  sum_r |dy_rj|) is the size of the terms column j is summed from and d bounds
  the number of fp32 roundings any one term meets on its way into the sum
  (three for forming dy * (x - mean) * rstd, then the additions along the
  kernel's summation tree: depth_fused, depth_colwalk). d * 2^-24 * A_j is the
  classical worst-case bound of fp32 summation (gamma_d * sum|t|), so where the
  column sum does not cancel (A_j ~ |ref_j|) the bound is 1e-3 relative to
  within d * 2^-24 (< 2e-5 here), and it widens only by as much as the terms
  cancel. When dgamma/dbeta are themselves stored in fp16 or bf16, the
  rounding of the stored value (at most 2^-11 or 2^-8 of it, to nearest even)
  is added to the bound.

* forward y: per element |got - ref| <= out_round*|ref| + k*T_y with
  T_y = |gamma|*(|xhat| + rstd*mean_k|x_k|) + |beta|, the size of the terms y
  is built from including the error a fp32 mean brings into xhat; k = 2^-16
  for fp16/bf16 outputs (out_round 2^-11 / 2^-8, plus half the subnormal
  spacing, 2^-25 for fp16, where the rounding error is absolute) and fp32
  outputs use
  1e-5 + 1e-5*|ref| + 2^-18*T_y. Statistics: |mean - ref| <= 2^-16 *
  mean_k|x_k| (+ 1e-7 * |ref| for its fp32 rounding), |rstd - ref| <= 2^-16 *
  rstd: the fp32 row sums carry at most ~90 ulps of the summed magnitudes.

* recompute mode (the backward computes mean/rstd itself): the reference is
  the oracle's backward on its fp64 statistics; dx uses the scale
  T_rec = 3 T + rstd^2 mean|x| (mean|dyhat xhat| + |xhat_j| mean|dyhat|) with
  coefficient 2^-16 for every dtype, and dgamma adds 2^-16 * sum_r |dy| (|xhat|
  + rstd mean|x|) (recompute_terms): the first-order effect of statistics
  within the forward's bounds.

Both sides read the same input bits (the oracle widens them exactly).
"""

from __future__ import annotations

import json
import os

import numpy as np
import torch

TAU = {torch.bfloat16: 2.0 ** -7, torch.float16: 2.0 ** -10}


def f64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu()
        if t.dtype in (torch.bfloat16, torch.float16):
            t = t.float()
        return t.double().numpy()
    return np.asarray(t, dtype=np.float64)


class Mismatch(AssertionError):
    pass


def _record(kind, what, io_dtype, **ratios):
    """With PARITY_LOG set to a file path, append one JSON line per check:
    the running test, the quantity, and the largest error over each bound
    (``plain``: the stated tolerance alone; ``used``: the bound checked)."""
    path = os.environ.get("PARITY_LOG")
    if not path:
        return
    rec = {"test": os.environ.get("PYTEST_CURRENT_TEST", "").split(" (")[0], "check": kind,
           "what": what, "io": str(io_dtype).replace("torch.", "")}
    rec.update({k: (None if v is None else float(v)) for k, v in ratios.items()})
    with open(path, "a") as f:
        f.write(json.dumps(rec) + "\n")


def _max_ratio(err, lim):
    if err.size == 0:
        return 0.0
    return float(np.max(err / np.maximum(lim, 1e-300)))


def _fail(what, got, ref, idx, extra=""):
    raise Mismatch(f"{what}: got {got[idx]!r} want {ref[idx]!r} at {idx} {extra}")


def dx_term_scale(kind, x, dy, gamma, mean, rstd) -> np.ndarray:
    """T[r, j] (see above) from the inputs, in fp64; a magnitude, not dx."""
    x, dy, gamma, rstd = f64(x), f64(dy), f64(gamma), f64(rstd)
    mu = f64(mean)[:, None] if kind == "layernorm" else 0.0
    xh = np.abs((x - mu) * rstd[:, None])
    dyh = np.abs(dy * gamma[None, :])
    m1 = dyh.mean(axis=1, keepdims=True) if kind == "layernorm" else 0.0
    m2 = (dyh * xh).mean(axis=1, keepdims=True)
    return rstd[:, None] * (dyh + m1 + xh * m2)


def recompute_terms(kind, x, dy, gamma, mean, rstd):
    """Scales for the recompute mode, where the kernel's own fp32 statistics
    stand in for the exact ones: (T_dx, T_dgamma).

    With |d rstd| <= 2^-16 rstd and |d mean| <= 2^-16 mean_k|x_k| (the bounds
    the forward statistics meet), dx_j = rstd*dyhat_j - rstd*m1 - xc_j*rstd^3*
    sum(dyhat*xc)/N moves by at most 2^-16 * (3 T_j + rstd^2 mean|x| (mean|dyhat
    xhat| + |xhat_j| mean|dyhat|)) to first order, and each term dy*xhat of
    dgamma by 2^-16 * |dy| (|xhat| + rstd mean|x|)."""
    x, dy, gamma, rstd = f64(x), f64(dy), f64(gamma), f64(rstd)
    mu = f64(mean)[:, None] if kind == "layernorm" else 0.0
    rs = rstd[:, None]
    xh = np.abs((x - mu) * rs)
    dyh = np.abs(dy * gamma[None, :])
    mx = np.abs(x).mean(axis=1, keepdims=True) if kind == "layernorm" else 0.0
    m1 = dyh.mean(axis=1, keepdims=True) if kind == "layernorm" else 0.0
    m2 = (dyh * xh).mean(axis=1, keepdims=True)
    t = rs * (dyh + m1 + xh * m2)
    t_dx = 3.0 * t + rs * rs * mx * (m2 + xh * m1)
    t_dg = (np.abs(dy) * (xh + rs * mx)).sum(axis=0)
    return t_dx, t_dg


def check_dx(io_dtype, got, ref, what="dx", scale=None, coef32=0.0):
    """`scale` (T per element) widens the fp16/bf16 per-row bound by
    2^-16 * max_j T_j; for fp32 I/O it is used only with a non-zero `coef32`,
    which a test passes for a named ill-conditioned case (see above)."""
    g, r = f64(got), f64(ref)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    if g.size == 0:
        return {}
    err = np.abs(g - r)
    if io_dtype == torch.float32:
        plain = 1e-5 + 1e-5 * np.abs(r)
        lim = plain
        if scale is not None and coef32:
            lim = plain + coef32 * f64(scale)
        _record("dx", what, io_dtype, plain=_max_ratio(err, plain), used=_max_ratio(err, lim),
                coef32=coef32)
        if not np.all(err <= lim):
            _fail(what, g, r, np.unravel_index(np.argmax(err - lim), err.shape))
        return {"max_abs": float(err.max()), "max_err_over_bound": _max_ratio(err, lim)}
    if not np.all(np.isfinite(g)):
        _fail(what + " (non-finite)", g, r, np.unravel_index(np.argmax(~np.isfinite(g)), g.shape))
    lim_abs = 2e-2 + OUT_ROUND[io_dtype] * np.abs(r)
    if not np.all(err <= lim_abs):
        _fail(what + " max-abs 2e-2 (+ output rounding)", g, r,
              np.unravel_index(np.argmax(err - lim_abs), err.shape))
    row_err = err.reshape(err.shape[0], -1).max(axis=1)
    row_ref = np.abs(r).reshape(r.shape[0], -1).max(axis=1)
    row_lim = TAU[io_dtype] * row_ref
    if scale is not None:
        row_lim = row_lim + 2.0 ** -16 * f64(scale).reshape(r.shape[0], -1).max(axis=1)
    _record("dx", what, io_dtype, plain=_max_ratio(err, 2e-2 + 0 * r),
            used=_max_ratio(err, lim_abs), row=_max_ratio(row_err, row_lim))
    bad = row_err > row_lim
    if bad.any():
        i = int(np.argmax(bad))
        raise Mismatch(f"{what}: row {i} max err {row_err[i]:.3g} > limit {row_lim[i]:.3g} "
                       f"(row max |ref| {row_ref[i]:.3g})")
    return {"max_abs": float(err.max()),
            "max_row_rel": float(np.max(row_err / np.maximum(row_ref, 1e-300)))}


OUT_ROUND = {torch.float32: 0.0, torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}


def check_wgrad(io_dtype, got, ref, what="dgamma", extra=None, absum=None, depth=None,
                sumsq=None):
    """dgamma/dbeta against the oracle. For fp16/bf16 I/O, `absum` (A_j, per
    column: abs_terms) and `depth` (d: depth_fused / depth_colwalk) are
    required and add d * 2^-24 * A_j to 1e-3 * |ref|. `extra` (optional, per
    element) is added to the bound: the recompute mode's 2^-16 * T_dgamma, the
    rounding of an accumulated old + sum, or fp32_long_sum_extra. (`sumsq`
    rides along in the wgrad_bounds dicts for fp32_long_sum_extra; the check
    itself does not use it.)"""
    out_round = OUT_ROUND[got.dtype] if isinstance(got, torch.Tensor) else 0.0
    g, r = f64(got), f64(ref)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    if g.size == 0:
        return {}
    err = np.abs(g - r)
    if io_dtype == torch.float32:
        plain = 1e-5 + 1e-5 * np.abs(r)
        lim = plain.copy()
    else:
        if absum is None or depth is None:
            raise TypeError(f"{what}: fp16/bf16 weight gradients need absum and depth")
        a = f64(absum)
        assert a.shape == r.shape, (what, a.shape, r.shape)
        plain = 1e-3 * np.abs(r)
        lim = plain + float(depth) * 2.0 ** -24 * a
    lim = lim + out_round * np.abs(r)
    plain = plain + out_round * np.abs(r)
    if extra is not None:
        lim = lim + f64(extra)
    _record("wgrad", what, io_dtype, plain=_max_ratio(err, plain), used=_max_ratio(err, lim),
            depth=depth)
    if not np.all(err <= lim):
        _fail(what, g, r, np.unravel_index(np.argmax(err - lim), err.shape))
    scale = max(float(np.max(np.abs(r))), 1e-300)
    return {"max_abs": float(err.max()), "max_rel_to_max": float(err.max() / scale),
            "max_err_over_bound": _max_ratio(err, lim)}


def term_sums(kind, x, dy, mean, rstd, block_rows=4096):
    """Per column, in fp64, over the terms t = dy * xhat (dgamma) and t = dy
    (dbeta): (sum_r |t| for dgamma, for dbeta, sum_r t^2 for dgamma, for
    dbeta). Row blocks keep full-size workloads within memory."""
    M, N = x.shape
    ag, ab, sg, sb = np.zeros(N), np.zeros(N), np.zeros(N), np.zeros(N)
    rs_all = f64(rstd)
    mu_all = f64(mean) if kind == "layernorm" else None
    for r0 in range(0, M, block_rows):
        r1 = min(M, r0 + block_rows)
        xb, yb = f64(x[r0:r1]), f64(dy[r0:r1])
        if mu_all is not None:
            xb = xb - mu_all[r0:r1, None]
        tg = yb * xb * rs_all[r0:r1, None]
        ag += np.abs(tg).sum(axis=0)
        ab += np.abs(yb).sum(axis=0)
        sg += (tg * tg).sum(axis=0)
        sb += (yb * yb).sum(axis=0)
    return ag, ab, sg, sb


def abs_terms(kind, x, dy, mean, rstd, block_rows=4096):
    """(A_gamma, A_beta) per column: sum_r |dy * xhat| and sum_r |dy| in fp64,
    the sizes of the terms dgamma and dbeta are summed from."""
    ag, ab, _, _ = term_sums(kind, x, dy, mean, rstd, block_rows)
    return ag, ab


# Rounding steps a term dy * (x - mean) * rstd meets before it is added: the
# subtraction, the product, the fused multiply-add into the sum; plus one
# for an accumulated old + sum.
_TERM_ROUNDINGS = 4


def depth_fused(M, groups=None):
    """An upper bound on the fp32 roundings of any term of a column sum formed
    by kernels A and B with `groups` row groups (None: any automatic plan,
    whose group count is at least min(256, ceil(M/4)) and at most 512): a
    row-lane of a group adds its rows in order (at most ceil(M/G)), at most 16
    row-lanes of a workgroup are combined in order, kernel B adds a slice of
    at most ceil(G/16) groups and then the 16 slice sums."""
    if M <= 0:
        return _TERM_ROUNDINGS
    if groups is None:
        g_lo, g_hi = max(1, min(256, -(-M // 4))), 512
    else:
        g_lo = g_hi = max(1, min(int(groups), M))
    return -(-M // g_lo) + 16 + -(-g_hi // 16) + 16 + _TERM_ROUNDINGS


def depth_colwalk(M):
    """The same bound for the column walk: a lane adds at most ceil(M/16) rows
    in order, an xor butterfly adds at most 64 row slots (6 levels), then 16
    wave sums in order."""
    return max(0, -(-M // 16)) + 6 + 16 + _TERM_ROUNDINGS


# Widest rows the fused kernels hold (the C header's NORM_BWD_MAX_N_*): wider
# rows take the row loop for dx and the column walk for dgamma/dbeta.
_MAX_N_16BIT, _MAX_N_16BIT_DBETA, _MAX_N_F32, _MAX_N_UNALIGNED = 32768, 16384, 16384, 8192


def depth_path(M, N, io_dtype, with_dbeta, groups=None, aligned=True):
    """depth_fused for rows the fused kernels hold, else depth_colwalk (the
    path the named entry points take for (M, N))."""
    eb = 4 if io_dtype == torch.float32 else 2
    full = aligned and N % (16 // eb) == 0
    limit = (_MAX_N_UNALIGNED if not full else _MAX_N_F32 if eb == 4 else
             _MAX_N_16BIT_DBETA if with_dbeta else _MAX_N_16BIT)
    return depth_fused(M, groups) if N <= limit else depth_colwalk(M)


# Named ill-conditioned fp32 weight-gradient case: long sums that cancel.
# A fixed-order fp32 sum errs by up to d * 2^-24 * A_j (the classical bound,
# d the summation depth), and in practice by the rounding of its partial
# sums: each term meets at most d roundings, each of about 2^-24 times the
# partial sum it lands in, and those partial sums are about
# sqrt(sum_r t_r^2) in size when the terms' signs are mixed. So
# 2^-24 * sqrt(d * sum_r t_r^2) is the scale of the rounding error, in any
# fixed order. Where that scale exceeds the plain bound 1e-5 + 1e-5 * |ref_j|
# (a column whose sum cancels far below its partial sums, over many rows or
# a deep chain) no fp32 evaluation can promise the plain bound: 302 rows in
# one group (d = 339) and 5835 rows in 256 groups (d = 91) each missed
# 1e-5 absolute on such a column. On those columns the fp32 summation bound
# is added; everywhere else the plain fp32 bound is asserted as stated (for
# the 128 x 512 workloads the scale is 4e-6 at most).


def fp32_long_sum_extra(io_dtype, bounds, ref):
    """For fp32 I/O: per column, the fp32 summation bound d * 2^-24 * A_j on
    the columns of the named long-sum case (2^-24 * sqrt(d * sum_r t_r^2) >
    1e-5 + 1e-5 * |ref_j|), 0 on the others; None for half precision or when
    no column is in the case. `bounds`: the wgrad_bounds dict of the
    gradient (absum, depth, sumsq); `ref`: the oracle's sums."""
    if io_dtype != torch.float32:
        return None
    d = float(bounds["depth"])
    scale = 2.0 ** -24 * np.sqrt(d * f64(bounds["sumsq"]))
    named = scale > 1e-5 + 1e-5 * np.abs(f64(ref))
    if not named.any():
        return None
    return np.where(named, d * 2.0 ** -24 * f64(bounds["absum"]), 0.0)


def add_extra(*terms):
    """Sum of the per-element bound terms that are not None (or None)."""
    out = None
    for t in terms:
        if t is not None:
            out = f64(t) if out is None else out + f64(t)
    return out


def wgrad_bounds(kind, x, dy, mean, rstd, depth):
    """Keyword arguments for check_wgrad of dgamma and of dbeta:
    ({absum, depth, sumsq}, {absum, depth, sumsq})."""
    ag, ab, sg, sb = term_sums(kind, x, dy, mean, rstd)
    return ({"absum": ag, "depth": depth, "sumsq": sg},
            {"absum": ab, "depth": depth, "sumsq": sb})


# Below the smallest normal number the formats are evenly spaced (fp16: 2^-24,
# bf16: 2^-133), so rounding to nearest errs there by up to half that spacing
# rather than by a fraction of |ref|.
SUBNORMAL_HALF_SPACING = {torch.float16: 2.0 ** -25, torch.bfloat16: 2.0 ** -134}


def check_forward(io_dtype, kind, x, gamma, beta, got_y, got_mean, got_rstd, ref_y, ref_mean,
                  ref_rstd):
    xs, g = f64(x), f64(gamma)
    b = f64(beta) if beta is not None else np.zeros_like(g)
    rm = f64(ref_mean)[:, None] if kind == "layernorm" else 0.0
    rr = f64(ref_rstd)[:, None]
    mabs = np.abs(xs).mean(axis=1, keepdims=True)
    ty = np.abs(g)[None, :] * (np.abs((xs - rm) * rr) + rr * mabs) + np.abs(b)[None, :]
    gy, ry = f64(got_y), f64(ref_y)
    err = np.abs(gy - ry)
    if io_dtype == torch.float32:
        lim = 1e-5 + 1e-5 * np.abs(ry) + 2.0 ** -18 * ty
    else:
        lim = OUT_ROUND[io_dtype] * np.abs(ry) + SUBNORMAL_HALF_SPACING[io_dtype] + \
            2.0 ** -16 * ty
    if not np.all(err <= lim):
        _fail("y", gy, ry, np.unravel_index(np.argmax(err - lim), err.shape))
    if got_rstd is not None:
        gr, rr1 = f64(got_rstd), f64(ref_rstd)
        e = np.abs(gr - rr1)
        if not np.all(e <= 2.0 ** -16 * rr1):
            _fail("rstd", gr, rr1, (int(np.argmax(e - 2.0 ** -16 * rr1)),))
    if kind == "layernorm" and got_mean is not None:
        gm, rm1 = f64(got_mean), f64(ref_mean)
        e = np.abs(gm - rm1)
        lim = 2.0 ** -16 * mabs[:, 0] + 1e-7 * np.abs(rm1)
        if not np.all(e <= lim):
            _fail("mean", gm, rm1, (int(np.argmax(e - lim)),))
    return {"y_max_abs": float(err.max()) if err.size else 0.0}
