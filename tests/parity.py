"""Comparison of the GPU path against the fp64 oracle, with the tolerances.

Tolerances (all comparisons in fp64, oracle unrounded):

* fp32 I/O: every element of dx, dgamma, dbeta within 1e-5 + 1e-5*|ref|; for
  dx plus 2^-18 * T_j (T_j below), the fp32 arithmetic bound with at most 16
  elements per lane, which only matters where the terms of dx_j cancel.
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
  1e-3*|ref| + 1e-3*max_j|ref_j|. The normwise floor is needed because a
  column sum of zero-mean terms can land near zero, where a purely relative
  test would fail on fp32 rounding alone. When dgamma/dbeta are themselves
  stored in fp16 or bf16, the rounding of the stored value (at most 2^-11 or
  2^-8 of it, to nearest even) is added to the bound.

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


def check_dx(io_dtype, got, ref, what="dx", scale=None, coef32=2.0 ** -18):
    g, r = f64(got), f64(ref)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    if g.size == 0:
        return {}
    err = np.abs(g - r)
    if io_dtype == torch.float32:
        lim = 1e-5 + 1e-5 * np.abs(r)
        if scale is not None:
            lim = lim + coef32 * f64(scale)
        if not np.all(err <= lim):
            _fail(what, g, r, np.unravel_index(np.argmax(err - lim), err.shape))
        return {"max_abs": float(err.max())}
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
    bad = row_err > row_lim
    if bad.any():
        i = int(np.argmax(bad))
        raise Mismatch(f"{what}: row {i} max err {row_err[i]:.3g} > limit {row_lim[i]:.3g} "
                       f"(row max |ref| {row_ref[i]:.3g})")
    return {"max_abs": float(err.max()),
            "max_row_rel": float(np.max(row_err / np.maximum(row_ref, 1e-300)))}


OUT_ROUND = {torch.float32: 0.0, torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}


def check_wgrad(io_dtype, got, ref, what="dgamma", extra=None):
    """`extra` (optional, per element) is added to the bound: the recompute
    mode's 2^-16 * T_dgamma."""
    out_round = OUT_ROUND[got.dtype] if isinstance(got, torch.Tensor) else 0.0
    g, r = f64(got), f64(ref)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    if g.size == 0:
        return {}
    err = np.abs(g - r)
    if io_dtype == torch.float32:
        lim = 1e-5 + 1e-5 * np.abs(r)
    else:
        lim = 1e-3 * np.abs(r) + 1e-3 * np.max(np.abs(r))
    lim = lim + out_round * np.abs(r)
    if extra is not None:
        lim = lim + f64(extra)
    if not np.all(err <= lim):
        _fail(what, g, r, np.unravel_index(np.argmax(err - lim), err.shape))
    scale = max(float(np.max(np.abs(r))), 1e-300)
    return {"max_abs": float(err.max()), "max_rel_to_max": float(err.max() / scale)}


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
