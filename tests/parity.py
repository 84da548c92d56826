"""Comparison of the GPU path against the fp64 oracle, with the tolerances.

Tolerances (all comparisons in fp64, oracle unrounded):

* fp32 I/O: every element of dx, dgamma, dbeta within 1e-5 + 1e-5*|ref|.
* fp16/bf16 I/O, dx:
  - max_j |got - ref| <= 2e-2 over the whole tensor, and
  - per row, max_j |got - ref| <= tau * max_j |ref| with tau = 2^-7 (bf16) or
    2^-10 (fp16). Rounding fp32 to bf16 (fp16) to nearest even moves a value
    by at most 2^-8 (2^-11) of itself, so tau is twice the output-rounding
    bound relative to the row's largest element; the fp32 arithmetic before it
    adds ~1e-6 relative. The absolute bound alone would be loose when dy is
    small (|dx| ~ 0.05 for dy ~ N(0, 1e-2)).
* fp16/bf16 I/O, dgamma/dbeta: every element within
  1e-3*|ref| + 1e-3*max_j|ref_j|. The normwise floor is needed because a
  column sum of zero-mean terms can land near zero, where a purely relative
  test would fail on fp32 rounding alone. fp16 outputs round by at most
  2^-11 < 1e-3 relative.

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


def check_dx(io_dtype, got, ref, what="dx"):
    g, r = f64(got), f64(ref)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    if g.size == 0:
        return {}
    err = np.abs(g - r)
    if io_dtype == torch.float32:
        lim = 1e-5 + 1e-5 * np.abs(r)
        if not np.all(err <= lim):
            _fail(what, g, r, np.unravel_index(np.argmax(err - lim), err.shape))
        return {"max_abs": float(err.max())}
    if not np.all(np.isfinite(g)):
        _fail(what + " (non-finite)", g, r, np.unravel_index(np.argmax(~np.isfinite(g)), g.shape))
    if err.max() > 2e-2:
        _fail(what + " max-abs 2e-2", g, r, np.unravel_index(np.argmax(err), err.shape))
    row_err = err.reshape(err.shape[0], -1).max(axis=1)
    row_ref = np.abs(r).reshape(r.shape[0], -1).max(axis=1)
    bad = row_err > TAU[io_dtype] * row_ref
    if bad.any():
        i = int(np.argmax(bad))
        raise Mismatch(f"{what}: row {i} max err {row_err[i]:.3g} > tau*{row_ref[i]:.3g}")
    return {"max_abs": float(err.max()),
            "max_row_rel": float(np.max(row_err / np.maximum(row_ref, 1e-300)))}


def check_wgrad(io_dtype, got, ref, what="dgamma"):
    g, r = f64(got), f64(ref)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    if g.size == 0:
        return {}
    err = np.abs(g - r)
    if io_dtype == torch.float32:
        lim = 1e-5 + 1e-5 * np.abs(r)
    else:
        lim = 1e-3 * np.abs(r) + 1e-3 * np.max(np.abs(r))
    if not np.all(err <= lim):
        _fail(what, g, r, np.unravel_index(np.argmax(err - lim), err.shape))
    scale = max(float(np.max(np.abs(r))), 1e-300)
    return {"max_abs": float(err.max()), "max_rel_to_max": float(err.max() / scale)}
