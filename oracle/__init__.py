"""fp64 CPU oracle for the LayerNorm / RMSNorm backward pass (ctypes wrapper).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The GPU library does
not load it and shares no code with it.

The arithmetic lives in ``norm_oracle.c`` (plain C, IEEE double, no FMA
contraction, ascending-order sums). This wrapper only widens inputs to
contiguous float64 NumPy arrays, allocates outputs and calls the C functions.
Widening bf16/fp16/fp32 to float64 is exact, so the oracle sees the very bits
the GPU was given.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(closed forms, invariants, finite differences, an explicit Jacobian, torch
fp64 autograd, hand-derived fixtures in ``tests/golden/``), and the same file
plants mistakes in copies of the C source to show the pins catch them.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "norm_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")
_KIND = {"layernorm": 0, "rmsnorm": 1}
_D = ctypes.POINTER(ctypes.c_double)


def compile_library(src: str, out: str) -> str:
    """gcc -O2, IEEE double, no FMA contraction, shared library."""
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compile norm_oracle.c into liboracle.so when missing or stale."""
    if force or not os.path.exists(LIBRARY) or \
            os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
        compile_library(SOURCE, LIBRARY)
    return LIBRARY


def _f64(a) -> Optional[np.ndarray]:
    """Exact widening to a contiguous float64 array (accepts torch tensors)."""
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch.Tensor, without importing torch here
        a = a.detach().cpu()
        if str(a.dtype) in ("torch.bfloat16", "torch.float16"):
            a = a.float()
        a = a.double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(_D)


def _kind(kind: str) -> int:
    try:
        return _KIND[kind]
    except KeyError:
        raise ValueError(f"kind must be 'layernorm' or 'rmsnorm', got {kind!r}")


class Oracle:
    """The oracle's functions bound to one compiled copy of norm_oracle.c."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        L, I = ctypes.c_long, ctypes.c_int
        lib.oracle_norm_fwd_stats.argtypes = [I, _D, L, L, ctypes.c_double, _D, _D]
        lib.oracle_norm_fwd.argtypes = [I, _D, _D, _D, L, L, ctypes.c_double, _D, _D, _D]
        lib.oracle_norm_bwd_dx.argtypes = [I, _D, _D, _D, _D, _D, L, L, _D]
        lib.oracle_norm_bwd_wgrad.argtypes = [I, _D, _D, _D, _D, L, L, _D, _D]
        for f in (lib.oracle_norm_fwd_stats, lib.oracle_norm_fwd,
                  lib.oracle_norm_bwd_dx, lib.oracle_norm_bwd_wgrad):
            f.restype = None
        self.lib = lib
        self.path = path

    def fwd_stats(self, kind: str, x, eps: float) -> Tuple[Optional[np.ndarray], np.ndarray]:
        """(mean, rstd) of each row of x[M, N]; mean is None for RMSNorm."""
        x = _f64(x)
        M, N = x.shape
        mean = np.empty(M) if kind == "layernorm" else None
        rstd = np.empty(M)
        self.lib.oracle_norm_fwd_stats(_kind(kind), _p(x), M, N, float(eps), _p(mean), _p(rstd))
        return mean, rstd

    def fwd(self, kind: str, x, gamma, beta, eps: float):
        """(y, mean, rstd) with y = gamma * xhat + beta; beta may be None."""
        x, gamma, beta = _f64(x), _f64(gamma), _f64(beta)
        M, N = x.shape
        y = np.empty((M, N))
        mean = np.empty(M)
        rstd = np.empty(M)
        self.lib.oracle_norm_fwd(_kind(kind), _p(x), _p(gamma), _p(beta), M, N, float(eps),
                                 _p(y), _p(mean), _p(rstd))
        return y, (mean if kind == "layernorm" else None), rstd

    def bwd_dx(self, kind: str, x, dy, gamma, mean, rstd) -> np.ndarray:
        """dx[M, N] from x, dy, gamma and the saved statistics."""
        x, dy, gamma, rstd = _f64(x), _f64(dy), _f64(gamma), _f64(rstd)
        mean = _f64(mean) if kind == "layernorm" else None
        M, N = x.shape
        if dy.shape != (M, N) or gamma.shape != (N,) or rstd.shape != (M,):
            raise ValueError("shape mismatch")
        if kind == "layernorm" and (mean is None or mean.shape != (M,)):
            raise ValueError("layernorm needs mean[M]")
        dx = np.empty((M, N))
        self.lib.oracle_norm_bwd_dx(_kind(kind), _p(x), _p(dy), _p(gamma), _p(mean),
                                    _p(rstd), M, N, _p(dx))
        return dx

    def bwd_wgrad(self, kind: str, x, dy, mean, rstd, want_dbeta: bool = True):
        """(dgamma[N], dbeta[N] or None) summed over all rows."""
        x, dy, rstd = _f64(x), _f64(dy), _f64(rstd)
        mean = _f64(mean) if kind == "layernorm" else None
        M, N = x.shape
        if dy.shape != x.shape or rstd.shape != (M,) or \
                (kind == "layernorm" and (mean is None or mean.shape != (M,))):
            raise ValueError("shape mismatch")
        dgamma = np.empty(N)
        dbeta = np.empty(N) if want_dbeta else None
        self.lib.oracle_norm_bwd_wgrad(_kind(kind), _p(x), _p(dy), _p(mean), _p(rstd),
                                       M, N, _p(dgamma), _p(dbeta))
        return dgamma, dbeta

    def bwd(self, kind: str, x, dy, gamma, mean, rstd, want_dbeta: bool = True):
        """(dx, dgamma, dbeta) in float64."""
        dx = self.bwd_dx(kind, x, dy, gamma, mean, rstd)
        dgamma, dbeta = self.bwd_wgrad(kind, x, dy, mean, rstd, want_dbeta)
        return dx, dgamma, dbeta


_lock = threading.Lock()
_default: Optional[Oracle] = None


def default() -> Oracle:
    """The oracle the tests use: liboracle.so, built when missing or stale;
    or, with NORM_ORACLE_LIBRARY set, that compiled copy of norm_oracle.c
    (the sanitizer test runs the pins against an instrumented build)."""
    global _default
    with _lock:
        if _default is None:
            _default = Oracle(os.environ.get("NORM_ORACLE_LIBRARY") or build())
    return _default


def fwd_stats(kind, x, eps):
    return default().fwd_stats(kind, x, eps)


def fwd(kind, x, gamma, beta, eps):
    return default().fwd(kind, x, gamma, beta, eps)


def bwd_dx(kind, x, dy, gamma, mean, rstd):
    return default().bwd_dx(kind, x, dy, gamma, mean, rstd)


def bwd_wgrad(kind, x, dy, mean, rstd, want_dbeta=True):
    return default().bwd_wgrad(kind, x, dy, mean, rstd, want_dbeta)


def bwd(kind, x, dy, gamma, mean, rstd, want_dbeta=True):
    return default().bwd(kind, x, dy, gamma, mean, rstd, want_dbeta)
