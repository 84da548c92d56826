"""Backward inputs for the tests: the seeded draws plus saved statistics.

The backward reads the per-row statistics a forward pass saved. Here they are
the fp64 oracle's forward statistics (mean = sum(x)/N, biased variance, rstd =
1/sqrt(var + eps); RMSNorm: rstd = 1/sqrt(sum(x^2)/N + eps)) rounded to fp32,
computed in row chunks so full-size workloads fit in memory.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle
from rmsnorm_backward_amd import workloads as W


def oracle_stats(x: torch.Tensor, kind: str, eps: float, chunk_rows: int = 4096):
    """fp32 (mean or None, rstd) of each row of x from the oracle's forward."""
    M = x.shape[0]
    o = oracle.default()
    rstd = np.empty(M, dtype=np.float32)
    mean = np.empty(M, dtype=np.float32) if kind == W.LAYERNORM else None
    for r0 in range(0, M, chunk_rows):
        m, r = o.fwd_stats(kind, x[r0:r0 + chunk_rows], eps)
        rstd[r0:r0 + chunk_rows] = r
        if mean is not None:
            mean[r0:r0 + chunk_rows] = m
    return (None if mean is None else torch.from_numpy(mean)), torch.from_numpy(rstd)


def backward_inputs(w: W.Workload):
    """W.make_inputs(w) plus fp32 ``rstd`` (and ``mean`` for LayerNorm)."""
    inp = W.make_inputs(w)
    mean, rstd = oracle_stats(inp["x"], w.kind, w.eps)
    inp["rstd"] = rstd
    if mean is not None:
        inp["mean"] = mean
    return inp
