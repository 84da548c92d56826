"""Seeded synthetic workloads for the LayerNorm / RMSNorm backward pass.

This module only draws inputs. It holds none of the forward or backward
arithmetic: the GPU path and the fp64 oracle each implement that on their own,
and both read their inputs from here.

What a workload carries (the norm backward consumes the forward's saved
per-row statistics, see "Norm backward in Triton — the dγ/dβ reduction",
section "The dx kernel — recompute the stat, don't store x̂"):

* ``x``, ``dy``, ``gamma`` in the I/O dtype (round-to-nearest-even casts of
  fp32 draws), and for LayerNorm workloads that list one, ``beta`` (it enters
  only the forward output, never the backward).
The saved statistics (fp32 ``rstd``, and ``mean`` for LayerNorm) are not drawn
here: they are what a forward pass computes from the cast ``x``, so each
consumer runs one (the tests and the CPU baseline the fp64 oracle's forward,
rounded to fp32; the benchmark the GPU forward).

Everything is drawn on the CPU from seeded ``torch.Generator`` objects, so
every consumer sees the same bits. The [M, N] draws (x, dy, an outlier mask)
come in blocks of 4096 rows; block b of draw t uses its own generator seeded
with ``block_seed(seed, t, b)``, so blocks can be filled in parallel and the
result does not depend on the thread count. The small draws (per-row shift and
scale, gamma, beta, outlier columns) come, in that order, from one generator
seeded with the workload's seed.
"""

from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional, Sequence

import torch

LAYERNORM = "layernorm"
RMSNORM = "rmsnorm"


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic backward problem: shapes, dtypes, distributions, seed."""

    name: str
    kind: str                     # LAYERNORM or RMSNORM
    M: int                        # rows (tokens)
    N: int                        # features
    io_dtype: torch.dtype         # x, dy, gamma, dx
    wgrad_dtype: torch.dtype      # dgamma, dbeta
    eps: float
    seed: int
    x_dist: str = "normal"        # "normal" | "row_shift_scale"
    dy_std: float = 1.0
    gamma_lo: float = 0.5
    gamma_hi: float = 1.5
    with_beta: bool = False       # draw beta ~ U(0,1) (forward-only input)
    outlier_frac: float = 0.0     # fraction of feature columns scaled
    outlier_scale: float = 1.0
    outlier_mode: str = "columns" # "columns" | "entries"

    @property
    def io_bytes(self) -> int:
        return torch.tensor([], dtype=self.io_dtype).element_size()

    @property
    def wgrad_bytes(self) -> int:
        return torch.tensor([], dtype=self.wgrad_dtype).element_size()

    def algorithmic_bytes(self, with_dbeta: Optional[bool] = None) -> int:
        """Bytes the method must move: read x, dy, gamma and the saved stats,
        write dx and the weight gradients. Workspace traffic is excluded."""
        if with_dbeta is None:
            with_dbeta = self.kind == LAYERNORM
        s = self.io_bytes
        w = torch.tensor([], dtype=self.wgrad_dtype).element_size()
        stats = (8 if self.kind == LAYERNORM else 4) * self.M
        nw = 2 if with_dbeta else 1
        return 3 * self.M * self.N * s + self.N * s + stats + nw * self.N * w


# The five problems the benchmark and the parity tests use. Shapes follow the
# pages' worked example (16384 x 4096 bf16 RMSNorm, "Norm & activation
# backward", "Worked number") and the Phobos tutorial's check (1151 x 8192
# fp16 LayerNorm, "05: Layer norm").
WORKLOADS: Dict[str, Workload] = {}


def _register(w: Workload) -> Workload:
    WORKLOADS[w.name] = w
    return w


LN_F32_128x512 = _register(Workload(
    "layernorm_f32_128x512", LAYERNORM, 128, 512, torch.float32, torch.float32,
    1e-5, 1001, dy_std=1.0, gamma_lo=0.5, gamma_hi=1.5))
RMS_F32_128x512 = _register(dataclasses.replace(
    LN_F32_128x512, name="rmsnorm_f32_128x512", kind=RMSNORM))
LN_F16_1151x8192 = _register(Workload(
    "layernorm_f16_1151x8192", LAYERNORM, 1151, 8192, torch.float16, torch.float16,
    1e-5, 1002, dy_std=0.1, gamma_lo=0.0, gamma_hi=1.0, with_beta=True))
RMS_BF16_16384x4096 = _register(Workload(
    "rmsnorm_bf16_16384x4096", RMSNORM, 16384, 4096, torch.bfloat16, torch.float32,
    1e-6, 1003, dy_std=1e-2, gamma_lo=0.8, gamma_hi=1.2))
LN_BF16_65536x8192 = _register(Workload(
    "layernorm_bf16_65536x8192", LAYERNORM, 65536, 8192, torch.bfloat16, torch.float32,
    1e-5, 1004, x_dist="row_shift_scale", dy_std=1e-2, gamma_lo=0.5, gamma_hi=1.5))
RMS_BF16_262144x768 = _register(Workload(
    "rmsnorm_bf16_262144x768", RMSNORM, 262144, 768, torch.bfloat16, torch.float32,
    1e-6, 1005, dy_std=1e-2, gamma_lo=0.5, gamma_hi=1.5,
    outlier_frac=0.01, outlier_scale=50.0, outlier_mode="columns"))

# The benchmark's headline problem.
HEADLINE = RMS_BF16_16384x4096


def scaled(w: Workload, M: Optional[int] = None, N: Optional[int] = None,
           **kw) -> Workload:
    """Same distributions at another size (for small parity cases)."""
    M = w.M if M is None else M
    N = w.N if N is None else N
    name = kw.pop("name", f"{w.kind}_{_dt(w.io_dtype)}_{M}x{N}")
    return dataclasses.replace(w, name=name, M=M, N=N, **kw)


def _dt(d: torch.dtype) -> str:
    return {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}[d]


def outlier_columns(w: Workload, gen: torch.Generator) -> torch.Tensor:
    k = int(round(w.outlier_frac * w.N))
    return torch.randperm(w.N, generator=gen)[:k]


BLOCK_ROWS = 4096
_X, _DY, _MASK = 1, 2, 3   # draw tags


def block_seed(seed: int, tag: int, block: int) -> int:
    """Seed of one 4096-row block of one [M, N] draw."""
    return (seed * 1_000_003 + tag * 65_537 + block * 8_191 + 12_345) % (1 << 62)


def _blocked(seed: int, tag: int, M: int, N: int, kind: str) -> torch.Tensor:
    """[M, N] fp32 draw (standard normal, or uniform [0,1)), block by block."""
    out = torch.empty(M, N, dtype=torch.float32)
    nblk = -(-M // BLOCK_ROWS)

    def fill(b):
        g = torch.Generator().manual_seed(block_seed(seed, tag, b))
        r0, r1 = b * BLOCK_ROWS, min(M, (b + 1) * BLOCK_ROWS)
        if kind == "normal":
            torch.randn(r1 - r0, N, generator=g, out=out[r0:r1])
        else:
            torch.rand(r1 - r0, N, generator=g, out=out[r0:r1])

    if nblk <= 1:
        for b in range(nblk):
            fill(b)
    else:
        with ThreadPoolExecutor(max_workers=min(nblk, os.cpu_count() or 4, 16)) as ex:
            list(ex.map(fill, range(nblk)))
    return out


def make_inputs(w: Workload) -> Dict[str, torch.Tensor]:
    """Draw the workload's inputs on the CPU (contiguous tensors).

    Returns x, dy, gamma (io dtype), beta (io dtype, only when the workload
    lists one), and ``outliers`` (column indices, or [k, 2] entry indices)
    when outliers are drawn. The saved statistics the backward reads are not
    drawn here: they are what a forward pass computes from x (the caller runs
    one).
    """
    g = torch.Generator().manual_seed(w.seed)
    M, N = w.M, w.N
    x = _blocked(w.seed, _X, M, N, "normal")
    if w.x_dist == "row_shift_scale":
        mu = torch.rand(M, 1, generator=g, dtype=torch.float32) * 4.0 - 2.0
        sc = torch.rand(M, 1, generator=g, dtype=torch.float32) * 3.5 + 0.5
        x.mul_(sc).add_(mu)
    elif w.x_dist != "normal":
        raise ValueError(w.x_dist)
    dy = _blocked(w.seed, _DY, M, N, "normal").mul_(w.dy_std)
    gamma = torch.rand(N, generator=g, dtype=torch.float32)
    gamma.mul_(w.gamma_hi - w.gamma_lo).add_(w.gamma_lo)
    out: Dict[str, torch.Tensor] = {}
    if w.with_beta:
        out["beta"] = torch.rand(N, generator=g, dtype=torch.float32).to(w.io_dtype)
    if w.outlier_frac > 0:
        if w.outlier_mode == "columns":
            cols = outlier_columns(w, g)
            if M and cols.numel():
                x[:, cols] *= w.outlier_scale
            out["outliers"] = cols
        elif w.outlier_mode == "entries":
            mask = _blocked(w.seed, _MASK, M, N, "uniform") < w.outlier_frac
            x[mask] *= w.outlier_scale
            out["outliers"] = mask.nonzero()
        else:
            raise ValueError(w.outlier_mode)
    out["x"] = x.to(w.io_dtype)
    del x
    out["dy"] = dy.to(w.io_dtype)
    del dy
    out["gamma"] = gamma.to(w.io_dtype)
    return out


def sample_rows(M: int, k: int, seed: int = 7, extra: Sequence[int] = ()) -> torch.Tensor:
    """Row indices for sampled checks: first, last, a seeded random set, and
    any extra rows (e.g. row-group boundaries), de-duplicated and sorted."""
    if M == 0:
        return torch.empty(0, dtype=torch.long)
    g = torch.Generator().manual_seed(seed)
    picks = set([0, M - 1]) | set(int(r) for r in extra if 0 <= r < M)
    picks |= set(torch.randint(0, M, (k,), generator=g).tolist())
    return torch.tensor(sorted(picks), dtype=torch.long)


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


__all__ = [
    "Workload", "WORKLOADS", "HEADLINE", "LAYERNORM", "RMSNORM", "make_inputs",
    "scaled", "sample_rows", "ceil_div",
]
