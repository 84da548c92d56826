"""torch.autograd Functions and nn.Modules over the library's forward and
backward, so a model can use them in place of torch's LayerNorm/RMSNorm.

Marshalling only: the forward is norm_fwd_layernorm / norm_fwd_rmsnorm (it
saves fp32 mean/rstd), the backward is norm_bwd_layernorm / norm_bwd_rmsnorm
on those statistics. Features are the last dimension; leading dimensions are
flattened into rows. gamma (and beta) share x's dtype; their gradients are
accumulated in fp32 by the kernels and rounded once to that dtype.
"""

from __future__ import annotations

from typing import Optional

import torch

from . import (norm_bwd_layernorm, norm_bwd_rmsnorm, norm_fwd_layernorm,
               norm_fwd_rmsnorm)


def _rows(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().view(-1, t.shape[-1])


class LayerNormFunction(torch.autograd.Function):
    """y = (x - mean) * rstd * gamma + beta over the last dimension."""

    @staticmethod
    def forward(ctx, x, gamma, beta, eps: float):
        x2 = _rows(x)
        y, mean, rstd = norm_fwd_layernorm(x2, gamma.contiguous(),
                                           None if beta is None else beta.contiguous(), eps)
        ctx.save_for_backward(x2, gamma, mean, rstd)
        ctx.eps = eps
        ctx.has_beta = beta is not None
        return y.view(x.shape)

    @staticmethod
    def backward(ctx, dy):
        x2, gamma, mean, rstd = ctx.saved_tensors
        dx, dg, db = norm_bwd_layernorm(x2, _rows(dy), gamma.contiguous(), mean, rstd, ctx.eps,
                                        wgrad_dtype=gamma.dtype, with_dbeta=ctx.has_beta)
        return dx.view(dy.shape), dg, db, None


class RMSNormFunction(torch.autograd.Function):
    """y = x * rstd * gamma over the last dimension, rstd = 1/sqrt(mean(x^2) + eps)."""

    @staticmethod
    def forward(ctx, x, gamma, eps: float):
        x2 = _rows(x)
        y, rstd = norm_fwd_rmsnorm(x2, gamma.contiguous(), eps)
        ctx.save_for_backward(x2, gamma, rstd)
        ctx.eps = eps
        return y.view(x.shape)

    @staticmethod
    def backward(ctx, dy):
        x2, gamma, rstd = ctx.saved_tensors
        dx, dg, _ = norm_bwd_rmsnorm(x2, _rows(dy), gamma.contiguous(), rstd, ctx.eps,
                                     wgrad_dtype=gamma.dtype)
        return dx.view(dy.shape), dg, None


class LayerNorm(torch.nn.Module):
    """LayerNorm over the last dimension (weight and optional bias)."""

    def __init__(self, features: int, eps: float = 1e-5, bias: bool = True,
                 device=None, dtype=None):
        super().__init__()
        self.eps = eps
        self.weight = torch.nn.Parameter(torch.ones(features, device=device, dtype=dtype))
        self.bias = (torch.nn.Parameter(torch.zeros(features, device=device, dtype=dtype))
                     if bias else None)

    def forward(self, x):
        return LayerNormFunction.apply(x, self.weight, self.bias, self.eps)


class RMSNorm(torch.nn.Module):
    """RMSNorm over the last dimension (weight only)."""

    def __init__(self, features: int, eps: float = 1e-6, device=None, dtype=None):
        super().__init__()
        self.eps = eps
        self.weight = torch.nn.Parameter(torch.ones(features, device=device, dtype=dtype))

    def forward(self, x):
        return RMSNormFunction.apply(x, self.weight, self.eps)


def layer_norm(x, gamma, beta: Optional[torch.Tensor] = None, eps: float = 1e-5):
    return LayerNormFunction.apply(x, gamma, beta, eps)


def rms_norm(x, gamma, eps: float = 1e-6):
    return RMSNormFunction.apply(x, gamma, eps)


__all__ = ["LayerNormFunction", "RMSNormFunction", "LayerNorm", "RMSNorm", "layer_norm",
           "rms_norm"]
