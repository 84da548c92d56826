"""The autograd wrappers (rmsnorm_backward_amd.autograd) against the oracle.

A model-level use: forward through the library's forward, backward through
its backward on the statistics the forward saved. The reference is the
oracle's forward and backward on its own fp64 statistics, with the
recompute-mode allowance for the GPU's fp32 statistics (parity.recompute_terms).
"""

from __future__ import annotations

import pytest
import torch

import oracle
import parity
from rmsnorm_backward_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ag():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    from rmsnorm_backward_amd import autograd
    return autograd


@pytest.mark.parametrize("kind,dt,shape", [
    ("layernorm", torch.float32, (4, 32, 512)),
    ("rmsnorm", torch.bfloat16, (2, 300, 4096)),
    ("layernorm", torch.float16, (1151, 8192)),
    ("rmsnorm", torch.float32, (3, 5, 40000)),           # wide rows
], ids=lambda v: str(v).replace("torch.", ""))
def test_module_forward_backward(ag, kind, dt, shape):
    N = shape[-1]
    M = 1
    for d in shape[:-1]:
        M *= d
    base = W.LN_F32_128x512 if kind == "layernorm" else W.RMS_F32_128x512
    w = W.scaled(base, M=M, N=N, io_dtype=dt, seed=60 + M)
    inp = W.make_inputs(w)
    x = inp["x"].view(shape).cuda().requires_grad_(True)
    dy = inp["dy"].view(shape).cuda()
    if kind == "layernorm":
        mod = ag.LayerNorm(N, eps=w.eps, device="cuda", dtype=dt)
        beta = torch.rand(N, generator=torch.Generator().manual_seed(2)).to(dt)
        with torch.no_grad():
            mod.bias.copy_(beta)
    else:
        mod = ag.RMSNorm(N, eps=w.eps, device="cuda", dtype=dt)
        beta = None
    with torch.no_grad():
        mod.weight.copy_(inp["gamma"])
    y = mod(x)
    y.backward(dy)
    torch.cuda.synchronize()
    x2, dy2 = inp["x"], inp["dy"]
    ry, rm, rr = oracle.fwd(kind, x2, inp["gamma"], beta, w.eps)
    # y against the oracle's forward (the statistics stay inside the Function)
    parity.check_forward(dt, kind, x2, inp["gamma"], beta, y.detach().view(M, N).cpu(), None,
                         None, ry, rm, rr)
    rdx = oracle.bwd_dx(kind, x2, dy2, inp["gamma"], rm, rr)
    rdg, rdb = oracle.bwd_wgrad(kind, x2, dy2, rm, rr)
    t_dx, t_dg = parity.recompute_terms(kind, x2, dy2, inp["gamma"], rm, rr)
    parity.check_dx(dt, x.grad.view(M, N).cpu(), rdx, scale=t_dx, coef32=2.0 ** -16)
    bg, bb = parity.wgrad_bounds(kind, x2, dy2, rm, rr,
                                 parity.depth_path(M, N, dt, kind == "layernorm"))
    parity.check_wgrad(dt, mod.weight.grad.cpu(), rdg, extra=2.0 ** -16 * t_dg, **bg)
    if kind == "layernorm":
        parity.check_wgrad(dt, mod.bias.grad.cpu(), rdb, "dbeta", **bb)
    assert x.grad.shape == x.shape and x.grad.dtype == dt


def test_functional_matches_module_and_is_deterministic(ag):
    g = torch.Generator(device="cuda").manual_seed(9)
    x = torch.randn(64, 1024, device="cuda", generator=g, dtype=torch.float32)
    gamma = torch.rand(1024, device="cuda", generator=g) + 0.5
    outs = []
    for _ in range(2):
        xx = x.clone().requires_grad_(True)
        gg = gamma.clone().requires_grad_(True)
        y = ag.rms_norm(xx, gg, 1e-6)
        y.sum().backward()
        outs.append((y.detach(), xx.grad, gg.grad))
    for a, b in zip(*outs):
        assert torch.equal(a, b)
