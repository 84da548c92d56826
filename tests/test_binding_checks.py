"""The Python binding's tensor checks (host only).

The library takes raw pointers, so the binding is what keeps a kernel from
reading or writing past a tensor: every tensor it hands over must be on x's
device, contiguous where no row stride is passed, and of the dtype and
element count the kernels assume; an explicit plan must match the tensors.

Here the device-type check is relaxed to accept CPU tensors, and the stream
lookup (the first step after the checks, before any library call) raises a
sentinel. A call that passes every check therefore ends in the sentinel; a
call that fails one raises ValueError. Nothing reaches the library's compute
entry points or a GPU.
"""

from __future__ import annotations

import pytest
import torch

import rmsnorm_backward_amd as nb


class Reached(Exception):
    """The call passed the binding's checks and was about to launch."""


@pytest.fixture
def cpu_binding(monkeypatch):
    def gpu_any(t, name):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device.type != "cpu":
            raise ValueError(f"{name}: test tensors live on the CPU")

    def stream(*_a, **_k):
        raise Reached()

    monkeypatch.setattr(nb, "_gpu_any", gpu_any)
    monkeypatch.setattr(nb, "_stream", stream)
    return nb


M, N = 12, 64
bf, f32 = torch.bfloat16, torch.float32


def inputs(dt=bf):
    return dict(x=torch.zeros(M, N, dtype=dt), dy=torch.zeros(M, N, dtype=dt),
                gamma=torch.zeros(N, dtype=dt), mean=torch.zeros(M), rstd=torch.ones(M))


def test_valid_calls_pass_the_checks(cpu_binding):
    i = inputs()
    with pytest.raises(Reached):
        nb.norm_bwd_layernorm(i["x"], i["dy"], i["gamma"], i["mean"], i["rstd"])
    with pytest.raises(Reached):
        nb.norm_bwd_rmsnorm(i["x"], i["dy"], i["gamma"], i["rstd"],
                            dx=torch.empty(M, N, dtype=bf), dgamma=torch.empty(N, dtype=bf))
    with pytest.raises(Reached):
        nb.norm_bwd_ex("layernorm", i["x"], i["dy"], i["gamma"], i["mean"], i["rstd"])
    with pytest.raises(Reached):
        nb.norm_bwd_wgrad("layernorm", i["x"], i["dy"], i["mean"], i["rstd"])
    with pytest.raises(Reached):
        nb.norm_fwd_layernorm(i["x"], i["gamma"], torch.zeros(N, dtype=bf))
    plan = nb.norm_bwd_make_plan("layernorm", M, N, bf, True)
    with pytest.raises(Reached):
        nb.norm_bwd_execute(plan, i["x"], i["dy"], i["gamma"], i["mean"], i["rstd"])
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8)
    with pytest.raises(Reached):
        nb.norm_bwd_execute_partials(plan, i["x"], i["dy"], i["gamma"], i["mean"], i["rstd"],
                                     torch.empty(M, N, dtype=bf), ws)
    with pytest.raises(Reached):
        nb.norm_bwd_reduce_partials(plan.groups, N, ws, torch.empty(N), torch.empty(N))


@pytest.mark.parametrize("over,match", [
    (dict(dx=torch.empty(M, N, dtype=f32)), "dx must be"),
    (dict(dx=torch.empty(M - 1, N, dtype=bf)), "dx must have"),
    (dict(dx=torch.empty(N, M, dtype=bf).t()), "dx must be contiguous"),
    (dict(dgamma=torch.empty(N - 1)), "dgamma must have"),
    (dict(dgamma=torch.empty(N, dtype=bf), wgrad_dtype=f32), "dgamma must be"),
    (dict(dbeta=torch.empty(2 * N)), "dbeta must have"),
    (dict(dgamma=torch.empty(N), dbeta=torch.empty(N, dtype=bf)), "dbeta must be"),
    (dict(mean=torch.zeros(M, dtype=torch.float64)), "mean must be"),
    (dict(rstd=torch.ones(M + 1)), "rstd must have"),
    (dict(gamma=torch.zeros(N + 1, dtype=bf)), "gamma must have"),
    (dict(gamma=torch.zeros(N, dtype=f32)), "gamma must be"),
    (dict(dy=torch.zeros(M, N, dtype=torch.float16)), "dy must be"),
    (dict(dy=torch.zeros(M, N + 1, dtype=bf)), "dy must have x's shape"),
    (dict(workspace=torch.empty(64, device="meta")), "workspace"),
])
def test_backward_rejects(cpu_binding, over, match):
    i = inputs()
    over = dict(over)
    i.update({k: over.pop(k) for k in list(over) if k in i})
    with pytest.raises(ValueError, match=match):
        nb.norm_bwd_layernorm(i["x"], i["dy"], i["gamma"], i["mean"], i["rstd"], **over)


def test_dgamma_dtype_sets_the_default_wgrad_dtype(cpu_binding, monkeypatch):
    """A bf16 dgamma with no wgrad_dtype is written as bf16 (not 4-byte fp32
    values into a 2-byte-per-element buffer)."""
    seen = {}
    real_code = nb._code

    def code(dtype, what):
        seen[what] = dtype
        return real_code(dtype, what)

    monkeypatch.setattr(nb, "_code", code)
    i = inputs()
    with pytest.raises(Reached):
        nb.norm_bwd_rmsnorm(i["x"], i["dy"], i["gamma"], i["rstd"],
                            dgamma=torch.empty(N, dtype=bf))
    assert seen["wgrad"] == bf


def test_plan_must_match_the_tensors(cpu_binding):
    i = inputs()
    big = nb.norm_bwd_make_plan("layernorm", 2 * M, N, bf, True)
    with pytest.raises(ValueError, match="the plan is for"):
        nb.norm_bwd_execute(big, i["x"], i["dy"], i["gamma"], i["mean"], i["rstd"])
    other = nb.norm_bwd_make_plan("layernorm", M, N, torch.float16, True)
    with pytest.raises(ValueError, match="the plan is for"):
        nb.norm_bwd_execute(other, i["x"], i["dy"], i["gamma"], i["mean"], i["rstd"])
    ws = torch.empty(big.workspace_bytes, dtype=torch.uint8)
    with pytest.raises(ValueError, match="x must have"):
        nb.norm_bwd_execute_partials(big, i["x"], i["dy"], i["gamma"], i["mean"], i["rstd"],
                                     torch.empty(M, N, dtype=bf), ws)
    plan = nb.norm_bwd_make_plan("layernorm", M, N, bf, True)
    with pytest.raises(ValueError, match="dx must have"):
        nb.norm_bwd_execute_partials(plan, i["x"], i["dy"], i["gamma"], i["mean"], i["rstd"],
                                     torch.empty(M, N - 8, dtype=bf), ws)
    with pytest.raises(ValueError, match="mean must have"):
        nb.norm_bwd_execute_partials(plan, i["x"], i["dy"], i["gamma"], i["mean"][:-1],
                                     i["rstd"], torch.empty(M, N, dtype=bf), ws)


def test_reduce_partials_rejects(cpu_binding):
    ws = torch.empty(4 * N * 4, dtype=torch.uint8)
    with pytest.raises(ValueError, match="dgamma must have"):
        nb.norm_bwd_reduce_partials(4, N, ws, torch.empty(N - 1))
    with pytest.raises(ValueError, match="dbeta must have"):
        nb.norm_bwd_reduce_partials(4, N, ws, torch.empty(N), torch.empty(N + 1))
    with pytest.raises(ValueError, match="dbeta must be"):
        nb.norm_bwd_reduce_partials(4, N, ws, torch.empty(N), torch.empty(N, dtype=bf))


def test_ex_and_wgrad_reject(cpu_binding):
    i = inputs()
    with pytest.raises(ValueError, match="dx must be"):
        nb.norm_bwd_ex("rmsnorm", i["x"], i["dy"], i["gamma"], None, i["rstd"],
                       dx=torch.empty(M, N, dtype=f32))
    with pytest.raises(ValueError, match="dgamma must have"):
        nb.norm_bwd_ex("rmsnorm", i["x"], i["dy"], i["gamma"], None, i["rstd"],
                       dgamma=torch.empty(N + 4))
    with pytest.raises(ValueError, match="rstd must have"):
        nb.norm_bwd_ex("rmsnorm", i["x"], i["dy"], i["gamma"], None, i["rstd"][:3])
    with pytest.raises(ValueError, match="rstd must have"):
        nb.norm_bwd_wgrad("rmsnorm", i["x"], i["dy"], None, i["rstd"][:3])
    with pytest.raises(ValueError, match="mean must be"):
        nb.norm_bwd_wgrad("layernorm", i["x"], i["dy"], i["mean"].half(), i["rstd"])
    with pytest.raises(ValueError, match="dbeta must have"):
        nb.norm_bwd_wgrad("layernorm", i["x"], i["dy"], i["mean"], i["rstd"],
                          dbeta=torch.empty(N - 1))


@pytest.mark.parametrize("over,match", [
    (dict(y=torch.empty(M, N, dtype=f32)), "y must be"),
    (dict(y=torch.empty(M * N - 1, dtype=bf)), "y must have"),
    (dict(mean=torch.empty(M - 1)), "mean must have"),
    (dict(rstd=torch.empty(M, dtype=bf)), "rstd must be"),
    (dict(beta=torch.zeros(N - 1, dtype=bf)), "beta must have"),
])
def test_forward_rejects(cpu_binding, over, match):
    i = inputs()
    kw = dict(beta=torch.zeros(N, dtype=bf))
    kw.update(over)
    beta = kw.pop("beta")
    with pytest.raises(ValueError, match=match):
        nb.norm_fwd_layernorm(i["x"], i["gamma"], beta, 1e-5, **kw)


def test_stream_of_another_device_is_refused(monkeypatch):
    """A torch stream object whose device differs from the tensors' is
    refused before any launch."""
    class FakeStream:
        cuda_stream = 1234
        device = torch.device("cuda", 1)

    with pytest.raises(ValueError, match="stream is on"):
        nb._stream(FakeStream(), torch.device("cuda", 0))

    class SameStream:
        cuda_stream = 1234
        device = torch.device("cuda", 0)

    assert nb._stream(SameStream(), torch.device("cuda", 0)).value == 1234
    assert nb._stream(5678, torch.device("cuda", 0)).value == 5678
