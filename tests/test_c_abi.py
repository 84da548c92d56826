"""The C ABI used from plain C (tests/c_abi_consumer.c), without Python or
torch in the calling process.

Host only: the consumer's host checks (status strings, workspace sizes,
plans, argument errors). On the GPU: the consumer runs the backward through
the named entry point, an explicit plan, and kernel A then kernel B on their
own; it checks that the three give the same bytes and that a call with too
little workspace launches nothing. Its output must equal, bit for bit, what
the Python binding returns for the same inputs (the same automatic plan), and
match the fp64 oracle within the parity tolerances.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import c_abi
import oracle
import parity
from inputs import backward_inputs
from rmsnorm_backward_amd import workloads as W

_CODE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}


def _raw(t: torch.Tensor) -> bytes:
    if t.numel() == 0:
        return b""
    return t.contiguous().view(torch.uint8).numpy().tobytes()


def _from_raw(buf: bytes, dtype, shape):
    n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
    assert len(buf) == n, (len(buf), n)
    if n == 0:
        return torch.empty(shape, dtype=dtype)
    return torch.frombuffer(bytearray(buf), dtype=torch.uint8).view(dtype).reshape(shape)


def test_host_checks():
    if not c_abi.is_current():
        c_abi.build()
    r = c_abi.run("host")
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host checks ok" in r.stdout


CASES = [
    # (base workload, M, N, wgrad dtype, with dbeta)
    (W.RMS_BF16_16384x4096, 300, 4096, torch.float32, False),
    (W.RMS_BF16_262144x768, 1000, 768, torch.bfloat16, True),
    (W.LN_F16_1151x8192, 129, 1000, torch.float16, True),
    (W.LN_F32_128x512, 128, 512, torch.float32, True),
    (W.LN_BF16_65536x8192, 17, 8192, torch.float32, True),
    (W.RMS_F32_128x512, 0, 64, torch.float32, False),
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0].kind}-{c[1]}x{c[2]}-"
                         f"{str(c[0].io_dtype)[6:]}-{str(c[3])[6:]}-db{int(c[4])}")
def test_c_consumer_matches_binding_and_oracle(case, tmp_path):
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    assert c_abi.is_current(), "build the C consumer first (__graft_entry__.build())"
    import rmsnorm_backward_amd as nb
    base, M, N, wg, with_db = case
    w = W.scaled(base, M=M, N=N, wgrad_dtype=wg)
    inp = backward_inputs(w)
    ln = w.kind == W.LAYERNORM
    blob = _raw(inp["x"]) + _raw(inp["dy"]) + _raw(inp["gamma"])
    if ln:
        blob += _raw(inp["mean"])
    blob += _raw(inp["rstd"])
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    src.write_bytes(blob)
    print(f"c consumer: {w.name} wgrad {wg} dbeta {with_db}", flush=True)
    r = c_abi.run("run", str(0 if ln else 1), str(M), str(N), str(_CODE[w.io_dtype]),
                  str(_CODE[wg]), str(int(with_db)), str(src), str(dst))
    assert r.returncode == 0, r.stdout + r.stderr
    out = dst.read_bytes()
    n_dx = M * N * w.io_bytes
    n_w = N * w.wgrad_bytes
    assert len(out) == n_dx + n_w * (2 if with_db else 1)
    c_dx = _from_raw(out[:n_dx], w.io_dtype, (M, N))
    c_dg = _from_raw(out[n_dx:n_dx + n_w], wg, (N,))
    c_db = _from_raw(out[n_dx + n_w:], wg, (N,)) if with_db else None

    # the Python binding on the same inputs: the same plan, the same bits
    dev = torch.device("cuda:0")
    x, dy, g = (inp[k].to(dev) for k in ("x", "dy", "gamma"))
    rstd = inp["rstd"].to(dev)
    if ln:
        dx, dg, db = nb.norm_bwd_layernorm(x, dy, g, inp["mean"].to(dev), rstd, w.eps,
                                           wgrad_dtype=wg, with_dbeta=with_db)
    else:
        dx, dg, db = nb.norm_bwd_rmsnorm(x, dy, g, rstd, w.eps, wgrad_dtype=wg,
                                         with_dbeta=with_db)
    torch.cuda.synchronize()
    assert torch.equal(c_dx.view(torch.uint8), dx.cpu().view(torch.uint8))
    assert torch.equal(c_dg.view(torch.uint8), dg.cpu().view(torch.uint8))
    if with_db:
        assert torch.equal(c_db.view(torch.uint8), db.cpu().view(torch.uint8))

    # and the oracle
    rdx, rdg, rdb = oracle.bwd(w.kind, inp["x"], inp["dy"], inp["gamma"], inp.get("mean"),
                               inp["rstd"])
    scale = parity.dx_term_scale(w.kind, inp["x"], inp["dy"], inp["gamma"], inp.get("mean"),
                                 inp["rstd"])
    parity.check_dx(w.io_dtype, c_dx, rdx, scale=scale)
    bg, bb = parity.wgrad_bounds(w.kind, inp["x"], inp["dy"], inp.get("mean"), inp["rstd"],
                                 parity.depth_path(w.M, w.N, w.io_dtype, with_db))
    parity.check_wgrad(w.io_dtype, c_dg, rdg, **bg)
    if with_db:
        parity.check_wgrad(w.io_dtype, c_db, rdb, "dbeta", **bb)
