"""Rows too wide for the fused kernels (the wide-row path) against the oracle.

Above the fused limits (fp32: 16384; fp16/bf16: 16384 with dbeta, 32768
without; unaligned rows: 8192) the named entry points compute dx with one
workgroup per row -- the row held in its registers when it fits (16-byte
aligned, up to 65536 16-bit or 32768 fp32 elements; 16385 fp32, 20000 bf16
with dbeta, 32776, 40000 strided and 65536 here), else streamed in chunks by
the row loop (40000 fp32, 100000, the unaligned rows, LayerNorm recompute at
8 chunks) -- and the weight gradients with the column walk. Same formulas ("Norm backward in
Triton", "The gradients"), same tolerances as the fused path.
"""

from __future__ import annotations

import pytest
import torch

import oracle
import parity
from inputs import backward_inputs
from rmsnorm_backward_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nb():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import rmsnorm_backward_amd as nbmod
    nbmod.load_library()
    return nbmod


def bwd(nb, w, g, with_db, recompute=False, **kw):
    mean = None if recompute else g.get("mean")
    rstd = None if recompute else g["rstd"]
    if w.kind == "layernorm":
        out = nb.norm_bwd_layernorm(g["x"], g["dy"], g["gamma"], mean, rstd, w.eps,
                                    wgrad_dtype=w.wgrad_dtype, with_dbeta=with_db, **kw)
    else:
        out = nb.norm_bwd_rmsnorm(g["x"], g["dy"], g["gamma"], rstd, w.eps,
                                  wgrad_dtype=w.wgrad_dtype, with_dbeta=with_db, **kw)
    torch.cuda.synchronize()
    return tuple(None if t is None else t.cpu() for t in out)


def check_saved(w, inp, out, with_db):
    dx, dg, db = out
    rdx, rdg, rdb = oracle.bwd(w.kind, inp["x"], inp["dy"], inp["gamma"], inp.get("mean"),
                               inp["rstd"])
    scale = parity.dx_term_scale(w.kind, inp["x"], inp["dy"], inp["gamma"], inp.get("mean"),
                                 inp["rstd"])
    parity.check_dx(w.io_dtype, dx, rdx, scale=scale)
    bg, bb = parity.wgrad_bounds(w.kind, inp["x"], inp["dy"], inp.get("mean"), inp["rstd"],
                                 parity.depth_colwalk(w.M))
    parity.check_wgrad(w.io_dtype, dg, rdg, **bg)
    if with_db:
        parity.check_wgrad(w.io_dtype, db, rdb, "dbeta", **bb)


def check_recompute(w, inp, out, with_db):
    dx, dg, db = out
    mean, rstd = oracle.fwd_stats(w.kind, inp["x"], w.eps)      # fp64, not rounded
    rdx = oracle.bwd_dx(w.kind, inp["x"], inp["dy"], inp["gamma"], mean, rstd)
    t_dx, t_dg = parity.recompute_terms(w.kind, inp["x"], inp["dy"], inp["gamma"], mean, rstd)
    parity.check_dx(w.io_dtype, dx, rdx, scale=t_dx, coef32=2.0 ** -16)
    rdg, rdb = oracle.bwd_wgrad(w.kind, inp["x"], inp["dy"], mean, rstd)
    bg, bb = parity.wgrad_bounds(w.kind, inp["x"], inp["dy"], mean, rstd,
                                 parity.depth_colwalk(w.M))
    parity.check_wgrad(w.io_dtype, dg, rdg, extra=2.0 ** -16 * t_dg, **bg)
    if with_db:
        parity.check_wgrad(w.io_dtype, db, rdb, "dbeta", **bb)


WIDE = [(kind, dt, M, N)
        for kind in ("layernorm", "rmsnorm")
        for dt, M, N in ((torch.float32, 37, 16385), (torch.float32, 5, 40000),
                         (torch.bfloat16, 64, 20000), (torch.float16, 3, 32776),
                         (torch.bfloat16, 9, 100000), (torch.bfloat16, 4, 100003),
                         (torch.float16, 21, 9001), (torch.bfloat16, 600, 65536),
                         # the register-held kernels at their edges: 4 and 8
                         # full chunks, a last chunk barely used, one row
                         (torch.bfloat16, 1, 32768), (torch.float32, 2, 32768),
                         (torch.float16, 3, 16392), (torch.bfloat16, 5, 65528))]


@pytest.mark.parametrize("kind,dt,M,N", WIDE, ids=lambda v: str(v).replace("torch.", ""))
def test_wide_rows(nb, kind, dt, M, N):
    base = W.LN_F32_128x512 if kind == "layernorm" else W.RMS_F32_128x512
    w = W.scaled(base, M=M, N=N, io_dtype=dt, wgrad_dtype=torch.float32, seed=700 + M + N)
    inp = backward_inputs(w)
    g = {k: v.cuda() for k, v in inp.items() if k != "outliers"}
    for with_db in (True, False):
        check_saved(w, inp, bwd(nb, w, g, with_db), with_db)
    check_recompute(w, inp, bwd(nb, w, g, True, recompute=True), True)


def test_wide_rows_half_wgrad_and_determinism(nb):
    w = W.scaled(W.LN_BF16_65536x8192, M=300, N=24576, wgrad_dtype=torch.bfloat16)
    inp = backward_inputs(w)
    g = {k: v.cuda() for k, v in inp.items() if k != "outliers"}
    a = bwd(nb, w, g, True)
    b = bwd(nb, w, g, True)
    for ta, tb in zip(a, b):
        assert torch.equal(ta, tb)
    assert a[1].dtype == torch.bfloat16
    check_saved(w, inp, a, True)


def test_wide_rows_strided_and_accumulated(nb):
    w = W.scaled(W.LN_BF16_65536x8192, M=77, N=40000)
    inp = backward_inputs(w)
    ld = w.N + 24                                   # 16-byte aligned rows
    def strided(t):
        buf = torch.zeros(w.M * ld, dtype=t.dtype, device="cuda")
        v = buf.view(w.M, ld)[:, :w.N]
        v.copy_(t.cuda())
        return v
    x, dy = strided(inp["x"]), strided(inp["dy"])
    old = torch.randn(w.N, generator=torch.Generator().manual_seed(4)).cuda()
    dg, db = old.clone(), old.clone()
    dx, _, _ = nb.norm_bwd_ex("layernorm", x, dy, inp["gamma"].cuda(), inp["mean"].cuda(),
                              inp["rstd"].cuda(), w.eps, dgamma=dg, dbeta=db, accumulate=True)
    torch.cuda.synchronize()
    rdx, rdg, rdb = oracle.bwd(w.kind, inp["x"], inp["dy"], inp["gamma"], inp["mean"],
                               inp["rstd"])
    scale = parity.dx_term_scale(w.kind, inp["x"], inp["dy"], inp["gamma"], inp["mean"],
                                 inp["rstd"])
    parity.check_dx(w.io_dtype, dx.cpu(), rdx, scale=scale)
    bg, bb = parity.wgrad_bounds(w.kind, inp["x"], inp["dy"], inp["mean"], inp["rstd"],
                                 parity.depth_colwalk(w.M))
    parity.check_wgrad(w.io_dtype, (dg - old).cpu(), rdg, extra=2.0 ** -24 * abs(old.cpu()),
                       **bg)
    parity.check_wgrad(w.io_dtype, (db - old).cpu(), rdb, "dbeta",
                       extra=2.0 ** -24 * abs(old.cpu()), **bb)
    # explicit groups are a fused-path notion
    with pytest.raises(nb.NormBwdError) as e:
        nb.norm_bwd_ex("layernorm", x, dy, inp["gamma"].cuda(), inp["mean"].cuda(),
                       inp["rstd"].cuda(), w.eps, groups=4)
    assert e.value.status == nb.ERR_UNSUPPORTED


def test_wide_recompute_workspace(nb):
    """Recompute mode stores the statistics in the workspace: 8 bytes per row
    for LayerNorm; a shorter workspace is refused before any launch."""
    w = W.scaled(W.LN_BF16_65536x8192, M=50, N=40000)
    inp = W.make_inputs(w)
    x, dy, g = inp["x"].cuda(), inp["dy"].cuda(), inp["gamma"].cuda()
    need = nb.norm_bwd_workspace_bytes("layernorm", w.M, w.N, w.io_dtype, True)
    assert need == 8 * w.M
    with pytest.raises(nb.NormBwdError) as e:
        nb.norm_bwd_layernorm(x, dy, g, None, None, w.eps,
                              workspace=torch.empty(need - 4, dtype=torch.uint8, device="cuda"))
    assert e.value.status == nb.ERR_WORKSPACE
    out = nb.norm_bwd_layernorm(x, dy, g, None, None, w.eps,
                                workspace=torch.empty(need, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    check_recompute(w, inp, tuple(t.cpu() for t in out), True)
