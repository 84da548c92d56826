"""Column-walk weight gradients (norm_bwd_wgrad) against the fp64 oracle.

dgamma = sum over rows of dy * xhat, dbeta = sum of dy ("Norm backward in
Triton", "The gradients"), by workgroups that each own a tile of columns and
walk all rows (the Phobos tutorial's ln_bwd_dwdb, "05: Layer norm"). No dx and
no workspace; any N up to INT32_MAX.
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


def run(nb, w, inp, with_db, wgrad=None, **kw):
    g = {k: v.cuda() for k, v in inp.items() if k in ("x", "dy", "mean", "rstd")}
    dg, db = nb.norm_bwd_wgrad(w.kind, g["x"], g["dy"], g.get("mean"), g["rstd"],
                               wgrad_dtype=wgrad or w.wgrad_dtype, with_dbeta=with_db, **kw)
    torch.cuda.synchronize()
    return dg.cpu(), (None if db is None else db.cpu())


def check(w, inp, dg, db, cols=None):
    x, dy = (inp["x"], inp["dy"]) if cols is None else (inp["x"][:, cols], inp["dy"][:, cols])
    rdg, rdb = oracle.bwd_wgrad(w.kind, x, dy, inp.get("mean"), inp["rstd"], want_dbeta=True)
    bg, bb = parity.wgrad_bounds(w.kind, x, dy, inp.get("mean"), inp["rstd"],
                                 parity.depth_colwalk(x.shape[0]))
    parity.check_wgrad(w.io_dtype, dg if cols is None else dg[cols], rdg, **bg)
    if db is not None:
        parity.check_wgrad(w.io_dtype, db if cols is None else db[cols], rdb, "dbeta", **bb)


SMALL = [
    W.LN_F32_128x512,
    W.RMS_F32_128x512,
    W.LN_F16_1151x8192,
    W.scaled(W.RMS_BF16_16384x4096, M=2003),
    W.scaled(W.LN_BF16_65536x8192, M=777),
    W.scaled(W.RMS_BF16_262144x768, M=5001),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_wgrad_parity(nb, w):
    inp = backward_inputs(w)
    for with_db in (True, False):
        dg, db = run(nb, w, inp, with_db)
        check(w, inp, dg, db)
        assert (db is None) == (not with_db)


@pytest.mark.parametrize("kind", ["layernorm", "rmsnorm"])
@pytest.mark.parametrize("dt,M,N", [
    (torch.float32, 1, 1), (torch.float32, 3, 3), (torch.float32, 513, 65),
    (torch.float16, 2, 7), (torch.float16, 64, 1000), (torch.float16, 9, 40000),
    (torch.bfloat16, 511, 8), (torch.bfloat16, 100, 4100), (torch.bfloat16, 3, 100000),
    (torch.bfloat16, 4097, 24),
], ids=lambda v: str(v).replace("torch.", ""))
def test_wgrad_edge_shapes(nb, kind, dt, M, N):
    """Ragged tiles, the one-element path (N not a multiple of the vector),
    single rows, and N beyond the fused path's limits."""
    base = W.LN_F32_128x512 if kind == "layernorm" else W.RMS_F32_128x512
    w = W.scaled(base, M=M, N=N, io_dtype=dt, wgrad_dtype=torch.float32, seed=900 + M + N)
    inp = backward_inputs(w)
    dg, db = run(nb, w, inp, True)
    check(w, inp, dg, db)


@pytest.mark.parametrize("wdt", [torch.float16, torch.bfloat16])
def test_wgrad_output_dtypes(nb, wdt):
    w = W.scaled(W.LN_F16_1151x8192, M=300, N=2000, io_dtype=wdt, wgrad_dtype=wdt)
    inp = backward_inputs(w)
    dg, db = run(nb, w, inp, True)
    assert dg.dtype == wdt and db.dtype == wdt
    check(w, inp, dg, db)


@pytest.mark.parametrize("w", [W.RMS_BF16_16384x4096, W.LN_BF16_65536x8192,
                               W.RMS_BF16_262144x768], ids=lambda w: w.name)
def test_wgrad_full_size_sampled(nb, w):
    print(f"[gen] {w.name}", flush=True)
    inp = backward_inputs(w)
    print(f"[run] {w.name}", flush=True)
    dg, db = run(nb, w, inp, w.kind == "layernorm")
    cols = W.sample_rows(w.N, 40, seed=w.seed + 3)
    if "outliers" in inp and inp["outliers"].dim() == 1:
        cols = torch.unique(torch.cat([cols, inp["outliers"]]))
    check(w, inp, dg, db, cols=cols)
    if db is not None:  # dbeta over every column is the column sum of dy
        _, ab = parity.abs_terms(w.kind, inp["x"], inp["dy"], inp.get("mean"), inp["rstd"])
        parity.check_wgrad(w.io_dtype, db, inp["dy"].double().sum(0), "dbeta(all)", absum=ab,
                           depth=parity.depth_colwalk(w.M))


def test_wgrad_agrees_with_fused_path_and_is_deterministic(nb):
    w = W.scaled(W.LN_BF16_65536x8192, M=3000, N=3072)
    inp = backward_inputs(w)
    a = run(nb, w, inp, True)
    b = run(nb, w, inp, True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    g = {k: v.cuda() for k, v in inp.items() if k != "outliers"}
    _, fg, fb = nb.norm_bwd_layernorm(g["x"], g["dy"], g["gamma"], g["mean"], g["rstd"], w.eps)
    torch.cuda.synchronize()
    rdg, rdb = oracle.bwd_wgrad(w.kind, inp["x"], inp["dy"], inp["mean"], inp["rstd"])
    bg, _ = parity.wgrad_bounds(w.kind, inp["x"], inp["dy"], inp["mean"], inp["rstd"], 0)
    parity.check_wgrad(w.io_dtype, fg.cpu(), rdg, absum=bg["absum"],
                       depth=parity.depth_fused(w.M))
    parity.check_wgrad(w.io_dtype, a[0], rdg, absum=bg["absum"],
                       depth=parity.depth_colwalk(w.M))
    # the two orders differ, so the bits may too, by rounding only
    assert torch.allclose(a[0], fg.cpu(), rtol=1e-4, atol=1e-4 * float(fg.abs().max()))


def test_wgrad_accumulate(nb):
    w = W.scaled(W.RMS_BF16_16384x4096, M=999)
    inp = backward_inputs(w)
    s, _ = run(nb, w, inp, False)
    old = torch.randn(w.N, generator=torch.Generator().manual_seed(3))
    acc = old.clone().cuda()
    g = {k: v.cuda() for k, v in inp.items() if k in ("x", "dy", "rstd")}
    nb.norm_bwd_wgrad("rmsnorm", g["x"], g["dy"], None, g["rstd"], dgamma=acc, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(acc.cpu(), old + s)
    # an empty batch adds nothing (the previous bits, -0.0 included, survive)
    e = torch.empty(0, w.N, dtype=w.io_dtype, device="cuda")
    keep = torch.full((w.N,), -0.0, device="cuda")
    nb.norm_bwd_wgrad("rmsnorm", e, e, None, torch.empty(0, device="cuda"), dgamma=keep,
                      accumulate=True)
    torch.cuda.synchronize()
    assert torch.all(keep.view(torch.int32) == torch.tensor(-0.0).view(torch.int32).item())


def test_wgrad_empty_batch_writes_zeros(nb):
    e = torch.empty(0, 96, dtype=torch.bfloat16, device="cuda")
    dg = torch.full((96,), float("nan"), device="cuda")
    db = torch.full((96,), float("nan"), device="cuda")
    st = torch.empty(0, device="cuda")
    nb.norm_bwd_wgrad("layernorm", e, e, st, st, dgamma=dg, dbeta=db)
    torch.cuda.synchronize()
    assert torch.all(dg == 0) and torch.all(db == 0)


def test_wgrad_misaligned_takes_the_scalar_path(nb):
    w = W.scaled(W.RMS_BF16_16384x4096, M=100, N=1024)
    inp = backward_inputs(w)
    buf = torch.zeros(2, w.M * w.N + 1, dtype=w.io_dtype, device="cuda")
    x = buf[0, 1:].view(w.M, w.N)
    dy = buf[1, 1:].view(w.M, w.N)
    x.copy_(inp["x"].cuda())
    dy.copy_(inp["dy"].cuda())
    dg, _ = nb.norm_bwd_wgrad("rmsnorm", x, dy, None, inp["rstd"].cuda())
    torch.cuda.synchronize()
    check(w, inp, dg.cpu(), None)
