"""HIP graph capture of the library's launches, and non-finite inputs.

* The forward and backward launch only kernels on the caller's stream (no
  allocation, no memset, no host synchronisation), so a captured graph
  replays them. Each replay, with new inputs copied in eagerly between
  replays, must equal the eager result bit for bit.
* NaN/Inf inputs propagate as the arithmetic does: compared position by
  position with the fp64 oracle run on the same bits.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from inputs import backward_inputs
from rmsnorm_backward_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nb():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import rmsnorm_backward_amd as nbmod
    nbmod.load_library()
    return nbmod


@pytest.mark.parametrize("kind", ["rmsnorm", "layernorm"])
def test_graph_replays_match_eager(nb, kind):
    base = W.RMS_BF16_16384x4096 if kind == "rmsnorm" else W.LN_BF16_65536x8192
    w = W.scaled(base, M=1000, N=2048)
    with_db = kind == "layernorm"
    dev = torch.device("cuda")
    x = torch.empty(w.M, w.N, dtype=w.io_dtype, device=dev)
    dy = torch.empty_like(x)
    g = torch.empty(w.N, dtype=w.io_dtype, device=dev)
    y, dx = torch.empty_like(x), torch.empty_like(x)
    mean = torch.empty(w.M, device=dev)
    rstd = torch.empty(w.M, device=dev)
    dg = torch.empty(w.N, device=dev)
    db = torch.empty(w.N, device=dev) if with_db else None
    ws = torch.empty(nb.norm_bwd_workspace_bytes(kind, w.M, w.N, w.io_dtype, with_db),
                     dtype=torch.uint8, device=dev)

    def step():
        if kind == "layernorm":
            nb.norm_fwd_layernorm(x, g, None, w.eps, y=y, mean=mean, rstd=rstd)
            nb.norm_bwd_layernorm(x, dy, g, mean, rstd, w.eps, dx=dx, dgamma=dg, dbeta=db,
                                  workspace=ws)
        else:
            nb.norm_fwd_rmsnorm(x, g, w.eps, y=y, rstd=rstd)
            nb.norm_bwd_rmsnorm(x, dy, g, rstd, w.eps, dx=dx, dgamma=dg, workspace=ws)

    def load(seed):
        inp = W.make_inputs(W.scaled(w, seed=seed))
        x.copy_(inp["x"])
        dy.copy_(inp["dy"])
        g.copy_(inp["gamma"])

    def snapshot():
        return [t.clone() for t in (y, rstd, dx, dg) + ((mean, db) if with_db else ())]

    # eager references for three input sets
    refs = []
    for seed in (11, 12, 13):
        load(seed)
        step()
        torch.cuda.synchronize()
        refs.append(snapshot())
    # capture once (warm up on a side stream first, as graph capture expects)
    load(11)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(2):
        for seed, ref in zip((11, 12, 13), refs):
            load(seed)                      # eager work between replays
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for a, b in zip(snapshot(), ref):
                assert torch.equal(a, b), (kind, rep, seed)


def _same_pattern(got, ref, what):
    g = got.double().numpy() if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    assert np.array_equal(np.isnan(g), np.isnan(r)), f"{what}: NaN positions differ"
    assert np.array_equal(np.isposinf(g), np.isposinf(r)), f"{what}: +inf positions differ"
    assert np.array_equal(np.isneginf(g), np.isneginf(r)), f"{what}: -inf positions differ"


@pytest.mark.parametrize("M,N", [(64, 512), (65, 384), (64, 128)],
                         ids=["one-row-per-wave", "two-rows-3-chunks", "two-rows-1-chunk"])
@pytest.mark.parametrize("kind", ["rmsnorm", "layernorm"])
def test_non_finite_inputs_propagate_like_the_arithmetic(nb, kind, M, N):
    base = W.RMS_F32_128x512 if kind == "rmsnorm" else W.LN_F32_128x512
    w = W.scaled(base, M=M, N=N)
    inp = backward_inputs(w)
    x, dy = inp["x"].clone(), inp["dy"].clone()
    x[3, 17] = float("nan")
    dy[9, 100] = float("inf")
    dy[9, 101] = float("-inf")           # inf - inf in the row sums -> NaN
    dy[20, 5] = float("inf")
    g = {k: v.cuda() for k, v in inp.items() if k in ("gamma", "mean", "rstd")}
    if kind == "layernorm":
        dx, dg, db = nb.norm_bwd_layernorm(x.cuda(), dy.cuda(), g["gamma"], g["mean"],
                                           g["rstd"], w.eps)
    else:
        dx, dg, db = nb.norm_bwd_rmsnorm(x.cuda(), dy.cuda(), g["gamma"], g["rstd"], w.eps,
                                         with_dbeta=True)
    cg, cb = nb.norm_bwd_wgrad(kind, x.cuda(), dy.cuda(), g.get("mean"), g["rstd"],
                               with_dbeta=True)
    torch.cuda.synchronize()
    rdx, rdg, rdb = oracle.bwd(kind, x, dy, inp["gamma"], inp.get("mean"), inp["rstd"])
    _same_pattern(dx.cpu(), rdx, "dx")
    _same_pattern(dg.cpu(), rdg, "dgamma")
    _same_pattern(db.cpu(), rdb, "dbeta")
    _same_pattern(cg.cpu(), rdg, "column-walk dgamma")
    _same_pattern(cb.cpu(), rdb, "column-walk dbeta")
    # rows without a non-finite input stay finite
    clean = [r for r in range(w.M) if r not in (3, 9, 20)]
    assert torch.isfinite(dx.cpu()[clean]).all()


@pytest.mark.parametrize("N", [512, 384, 128])
@pytest.mark.parametrize("kind", ["rmsnorm", "layernorm"])
def test_forward_non_finite_rows(nb, kind, N):
    """A NaN or an infinity in a row of x makes that row's statistics and y
    non-finite as the oracle's arithmetic does; the other rows, including
    the other row of a two-row pair, stay finite."""
    base = W.RMS_F32_128x512 if kind == "rmsnorm" else W.LN_F32_128x512
    w = W.scaled(base, M=33, N=N)
    inp = W.make_inputs(w)
    x = inp["x"].clone()
    x[4, 7] = float("nan")
    x[11, N - 1] = float("inf")
    x[32, 0] = float("-inf")                 # the last row: a pair of one row
    g = inp["gamma"]
    if kind == "layernorm":
        y, mean, rstd = nb.norm_fwd_layernorm(x.cuda(), g.cuda(), None, w.eps)
    else:
        y, rstd = nb.norm_fwd_rmsnorm(x.cuda(), g.cuda(), w.eps)
        mean = None
    torch.cuda.synchronize()
    ry, rm, rr = oracle.fwd(kind, x, g, None, w.eps)
    _same_pattern(y.cpu(), ry, "y")
    _same_pattern(rstd.cpu(), rr, "rstd")
    if mean is not None:
        _same_pattern(mean.cpu(), rm, "mean")
    clean = [r for r in range(w.M) if r not in (4, 11, 32)]
    assert torch.isfinite(y.cpu()[clean]).all() and torch.isfinite(rstd.cpu()[clean]).all()
