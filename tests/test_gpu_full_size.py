"""The three large workloads at their full size, in the launch configuration
the benchmark times (the automatic plan), against the fp64 oracle on every
output element, and bitwise over repeated runs (needs a gfx950 GPU).

dx is compared in row blocks (it is row-local, so a block of rows is an
oracle call of its own); dgamma and dbeta in column blocks, each an oracle
call over all M rows of those columns, which keeps the oracle's ascending-row
order. Blocks run on the host's cores (the oracle's C calls and NumPy release
the interpreter lock). The shapes are the worked example of "Norm backward in
Triton -- the dγ/dβ reduction" ("Worked numbers", 16384 x 4096 bf16), a wide
LayerNorm of 65536 x 8192 whose row groups sweep 4 MiB of each operand, and
262144 narrow rows of 768 features with outlier columns.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import parity
from inputs import backward_inputs
from rmsnorm_backward_amd import workloads as W

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

FULL = [W.RMS_BF16_16384x4096, W.LN_BF16_65536x8192, W.RMS_BF16_262144x768]
REPEATS = 5
BLOCK_ELEMS = 1 << 23          # elements of one oracle block (64 MiB in fp64)


@pytest.fixture(scope="module")
def nb():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import rmsnorm_backward_amd as nbmod
    nbmod.load_library()
    return nbmod


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int32 if t.element_size() == 4 else torch.int16)


def _call(nb, w, g, with_db):
    if w.kind == "layernorm":
        return nb.norm_bwd_layernorm(g["x"], g["dy"], g["gamma"], g["mean"], g["rstd"], w.eps,
                                     wgrad_dtype=w.wgrad_dtype, with_dbeta=with_db)
    return nb.norm_bwd_rmsnorm(g["x"], g["dy"], g["gamma"], g["rstd"], w.eps,
                               wgrad_dtype=w.wgrad_dtype, with_dbeta=with_db)


def _blocks(n, size):
    return [(a, min(n, a + size)) for a in range(0, n, size)]


@pytest.mark.parametrize("w", FULL, ids=lambda w: w.name)
def test_full_size_every_element_and_repeats(nb, w):
    print(f"[gen] {w.name}", flush=True)
    inp = backward_inputs(w)
    with_db = w.kind == "layernorm"
    plan = nb.norm_bwd_make_plan(w.kind, w.M, w.N, w.io_dtype, with_db)
    print(f"[run] {w.name} plan={plan.as_dict()}", flush=True)
    g = {k: v.cuda() for k, v in inp.items() if isinstance(v, torch.Tensor) and k != "outliers"}
    first = _call(nb, w, g, with_db)
    torch.cuda.synchronize()

    # bitwise over repeats, with unrelated work on another stream perturbing
    # the order in which workgroups are scheduled
    side = torch.cuda.Stream()
    junk = torch.randn(4096, 4096, device="cuda")
    for i in range(REPEATS):
        with torch.cuda.stream(side):
            junk = junk @ junk
            junk = junk / junk.abs().max()
        out = _call(nb, w, g, with_db)
        torch.cuda.synchronize()
        for a, b, name in zip(out, first, ("dx", "dgamma", "dbeta")):
            if b is None:
                assert a is None
                continue
            assert torch.equal(_bits(a), _bits(b)), f"{name} changed on repeat {i}"
        del out
    print(f"[repeat] {w.name}: {REPEATS} repeats bitwise equal", flush=True)

    dx = first[0].cpu()
    dg = first[1].cpu()
    db = first[2].cpu() if with_db else None
    del first, g, junk
    torch.cuda.empty_cache()

    x, dy, gamma, rstd = inp["x"], inp["dy"], inp["gamma"], inp["rstd"]
    mean = inp.get("mean")

    # dx, every element, in row blocks
    def rows(blk):
        r0, r1 = blk
        mb = None if mean is None else mean[r0:r1]
        rdx = oracle.bwd_dx(w.kind, x[r0:r1], dy[r0:r1], gamma, mb, rstd[r0:r1])
        scale = parity.dx_term_scale(w.kind, x[r0:r1], dy[r0:r1], gamma, mb, rstd[r0:r1])
        return parity.check_dx(w.io_dtype, dx[r0:r1], rdx, scale=scale)

    rblocks = _blocks(w.M, max(1, BLOCK_ELEMS // w.N))
    with ThreadPoolExecutor(max_workers=_threads()) as ex:
        res = list(ex.map(rows, rblocks))
    print(f"[dx] {w.name}: {w.M * w.N} elements in {len(rblocks)} row blocks, max |err| "
          f"{max(r['max_abs'] for r in res):.3g}", flush=True)

    # dgamma (dbeta), every column, in column blocks over all rows
    depth = parity.depth_fused(w.M, plan.groups)

    def cols(blk):
        c0, c1 = blk
        xc, dyc = x[:, c0:c1], dy[:, c0:c1]
        rdg, rdb = oracle.bwd_wgrad(w.kind, xc, dyc, mean, rstd, want_dbeta=with_db)
        ag, ab = parity.abs_terms(w.kind, xc, dyc, mean, rstd)
        out = [parity.check_wgrad(w.io_dtype, dg[c0:c1], rdg, absum=ag, depth=depth)]
        if with_db:
            out.append(parity.check_wgrad(w.io_dtype, db[c0:c1], rdb, "dbeta", absum=ab,
                                          depth=depth))
        return out, ab

    cblocks = _blocks(w.N, max(1, BLOCK_ELEMS // w.M))
    with ThreadPoolExecutor(max_workers=_threads()) as ex:
        res = list(ex.map(cols, cblocks))
    worst = max(r["max_err_over_bound"] for rr, _ in res for r in rr)
    print(f"[wgrad] {w.name}: {w.N} columns in {len(cblocks)} blocks, max err/bound "
          f"{worst:.3g}", flush=True)

    # dbeta is also the plain column sum of dy (a closed form)
    if with_db:
        ref = np.zeros(w.N)
        for r0, r1 in _blocks(w.M, max(1, BLOCK_ELEMS // w.N)):
            ref += parity.f64(dy[r0:r1]).sum(axis=0)
        ab = np.concatenate([a for _, a in res])
        parity.check_wgrad(w.io_dtype, db, ref, "dbeta(all)", absum=ab, depth=depth)
