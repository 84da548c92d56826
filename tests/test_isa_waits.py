"""The steady-state loops of kernel A keep their register ring in flight.

Read from the gfx950 assembly of this repository's own kernel sources
(compiled here with the library's flags; no GPU): in each steady-state loop
(the loop whose accesses are all buffer loads and stores) every
`s_waitcnt vmcnt(n)` leaves n accesses in flight. vmcnt counts loads and
stores in issue order, so a wait with a small n also waits for the row pairs
loaded ahead: the ring drains. The two-rows-per-wave RMSNorm kernel needed a
scheduling fence between row pairs for this (without it, waits went down to
1 of 18 loads); the one-row-per-wave kernels of the large workloads keep
their waits through the per-row barrier.
"""

from __future__ import annotations

import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from rmsnorm_backward_amd import _build as B  # noqa: E402


def _assembly(tmp, src):
    out = os.path.join(tmp, os.path.splitext(src)[0] + ".s")
    flags = [f for f in B.common_flags() if f != "-fPIC"]
    subprocess.run([B.hipcc(), *flags, "--cuda-device-only", "-S", os.path.join(B.CSRC, src),
                    "-o", out], check=True, capture_output=True, text=True)
    return open(out).read()


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    try:
        B.hipcc()
    except Exception as e:  # pragma: no cover - the toolchain is part of the image
        pytest.skip(f"hipcc unavailable: {e}")
    tmp = str(tmp_path_factory.mktemp("asm"))
    with ThreadPoolExecutor(2) as ex:
        texts = list(ex.map(lambda s: _assembly(tmp, s), ("tworow.hip", "kernels_bf16.hip")))
    return "\n".join(texts)


def steady_loop(text, prefix):
    """The instructions of the steady-state loop of the kernel whose mangled
    name starts with `prefix`: the backward branch's body that holds buffer
    loads and no global loads."""
    m = re.search(r"^(" + re.escape(prefix) + r"\S*):", text, re.M)
    assert m, prefix
    lines = text[m.start():].split("\n")
    end = next(i for i, l in enumerate(lines) if l.strip().startswith(".Lfunc_end"))
    body = lines[:end]
    labels = {}
    for i, l in enumerate(body):
        lm = re.match(r"^(\.LBB\d+_\d+):", l)
        if lm:
            labels[lm.group(1)] = i
    for i, l in enumerate(body):
        bm = re.search(r"s_c?branch\w*\s+(\.LBB\d+_\d+)", l)
        if bm and bm.group(1) in labels and labels[bm.group(1)] < i:
            seg = [x.strip() for x in body[labels[bm.group(1)]:i + 1]
                   if x.strip() and not x.strip().startswith((";", "."))]
            if any(x.startswith("buffer_load") for x in seg) and \
                    not any(x.startswith("global_load_dwordx4") for x in seg):
                return seg
    raise AssertionError(f"no steady-state loop in {prefix}")


def waits(seg):
    return [int(re.search(r"vmcnt\((\d+)\)", x).group(1))
            for x in seg if x.startswith("s_waitcnt") and "vmcnt" in x]


# (kernel, fewest accesses every wait must leave in flight)
# (unfenced, the two-row RMSNorm loops waited down to 7, 3 and 1; fenced they
# keep 9, 6 and 14)
CASES = [
    # 262144 x 768 bf16 RMSNorm: two rows per wave, 3 chunks, saved statistics
    ("_ZN2nb25dx_partials_tworow_kernelILi1ELb0ENS_5TBF16ELi3ELi1ELb0E", 8),
    # 1048576 x 256 bf16 RMSNorm: two rows per wave, 1 chunk
    ("_ZN2nb25dx_partials_tworow_kernelILi1ELb0ENS_5TBF16ELi1ELi1ELb0E", 5),
    # 262144 x 384 fp32 RMSNorm: two rows per wave, 3 chunks
    ("_ZN2nb25dx_partials_tworow_kernelILi1ELb0ENS_4TF32ELi3ELi1ELb0E", 10),
    # 16384 x 4096 bf16 RMSNorm: one row per wave, 2 chunks, 4 waves a row
    ("_ZN2nb18dx_partials_kernelILi1ELb0ENS_5TBF16ELi8ELi2ELi1ELb0ELi1024E", 8),
    # 65536 x 8192 bf16 LayerNorm with dbeta, non-temporal partials
    ("_ZN2nb18dx_partials_kernelILi0ELb0ENS_5TBF16ELi8ELi2ELi2ELb1ELi1024E", 6),
    # the two-row forward on rows of 3 chunks (a ring of two row pairs): the
    # next pair's 3 loads stay in flight (unfenced, the waits went down to 0)
    ("_ZN2nb22norm_fwd_tworow_kernelILi0ENS_5TBF16ELi3ELb0E", 3),
    ("_ZN2nb22norm_fwd_tworow_kernelILi1ENS_5TBF16ELi3ELb0E", 3),
]


@pytest.mark.parametrize("prefix,least", CASES, ids=[c[0][9:60] for c in CASES])
def test_steady_loops_keep_loads_in_flight(asm, prefix, least):
    seg = steady_loop(asm, prefix)
    w = waits(seg)
    loads = sum(x.startswith("buffer_load") for x in seg)
    assert loads >= 6 and w, (prefix, loads, w)
    assert min(w) >= least, (prefix, w)
