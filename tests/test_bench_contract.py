"""The benchmark's host-side contract (no GPU): byte accounting, the refusal
of several GPUs, and reading the committed counter summaries."""

from __future__ import annotations

import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from rmsnorm_backward_amd import profiling  # noqa: E402
from rmsnorm_backward_amd import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.parametrize("w", list(W.WORKLOADS.values()), ids=lambda w: w.name)
def test_byte_accounting(w):
    s = w.io_bytes
    stats = 8 if w.kind == "layernorm" else 4
    # kernel A: x, dy read, dx written, statistics, gamma once
    assert bench.kernel_a_bytes(w) == w.M * (3 * w.N * s + stats) + w.N * s
    # the whole step adds the weight gradients written
    nw = 2 if w.kind == "layernorm" else 1
    assert w.algorithmic_bytes() == bench.kernel_a_bytes(w) + nw * w.N * w.wgrad_bytes
    # forward: x read, y written, statistics written, gamma (and beta)
    assert bench.forward_bytes(w, False) == w.M * (2 * w.N * s + stats) + w.N * s
    assert bench.forward_bytes(w, True) == bench.forward_bytes(w, False) + w.N * s


def _summaries():
    d = os.path.join(ROOT, "profiles")
    return sorted(f for f in os.listdir(d) if f.startswith("pmc_dx_partials_"))


@pytest.mark.parametrize("name", _summaries())
def test_committed_traffic_is_read_from_the_right_lines(name):
    """Each summary names kernel A's and the forward's traffic on lines of their
    own; the reader must take kernel A's line, not the forward's (whose key
    contains kernel A's key)."""
    workload = name[len("pmc_dx_partials_"):-len(".md")]
    w = W.WORKLOADS[workload]
    text = open(os.path.join(ROOT, "profiles", name)).read()
    a = int(re.search(r"^traffic_bytes_per_launch:\s*([0-9]+)", text, re.M).group(1))
    assert a >= bench.kernel_a_bytes(w)
    got_a = bench.committed_traffic(workload)
    got_f = bench.committed_forward_traffic(workload)
    fm = re.search(r"^forward_traffic_bytes_per_launch:\s*([0-9]+)", text, re.M)
    if re.search(r"^kernel_source_sha256_16:\s*(\S+)", text, re.M).group(1) == \
            profiling.kernel_source_hash():
        assert got_a == a
    else:
        assert got_a is None          # a stale summary is never reported
    if fm is None:                    # a summary of kernel A alone
        assert got_f is None
        return
    f = int(fm.group(1))
    assert f >= bench.forward_bytes(w, False)
    if re.search(r"^forward_source_sha256_16:\s*(\S+)", text, re.M).group(1) == \
            profiling.forward_source_hash():
        assert got_f == f
    else:
        assert got_f is None


def test_profile_summaries_pick_the_step_kernel():
    """The trace and counter summaries compare the benchmark's kernel A (saved
    statistics) with the events, not the recompute-mode instantiation the same
    run also launches."""
    is_step_kernel_a = profiling.is_step_kernel_a
    assert is_step_kernel_a("void nb::dx_partials_kernel<1, false, nb::TBF16, 8, 2, 1, false>(a)")
    assert is_step_kernel_a("nb::dx_partials_kernel<0, false, nb::TF16, 8, 2, 2, true>")
    assert not is_step_kernel_a("void nb::dx_partials_kernel<1, true, nb::TBF16, 8, 2, 1, false>")
    assert not is_step_kernel_a("nb::reduce_partials_kernel<nb::TF32>")
    assert is_step_kernel_a("void nb::dx_partials_tworow_kernel<1, false, nb::TBF16, 3, 1, false>(a)")
    assert not is_step_kernel_a("void nb::dx_partials_tworow_kernel<0, true, nb::TBF16, 3, 2, false>")
    assert profiling.is_forward("void nb::norm_fwd_tworow_kernel<1, nb::TBF16, 3, false>(a)")
    assert profiling.is_forward("void nb::norm_fwd_kernel<1, nb::TBF16, 8, 1, false>(a)")
    assert not profiling.is_forward("void nb::fwd_rowloop_kernel<1, nb::TBF16>(a)")
    for name in ("rmsnorm_bf16_16384x4096", "layernorm_bf16_65536x8192"):
        text = open(os.path.join(ROOT, "profiles", f"kernels_{name}.md")).read()
        ratio = float(re.search(r"kernel A by the trace: [\d.]+ us \(events / trace = ([\d.]+)\)",
                                text).group(1))
        assert 0.95 < ratio < 1.05, (name, ratio)


@pytest.mark.parametrize("spec", ["rmsnorm_bf16_262144x768", "layernorm_f16_1151x8192",
                                  "rmsnorm_f32_1000x384", "layernorm_bf16_4096x4096",
                                  "rmsnorm_f16_100000x256", "layernorm_f32_128x512"])
def test_shape_and_plan_options(spec):
    """--shape builds the named shape; --plan with no edits reproduces the
    planner's threads and LDS (so an edit changes only what it names)."""
    import torch
    import rmsnorm_backward_amd as nb
    w = bench.parse_shape(W, torch, spec)
    kind, dt, mn = spec.split("_")
    assert (w.kind, W._dt(w.io_dtype), f"{w.M}x{w.N}") == (kind, dt, mn)
    with_db = w.kind == "layernorm"
    p = nb.norm_bwd_make_plan(w.kind, w.M, w.N, w.io_dtype, with_db)
    want = (p.threads, p.lds_bytes)
    q = bench.edit_plan(p.copy(), "", with_db)
    assert (q.threads, q.lds_bytes) == want
    if p.rows_per_wave == 2:
        q = bench.edit_plan(p.copy(), "rows_in_flight=8", with_db)
        assert q.threads == 256
    with pytest.raises(ValueError):
        bench.edit_plan(p.copy(), "groups=3", with_db)


@pytest.mark.parametrize("shape,count", [((4096, 1024), 12), ((128, 512), 9), ((1151, 77), 5)])
def test_placed_buffers_are_disjoint_aligned_and_seeded(shape, count):
    """The bench's buffer sets: disjoint views inside one pool, at 2 MiB (or,
    under 2 MiB, 4 KiB) offsets from the pool's start, the same for the same
    seed and different for another."""
    import torch
    bufs, pool = bench.placed_buffers(torch, "cpu", torch.bfloat16, shape, count, 7)
    nbytes = shape[0] * shape[1] * 2
    align = (2 << 20) if nbytes >= (2 << 20) else 4096
    base, end = pool.data_ptr(), pool.data_ptr() + pool.numel() * 2
    offs = sorted(b.data_ptr() - base for b in bufs)
    assert all(b.shape == shape and b.is_contiguous() for b in bufs)
    assert all(o % align == 0 for o in offs)
    assert all(b - a >= nbytes for a, b in zip(offs, offs[1:]))
    assert base + offs[-1] + nbytes <= end
    again, _ = bench.placed_buffers(torch, "cpu", torch.bfloat16, shape, count, 7)
    assert [b.data_ptr() - base for b in bufs] == [b.data_ptr() - _.data_ptr() for b in again]
    other, p2 = bench.placed_buffers(torch, "cpu", torch.bfloat16, shape, count, 8)
    assert [b.data_ptr() - base for b in bufs] != [b.data_ptr() - p2.data_ptr() for b in other]


def test_source_hash_ignores_comments_only():
    """The counters stay valid across comment edits of the kernel sources,
    and not across code edits."""
    code = "int f(int a) {\n  return a + 1;  // one more\n}\n/* a\n   block */\n"
    base = profiling._code_only(code)
    assert base == profiling._code_only(code.replace("one more", "plus one") + "\n\n// end\n")
    assert base != profiling._code_only(code.replace("a + 1", "a + 2"))
    assert "one more" not in base and "block" not in base


def test_compare_lib_loads_another_build():
    """--compare-lib takes a path to another build; the binding loads it
    beside the default library with its entry points declared, and refuses a
    missing path."""
    import rmsnorm_backward_amd as nb
    assert bench.parse_args(["--compare-lib", "/tmp/x.so"]).compare_lib == "/tmp/x.so"
    assert bench.parse_args([]).compare_lib is None
    other = nb.load_library_at(nb.library_path())
    assert other.norm_bwd_rmsnorm.argtypes is not None
    assert other.norm_bwd_workspace_bytes.restype is not None
    assert other.norm_bwd_workspace_bytes(1, 16384, 4096, 2, 0) == \
        nb.load_library().norm_bwd_workspace_bytes(1, 16384, 4096, 2, 0)
    with pytest.raises(RuntimeError):
        nb.load_library_at("/nonexistent/libnorm_bwd.so")


def test_stats_summary_names_the_instantiations(tmp_path):
    """In a run over several workloads, --kernel and --forward pick the
    named instantiations; without them the saved-statistics kernel A with the
    most calls is taken."""
    import json
    head = "Name,Calls,TotalDurationNs,AverageNs,Percentage,MinNs,MaxNs,StdDev\n"
    rows = [("void nb::dx_partials_kernel<1, false, nb::TBF16, 8, 2, 1, false, 1024>(a)", 100, 66000),
            ("void nb::dx_partials_kernel<0, false, nb::TBF16, 8, 2, 2, true, 1024>(a)", 120, 540000),
            ("void nb::dx_partials_kernel<1, true, nb::TBF16, 8, 2, 1, false, 512>(a)", 500, 70000),
            ("void nb::norm_fwd_kernel<1, nb::TBF16, 8, 2, false>(a)", 50, 46000),
            ("void nb::norm_fwd_kernel<0, nb::TBF16, 8, 2, false>(a)", 50, 370000)]
    csv_path = tmp_path / "stats.csv"
    csv_path.write_text(head + "".join(f'"{n}",{c},{c * a},{a},1.0,{a},{a},0\n' for n, c, a in rows))
    cfg = {"workload": "rmsnorm_bf16_16384x4096", "pct_of_peak": 73.0, "kernel_a_us": 66.0,
           "plan": {}, "forward": {"us": 46.0, "GBps": 5800, "pct_of_peak": 72.5}}
    bj = tmp_path / "b.json"
    bj.write_text(json.dumps({"ms_per_step": 0.0688, "value": 5850, "config": cfg}) + "\n")
    text = profiling.stats_summary(str(csv_path), str(bj), ["cmd"],
                                   kernel="dx_partials_kernel<1, false, nb::TBF16, 8, 2, 1, false, 1024>",
                                   forward="norm_fwd_kernel<1, nb::TBF16, 8, 2, false>")
    assert "kernel A by the trace: 66.00 us (events / trace = 1.000)" in text
    assert "forward by the trace: 46.00 us (events / trace = 1.000)" in text
    default = profiling.stats_summary(str(csv_path), str(bj), ["cmd"])
    assert "kernel A by the trace: 540.00 us" in default
