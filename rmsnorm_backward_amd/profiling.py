"""Summaries of rocprofv3 output for the profiles/ directory.

Two summaries, each a short Markdown text that records the exact commands
that produced it:

* ``stats``: per-kernel durations from ``rocprofv3 --kernel-trace --stats``
  (kernel_stats.csv), next to the kernel-A time the benchmark measured with
  HIP events in the same run (its JSON line), so the two can be compared.

* ``pmc``: HBM traffic of kernel A from two counter runs, ``--pmc
  FETCH_SIZE`` and ``--pmc WRITE_SIZE`` (counter_collection.csv, KiB per
  dispatch). Each counter is calibrated on the benchmark's plain copy kernel
  of known size in the same run: scale = bytes the copy moves / bytes the
  counter reports for it. The summary carries the kernel source hash, so the
  benchmark reports the traffic only while the kernel is unchanged.

Usage:
  python -m rmsnorm_backward_amd.profiling stats KERNEL_STATS_CSV BENCH_JSON --cmd "..."
  python -m rmsnorm_backward_amd.profiling pmc FETCH_CSV WRITE_CSV BENCH_JSON --cmd "..." --cmd "..."
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import statistics
import sys

KERNEL_A = "dx_partials_kernel"
KERNEL_A_TWOROW = "dx_partials_tworow_kernel"
KERNEL_B = "reduce_partials_kernel"
FORWARD = "norm_fwd_kernel"
FORWARD_TWOROW = "norm_fwd_tworow_kernel"
COLWALK = "wgrad_colwalk_kernel"
COPY = "copy_probe_kernel"
TRIAD = "triad_probe_kernel"
_HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCE = os.path.join(_HERE, "csrc", "nb_device.hpp")
# kernel A's sources: the one-row-per-wave kernel and the two-rows-per-wave one
KERNEL_A_SOURCES = (KERNEL_SOURCE, os.path.join(_HERE, "csrc", "nb_tworow.hpp"))
FORWARD_SOURCES = (KERNEL_SOURCE, os.path.join(_HERE, "csrc", "nb_forward.hpp"),
                   os.path.join(_HERE, "csrc", "nb_tworow.hpp"))


def _code_only(text: str) -> str:
    """The source without its comments, trailing blanks and empty lines: an
    edit of a comment does not change the kernel the counters were taken on.
    (The kernel sources hold no string literals that contain comment
    markers.)"""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", line).rstrip() for line in text.splitlines())
    return "\n".join(line for line in lines if line)


def _hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(p, encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def kernel_source_hash() -> str:
    """Hash of kernel A's sources (the counters are valid while it holds)."""
    return _hash(KERNEL_A_SOURCES)


def forward_source_hash() -> str:
    """Hash of the forward kernel's sources."""
    return _hash(FORWARD_SOURCES)


def _bench(path):
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("{"):
                return json.loads(line)
    raise ValueError(f"no JSON line in {path}")


def is_step_kernel_a(name: str) -> bool:
    """Kernel A as the benchmark's step and roofline time it: the instantiation
    that reads the saved statistics (template argument RECOMP = false), not
    the recompute-mode one the same run also launches, of either layout (one
    or two rows per wave)."""
    return re.search("(" + KERNEL_A + "|" + KERNEL_A_TWOROW + r")<\s*\d+\s*,\s*false\s*,",
                     name) is not None


def is_forward(name: str) -> bool:
    """The fused forward of either layout (not the row-loop forward)."""
    return FORWARD in name or FORWARD_TWOROW in name


def stats_summary(stats_csv: str, bench_json: str, cmds, kernel=None, forward=None) -> str:
    """`kernel` / `forward`: substrings naming the instantiations to compare
    with the events (a run over several workloads launches several); by
    default the saved-statistics kernel A with the most calls and any fused
    forward."""
    rows = list(csv.DictReader(open(stats_csv)))
    b = _bench(bench_json)
    c = b["config"]
    out = [f"# Kernel durations: {c['workload']}", "",
           "Commands (run from the repository root on one MI355X):", "", "```"]
    out += list(cmds) + ["```", "",
                         "| kernel | calls | average (us) | min (us) | max (us) | share |",
                         "|---|---|---|---|---|---|"]
    avg_a = avg_f = avg_b = None
    calls_a = -1
    for r in rows:
        name = r["Name"]
        short = name.split("(")[0].replace("void ", "")
        avg = float(r["AverageNs"]) / 1e3
        if kernel is not None:
            if kernel in name:
                avg_a = avg
        elif is_step_kernel_a(name) and int(r["Calls"]) > calls_a:
            avg_a, calls_a = avg, int(r["Calls"])
        if (forward in name) if forward is not None else is_forward(name):
            avg_f = avg
        if KERNEL_B in name:
            avg_b = avg
        out.append(f"| `{short}` | {r['Calls']} | {avg:.2f} | {float(r['MinNs'])/1e3:.2f} | "
                   f"{float(r['MaxNs'])/1e3:.2f} | {float(r['Percentage']):.1f}% |")
    out += ["", "Benchmark line of the same run (HIP events on the launch stream):", "",
            f"- step: {b['ms_per_step']*1e3:.2f} us, {b['value']} GB/s ({c['pct_of_peak']}% of 8 TB/s)",
            f"- kernel A by events: {c['kernel_a_us']} us",
            f"- plan: {json.dumps(c['plan'])}"]
    if "kernel_b_in_place_us" in c:
        out.append(f"- kernel B in place (step minus kernel A, events): "
                   f"{c['kernel_b_in_place_us']} us")
    if avg_b is not None:
        out.append(f"- kernel B by the trace (average over every launch of the run): "
                   f"{avg_b:.2f} us")
    tri = c.get("triad_probe")
    if tri:
        out.append(f"- triad ceiling by events: {tri['GBps']} GB/s (grid {tri['grid']}, unroll "
                   f"{tri['unroll']}); step at {c.get('pct_of_triad')}% of it")
    if avg_a is not None:
        out.append(f"- kernel A by the trace: {avg_a:.2f} us "
                   f"(events / trace = {c['kernel_a_us'] / avg_a:.3f})")
    fw = c.get("forward")
    if fw:
        out.append(f"- forward by events: {fw['us']} us, {fw['GBps']} GB/s "
                   f"({fw['pct_of_peak']}% of 8 TB/s)")
        if avg_f is not None:
            out.append(f"- forward by the trace: {avg_f:.2f} us "
                       f"(events / trace = {fw['us'] / avg_f:.3f})")
    out += ["", f"kernel_source_sha256_16: {kernel_source_hash()}",
            f"forward_source_sha256_16: {forward_source_hash()}", ""]
    return "\n".join(out)


def _counter_rows(path, counter):
    rows = list(csv.DictReader(open(path)))
    per_dispatch = {}
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        key = (int(r["Dispatch_Id"]), r["Kernel_Name"], r.get("Grid_Size", ""))
        per_dispatch[key] = per_dispatch.get(key, 0.0) + float(r["Counter_Value"])
    return per_dispatch


def _mean_for(per_dispatch, needle):
    """Median counter value per dispatch of a kernel, and the dispatch count.
    For the column walk only the launches of the benchmarked workload count:
    bench.py also runs it for the wide-row workload, after the benchmarked
    one, so the (kernel, grid) pair dispatched first is taken."""
    if needle == KERNEL_A:
        vals = [v for (d, name, g), v in per_dispatch.items() if is_step_kernel_a(name)]
    elif needle == FORWARD:
        vals = [v for (d, name, g), v in per_dispatch.items() if is_forward(name)]
    elif needle == COLWALK:
        hits = sorted((d, name, g, v) for (d, name, g), v in per_dispatch.items() if needle in name)
        vals = [v for d, name, g, v in hits if hits and (name, g) == hits[0][1:3]]
    else:
        vals = [v for (d, name, g), v in per_dispatch.items() if needle in name]
    return (statistics.median(vals), len(vals)) if vals else (None, 0)


def pmc_summary(fetch_csv: str, write_csv: str, bench_json: str, cmds) -> str:
    b = _bench(bench_json)
    c = b["config"]
    copy_bytes = c["copy_probe_bytes"]
    f = _counter_rows(fetch_csv, "FETCH_SIZE")
    w = _counter_rows(write_csv, "WRITE_SIZE")
    fa, na = _mean_for(f, KERNEL_A)
    wa, _ = _mean_for(w, KERNEL_A)
    fc, nc = _mean_for(f, COPY)
    wc, _ = _mean_for(w, COPY)
    fb, _ = _mean_for(f, KERNEL_B)
    wb, _ = _mean_for(w, KERNEL_B)
    if fa is None or fc is None or wc is None or wa is None:
        raise ValueError("counter rows for kernel A or the copy kernel are missing")
    fscale = copy_bytes / (fc * 1024.0)
    wscale = copy_bytes / (wc * 1024.0)
    read_bytes = fa * 1024.0 * fscale
    write_bytes = wa * 1024.0 * wscale
    alg = b["roofline"]["bytes_per_launch"]
    alg_read = alg - c["M"] * c["N"] * (2 if c["io_dtype"] != "f32" else 4)
    alg_write = alg - alg_read
    ws = c["workspace_bytes"]
    traffic = int(round(read_bytes + write_bytes))
    out = [f"# HBM traffic of kernel A: {c['workload']}", "",
           "Commands (run from the repository root on one MI355X; counters in runs of their own):",
           "", "```"] + list(cmds) + ["```", "",
           f"Calibration on the copy kernel ({copy_bytes} bytes read and written per launch,",
           f"{nc} launches): FETCH_SIZE reads {fc:.1f} KiB -> scale {fscale:.4f}; "
           f"WRITE_SIZE reads {wc:.1f} KiB -> scale {wscale:.4f}.", "",
           "| kernel A, per launch | counter (KiB) | scaled bytes | algorithmic bytes | ratio |",
           "|---|---|---|---|---|",
           f"| read (FETCH_SIZE) | {fa:.1f} | {read_bytes:.0f} | {alg_read} | {read_bytes/alg_read:.4f} |",
           f"| write (WRITE_SIZE) | {wa:.1f} | {write_bytes:.0f} | {alg_write} (+{ws} workspace) | "
           f"{write_bytes/(alg_write + ws):.4f} |",
           f"| total | | {traffic} | {alg} (+{ws}) | {traffic/(alg + ws):.4f} |", ""]
    if fb is not None and wb is not None:
        out.append(f"Kernel B per launch: FETCH_SIZE {fb:.1f} KiB ({fb*1024*fscale:.0f} B), "
                   f"WRITE_SIZE {wb:.1f} KiB ({wb*1024*wscale:.0f} B); workspace {ws} B.")
    ff, nf = _mean_for(f, FORWARD)
    wf, _ = _mean_for(w, FORWARD)
    fw = c.get("forward")
    ftraffic = None
    if ff is not None and wf is not None and fw:
        fr, fwb = ff * 1024.0 * fscale, wf * 1024.0 * wscale
        ftraffic = int(round(fr + fwb))
        falg = fw["bytes_per_launch"]
        out += ["", "| forward, per launch | counter (KiB) | scaled bytes |", "|---|---|---|",
                f"| read (FETCH_SIZE) | {ff:.1f} | {fr:.0f} |",
                f"| write (WRITE_SIZE) | {wf:.1f} | {fwb:.0f} |",
                f"| total | | {ftraffic} (algorithmic {falg}, ratio {ftraffic / falg:.4f}) |",
                "", f"forward launches counted: {nf}",
                f"forward_traffic_bytes_per_launch: {ftraffic}",
                f"forward_source_sha256_16: {forward_source_hash()}"]
    fc_, ncw = _mean_for(f, COLWALK)
    wc_, _ = _mean_for(w, COLWALK)
    cw = c.get("colwalk_wgrad")
    if fc_ is not None and wc_ is not None and cw:
        cr, cwb = fc_ * 1024.0 * fscale, wc_ * 1024.0 * wscale
        ct = int(round(cr + cwb))
        out += ["", "| column walk, per launch | counter (KiB) | scaled bytes |", "|---|---|---|",
                f"| read (FETCH_SIZE) | {fc_:.1f} | {cr:.0f} |",
                f"| write (WRITE_SIZE) | {wc_:.1f} | {cwb:.0f} |",
                f"| total | | {ct} (algorithmic {cw['bytes']}, ratio {ct / cw['bytes']:.4f}) |",
                "", f"column-walk launches counted: {ncw}"]
    out += ["", f"kernel A launches counted: {na}",
            f"traffic_bytes_per_launch: {traffic}",
            f"kernel_source_sha256_16: {kernel_source_hash()}", ""]
    return "\n".join(out)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("stats_csv")
    s.add_argument("bench_json")
    s.add_argument("--cmd", action="append", default=[])
    s.add_argument("--kernel", default=None, help="substring naming kernel A's instantiation")
    s.add_argument("--forward", default=None, help="substring naming the forward's")
    p = sub.add_parser("pmc")
    p.add_argument("fetch_csv")
    p.add_argument("write_csv")
    p.add_argument("bench_json")
    p.add_argument("--cmd", action="append", default=[])
    a = ap.parse_args(argv)
    if a.what == "stats":
        sys.stdout.write(stats_summary(a.stats_csv, a.bench_json, a.cmd, a.kernel, a.forward))
    else:
        sys.stdout.write(pmc_summary(a.fetch_csv, a.write_csv, a.bench_json, a.cmd))


if __name__ == "__main__":
    main()
