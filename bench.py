#!/usr/bin/env python3
"""Benchmark the LayerNorm / RMSNorm backward pass on one MI355X.

One step = one full backward pass (kernel A: dx + per-group partial
dgamma/dbeta; kernel B: fixed-order reduction of the partials) over one batch
of synthetic, seeded inputs already resident in HBM. The headline workload is
the 16384 x 4096 bf16 RMSNorm backward (fp32 rstd and dgamma), the worked
example of "Norm backward in Triton -- the dγ/dβ reduction".

A default run measures, in this order: the streaming ceiling (a
2-read:1-write non-temporal triad probe swept over launch shapes), the
headline workload (exactly --steps timed steps after --warmup untimed ones,
plus its forward, recompute mode, strided/accumulating call and column walk),
then each other workload (128 x 512 fp32 LayerNorm and RMSNorm, 1151 x 8192
fp16 LayerNorm, 65536 x 8192 bf16 LayerNorm, 262144 x 768 bf16 RMSNorm), and
last the fp64 CPU oracle on each workload's inputs, on one thread and on
every core. --workload NAME measures that one workload alone.

Timing: HIP events recorded on the stream the library launches on (torch's
current stream). Input/output buffer sets are rotated so that consecutive
steps touch different memory (the set count makes the rotation exceed the
256 MB Infinity Cache several times over): every step streams from HBM,
except where all sets together fit in that cache (128 x 512, flagged
cache_resident). The x, dy and dx buffers of the sets (at least four) are
carved from one pool in a seeded random order with random gaps, so the
rotation averages over the operands' relative placement in HBM: kernel A on
long row groups moves by up to 10% with it (65536 x 8192 bf16 LayerNorm,
527-578 us over ten placements) while the triad does not (512-517 us); a
single placement would inherit whatever the run's earlier allocations left.
The same-size triad runs on the same buffers.

The saved statistics the backward reads are produced by the library's GPU
forward; the forward is also timed on its own (config.forward).

Prints ONE JSON line. `value` is algorithmic GB/s of the headline's whole
step: bytes = read x, dy, gamma, saved stats; write dx, dgamma(, dbeta)
(workspace traffic excluded). `roofline` is kernel A alone against the 8 TB/s
HBM peak; `cpu_baseline` is the fp64 CPU oracle timed on this host;
`config.workloads` holds one entry per workload with the same figures.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import random
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "norm-backward achieved HBM GB/s and % of peak (16384×4096 bf16 RMSNorm)"
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E, published
MALL_BYTES = 256 << 20        # Infinity Cache
PROFILES = os.path.join(ROOT, "profiles")


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--workload", default=None, help="workload name (default: the headline)")
    ap.add_argument("--shape", default=None,
                    help="KIND_DTYPE_MxN (e.g. rmsnorm_bf16_65536x1024): that shape alone, with "
                         "the distributions of the headline (RMSNorm) or of 65536x8192 "
                         "(LayerNorm)")
    ap.add_argument("--plan", default=None,
                    help="plan field overrides, e.g. rows_in_flight=8,rows_per_wave=1 (the "
                         "explicit-plan path; the library validates the edited plan)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="one-thread oracle time on the primary workload")
    ap.add_argument("--cpu-seconds-other", type=float, default=3.0,
                    help="one-thread oracle time on each other workload")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the forward, recompute, strided and column-walk measurements")
    ap.add_argument("--no-wide", action="store_true", help="skip the wide-row measurement")
    ap.add_argument("--no-triad", action="store_true", help="skip the triad ceiling sweep")
    ap.add_argument("--sets", type=int, default=0, help="buffer sets to rotate (0 = auto)")
    ap.add_argument("--groups", type=int, default=0, help="explicit row-group count (0 = auto)")
    ap.add_argument("--triad-policies", action="store_true",
                    help="also sweep the triad over every load/store cache policy, at 512 MiB "
                         "and at the first workload's x size (config.triad_policies)")
    ap.add_argument("--widths", default=None,
                    help="also time bf16 RMSNorm and LayerNorm at these row widths (comma "
                         "separated), about 64M elements per operand each "
                         "(config.widths)")
    ap.add_argument("--placements", type=int, default=0,
                    help="also time the workload over this many seeded random placements of its "
                         "operands, with the triad on the same buffers (config.workloads[]."
                         "placements)")
    ap.add_argument("--compare-lib", default=None,
                    help="another build of the library (a .so path): time its backward step, "
                         "recompute mode and forward against this build's on the same buffers, "
                         "in alternating loops, and check that one call of each gives the same "
                         "bytes (config.workloads[].compare_lib)")
    ap.add_argument("--compare-plan", default=None,
                    help="with --placements: also time this edited plan (as --plan) on the same "
                         "buffers of every placement")
    return ap.parse_args(argv)


def kernel_source_hash() -> str:
    """Hash of kernel A's sources (the committed counters hold while it does)."""
    from rmsnorm_backward_amd import profiling
    return profiling.kernel_source_hash()


def committed_traffic(workload: str):
    """HBM bytes per kernel-A launch from the committed counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, f"pmc_dx_partials_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"^kernel_source_sha256_16:\s*([0-9a-f]{16})", text, re.M)
    t = re.search(r"^traffic_bytes_per_launch:\s*([0-9]+)", text, re.M)
    if not m or not t or m.group(1) != kernel_source_hash():
        return None
    return int(t.group(1))


def committed_forward_traffic(workload: str):
    """HBM bytes per forward launch from the same counter summary, if it was
    taken on the current forward source; else None."""
    from rmsnorm_backward_amd import profiling
    path = os.path.join(PROFILES, f"pmc_dx_partials_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"^forward_source_sha256_16:\s*([0-9a-f]{16})", text, re.M)
    t = re.search(r"^forward_traffic_bytes_per_launch:\s*([0-9]+)", text, re.M)
    if not m or not t or m.group(1) != profiling.forward_source_hash():
        return None
    return int(t.group(1))


def kernel_a_bytes(w) -> int:
    """Algorithmic bytes of one kernel-A launch: x, dy read and dx written
    (3*N*s per row), the saved statistics (4 or 8 B per row), gamma once."""
    s = w.io_bytes
    stats = 8 if w.kind == "layernorm" else 4
    return w.M * (3 * w.N * s + stats) + w.N * s


def forward_bytes(w, with_beta: bool) -> int:
    """Algorithmic bytes of one forward launch: x read and y written (2*N*s
    per row), the statistics written (4 or 8 B per row), gamma (and beta)."""
    s = w.io_bytes
    stats = 8 if w.kind == "layernorm" else 4
    return w.M * (2 * w.N * s + stats) + w.N * s * (2 if with_beta else 1)


def parse_shape(W, torch, spec: str):
    """KIND_DTYPE_MxN -> a workload of that shape with the distributions of
    the headline (RMSNorm) or of 65536 x 8192 (LayerNorm)."""
    kind, dt, mn = spec.split("_")
    M, N = (int(v) for v in mn.split("x"))
    dtype = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dt]
    base = W.LN_BF16_65536x8192 if kind == "layernorm" else W.HEADLINE
    if kind not in ("layernorm", "rmsnorm"):
        raise ValueError(f"unknown kind in --shape {spec}")
    return W.scaled(base, M=M, N=N, io_dtype=dtype, name=spec)


def edit_plan(plan, spec: str, with_db: bool):
    """Apply --plan overrides (field=value, comma separated) and make threads
    and lds_bytes consistent with them, as the planner would."""
    for item in filter(None, spec.split(",")):
        k, v = item.split("=")
        if k not in ("rows_in_flight", "rows_per_wave", "waves_per_row", "chunks"):
            raise ValueError(f"--plan: cannot set {k}")
        setattr(plan, k, int(v))
    nacc = 2 if with_db else 1
    S, C, P, vec = plan.waves_per_row, plan.chunks, plan.rows_in_flight, plan.vec
    M = plan.M
    if plan.rows_per_wave == 2:
        plan.threads = 32 * P
        plan.lds_bytes = nacc * C * 32 * vec * 4 if P > 2 else 0
        # groups of adjacent row pairs
        pairs = -(-M // 2)
        plan.groups = min(plan.groups, pairs)
        plan.rows_per_group = 2 * -(-pairs // plan.groups) if plan.groups else 0
    else:
        plan.threads = 64 * S * P
        plan.lds_bytes = S * C * 64 * vec * 4 if P > 1 else 0
        plan.rows_per_group = -(-M // plan.groups) if plan.groups else 1
    plan.grid = min(plan.groups, 1 << 20)
    plan.workspace_bytes = nacc * plan.groups * plan.N * 4
    return plan


def time_loop(torch, fn, steps, stream):
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(steps):
        fn(i)
    end.record(stream)
    end.synchronize()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps  # ms per call


def measure_wide(torch, nb, W, lib, dev, stream, args):
    """The wide-row path (rows beyond the fused limits): 1024 x 65536 bf16
    RMSNorm, backward step (row-loop dx + column walk) and forward. Bytes are
    the same algorithmic count as the fused path's; the row loop reads each
    row twice and the column walk once more, so traffic exceeds them."""
    w = W.scaled(W.HEADLINE, M=1024, N=65536, name="rmsnorm_bf16_1024x65536")
    inp = W.make_inputs(w)
    sets = []
    for i in range(3):
        s = {k: inp[k].to(dev) for k in ("x", "dy", "gamma")}
        s["y"] = torch.empty_like(s["x"])
        s["rstd"] = torch.empty(w.M, device=dev)
        s["dx"] = torch.empty_like(s["x"])
        sets.append(s)
    dg = torch.empty(w.N, device=dev)
    io = nb._DTYPE_CODE[w.io_dtype]
    P = ctypes.c_void_p
    sh = P(stream.cuda_stream)
    pt = lambda t: P(t.data_ptr())  # noqa: E731
    for s in sets:
        lib.norm_fwd_rmsnorm(pt(s["x"]), pt(s["gamma"]), w.M, w.N, io, w.eps, pt(s["y"]),
                             pt(s["rstd"]), sh)

    def fwd(i):
        s = sets[i % 3]
        if lib.norm_fwd_rmsnorm(pt(s["x"]), pt(s["gamma"]), w.M, w.N, io, w.eps, pt(s["y"]),
                                pt(s["rstd"]), sh):
            raise RuntimeError(nb.norm_bwd_last_error())

    def bwd(i):
        s = sets[i % 3]
        if lib.norm_bwd_rmsnorm(pt(s["x"]), pt(s["dy"]), pt(s["gamma"]), pt(s["rstd"]), w.M,
                                w.N, io, 0, w.eps, pt(s["dx"]), pt(dg), None, None, 0, sh):
            raise RuntimeError(nb.norm_bwd_last_error())

    steps = max(args.steps // 5, 20)
    for i in range(20):
        bwd(i)
        fwd(i)
    ms_b = time_loop(torch, bwd, steps, stream)
    ms_f = time_loop(torch, fwd, steps, stream)
    b_bytes = w.algorithmic_bytes()
    f_bytes = forward_bytes(w, False)
    return {"workload": w.name, "backward_us": round(ms_b * 1e3, 2),
            "backward_GBps": round(b_bytes / (ms_b * 1e-3) / 1e9, 1),
            "backward_pct_of_peak": round(100 * b_bytes / (ms_b * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2),
            "forward_us": round(ms_f * 1e3, 2),
            "forward_GBps": round(f_bytes / (ms_f * 1e-3) / 1e9, 1),
            "forward_pct_of_peak": round(100 * f_bytes / (ms_f * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2)}


def cpu_baseline(w, inp, seconds=10.0, seconds_threads=5.0):
    """The fp64 oracle (plain C, one thread) on the same workload, timed on
    this host for about `seconds`; then on every core for `seconds_threads`.
    Inputs are widened to fp64 before the clock starts."""
    import numpy as np

    import oracle
    o = oracle.default()
    max_rows = max(1, (1 << 27) // max(w.N, 1))      # bound the sample (~1-20 s)
    rows = min(w.M, max_rows)
    x = inp["x"][:rows].double().numpy()
    dy = inp["dy"][:rows].double().numpy()
    gamma = inp["gamma"].double().numpy()
    # the saved statistics: the oracle's forward, rounded to fp32 (untimed)
    m64, r64 = o.fwd_stats(w.kind, x, w.eps)
    rstd = r64.astype(np.float32).astype(np.float64)
    mean = m64.astype(np.float32).astype(np.float64) if w.kind == "layernorm" else None
    # repeat the pass until about `seconds` of CPU time has accumulated (at
    # most 200 passes)
    reps, total = 0, 0.0
    while reps < 200 and (total < seconds or reps < 1):
        t0 = time.perf_counter()
        o.bwd(w.kind, x, dy, gamma, mean, rstd, want_dbeta=w.kind == "layernorm")
        total += time.perf_counter() - t0
        reps += 1
    dt = total / reps
    import dataclasses
    ws = dataclasses.replace(w, M=rows)
    sample = (f"full {w.M}x{w.N} workload" if rows == w.M else
              f"first {rows} of {w.M} rows x {w.N}") + \
        f", fp64 passes (dx, dgamma{', dbeta' if w.kind == 'layernorm' else ''}) repeated " \
        f"{reps}x, {total:.1f} s total, mean per pass"
    out = {"value": round(ws.algorithmic_bytes() / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
           "kind": "oracle", "sample": sample, "seconds_per_pass": round(dt, 4),
           "cpu_model": cpu_model()}
    out["all_cores"] = cpu_baseline_threads(o, w, x, dy, gamma, mean, rstd,
                                            ws.algorithmic_bytes(), seconds_threads)
    return out


def cpu_baseline_threads(o, w, x, dy, gamma, mean, rstd, nbytes, seconds=5.0):
    """The same, unchanged oracle run on every core this process may use (at
    most 16): each thread takes a contiguous slice of the sample's rows (the
    C calls release the interpreter lock), and the slices' dgamma (dbeta)
    sums are added in slice order. Reported beside the one-thread figure."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    try:
        threads = len(os.sched_getaffinity(0))
    except AttributeError:
        threads = os.cpu_count() or 1
    threads = max(1, min(threads, 16, x.shape[0]))
    bounds = np.linspace(0, x.shape[0], threads + 1).astype(int)
    want_db = w.kind == "layernorm"

    def part(i):
        lo, hi = bounds[i], bounds[i + 1]
        return o.bwd(w.kind, x[lo:hi], dy[lo:hi], gamma,
                     None if mean is None else mean[lo:hi], rstd[lo:hi], want_dbeta=want_db)

    reps, total = 0, 0.0
    with ThreadPoolExecutor(max_workers=threads) as ex:
        while reps < 200 and (total < seconds or reps < 1):
            t0 = time.perf_counter()
            res = list(ex.map(part, range(threads)))
            for k in (1, 2) if want_db else (1,):
                acc = res[0][k].copy()
                for r in res[1:]:
                    acc += r[k]
            total += time.perf_counter() - t0
            reps += 1
    dt = total / reps
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "seconds_per_pass": round(dt, 4), "reps": reps}


def cpu_model() -> str:
    """The host CPU's model name (Linux /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def triad_sweep(torch, nb, dev, stream, operand_bytes):
    """The 2-read:1-write streaming ceiling: norm_bwd_probe_triad over three
    operands of `operand_bytes` each (together several times the 256 MB
    Infinity Cache), swept over launch shapes; the fastest is the ceiling."""
    n = operand_bytes // 4
    a = torch.empty(n, dtype=torch.int32, device=dev).fill_(1)
    b = torch.empty_like(a).fill_(2)
    c = torch.empty_like(a)
    sweep = []
    for grid in (1024, 2048, 4096, 8192, 0):
        for unroll in (1, 2, 4, 8):
            for _ in range(3):
                nb.norm_bwd_probe_triad(a, b, c, grid, unroll)
            ms = time_loop(torch, lambda i: nb.norm_bwd_probe_triad(a, b, c, grid, unroll), 10,
                           stream)
            sweep.append((grid, unroll, 3 * operand_bytes / (ms * 1e-3) / 1e9))
    # the one-pass buffer-load form (kernel A's addressing), non-temporal
    for unroll in (1, 2, 4):
        def go(i, unroll=unroll):
            nb.norm_bwd_probe_triad_policy(a, b, c, unroll, nb.POLICY_NT, nb.POLICY_NT)
        for i in range(3):
            go(i)
        ms = time_loop(torch, go, 10, stream)
        sweep.append(("buffer", unroll, 3 * operand_bytes / (ms * 1e-3) / 1e9))
    torch.cuda.synchronize()
    ok = bool(torch.all(c == 3).item())
    del a, b, c
    torch.cuda.empty_cache()
    best = max(sweep, key=lambda t: t[2])
    return {"kernel": "triad_policy_kernel" if best[0] == "buffer" else "triad_probe_kernel",
            "what": "c = a + b, 16-byte non-temporal loads and stores, 2 reads : 1 write as "
            "kernel A (grid 'buffer': the one-pass buffer-load form)",
            "bytes_per_operand": operand_bytes,
            "GBps": round(best[2], 1), "grid": best[0], "unroll": best[1],
            "pct_of_peak": round(100 * best[2] / PEAK_HBM_GBPS, 2), "result_ok": ok,
            "sweep_min_GBps": round(min(t[2] for t in sweep), 1), "launch_shapes": len(sweep),
            "sweep": [[g, u, round(v, 1)] for g, u, v in sweep]}


def triad_policy_sweep(torch, nb, lib, dev, stream, operand_bytes, steps):
    """norm_bwd_probe_triad_policy over every pair of load and store cache
    policies (ORs of sc0, nt, sc1) and 1, 2, 4 vectors per thread, on
    operands of `operand_bytes` (rounded down to 16 KiB) rotated over enough
    sets to stream from HBM; best of two rounds per variant."""
    nbytes = min(operand_bytes, 0xFFFFFFFF - 16383) // 16384 * 16384
    n = nbytes // 4
    nsets = max(1, min(16, math.ceil(4 * MALL_BYTES / (3 * nbytes))))
    sets = [[torch.empty(n, dtype=torch.int32, device=dev).fill_(k) for k in (1, 2, 0)]
            for _ in range(nsets)]
    P = ctypes.c_void_p
    sh = P(stream.cuda_stream)
    ptrs = [[P(t.data_ptr()) for t in s] for s in sets]
    times = {}
    for _ in range(2):
        for unroll in (1, 2, 4):
            for lp in nb.POLICIES:
                for sp in nb.POLICIES:
                    def go(i):
                        a, b, c = ptrs[i % nsets]
                        if lib.norm_bwd_probe_triad_policy(a, b, c, nbytes, unroll, lp, sp, sh):
                            raise RuntimeError(nb.norm_bwd_last_error())
                    for i in range(3):
                        go(i)
                    ms = time_loop(torch, go, steps, stream)
                    key = (lp, sp, unroll)
                    times[key] = min(times.get(key, ms), ms)
    torch.cuda.synchronize()
    ok = all(bool(torch.all(s[2] == 3).item()) for s in sets)
    del sets
    torch.cuda.empty_cache()
    gbps = {k: 3 * nbytes / (ms * 1e-3) / 1e9 for k, ms in times.items()}
    nt_both = [v for (lp, sp, _), v in gbps.items() if lp & nb.POLICY_NT and sp & nb.POLICY_NT]
    other = [v for (lp, sp, _), v in gbps.items()
             if not (lp & nb.POLICY_NT and sp & nb.POLICY_NT)]
    best = max(gbps, key=gbps.get)
    return {"what": "c = a + b in one pass, 16-byte buffer loads and stores under each load and "
                    "store cache policy (1 sc0, 2 nt, 16 sc1, and their ORs), 1-4 vectors a "
                    "thread", "bytes_per_operand": nbytes, "buffer_sets": nsets,
            "result_ok": ok, "best": {"load_policy": best[0], "store_policy": best[1],
                                      "unroll": best[2], "GBps": round(gbps[best], 1)},
            "nt_on_both_GBps": [round(min(nt_both), 1), round(max(nt_both), 1)],
            "otherwise_GBps": [round(min(other), 1), round(max(other), 1)],
            "all": [[lp, sp, u, round(v, 1)] for (lp, sp, u), v in
                    sorted(gbps.items(), key=lambda kv: -kv[1])]}


# Launch shapes of the same-size triad (grid, unroll); grid 0 = one pass.
SAME_SIZE_SHAPES = ((0, 1), (0, 2), (0, 4), (256, 4), (512, 4), (1024, 2), (1024, 4), (2048, 2))


def placed_buffers(torch, dev, dtype, shape, count, seed):
    """`count` tensors of `shape` carved from one pool (returned second) in a
    seeded random order with random gaps of up to half a tensor between them,
    at 2 MiB granularity (4 KiB for tensors under 2 MiB): each buffer set's x,
    dy and dx then sit at random relative offsets, and a timing that rotates
    over the sets averages over the placement."""
    eb = torch.tensor([], dtype=dtype).element_size()
    numel = math.prod(shape)
    align = (2 << 20) if numel * eb >= (2 << 20) else 4096
    slots = -(-numel * eb // align)
    rng = random.Random(seed)
    gaps = [rng.randrange(0, slots // 2 + 1) for _ in range(count)]
    order = list(range(count))
    rng.shuffle(order)
    pool = torch.empty((sum(gaps) + count * slots) * align // eb, dtype=dtype, device=dev)
    out, pos = [None] * count, 0
    for gap, k in zip(gaps, order):
        pos += gap
        out[k] = pool[pos * align // eb:pos * align // eb + numel].view(shape)
        pos += slots
    return out, pool


def triad_launchers(nb, lib, nbytes, sh, shapes=SAME_SIZE_SHAPES):
    """(label, call(a, b, c)) for every triad form tried as a ceiling on
    operands of nbytes: norm_bwd_probe_triad at each (grid, unroll) of
    `shapes` (global loads), and norm_bwd_probe_triad_policy with
    non-temporal loads and stores at 1, 2 and 4 vectors a thread (buffer
    loads, as kernel A streams) where nbytes allows it."""
    out = []
    for grid, unroll in shapes:
        def call(a, b, c, grid=grid, unroll=unroll):
            if lib.norm_bwd_probe_triad(a, b, c, nbytes, grid, unroll, sh):
                raise RuntimeError(nb.norm_bwd_last_error())
        out.append((f"global grid {grid} unroll {unroll}", call))
    for unroll in (1, 2, 4):
        if nbytes % (4096 * unroll) or nbytes > 0xFFFFFFFF - 16383:
            continue
        def call(a, b, c, unroll=unroll):
            if lib.norm_bwd_probe_triad_policy(a, b, c, nbytes, unroll, nb.POLICY_NT,
                                               nb.POLICY_NT, sh):
                raise RuntimeError(nb.norm_bwd_last_error())
        out.append((f"buffer nt unroll {unroll}", call))
    return out


def triad_same_size(torch, nb, lib, dev, stream, sets, operand_bytes, steps):
    """The triad over one workload's own x and dy into its dx (as 32-bit
    words), rotating over the same buffer sets as kernel A: the achievable
    rate for that many bytes per launch at the same placement, fixed costs
    included, best of the forms triad_launchers lists. Launched through the C
    entry points with prepared arguments, as kernel A is timed. Overwrites
    dx."""
    nbytes = operand_bytes // 16 * 16
    nsets = len(sets)
    P = ctypes.c_void_p
    sh = P(stream.cuda_stream)
    ptrs = [[P(s[k].data_ptr()) for k in ("x", "dy", "dx")] for s in sets]
    best = (0.0, None, None)
    for label, call in triad_launchers(nb, lib, nbytes, sh):
        def go(i):
            call(*ptrs[i % nsets])
        for i in range(5):
            go(i)
        ms = time_loop(torch, go, steps, stream)
        gbps = 3 * nbytes / (ms * 1e-3) / 1e9
        if gbps > best[0]:
            best = (gbps, label, ms)
    return {"GBps": round(best[0], 1), "us": round(best[2] * 1e3, 3), "form": best[1],
            "bytes_per_launch": 3 * nbytes}


def backward_args(w, sets, plan, dgamma, dbeta, ws, io, wg, sh):
    """Prepared C arguments per buffer set: those of the named entry point
    (automatic plan) and those of norm_bwd_execute_partials (explicit plan)."""
    P = ctypes.c_void_p
    ptr = lambda t: None if t is None else P(t.data_ptr())  # noqa: E731
    full_args, part_args = [], []
    for s in sets:
        if w.kind == "layernorm":
            full_args.append((ptr(s["x"]), ptr(s["dy"]), ptr(s["gamma"]), ptr(s["mean"]),
                              ptr(s["rstd"]), w.M, w.N, io, wg, w.eps, ptr(s["dx"]), ptr(dgamma),
                              ptr(dbeta), ptr(ws), ws.numel(), sh))
        else:
            full_args.append((ptr(s["x"]), ptr(s["dy"]), ptr(s["gamma"]), ptr(s["rstd"]), w.M,
                              w.N, io, wg, w.eps, ptr(s["dx"]), ptr(dgamma), ptr(dbeta), ptr(ws),
                              ws.numel(), sh))
        part_args.append((ctypes.byref(plan), ptr(s["x"]), ptr(s["dy"]), ptr(s["gamma"]),
                          ptr(s.get("mean")), ptr(s["rstd"]), ptr(s["dx"]), ptr(ws), ws.numel(),
                          sh))
    return full_args, part_args


def backward_step(nb, lib, w, explicit, full_args, part_args, wg, dgamma, dbeta):
    """step(i): the whole backward on buffer set i mod len(sets), through the
    named entry point or, with an explicit plan, norm_bwd_execute."""
    P = ctypes.c_void_p
    dg = P(dgamma.data_ptr())
    db = None if dbeta is None else P(dbeta.data_ptr())
    fn = lib.norm_bwd_layernorm if w.kind == "layernorm" else lib.norm_bwd_rmsnorm
    n = len(full_args)

    def step(i):
        if explicit:
            a = part_args[i % n]
            st = lib.norm_bwd_execute(a[0], a[1], a[2], a[3], a[4], a[5], wg, a[6], dg, db, a[7],
                                      a[8], a[9])
        else:
            st = fn(*full_args[i % n])
        if st:
            raise RuntimeError(nb.norm_bwd_last_error())
    return step


def compare_builds(torch, nb, lib, other, w, sets, full_args, dgamma, dbeta, ws, io, stream,
                   steps, path, rounds=8):
    """This build and `other`, another build of the library, on the same
    buffer sets and workspace: the backward step (named entry point,
    automatic plan), the backward in recompute mode (NULL statistics) and the
    forward, each timed in alternating loops of `steps` steps (`rounds`
    each), and whether one call of each build on buffer set 0 writes the
    same bytes."""
    with_db = dbeta is not None
    kind = 0 if w.kind == "layernorm" else 1
    need = other.norm_bwd_workspace_bytes(kind, w.M, w.N, io, int(with_db))
    if need > ws.numel():
        raise RuntimeError(f"{path} needs a {need}-byte workspace, the bench holds {ws.numel()}")
    P = ctypes.c_void_p
    sh = P(stream.cuda_stream)
    ptr = lambda t: None if t is None else P(t.data_ptr())  # noqa: E731
    rc_args = [(a[0], a[1], a[2], None, None) + a[5:] if kind == 0
               else (a[0], a[1], a[2], None) + a[4:] for a in full_args]
    fwd_args = [(ptr(s["x"]), ptr(s["gamma"]), ptr(s.get("beta")), w.M, w.N, io, w.eps,
                 ptr(s["dx"]), ptr(s["f_mean"]), ptr(s["f_rstd"]), sh) if kind == 0
                else (ptr(s["x"]), ptr(s["gamma"]), w.M, w.N, io, w.eps, ptr(s["dx"]),
                      ptr(s["f_rstd"]), sh) for s in sets]
    bwd = "norm_bwd_layernorm" if kind == 0 else "norm_bwd_rmsnorm"
    fwd = "norm_fwd_layernorm" if kind == 0 else "norm_fwd_rmsnorm"
    s0 = sets[0]
    modes = {
        "backward": (bwd, full_args, (s0["dx"], dgamma, dbeta)),
        "recompute": (bwd, rc_args, (s0["dx"], dgamma, dbeta)),
        "forward": (fwd, fwd_args, (s0["dx"], s0["f_mean"] if kind == 0 else None, s0["f_rstd"])),
    }
    out = {"path": path, "rounds": rounds, "steps_per_round": steps}
    for mode, (name, args, outputs) in modes.items():
        def make(L, name=name, args=args):
            fn = getattr(L, name)

            def step(i):
                st = fn(*args[i % len(args)])
                if st:
                    raise RuntimeError(f"{name} returned {st}")
            return step
        fa, fb = make(lib), make(other)
        snaps = []
        for f in (fa, fb):
            f(0)
            torch.cuda.synchronize()
            snaps.append([t.clone() for t in outputs if t is not None])
        same = all(torch.equal(a.view(torch.uint8), b.view(torch.uint8))
                   for a, b in zip(snaps[0], snaps[1]))
        for i in range(max(10, steps // 2)):
            fa(i)
            fb(i)
        ta, tb = [], []
        for _ in range(rounds):
            ta.append(time_loop(torch, fa, steps, stream))
            tb.append(time_loop(torch, fb, steps, stream))
        ma, mb = sorted(ta)[len(ta) // 2], sorted(tb)[len(tb) // 2]
        out[mode] = {"this_us": round(ma * 1e3, 3), "other_us": round(mb * 1e3, 3),
                     "other_over_this": round(mb / ma, 4), "bitwise_equal": bool(same)}
    return out


def graph_step_time(torch, nb, w, sets, dgamma, dbeta, ws, steps):
    """ms per backward step replayed from a captured HIP graph: one capture
    of a step on every buffer set in turn (the named entry point through the
    binding, on the capturing stream), warmed up on a side stream first,
    replayed until at least `steps` steps have run. The launches' host cost
    drops out, so on small workloads this is the GPU's own time per step."""
    def call(s):
        if w.kind == "layernorm":
            nb.norm_bwd_layernorm(s["x"], s["dy"], s["gamma"], s["mean"], s["rstd"], w.eps,
                                  wgrad_dtype=w.wgrad_dtype, dx=s["dx"], dgamma=dgamma,
                                  dbeta=dbeta, with_dbeta=dbeta is not None, workspace=ws)
        else:
            nb.norm_bwd_rmsnorm(s["x"], s["dy"], s["gamma"], s["rstd"], w.eps,
                                wgrad_dtype=w.wgrad_dtype, dx=s["dx"], dgamma=dgamma,
                                dbeta=dbeta, with_dbeta=dbeta is not None, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for s in sets:
            call(s)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for s in sets:
            call(s)
    replays = max(2, math.ceil(steps / len(sets)))
    graph.replay()
    stream = torch.cuda.current_stream()
    ms = time_loop(torch, lambda i: graph.replay(), replays, stream) / len(sets)
    del graph
    return ms


def placement_study(torch, nb, lib, dev, stream, w, args, base, plan, count):
    """The backward step and the triad over `count` placements of the
    operands: for each, two buffer sets whose x, dy and dx are carved from
    one pool at seeded random offsets (placed_buffers), timed with the
    benchmark's plan and, with --compare-plan, with the edited plan on the
    same buffers, then the triad on the same buffers (best of its one-pass
    global-load and buffer-load forms). Returns per-placement times and their summary."""
    sh = ctypes.c_void_p(stream.cuda_stream)
    with_db = w.kind == "layernorm"
    io = nb._DTYPE_CODE[w.io_dtype]
    wg = nb._DTYPE_CODE[w.wgrad_dtype]
    variants = [("plan", plan, bool(args.groups or args.plan))]
    if args.compare_plan:
        other = nb.norm_bwd_make_plan(w.kind, w.M, w.N, w.io_dtype, with_db, args.groups)
        variants.append(("compare_plan", edit_plan(other, args.compare_plan, with_db), True))
    ws_bytes = max([p.workspace_bytes for _, p, _ in variants] +
                   [nb.norm_bwd_workspace_bytes(w.kind, w.M, w.N, io, with_db)])
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    dgamma = torch.empty(w.N, dtype=w.wgrad_dtype, device=dev)
    dbeta = torch.empty(w.N, dtype=w.wgrad_dtype, device=dev) if with_db else None
    steps = max(50, int(0.2e6 / max(1.0, w.algorithmic_bytes() / 6.0e6)))
    nbytes = w.M * w.N * w.io_bytes // 16 * 16
    rows = []
    for j in range(count):
        big, pool = placed_buffers(torch, dev, w.io_dtype, (w.M, w.N), 6,
                                   w.seed * 1000003 + 7919 * (j + 1))
        sets = []
        for i in range(2):
            s = {k: v for k, v in base.items() if k not in ("x", "dy")}
            s["x"], s["dy"], s["dx"] = big[3 * i], big[3 * i + 1], big[3 * i + 2]
            s["x"].copy_(base["x"])
            s["dy"].copy_(base["dy"])
            sets.append(s)
        row = {"placement": j,
               "offsets_MiB": [round((t.data_ptr() - pool.data_ptr()) / 2**20) for t in big]}
        for name, p, explicit in variants:
            full_args, part_args = backward_args(w, sets, p, dgamma, dbeta, ws, io, wg, sh)
            step = backward_step(nb, lib, w, explicit, full_args, part_args, wg, dgamma, dbeta)
            for i in range(steps // 4):
                step(i)
            row[name + "_us"] = round(min(time_loop(torch, step, steps, stream)
                                          for _ in range(2)) * 1e3, 2)
        ptrs = [[ctypes.c_void_p(s[k].data_ptr()) for k in ("x", "dy", "dx")] for s in sets]
        best = None
        for _, call in triad_launchers(nb, lib, nbytes, sh, ((0, 1), (0, 4))):
            def go(i):
                call(*ptrs[i % 2])
            for i in range(4):
                go(i)
            ms = time_loop(torch, go, steps, stream)
            best = ms if best is None else min(best, ms)
        row["triad_us"] = round(best * 1e3, 2)
        rows.append(row)
        print(f"bench.py: placement {j}: " + ", ".join(f"{k} {v}" for k, v in row.items()
                                                       if k.endswith("_us")),
              file=sys.stderr, flush=True)
        del sets, big, pool
        torch.cuda.empty_cache()
    out = {"what": "backward step (kernel A + B) and the triad on the same buffers, per "
                   "placement of x, dy, dx (two sets each)", "count": count, "steps": steps,
           "per_placement": rows}
    for key in [k for k in rows[0] if k.endswith("_us")]:
        v = [r[key] for r in rows]
        out[key.replace("_us", "")] = {"mean_us": round(sum(v) / len(v), 2), "min_us": min(v),
                                       "max_us": max(v)}
    if args.compare_plan:
        out["compare_plan_spec"] = args.compare_plan
        out["plan_faster_in"] = sum(r["plan_us"] < r["compare_plan_us"] for r in rows)
    return out


def measure_workload(torch, nb, W, lib, dev, stream, w, args, steps, warmup, extras, triad):
    """Time one workload's backward step (kernel A + kernel B through the named
    entry point), kernel A alone and kernel B alone on rotating buffer sets;
    with `extras` also the forward, recompute mode, the strided/accumulating
    call and the column walk. Returns (entry, plan dict, extras dict, inputs)."""
    sh = ctypes.c_void_p(stream.cuda_stream)
    inp = W.make_inputs(w)
    with_db = w.kind == "layernorm"
    io = nb._DTYPE_CODE[w.io_dtype]
    wg = nb._DTYPE_CODE[w.wgrad_dtype]
    plan = nb.norm_bwd_make_plan(w.kind, w.M, w.N, w.io_dtype, with_db, args.groups)
    if args.plan:
        plan = edit_plan(plan, args.plan, with_db)
    set_bytes = 3 * w.M * w.N * w.io_bytes
    nsets = args.sets or max(4, math.ceil(4 * MALL_BYTES / max(set_bytes, 1)))
    nsets = min(nsets, 64)
    base = {k: inp[k].to(dev) for k in ("x", "dy", "gamma", "beta") if k in inp}
    # the saved statistics the backward reads come from the GPU forward
    if w.kind == "layernorm":
        _, base["mean"], base["rstd"] = nb.norm_fwd_layernorm(base["x"], base["gamma"],
                                                             base.get("beta"), w.eps)
    else:
        _, base["rstd"] = nb.norm_fwd_rmsnorm(base["x"], base["gamma"], w.eps)
    torch.cuda.synchronize()
    big, pool = placed_buffers(torch, dev, w.io_dtype, (w.M, w.N), 3 * nsets, w.seed)
    sets = []
    for i in range(nsets):
        s = {k: (v if i == 0 else v.clone()) for k, v in base.items() if k not in ("x", "dy")}
        s["x"], s["dy"], s["dx"] = big[3 * i], big[3 * i + 1], big[3 * i + 2]
        s["x"].copy_(base["x"])
        s["dy"].copy_(base["dy"])
        s["f_mean"] = torch.empty_like(base["rstd"])
        s["f_rstd"] = torch.empty_like(base["rstd"])
        sets.append(s)
    dgamma = torch.empty(w.N, dtype=w.wgrad_dtype, device=dev)
    dbeta = torch.empty(w.N, dtype=w.wgrad_dtype, device=dev) if with_db else None
    # enough for the explicit plan and for the automatic plan of either
    # statistics mode (LayerNorm recompute plans more row groups)
    ws_bytes = max(plan.workspace_bytes, nb.norm_bwd_workspace_bytes(w.kind, w.M, w.N, io, with_db))
    # another build to compare with may plan a larger workspace
    other = nb.load_library_at(args.compare_lib) if args.compare_lib else None
    if other is not None:
        ws_bytes = max(ws_bytes, other.norm_bwd_workspace_bytes(
            0 if w.kind == "layernorm" else 1, w.M, w.N, io, int(with_db)))
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    P = ctypes.c_void_p
    ptr = lambda t: None if t is None else P(t.data_ptr())  # noqa: E731

    full_args, part_args = backward_args(w, sets, plan, dgamma, dbeta, ws, io, wg, sh)
    step = backward_step(nb, lib, w, bool(args.groups or args.plan), full_args, part_args, wg,
                         dgamma, dbeta)

    def step_a(i):
        st = lib.norm_bwd_execute_partials(*part_args[i % nsets])
        if st:
            raise RuntimeError(nb.norm_bwd_last_error())

    def step_b(i):
        st = lib.norm_bwd_reduce_partials(plan.groups, w.N, wg, ptr(ws), ws.numel(), ptr(dgamma),
                                          ptr(dbeta), sh)
        if st:
            raise RuntimeError(nb.norm_bwd_last_error())

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ms = time_loop(torch, step, steps, stream)
    ms_graph = graph_step_time(torch, nb, w, sets, dgamma, dbeta, ws, steps)
    cmp = None
    if args.compare_lib:
        cmp = compare_builds(torch, nb, lib, other, w, sets, full_args, dgamma, dbeta, ws, io,
                             stream, steps, args.compare_lib)
    # the spread of the step time: 20 loops of 25 steps, each loop's mean
    chunks = sorted(time_loop(torch, step, 25, stream) for _ in range(20))
    ms_a = time_loop(torch, step_a, steps, stream)
    ms_b = time_loop(torch, step_b, max(steps, 50), stream)
    # the kernel boundary: kernel A, then a dependent 16-byte copy on the stream
    tiny = torch.zeros(8, dtype=torch.int32, device=dev)
    tiny_src, tiny_dst = ptr(tiny[:4]), ptr(tiny[4:])

    def step_a_gap(i):
        step_a(i)
        if lib.norm_bwd_probe_copy(tiny_src, tiny_dst, 16, sh):
            raise RuntimeError(nb.norm_bwd_last_error())

    ms_a_gap = time_loop(torch, step_a_gap, steps, stream)

    alg = w.algorithmic_bytes()
    value = alg / (ms * 1e-3) / 1e9
    a_bytes = kernel_a_bytes(w)
    achieved = a_bytes / (ms_a * 1e-3) / 1e9
    entry = {
        "workload": w.name, "kind": w.kind, "M": w.M, "N": w.N,
        "io_dtype": W._dt(w.io_dtype), "wgrad_dtype": W._dt(w.wgrad_dtype), "eps": w.eps,
        "seed": w.seed, "algorithmic_bytes": alg, "steps": steps,
        "step_us": round(ms * 1e3, 3), "GBps": round(value, 2),
        "pct_of_peak": round(100 * value / PEAK_HBM_GBPS, 2),
        "rows_per_s": round(w.M / (ms * 1e-3), 1),
        "graph_step_us": round(ms_graph * 1e3, 3),
        **({"compare_lib": cmp} if cmp else {}),
        "graph_GBps": round(alg / (ms_graph * 1e-3) / 1e9, 2),
        "step_us_spread": {"loops": len(chunks), "steps_per_loop": 25,
                           "median": round(chunks[len(chunks) // 2] * 1e3, 3),
                           "min": round(chunks[0] * 1e3, 3), "max": round(chunks[-1] * 1e3, 3)},
        "kernel_a_us": round(ms_a * 1e3, 3), "kernel_a_bytes": a_bytes,
        "kernel_a_GBps": round(achieved, 2),
        "kernel_a_frac": round(achieved / PEAK_HBM_GBPS, 4),
        "kernel_a_traffic": committed_traffic(w.name),
        "kernel_b_alone_us": round(ms_b * 1e3, 3),
        "kernel_b_in_place_us": round((ms - ms_a) * 1e3, 3),
        "kernel_boundary_us": round((ms_a_gap - ms_a) * 1e3, 3),
        "workspace_bytes": plan.workspace_bytes,
        "counted_GBps_incl_workspace": round((alg + 2 * plan.workspace_bytes) / (ms * 1e-3) / 1e9,
                                             2),
        "buffer_sets": nsets,
        "placement": "x, dy, dx of the sets at seeded random offsets in one pool",
        "cache_resident": nsets * set_bytes <= MALL_BYTES,
    }
    if triad:
        entry["pct_of_triad"] = round(100 * value / triad["GBps"], 2)
        entry["kernel_a_pct_of_triad"] = round(100 * achieved / triad["GBps"], 2)
        same = triad_same_size(torch, nb, lib, dev, stream, sets, w.M * w.N * w.io_bytes,
                               max(steps, 50))
        entry["triad_same_bytes"] = same
        entry["kernel_a_pct_of_triad_same_bytes"] = round(100 * achieved / same["GBps"], 2)
    plan_d = {k: v for k, v in plan.as_dict().items()
              if k in ("groups", "rows_per_group", "vec", "chunks", "waves_per_row",
                       "rows_in_flight", "rows_per_wave", "threads", "grid")}
    entry["plan"] = plan_d
    if args.placements and w.name == args.primary_name:
        entry["placements"] = placement_study(torch, nb, lib, dev, stream, w, args, base, plan,
                                              args.placements)
    more = {}
    if extras:
        more = measure_extras(torch, nb, W, lib, dev, stream, w, args, steps, warmup, sets,
                              base, full_args, dgamma, dbeta, ws, io, wg, set_bytes)
    del sets, big, pool, base, ws, dgamma, dbeta, full_args, part_args
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return entry, more, inp


def measure_extras(torch, nb, W, lib, dev, stream, w, args, steps, warmup, sets, base, full_args,
                   dgamma, dbeta, ws, io, wg, set_bytes):
    """The forward, recompute mode, norm_bwd_ex (strided, accumulating) and the
    column walk on the same buffers; the copy probe; wide rows."""
    sh = ctypes.c_void_p(stream.cuda_stream)
    nsets = len(sets)
    with_db = w.kind == "layernorm"
    P = ctypes.c_void_p
    ptr = lambda t: None if t is None else P(t.data_ptr())  # noqa: E731
    # the forward that produces the statistics, into per-set y and stats
    # buffers (y lands in the dx buffer of the set, which the backward rewrites)
    fwd_args = []
    for s in sets:
        if w.kind == "layernorm":
            fwd_args.append((ptr(s["x"]), ptr(s["gamma"]), ptr(s.get("beta")), w.M, w.N, io,
                             w.eps, ptr(s["dx"]), ptr(s["f_mean"]), ptr(s["f_rstd"]), sh))
        else:
            fwd_args.append((ptr(s["x"]), ptr(s["gamma"]), w.M, w.N, io, w.eps, ptr(s["dx"]),
                             ptr(s["f_rstd"]), sh))
    ffn = lib.norm_fwd_layernorm if w.kind == "layernorm" else lib.norm_fwd_rmsnorm

    def step_f(i):
        st = ffn(*fwd_args[i % nsets])
        if st:
            raise RuntimeError(nb.norm_bwd_last_error())

    for i in range(min(warmup, 50)):
        step_f(i)
    ms_f = time_loop(torch, step_f, steps, stream)
    f_bytes = forward_bytes(w, "beta" in base)
    # the forward's own ceiling: one read and one write (the triad probe
    # reading x twice, so HBM sees x once), on the same buffers into y
    f_ceiling = None
    nbytes = w.M * w.N * w.io_bytes
    for unroll in (1, 2, 4):
        if nbytes % (4096 * unroll) or nbytes > 0xFFFFFFFF - 16383:
            continue
        one = [(P(s["x"].data_ptr()), P(s["dx"].data_ptr())) for s in sets]

        def step_c(i, unroll=unroll):
            xp, yp = one[i % nsets]
            if lib.norm_bwd_probe_triad_policy(xp, xp, yp, nbytes, unroll, nb.POLICY_NT,
                                               nb.POLICY_NT, sh):
                raise RuntimeError(nb.norm_bwd_last_error())
        for i in range(5):
            step_c(i)
        ms_c = time_loop(torch, step_c, steps, stream)
        f_ceiling = ms_c if f_ceiling is None else min(f_ceiling, ms_c)

    # the backward in recompute mode: NULL statistics, recomputed from x
    rc_args = [(a[0], a[1], a[2], None, None) + a[5:] if w.kind == "layernorm"
               else (a[0], a[1], a[2], None) + a[4:] for a in full_args]
    fn_rc = lib.norm_bwd_layernorm if w.kind == "layernorm" else lib.norm_bwd_rmsnorm

    def step_rc(i):
        st = fn_rc(*rc_args[i % nsets])
        if st:
            raise RuntimeError(nb.norm_bwd_last_error())

    for i in range(min(warmup, 50)):
        step_rc(i)
    ms_rc = time_loop(torch, step_rc, steps, stream)
    rc_bytes = w.algorithmic_bytes() - w.M * (8 if w.kind == "layernorm" else 4)

    # norm_bwd_ex: x, dy, dx as row-strided views (row stride N + 64 elements)
    # and the weight gradients accumulated into (read, added, written)
    ld = w.N + 64
    ex_args, ex_keep = [], []
    for s in sets:
        views = {}
        for k in ("x", "dy", "dx"):
            buf = torch.empty(w.M * ld, dtype=w.io_dtype, device=dev)
            v = buf.view(w.M, ld)[:, :w.N]
            v.copy_(s[k])
            views[k] = v
        ex_keep.append(views)
        a = nb.NormBwdArgs()
        a.kind, a.io_dtype, a.wgrad_dtype = (0 if w.kind == "layernorm" else 1), io, wg
        a.flags, a.M, a.N, a.groups = nb.ACCUMULATE, w.M, w.N, 0
        a.x, a.ldx, a.dy, a.lddy = views["x"].data_ptr(), ld, views["dy"].data_ptr(), ld
        a.gamma = s["gamma"].data_ptr()
        a.mean = s["mean"].data_ptr() if w.kind == "layernorm" else None
        a.rstd = s["rstd"].data_ptr()
        a.dx, a.lddx = views["dx"].data_ptr(), ld
        a.dgamma = dgamma.data_ptr()
        a.dbeta = dbeta.data_ptr() if dbeta is not None else None
        a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
        a.stream, a.eps = stream.cuda_stream, w.eps
        ex_args.append(a)

    def step_ex(i):
        st = lib.norm_bwd_ex(ctypes.byref(ex_args[i % nsets]))
        if st:
            raise RuntimeError(nb.norm_bwd_last_error())

    dgamma.zero_()
    if dbeta is not None:
        dbeta.zero_()
    for i in range(min(warmup, 50)):
        step_ex(i)
    ms_ex = time_loop(torch, step_ex, steps, stream)

    # weight gradients alone by the column walk (no dx, no workspace)
    def step_cw(i):
        s = sets[i % nsets]
        st = lib.norm_bwd_wgrad(0 if w.kind == "layernorm" else 1, ptr(s["x"]), ptr(s["dy"]),
                                ptr(s.get("mean")), ptr(s["rstd"]), w.M, w.N, io, wg,
                                ptr(dgamma), ptr(dbeta), 0, sh)
        if st:
            raise RuntimeError(nb.norm_bwd_last_error())

    for i in range(min(warmup, 50)):
        step_cw(i)
    ms_cw = time_loop(torch, step_cw, steps, stream)
    cw_bytes = w.M * (2 * w.N * w.io_bytes + (8 if with_db else 4)) + \
        w.N * w.wgrad_bytes * (2 if with_db else 1)
    ex_bytes = w.algorithmic_bytes() + w.N * w.wgrad_bytes * (2 if with_db else 1)
    del ex_keep, ex_args
    torch.cuda.empty_cache()

    wide = measure_wide(torch, nb, W, lib, dev, stream, args) if not args.no_wide else None
    # the forward takes the backward's lane layout (two rows per wave or one)
    two_row = nb.norm_bwd_make_plan(w.kind, w.M, w.N, io, with_db).rows_per_wave == 2
    out = {
        "forward": {
            "kernel": "norm_fwd_tworow_kernel" if two_row else "norm_fwd_kernel",
            "us": round(ms_f * 1e3, 3),
            "bytes_per_launch": f_bytes, "with_beta": "beta" in base,
            "GBps": round(f_bytes / (ms_f * 1e-3) / 1e9, 2),
            "traffic": committed_forward_traffic(w.name),
            "pct_of_peak": round(100 * f_bytes / (ms_f * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2),
            "one_read_one_write_ceiling_us": None if f_ceiling is None else
            round(f_ceiling * 1e3, 3),
            "pct_of_ceiling": None if f_ceiling is None else round(100 * f_ceiling / ms_f, 2),
        },
        "recompute": {
            "what": "whole backward step with mean/rstd recomputed from x (no stats read)",
            "workspace_bytes": nb.norm_bwd_workspace_bytes(w.kind, w.M, w.N, io, with_db),
            "us": round(ms_rc * 1e3, 3), "bytes": rc_bytes,
            "GBps": round(rc_bytes / (ms_rc * 1e-3) / 1e9, 2),
            "pct_of_peak": round(100 * rc_bytes / (ms_rc * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2),
        },
        "strided_accumulate": {
            "what": "norm_bwd_ex: x, dy, dx row stride N+64, dgamma/dbeta accumulated",
            "us": round(ms_ex * 1e3, 3), "bytes": ex_bytes,
            "GBps": round(ex_bytes / (ms_ex * 1e-3) / 1e9, 2),
            "pct_of_peak": round(100 * ex_bytes / (ms_ex * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2),
        },
        "colwalk_wgrad": {
            "what": "dgamma/dbeta alone by the column walk (reads x, dy, stats; no dx)",
            "kernel": "wgrad_colwalk_kernel", "us": round(ms_cw * 1e3, 3), "bytes": cw_bytes,
            "GBps": round(cw_bytes / (ms_cw * 1e-3) / 1e9, 2),
            "pct_of_peak": round(100 * cw_bytes / (ms_cw * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2),
        },
    }
    if wide is not None:
        out["wide_rows"] = wide
    return out


def copy_probe(torch, nb, dev, stream, nbytes):
    """The library's plain copy kernel over `nbytes` (the counter calibration
    reference of the profiles)."""
    cp_bytes = nbytes // 16 * 16
    src = torch.empty(cp_bytes // 4, dtype=torch.int32, device=dev).fill_(1)
    dsts = [torch.empty_like(src) for _ in range(2)]
    srcs = [src, src.clone()]
    for i in range(3):
        nb.norm_bwd_probe_copy(srcs[i % 2], dsts[i % 2])
    ms_cp = time_loop(torch, lambda i: nb.norm_bwd_probe_copy(srcs[i % 2], dsts[i % 2]),
                      20, stream)
    del src, dsts, srcs
    torch.cuda.empty_cache()
    return cp_bytes, 2 * cp_bytes / (ms_cp * 1e-3) / 1e9


# The default run: the five workloads (the first with its RMSNorm variant),
# in their order; the headline is measured first and carries the line's
# top-level fields.
DEFAULT_ORDER = ("layernorm_f32_128x512", "rmsnorm_f32_128x512", "layernorm_f16_1151x8192",
                 "rmsnorm_bf16_16384x4096", "layernorm_bf16_65536x8192",
                 "rmsnorm_bf16_262144x768")


def main(argv=None) -> int:
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: the library and this benchmark "
              "run on one GPU (the sharding across GPUs is described, not implemented). "
              "Use --gpus 1.", file=sys.stderr)
        return 2

    import torch

    import rmsnorm_backward_amd as nb
    from rmsnorm_backward_amd import workloads as W

    if not os.path.exists(nb.LIB_PATH):
        from rmsnorm_backward_amd import _build
        _build.build()
    lib = nb.load_library()
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    if args.shape:
        primary = parse_shape(W, torch, args.shape)
    else:
        primary = W.WORKLOADS[args.workload] if args.workload else W.HEADLINE
    args.primary_name = primary.name
    if args.compare_plan and not args.placements:
        print("bench.py: --compare-plan needs --placements", file=sys.stderr)
        return 2
    single = bool(args.workload or args.shape or args.plan or args.groups)
    others = [] if single else [W.WORKLOADS[n] for n in DEFAULT_ORDER if n != primary.name]

    # the streaming ceiling (first: it also brings the GPU clock up)
    triad = triad_sweep(torch, nb, dev, stream, 512 << 20) if not args.no_triad else None
    print(f"bench.py: triad ceiling {triad and triad['GBps']} GB/s", file=sys.stderr, flush=True)
    policies = None
    if args.triad_policies:
        policies = [triad_policy_sweep(torch, nb, lib, dev, stream, nbytes, 20)
                    for nbytes in (512 << 20, primary.M * primary.N * primary.io_bytes)]
        for p in policies:
            print(f"bench.py: triad policies at {p['bytes_per_operand']} B: best {p['best']}, "
                  f"nt on both {p['nt_on_both_GBps']}, otherwise {p['otherwise_GBps']} GB/s",
                  file=sys.stderr, flush=True)

    entries = {}
    cpu_inputs = {}
    entry, extras, inp = measure_workload(torch, nb, W, lib, dev, stream, primary, args,
                                          args.steps, args.warmup, not args.no_extras, triad)
    entries[primary.name] = entry
    cpu_inputs[primary.name] = inp
    print(f"bench.py: {primary.name} step {entry['step_us']} us", file=sys.stderr, flush=True)
    cp_bytes, copy_gbps = copy_probe(torch, nb, dev, stream,
                                     min(512 << 20, max(2 * primary.M * primary.N *
                                                        primary.io_bytes, 64 << 20)))
    for w in others:
        e, _, inp = measure_workload(torch, nb, W, lib, dev, stream, w, args,
                                     max(args.steps, 200), max(args.warmup, 20), False, triad)
        entries[w.name] = e
        cpu_inputs[w.name] = inp
        print(f"bench.py: {w.name} step {e['step_us']} us", file=sys.stderr, flush=True)

    # row widths of common models: the lane layout the planner takes for each
    width_entries = []
    if args.widths:
        for n in (int(v) for v in args.widths.split(",") if v):
            m = max(256, (64 << 20) // n)
            for kind, base in (("rmsnorm", W.HEADLINE), ("layernorm", W.LN_BF16_65536x8192)):
                w = W.scaled(base, M=m, N=n, name=f"{kind}_bf16_{m}x{n}")
                e, _, _ = measure_workload(torch, nb, W, lib, dev, stream, w, args,
                                           max(args.steps, 200), max(args.warmup, 50), False,
                                           triad)
                width_entries.append({k: e.get(k) for k in (
                    "workload", "kind", "M", "N", "step_us", "GBps", "pct_of_peak",
                    "kernel_a_us", "kernel_a_frac", "kernel_a_pct_of_triad_same_bytes",
                    "plan")})
                print(f"bench.py: {w.name} step {e['step_us']} us, kernel A "
                      f"{e['kernel_a_frac']} of 8 TB/s", file=sys.stderr, flush=True)

    # the CPU oracle on the same inputs (after every GPU measurement)
    if not args.no_cpu_baseline:
        for name, e in entries.items():
            w = primary if name == primary.name else W.WORKLOADS[name]
            secs = args.cpu_seconds if name == primary.name else args.cpu_seconds_other
            e["cpu_oracle"] = cpu_baseline(w, cpu_inputs[name], secs, max(secs / 2, 1.0))
            print(f"bench.py: {name} cpu oracle {e['cpu_oracle']['value']} GB/s",
                  file=sys.stderr, flush=True)
    del cpu_inputs

    e = entries[primary.name]
    order = [n for n in DEFAULT_ORDER if n in entries] + \
        [n for n in entries if n not in DEFAULT_ORDER]
    config = {
        "workload": primary.name, "kind": primary.kind, "M": primary.M, "N": primary.N,
        "io_dtype": e["io_dtype"], "wgrad_dtype": e["wgrad_dtype"], "stats_dtype": "f32",
        "eps": primary.eps, "seed": primary.seed, "algorithmic_bytes": e["algorithmic_bytes"],
        "pct_of_peak": e["pct_of_peak"], "rows_per_s": e["rows_per_s"],
        "step_us_spread": e["step_us_spread"],
        "kernel_a_us": e["kernel_a_us"], "kernel_b_us": e["kernel_b_alone_us"],
        "kernel_b_in_place_us": e["kernel_b_in_place_us"],
        "copy_probe_GBps": round(copy_gbps, 1), "copy_probe_bytes": cp_bytes,
        "triad_probe": triad,
        "pct_of_triad": e.get("pct_of_triad"),
        "triad_policies": policies,
        "buffer_sets": e["buffer_sets"], "workspace_bytes": e["workspace_bytes"],
        "counted_GBps_incl_workspace": e["counted_GBps_incl_workspace"],
        "plan": e["plan"],
    }
    config.update(extras)
    config["workloads"] = [entries[n] for n in order]
    if width_entries:
        config["widths"] = width_entries
    result = {
        "metric": METRIC,
        "value": e["GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(e["step_us"] / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": config,
        "roofline": {
            "bound": "hbm", "achieved": e["kernel_a_GBps"], "peak": PEAK_HBM_GBPS,
            "unit": "GB/s", "frac": e["kernel_a_frac"], "traffic": e["kernel_a_traffic"],
            "kernel": "dx_partials_tworow_kernel" if e["plan"].get("rows_per_wave") == 2
            else "dx_partials_kernel", "bytes_per_launch": e["kernel_a_bytes"],
        },
    }
    if "cpu_oracle" in e:
        result["cpu_baseline"] = e["cpu_oracle"]
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
