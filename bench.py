#!/usr/bin/env python3
"""Benchmark of the Ulysses 4D relayout on one MI355X.

One step = one mode-0 relayout plus one mode-1 relayout of the video-DiT
attention operand the fast-ulysses pages measure on (Wan 720p, bf16):
W = 8 emulated ranks, 75,600 tokens (9,450 per rank), 40 heads (5 per rank),
head dim 128, batch 1.  Synthetic N(0, 1) inputs, resident in HBM before
the timed region.  Mode 1 reads a separately generated head-sharded input,
so no step reads what the previous kernel just wrote (no help from the
256 MB Infinity Cache).

Prints ONE JSON line on stdout (progress goes to stderr):
  value      whole-step throughput, algorithmic bytes (every element read
             once and written once) / step time, in GB/s;
  roofline   the relayout kernel: algorithmic bytes per launch / its
             average launch time, the timed region's event time over its 2K
             launches (every launch of the region is that kernel), against
             8 TB/s; per-mode medians come from a pass of at least 100
             steps with an event pair around each launch, run before the
             warm-up so the timed region carries no events; `traffic` comes from the
             rocprofv3 counter summary in profiles/ when it was taken on the
             current kernel source, else null;
  value_mall_cold  the same step with 1 GiB of other data read between
             launches, so the 256 MB Infinity Cache holds none of the
             launch's bytes (per-mode medians), beside `value`;
  cpu_baseline  the CPU oracle on the step's geometry: its loops on all
             the host cores the process may use (value), and single-threaded;
  rows       the other hot-path rows timed after the step: uneven W=7 in
             four dtypes, unequal head widths, q/k/v in one launch, the
             plane-at-a-time QKV pack through windows and straight into the
             destination, the fused QK-norm + RoPE pass; plus a same-run
             device-to-device copy (torch) and this GPU's read / write / copy
             ceilings for 16-byte vectors (hbm_probe, run as a child process
             first).
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_GBS = 8000.0   # MI355X HBM3E, AMD's published peak
METRIC = "relayout HBM GB/s & % of MI355X peak, W=8 75.6k-token bf16 mode0+mode1"
COUNTERS = os.path.join(ROOT, "profiles", "relayout_w8_wan720p_counters.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


PROBE_SRC = os.path.join(ROOT, "hbm_probe.hip")
PROBE = os.path.join(ROOT, "hbm_probe")


def build_probe(verbose=False):
    """Compiles hbm_probe.hip (this GPU's HBM read / write / copy ceilings),
    a standalone gfx950 program that only this benchmark runs."""
    import subprocess
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = [os.path.join(rocm, "bin", "hipcc"), "-O3", "-std=c++17", "--offload-arch=gfx950",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", PROBE_SRC, "-o", PROBE]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return PROBE


def kernel_source_hash():
    """SHA-256 of the kernel sources with comments and layout removed, so a
    counter summary stays attached to the code it measured and edits to
    comments alone do not detach it."""
    import re
    h = hashlib.sha256()
    for f in ("kernels.hip", "args.hpp"):
        with open(os.path.join(ROOT, "sequence_attention_relayout_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def traffic_from_profile():
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return c.get("traffic_bytes_per_launch")


def timed(fn, reps, stream, torch, warmup=3, inner=10):
    """Median and min milliseconds per call of fn(), timed like the step:
    `inner` calls back to back between one pair of HIP events on `stream`,
    `reps` such pairs after `warmup` untimed calls.  (An event pair around
    every single call measured some launches up to 10% slower: the
    per-call events, not the kernels, set those figures.)"""
    for _ in range(warmup):
        fn()
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(reps)]
    for a, b in pairs:
        a.record(stream)
        for _ in range(inner):
            fn()
        b.record(stream)
    torch.cuda.synchronize()
    ts = [a.elapsed_time(b) / inner for a, b in pairs]
    return statistics.median(ts), min(ts)


def cpu_baseline(reps=3):
    """The oracle as it is on the whole step's geometry (one mode 0 and one
    mode 1 per run, median of `reps` runs): its loops on every host core this
    process may use (the threaded entry point hands destination rows to
    threads), and single-threaded."""
    import numpy as np
    import oracle
    world, per_rank, heads, d = 8, 9450, 5, 128
    seq, head = [per_rank] * world, [heads] * world
    rng = np.random.default_rng(7)
    xs = [rng.integers(0, 1 << 16, (1, per_rank, heads * world, d), dtype=np.uint16)
          for _ in range(world)]
    ys_in = [rng.integers(0, 1 << 16, (1, per_rank * world, heads, d), dtype=np.uint16)
             for _ in range(world)]
    nbytes = 2 * 2 * (per_rank * world) * (heads * world) * d * 2
    cores = len(os.sched_getaffinity(0))

    def rate(threads):
        times = []
        for _ in range(reps):
            t0 = time.perf_counter()
            oracle.a2a_4d(0, 1, d, seq, head, xs, threads=threads)
            oracle.a2a_4d(1, 1, d, seq, head, ys_in, threads=threads)
            times.append(time.perf_counter() - t0)
        return nbytes / statistics.median(times) / 1e9, statistics.median(times), sum(times)

    all_gbs, all_dt, all_s = rate(cores)
    one_gbs, one_dt, one_s = rate(1)
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    sample = ("the full step's geometry (W=8, 75,600 tokens, n=40, d=128, bf16): one mode 0 and "
              f"one mode 1 on the oracle's plain index loops, median of {reps} runs")
    return {"value": round(all_gbs, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "cpu": cpu, "sample": sample + f" ({all_dt:.2f} s each, {cores} threads)",
            "single_thread": {"value": round(one_gbs, 3), "unit": "GB/s", "cores": 1,
                              "seconds_per_run": round(one_dt, 2)},
            "seconds": round(all_s + one_s, 2)}


def hbm_ceilings():
    """Runs the HBM-ceiling probe (built next to the library) as a child
    process; returns the best of its launch shapes for each kind,
    {"copy": GB/s, "read": GB/s, "write": GB/s}, or None."""
    import subprocess
    exe = PROBE
    if not os.path.exists(exe):
        log("hbm probe not built; skipping the ceilings")
        return None
    try:
        out = subprocess.run([exe], capture_output=True, text=True, timeout=120).stdout
    except subprocess.TimeoutExpired:
        log("hbm probe timed out")
        return None
    res = {}
    for line in out.splitlines():
        if line.startswith("{"):
            rec = json.loads(line)
            if "kernel" in rec and rec["gbs"] > res.get(rec["kernel"], 0.0):
                res[rec["kernel"]] = rec["gbs"]   # the best launch shape of each kind
            if "device_props" in rec:
                res["device_props"] = rec["device_props"]
    return res or None


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true", help="time the step only")
    ap.add_argument("--rows", default=",".join(ROW_GROUPS),
                    help="comma-separated row groups to time after the step "
                         f"(of {', '.join(ROW_GROUPS)}); each runs only its own launches")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the HBM read/write/copy ceiling probe")
    args = ap.parse_args()
    groups = [g for g in args.rows.split(",") if g]
    bad = [g for g in groups if g not in ROW_GROUPS]
    if bad:
        print(f"unknown row groups {bad}; known: {list(ROW_GROUPS)}", file=sys.stderr)
        sys.exit(2)
    world_env = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world_env != 1:
        print("bench.py measures one GPU: the W ranks are emulated as shard buffers in one "
              "GPU's HBM, and the library has no multi-GPU path. Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    # the ceiling probe runs first, in a child process, before this process
    # touches the GPU
    ceilings = None if args.no_ceilings else hbm_ceilings()

    import torch
    sys.path.insert(0, ROOT)
    from sequence_attention_relayout_amd import ulysses as U
    from sequence_attention_relayout_amd import workloads as W

    if not torch.cuda.is_available():
        print("no HIP device visible", file=sys.stderr)
        sys.exit(1)
    U.library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    props = torch.cuda.get_device_properties(dev)
    log(f"device: {props.name} ({getattr(props, 'gcnArchName', '?')}), "
        f"{props.multi_processor_count} CUs, {props.total_memory / 2**30:.0f} GiB")

    wl = W.workloads()["w8_wan720p"]
    plan = U.ulysses_plan_create(wl.world, wl.b, wl.d, wl.seq_splits, wl.head_splits, "bf16")
    bytes0, bytes1 = U.ulysses_plan_bytes(plan, 0), U.ulysses_plan_bytes(plan, 1)
    step_bytes = bytes0 + bytes1
    x0 = W.make_shards(wl, 0, "bf16", wl.seed, dev)
    y0 = [torch.empty(U.ulysses_plan_shape(plan, 0, r, True), dtype=torch.bfloat16, device=dev)
          for r in range(wl.world)]
    y1 = W.make_shards(wl, 1, "bf16", wl.seed + 1, dev)
    x1 = [torch.empty(U.ulysses_plan_shape(plan, 1, r, True), dtype=torch.bfloat16, device=dev)
          for r in range(wl.world)]
    torch.cuda.synchronize()
    h = stream.cuda_stream
    # what the step reads: a checksum of both inputs' 32-bit words, summed on
    # the device before anything is timed
    checksum = int(sum(int(x.view(torch.int32).sum(dtype=torch.int64)) for x in x0 + y1))
    inputs = {"generator": "torch.Generator on the device, one per shard set",
              "seeds": {"mode0_input": wl.seed, "mode1_input": wl.seed + 1},
              "values": "N(0,1) in fp32, rounded to bf16 by torch",
              "checksum_int32_words": checksum}

    def mode0():
        U.ulysses_a2a_4d(plan, 0, x0, y0, h)

    def mode1():
        U.ulysses_a2a_4d(plan, 1, y1, x1, h)

    K = args.steps
    # Per-launch durations of the relayout kernel: at least 100 steps with
    # each launch between its own pair of events on the launch stream, after
    # three untimed steps of their own (the first launches of a process load
    # code, and the clocks take tens of milliseconds to come up; the medians
    # absorb that).  They run before the timed region, which carries no events
    # of its own.
    for _ in range(3):
        mode0()
        mode1()
    KE = max(K, 100)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(KE)]
    for k in range(KE):
        evs[k][0].record(stream)
        mode0()
        evs[k][1].record(stream)
        mode1()
        evs[k][2].record(stream)
    torch.cuda.synchronize()
    m0 = [e[0].elapsed_time(e[1]) for e in evs]
    m1 = [e[1].elapsed_time(e[2]) for e in evs]

    # The same launches with the 256 MB Infinity Cache (MALL) cold: 1 GiB of
    # other data is read between launches, outside the events.  Reading (not
    # writing) leaves only clean lines behind, so the next launch pays no
    # write-back of the flush itself.
    flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    cold = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    sink = torch.zeros((), dtype=torch.int64, device=dev)
    for k in range(K):
        sink += flush.sum()
        cold[k][0].record(stream)
        mode0()
        cold[k][1].record(stream)
        sink += flush.sum()
        cold[k][2].record(stream)
        mode1()
        cold[k][3].record(stream)
    torch.cuda.synchronize()
    c0 = [e[0].elapsed_time(e[1]) for e in cold]
    c1 = [e[2].elapsed_time(e[3]) for e in cold]
    del flush, sink

    for _ in range(args.warmup):
        mode0()
        mode1()
    torch.cuda.synchronize()

    # The timed region: K steps back to back, events only at its two ends.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for _ in range(K):
        mode0()
        mode1()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = start.elapsed_time(end) / K
    # Every launch of the timed region is the relayout kernel (mode 0 and
    # mode 1 move the same bytes), so its average launch duration is the
    # region's event time over its 2K launches; the per-launch event pairs
    # above give the per-mode medians (they add the events' own overhead).
    launch_ms = ms_step / 2
    launch_ms_event_pairs = statistics.median(m0 + m1)

    # A second timed region like the first, for the spread between two
    # invocations of the same K steps.
    start.record(stream)
    for _ in range(K):
        mode0()
        mode1()
    end.record(stream)
    torch.cuda.synchronize()
    ms_step_repeat = start.elapsed_time(end) / K
    value = step_bytes / (ms_step * 1e-3) / 1e9
    achieved = (step_bytes / 2) / (launch_ms * 1e-3) / 1e9
    log(f"step {ms_step * 1e3:.1f} us ({value:.0f} GB/s); mode 0 median "
        f"{statistics.median(m0) * 1e3:.1f} us, mode 1 median {statistics.median(m1) * 1e3:.1f} us;"
        f" host wall {wall / K * 1e6:.1f} us/step")

    # same-run device-to-device copy of one shard set's bytes: the flat-copy
    # ceiling ("of the fabric" in the pages' terms)
    flat_src = torch.empty(bytes0 // 2, dtype=torch.uint8, device=dev)
    flat_dst = torch.empty_like(flat_src)
    d2d_ms, _ = timed(lambda: flat_dst.copy_(flat_src), 5, stream, torch)
    d2d = bytes0 / (d2d_ms * 1e-3) / 1e9
    del flat_src, flat_dst

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "w8_wan720p: mode 0 + mode 1, W=8 emulated ranks, b=1, "
                               "s_global=75,600 (9,450/rank), n_global=40 (5/rank), d=128",
                   "world": 8, "b": 1, "s_global": 75600, "n_global": 40, "d": 128,
                   "bytes_per_step": step_bytes, "parallelism": "none (one GPU)",
                   "inputs": inputs},
        "pct_of_peak": round(100 * value / PEAK_GBS, 2),
        "value_mall_cold": round(step_bytes / ((statistics.median(c0) + statistics.median(c1))
                                               * 1e-3) / 1e9, 1),
        "roofline": {"bound": "hbm", "kernel": "relayout_kernel", "achieved": round(achieved, 1),
                     "peak": PEAK_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_GBS, 4),
                     "traffic": traffic_from_profile(),
                     "bytes_per_launch": bytes0, "avg_launch_us": round(launch_ms * 1e3, 2),
                     "launches_timed": 2 * K,
                     "median_launch_us_event_pairs": round(launch_ms_event_pairs * 1e3, 2),
                     "launches_event_pairs": 2 * KE,
                     "mode0_median_us": round(statistics.median(m0) * 1e3, 2),
                     "mode1_median_us": round(statistics.median(m1) * 1e3, 2),
                     "mode0_min_us": round(min(m0) * 1e3, 2),
                     "mode1_min_us": round(min(m1) * 1e3, 2),
                     "mode0_mall_cold_median_us": round(statistics.median(c0) * 1e3, 2),
                     "mode1_mall_cold_median_us": round(statistics.median(c1) * 1e3, 2)},
        "ms_per_step_repeat": round(ms_step_repeat, 5),
        "step_spread_pct": round(100 * abs(ms_step_repeat - ms_step) / ms_step, 2),
        "d2d_copy_ceiling_gbs": round(d2d, 1),
    }
    if ceilings and "device_props" in ceilings:
        # 2 x memory clock x bus width as the runtime reports them; on this
        # part the reported clock does not give HBM3E's data rate, so the
        # figure sits below the measured read ceiling and is not the peak
        # the fraction is taken against.
        result["device_props_hbm"] = ceilings.pop("device_props")
    if ceilings:
        result["hbm_ceilings_gbs"] = ceilings
        if "copy" in ceilings:
            result["relayout_over_copy_ceiling"] = round(value / ceilings["copy"], 4)
    del x0, y0, y1, x1
    torch.cuda.empty_cache()

    if not args.no_rows:
        result["rows"] = time_rows(U, W, torch, dev, stream, groups)
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on a bounded sample ...")
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


ROW_GROUPS = ("uneven", "heads", "tiny", "qkv", "chunked", "fused")


def time_rows(U, W, torch, dev, stream, groups=ROW_GROUPS, reps=7):
    """The other hot-path rows, each timed on its own (median of reps)."""
    rows = {}
    if "uneven" in groups:
        rows.update(rows_uneven(U, W, torch, dev, stream, reps))
    if "heads" in groups:
        rows.update(rows_heads(U, W, torch, dev, stream, reps))
    if "tiny" in groups:
        rows.update(rows_tiny(U, W, torch, dev, stream))
    if "qkv" in groups:
        rows.update(rows_qkv(U, W, torch, dev, stream, reps))
    if "chunked" in groups:
        rows.update(rows_chunked(U, W, torch, dev, stream))
    if "fused" in groups:
        rows.update(rows_fused(U, W, torch, dev, stream, reps))
    return rows


def rows_uneven(U, W, torch, dev, stream, reps):
    rows = {}
    h = stream.cuda_stream
    wl = W.workloads()["w7_uneven"]
    for dt in wl.dtypes:
        plan = U.ulysses_plan_create(wl.world, wl.b, wl.d, wl.seq_splits, wl.head_splits, dt)
        for mode in (0, 1):
            xs = W.make_shards(wl, mode, dt, 40 + mode, dev)
            ys = [torch.empty(U.ulysses_plan_shape(plan, mode, r, True),
                              dtype=W.torch_dtype(dt), device=dev) for r in range(wl.world)]
            med, mn = timed(lambda: U.ulysses_a2a_4d(plan, mode, xs, ys, h), reps, stream, torch)
            nb = U.ulysses_plan_bytes(plan, mode)
            rows[f"w7_uneven_{dt}_mode{mode}"] = {
                "gbs": round(nb / (med * 1e-3) / 1e9, 1), "median_us": round(med * 1e3, 1),
                "bytes": nb}
            del xs, ys
        torch.cuda.empty_cache()
    log("uneven rows done")
    return rows


def rows_heads(U, W, torch, dev, stream, reps):
    # unequal head widths (6 and 4 heads per rank)
    rows = {}
    h = stream.cuda_stream
    world, heads = 8, [6, 6, 6, 6, 4, 4, 4, 4]
    seq = W.even_splits(75600, world)
    plan = U.ulysses_plan_create(world, 1, 128, seq, heads, "bf16")
    wlu = W.Workload("w8 unequal heads", world, 1, 128, seq, heads)
    for mode in (0, 1):
        xs = W.make_shards(wlu, mode, "bf16", 45 + mode, dev)
        ys = [torch.empty(U.ulysses_plan_shape(plan, mode, r, True), dtype=torch.bfloat16,
                          device=dev) for r in range(world)]
        med, _ = timed(lambda: U.ulysses_a2a_4d(plan, mode, xs, ys, h), reps, stream, torch)
        nb = U.ulysses_plan_bytes(plan, mode)
        rows[f"w8_heads_6x4_4x4_mode{mode}"] = {
            "gbs": round(nb / (med * 1e-3) / 1e9, 1), "median_us": round(med * 1e3, 1),
            "bytes": nb}
        del xs, ys
    torch.cuda.empty_cache()
    log("unequal-heads rows done")
    return rows


def rows_tiny(U, W, torch, dev, stream):
    # the two-rank example: launch-bound, so this is latency, not bandwidth
    rows = {}
    h = stream.cuda_stream
    wl = W.workloads()["w2_tiny"]
    plan = U.ulysses_plan_create(wl.world, wl.b, wl.d, wl.seq_splits, wl.head_splits, "bf16")
    xs = W.make_shards(wl, 0, "bf16", wl.seed, dev)
    ys = [torch.empty(U.ulysses_plan_shape(plan, 0, r, True), dtype=torch.bfloat16, device=dev)
          for r in range(wl.world)]
    zs = [torch.empty_like(x) for x in xs]

    def tiny_step():
        U.ulysses_a2a_4d(plan, 0, xs, ys, h)
        U.ulysses_a2a_4d(plan, 1, ys, zs, h)

    med_tiny, _ = timed(tiny_step, 10, stream, torch)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(500):
        tiny_step()
    torch.cuda.synchronize()
    host_us = (time.perf_counter() - t0) / 1000 * 1e6
    rows["w2_tiny_latency"] = {"step_median_us": round(med_tiny * 1e3, 2),
                               "host_us_per_call": round(host_us, 2),
                               "note": "mode 0 + mode 1 of the two-rank example (65,536 B "
                                       "per mode); host time per ABI call through Python"}
    del xs, ys, zs
    return rows


def rows_qkv(U, W, torch, dev, stream, reps):
    # q, k and v of the timed geometry: one launch against three
    rows = {}
    h = stream.cuda_stream
    wl = W.workloads()["w8_wan720p"]
    plan = U.ulysses_plan_create(wl.world, wl.b, wl.d, wl.seq_splits, wl.head_splits, "bf16")
    xs = [W.make_shards(wl, 0, "bf16", 130 + t, dev) for t in range(3)]
    ys = [[torch.empty(U.ulysses_plan_shape(plan, 0, r, True), dtype=torch.bfloat16,
                       device=dev) for r in range(wl.world)] for _ in range(3)]
    nb = 3 * U.ulysses_plan_bytes(plan, 0)
    med_multi, _ = timed(lambda: U.ulysses_a2a_4d_multi(plan, 0, xs, ys, h), reps, stream, torch)

    def three():
        for t in range(3):
            U.ulysses_a2a_4d(plan, 0, xs[t], ys[t], h)

    med_three, _ = timed(three, reps, stream, torch)

    def host_us(fn, n=20):
        # host time to enqueue one q/k/v relayout while the GPU is busy with
        # the previous ones (the calls return before their kernels run)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        t = (time.perf_counter() - t0) / n * 1e6
        torch.cuda.synchronize()
        return round(t, 2)

    rows["w8_qkv_mode0_one_launch"] = {"gbs": round(nb / (med_multi * 1e-3) / 1e9, 1),
                                       "median_us": round(med_multi * 1e3, 1), "bytes": nb,
                                       "host_us_per_qkv": host_us(
                                           lambda: U.ulysses_a2a_4d_multi(plan, 0, xs, ys, h))}
    rows["w8_qkv_mode0_three_launches"] = {"gbs": round(nb / (med_three * 1e-3) / 1e9, 1),
                                           "median_us": round(med_three * 1e3, 1),
                                           "host_us_per_qkv": host_us(three)}
    # autograd: forward (mode 0) and backward (mode 1, same plan) of one tensor
    from sequence_attention_relayout_amd.autograd import all_to_all_4d
    xg = [x.detach().requires_grad_() for x in xs[0]]
    gy = [torch.ones_like(y) for y in ys[0]]

    def fwd_bwd():
        for x in xg:
            x.grad = None   # no accumulation pass: each backward writes fresh grads
        outs = all_to_all_4d(plan, xg, 0)
        torch.autograd.backward(outs, gy)

    med_ag, _ = timed(fwd_bwd, reps, stream, torch)
    rows["w8_autograd_fwd_bwd"] = {
        "gbs": round(2 * U.ulysses_plan_bytes(plan, 0) / (med_ag * 1e-3) / 1e9, 1),
        "median_us": round(med_ag * 1e3, 1)}
    del xs, ys, xg, gy
    torch.cuda.empty_cache()
    log("multi-tensor rows done")
    return rows


def rows_chunked(U, W, torch, dev, stream):
    # the FastVideo pack, plane at a time: through the windows (relayout,
    # then copy-out), straight into the destination planes, and in one pass
    rows = {}
    h = stream.cuda_stream
    wl = W.workloads()["w4_qkv_chunked"]
    plan = U.ulysses_plan_create(wl.world, wl.b, wl.d, wl.seq_splits, wl.head_splits, "bf16",
                                 wl.window_cap_bytes)
    xs = W.make_shards(wl, 0, "bf16", wl.seed, dev)
    ys = [torch.empty(U.ulysses_plan_shape(plan, 0, r, True), dtype=torch.bfloat16, device=dev)
          for r in range(wl.world)]
    win = [torch.empty(U.ulysses_plan_window_bytes(plan, 0), dtype=torch.uint8, device=dev)
           for _ in range(wl.world)]
    relayout_bytes = U.ulysses_plan_bytes(plan, 0)
    staged, _ = timed(lambda: U.ulysses_a2a_4d_chunked(plan, 0, xs, ys, win, h), 3, stream,
                      torch, inner=3)
    direct, _ = timed(lambda: U.ulysses_a2a_4d_chunked(plan, 0, xs, ys, None, h), 3, stream,
                      torch, inner=3)
    one_pass, _ = timed(lambda: U.ulysses_a2a_4d(plan, 0, xs, ys, h), 3, stream, torch, inner=3)
    rows["w4_qkv_chunked_mode0"] = {
        "staged_gbs_relayout_bytes": round(relayout_bytes / (staged * 1e-3) / 1e9, 1),
        "staged_gbs_moved_bytes": round(2 * relayout_bytes / (staged * 1e-3) / 1e9, 1),
        "staged_median_us": round(staged * 1e3, 1),
        "direct_gbs": round(relayout_bytes / (direct * 1e-3) / 1e9, 1),
        "direct_median_us": round(direct * 1e3, 1),
        "staged_over_direct": round(staged / direct, 3),
        "one_pass_gbs": round(relayout_bytes / (one_pass * 1e-3) / 1e9, 1),
        "one_pass_median_us": round(one_pass * 1e3, 1),
        "relayout_bytes": relayout_bytes,
        "note": "staged: per plane, relayout into the W windows then copy-out (twice the "
                "bytes); direct: per plane, relayout straight into the destination plane (the "
                "window is the output slice); one pass: all three planes in one launch"}
    del xs, ys, win
    torch.cuda.empty_cache()
    log("chunked rows done")
    return rows


def rows_fused(U, W, torch, dev, stream, reps):
    rows = {}
    h = stream.cuda_stream
    wl = W.workloads()["w8_fused_qknorm_rope"]
    plan = U.ulysses_plan_create(wl.world, wl.b, wl.d, wl.seq_splits, wl.head_splits, "bf16")
    q = W.make_shards(wl, 0, "bf16", 70, dev)
    k = W.make_shards(wl, 0, "bf16", 71, dev)
    v = W.make_shards(wl, 0, "bf16", 72, dev)
    outs = [[torch.empty(U.ulysses_plan_shape(plan, 0, r, True), dtype=torch.bfloat16,
                         device=dev) for r in range(wl.world)] for _ in range(3)]
    gq, gk = W.make_gamma(wl.d, 73, dev), W.make_gamma(wl.d, 74, dev)
    c, s = U.ulysses_rope_table(10000.0, wl.s_global, wl.d)
    tc, ts = torch.from_numpy(c).to(dev), torch.from_numpy(s).to(dev)

    def fused():
        U.ulysses_a2a_4d_qknorm_rope(plan, q, outs[0], k, outs[1], gq, gk, 1e-6, tc, ts, h)

    def plain_v():
        U.ulysses_a2a_4d(plan, 0, v, outs[2], h)

    fmed, _ = timed(fused, reps, stream, torch)
    vmed, _ = timed(plain_v, reps, stream, torch)
    qk_bytes = 2 * U.ulysses_plan_bytes(plan, 0) + c.nbytes + s.nbytes + 2 * wl.d * 4
    v_bytes = U.ulysses_plan_bytes(plan, 0)
    rows["w8_fused_qknorm_rope"] = {
        "fused_qk_gbs": round(qk_bytes / (fmed * 1e-3) / 1e9, 1),
        "fused_qk_median_us": round(fmed * 1e3, 1),
        "plain_v_gbs": round(v_bytes / (vmed * 1e-3) / 1e9, 1),
        "total_gbs": round((qk_bytes + v_bytes) / ((fmed + vmed) * 1e-3) / 1e9, 1),
        "bytes": qk_bytes + v_bytes}
    del q, k, v, outs
    torch.cuda.empty_cache()
    log("fused rows done")
    return rows


if __name__ == "__main__":
    main()
