#!/usr/bin/env python3
"""Writes the summaries under profiles/ from rocprofv3 output of bench.py.

    python3 summarize_profiles.py OUT
    python3 summarize_profiles.py --commands REPO OUT   (prints the runs below)

OUT holds rocprofv3 output directories (--output-format csv -o run) of
bench.py runs on one MI355X, made from /tmp with TMPDIR=/tmp:

  ktrace/   TRACE_CMD (its stdout and stderr in OUT/ktrace.log)
  <pass>/   one per entry of PASSES (pmc_cmd)

Every counter is averaged per (kernel, grid size) over its dispatches.  The
summaries name the kernels by what they run (the W=8 relayout step, the
fused pass, the W=4 plane-at-a-time pack) and carry the commands above.
"""
import csv
import json
import os
import statistics
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")
sys.path.insert(0, ROOT)
import bench  # noqa: E402  (kernel_source_hash, PEAK_GBS)

BENCH_PMC_ARGS = ("--no-cpu-baseline --no-ceilings --steps 5 --warmup 1 "
                  "--rows uneven,chunked,fused")
# The unequal-heads rows launch the relayout with the same grid as the W=8
# step, so the trace run leaves them out.
TRACE_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d OUT/ktrace -o run "
             "-- python3 REPO/bench.py --no-cpu-baseline --no-ceilings "
             "--rows uneven,tiny,qkv,chunked,fused")
# One counter pass per run: rocprofv3 does not split counters over passes.
PASSES = {
    "fetch": ["FETCH_SIZE"],
    "write": ["WRITE_SIZE"],
    "rdreq": ["TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_BUBBLE_sum"],
    "wrreq": ["TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum"],
    "sq1": ["SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_VMEM_RD", "SQ_INSTS_VMEM_WR",
            "SQ_INSTS_SMEM", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE", "GRBM_COUNT"],
    "sq2": ["SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_SCA", "SQ_ACTIVE_INST_VMEM",
            "SQ_ACTIVE_INST_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_ANY", "SQ_INST_CYCLES_SALU",
            "SQ_BUSY_CU_CYCLES", "TA_TA_BUSY_sum", "TA_FLAT_READ_WAVEFRONTS_sum", "TD_TD_BUSY_sum"],
    "tcp": ["TCP_TOTAL_CACHE_ACCESSES_sum", "TCP_TCC_READ_REQ_sum", "TCP_TCC_WRITE_REQ_sum",
            "TCP_TCP_TA_DATA_STALL_CYCLES_sum", "SQ_INST_LEVEL_VMEM", "SQ_LEVEL_WAVES",
            "SQ_INST_CYCLES_VMEM_RD", "SQ_INST_CYCLES_VMEM_WR"],
}


def pmc_cmd(name):
    return (f"timeout -s KILL 300 rocprofv3 --pmc {' '.join(PASSES[name])} --output-format csv "
            f"-d OUT/{name} -o run -- python3 REPO/bench.py {BENCH_PMC_ARGS}")


# MI355X: 256 CUs of 4 SIMDs in 8 XCDs; a wave64 VALU instruction holds its
# 16-lane SIMD for 4 cycles.
CUS, SIMDS, XCDS = 256, 1024, 8
CALIBRATION = ("__amd_rocclr_copyBuffer", 131072)
CALIBRATION_BYTES = 774144000   # each way: bench.py's same-run device-to-device copy

# Mode-0 and mode-1 launches of the one-plane relayout (mode 0 runs its
# blocks in the two-halves order).
MODE0, MODE1 = "relayout_kernel<false, true>", "relayout_kernel<false, false>"

# (file stem, kernels whose dispatches are pooled, total grid threads,
# algorithmic bytes per launch, what)
WORKLOADS = [
    ("relayout_w8_wan720p", (MODE0, MODE1), 48384000, 1548288000,
     "the relayout at W=8, 75,600 tokens (9,450 per rank), 40 heads (5 per rank), d=128, bf16: "
     "the step's mode-0 and mode-1 launches and the rows' launches of the same geometry "
     "(q/k/v one at a time, the autograd forward and backward, the fused row's plain v)"),
    ("fused_qknorm_rope_w8_wan720p", ("fused_kernel<16, false>",), 48384000,
     2 * 1548288000 + 2 * 75600 * 64 * 4 + 2 * 128 * 4,
     "the fused QK RMSNorm + RoPE mode-0 pass at the same W=8 geometry, q and k in one launch "
     "(algorithmic bytes: q and k each read and written once, the two 75,600 x 64 fp32 rotary "
     "tables and the two 128-float gains read once)"),
    ("chunked_w4_qkv_plane_relayout", (MODE0,), 224000000, 7168000000,
     "the plane-at-a-time W=4 QKV pack (250,000 tokens, 56 heads, d=128, bf16, 3 planes): the "
     "relayout of one plane, into the windows (staged) or straight into the destination plane "
     "(direct); the whole-pack call launches the same kernel once per plane (each plane moves "
     "7.2 GB)"),
    ("chunked_w4_qkv_plane_copy", ("plane_copy_kernel",), 224000000, 7168000000,
     "the same pack's copy of one plane from the W windows into the destination shards "
     "(staged mode only)"),
]


def relayout_threads(world, b, d, S, H, esz, mode):
    """Threads of one relayout launch: 64-vector blocks per destination shard,
    b planes along grid.y."""
    s_global, n_global = sum(S), sum(H)
    blocks = 0
    for r in range(world):
        rows, per_row = (s_global, H[r]) if mode == 0 else (S[r], n_global)
        blocks += -(-(rows * per_row * d * esz // 16) // 64)
    return blocks * 64 * b


def uneven_workloads():
    """The W=7 uneven relayout rows: one entry per byte width and mode (the
    fp8 and int8 rows share a geometry, so they are summarised together).
    Each of their two batch planes moves 0.77-3.1 GB, so every plane gets a
    launch of its own: one-plane grids and bytes per launch."""
    from sequence_attention_relayout_amd import workloads as W
    wl = W.workloads()["w7_uneven"]
    out = []
    for esz, name in ((2, "bf16"), (4, "fp32"), (1, "fp8_int8")):
        for mode in (0, 1):
            out.append((
                f"w7_uneven_{name}_mode{mode}", (MODE1 if mode else MODE0,),
                relayout_threads(wl.world, 1, wl.d, wl.seq_splits, wl.head_splits, esz, mode),
                2 * sum(wl.seq_splits) * sum(wl.head_splits) * wl.d * esz,
                f"the uneven W=7 relayout, mode {mode}, one batch plane per launch (b=2): "
                f"s_global=75,597 as "
                f"{', '.join(f'{x:,}' for x in wl.seq_splits)}, heads "
                f"{', '.join(map(str, wl.head_splits))}, d=128, "
                + ("bf16" if esz == 2 else "fp32" if esz == 4 else
                   "1-byte elements (the fp8 e4m3 and int8 rows together)")))
    return out


def short(name):
    n = name.replace("void ", "").replace("ulysses::", "")
    return n[:n.index("(")] if "(" in n else n


def trace_durations(out):
    """(kernel, grid threads) -> [durations in us] from the kernel trace."""
    d = defaultdict(list)
    with open(os.path.join(out, "ktrace", "run_kernel_trace.csv")) as f:
        for r in csv.DictReader(f):
            g = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            d[(short(r["Kernel_Name"]), g)].append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return d


def counters(out):
    """(kernel, grid threads) -> {counter: mean per dispatch}, and the counts."""
    vals = defaultdict(lambda: defaultdict(list))
    for p in PASSES:
        path = os.path.join(out, p, "run_counter_collection.csv")
        if not os.path.exists(path):
            continue
        with open(path) as f:
            for r in csv.DictReader(f):
                vals[(short(r["Kernel_Name"]), int(r["Grid_Size"]))][r["Counter_Name"]].append(
                    float(r["Counter_Value"]))
    means = {k: {c: statistics.mean(v) for c, v in cs.items()} for k, cs in vals.items()}
    counts = {k: {c: len(v) for c, v in cs.items()} for k, cs in vals.items()}
    return means, counts


def bench_line(out):
    with open(os.path.join(out, "ktrace.log")) as f:
        lines = [ln for ln in f if ln.startswith('{"metric"')]
    return json.loads(lines[-1]) if lines else None


def pooled(tr, cm, cn, kerns, grid):
    """Trace durations, mean counters and dispatch counts of every kernel in
    kerns at this grid size, pooled over their dispatches."""
    ds = [x for k in kerns for x in tr.get((k, grid), [])]
    tot, cnt = defaultdict(float), defaultdict(int)
    for k in kerns:
        for c, v in cm.get((k, grid), {}).items():
            n = cn[(k, grid)][c]
            tot[c] += v * n
            cnt[c] += n
    return ds, {c: tot[c] / cnt[c] for c in tot}, dict(cnt)


def stats_row(name, ds):
    return (f"| `{name}` | {len(ds)} | {statistics.mean(ds):.1f} | {statistics.median(ds):.1f} "
            f"| {min(ds):.1f} | {max(ds):.1f} |")


def commands(repo, out):
    """The rocprofv3 runs that make OUT, one per line, each with its own time
    limit (run them from /tmp with TMPDIR=/tmp)."""
    cmds = ["timeout -k 10 600 " + TRACE_CMD + " > OUT/ktrace.log 2>&1"]
    cmds += [pmc_cmd(p) + f" > OUT/{p}.log 2>&1" for p in PASSES]
    return [c.replace("REPO", repo).replace("OUT", out) for c in cmds]


def main():
    if len(sys.argv) == 4 and sys.argv[1] == "--commands":
        print("\n".join(commands(sys.argv[2], sys.argv[3])))
        return
    if len(sys.argv) != 2:
        print(__doc__, file=sys.stderr)
        sys.exit(2)
    out = sys.argv[1]
    os.makedirs(PROFILES, exist_ok=True)
    tr = trace_durations(out)
    cm, cn = counters(out)
    bl = bench_line(out)
    sha = bench.kernel_source_hash()
    cal = cm.get(CALIBRATION, {})
    fetch_factor = CALIBRATION_BYTES / (cal["FETCH_SIZE"] * 1024) if "FETCH_SIZE" in cal else None
    write_factor = CALIBRATION_BYTES / (cal["WRITE_SIZE"] * 1024) if "WRITE_SIZE" in cal else None
    cal_trace = tr.get(CALIBRATION, [])
    table = []
    for stem, kerns, grid, nbytes, what in WORKLOADS + uneven_workloads():
        ds, c, counts = pooled(tr, cm, cn, kerns, grid)
        kern = " + ".join(kerns)
        if not ds:
            print(f"{stem}: no dispatches of {kern} with {grid} threads in the trace",
                  file=sys.stderr)
            continue
        avg = statistics.mean(ds)
        gbs = nbytes / (avg * 1e-6) / 1e9
        lines = [
            f"# {kern} — {stem.replace('_', ' ')} (kernel trace)", "",
            f"What: {what}.", "",
            "Command (from /tmp with TMPDIR=/tmp, on one MI355X; REPO is this repository, OUT "
            "any output folder), then `python3 REPO/summarize_profiles.py OUT`:", "",
            "```", TRACE_CMD, "```", "",
            f"Dispatches summarised: every {' and every '.join(f'`{k}`' for k in kerns)} launch "
            f"of {grid:,} threads.", "",
            "| Kernel | Dispatches | Average (us) | Median (us) | Min (us) | Max (us) |",
            "|---|---|---|---|---|---|"]
        lines += [stats_row(k, tr[(k, grid)]) for k in kerns if tr.get((k, grid))]
        if len(kerns) > 1:
            lines.append(stats_row("all of the above", ds).replace("`", ""))
        if cal_trace:
            lines.append(stats_row("__amd_rocclr_copyBuffer", cal_trace)
                         + "  (torch device-to-device copy of 774,144,000 B, same run)")
        lines += ["", f"Algorithmic bytes per launch: {nbytes:,}.",
                  f"From the trace average: {gbs:.0f} GB/s = {100 * gbs / bench.PEAK_GBS:.1f}% "
                  f"of 8 TB/s."]
        if stem == "relayout_w8_wan720p" and bl:
            rf = bl["roofline"]
            lines.append(
                f"The profiled bench process's own HIP-event average over the "
                f"{rf['launches_timed']} launches of its timed region: {rf['avg_launch_us']} us "
                f"(achieved {rf['achieved']} GB/s); trace / events = "
                f"{avg / rf['avg_launch_us']:.4f}.  That process's whole-step value: "
                f"{bl['value']} GB/s ({bl['pct_of_peak']}% of 8 TB/s).")
        if stem == "fused_qknorm_rope_w8_wan720p" and bl and "rows" in bl:
            fr = bl["rows"].get("w8_fused_qknorm_rope", {})
            if fr:
                lines.append(f"The profiled bench process's own median for the fused row: "
                             f"{fr['fused_qk_median_us']} us ({fr['fused_qk_gbs']} GB/s).")
        if "FETCH_SIZE" in c and "WRITE_SIZE" in c and fetch_factor:
            traffic = (c["FETCH_SIZE"] * fetch_factor + c["WRITE_SIZE"] * write_factor) * 1024
            lines.append(f"HBM traffic from the FETCH_SIZE / WRITE_SIZE passes: {stem}_counters.json"
                         f" (calibrated traffic / algorithmic bytes = {traffic / nbytes:.5f}).")
            j = {
                "kernel": kern, "grid_threads": grid, "what": what,
                "dispatches_counted": [counts["FETCH_SIZE"], counts["WRITE_SIZE"]],
                "commands": [pmc_cmd("fetch"), pmc_cmd("write"), pmc_cmd("rdreq"),
                             pmc_cmd("wrreq")],
                "fetch_kib_per_dispatch": round(c["FETCH_SIZE"], 2),
                "write_kib_per_dispatch": round(c["WRITE_SIZE"], 2),
                "calibration": {
                    "kernel": CALIBRATION[0],
                    "what": "torch device-to-device copy of 774,144,000 bytes in the same run",
                    "bytes_read": CALIBRATION_BYTES, "bytes_written": CALIBRATION_BYTES,
                    "fetch_kib_per_dispatch": round(cal["FETCH_SIZE"], 2),
                    "write_kib_per_dispatch": round(cal["WRITE_SIZE"], 2),
                    "fetch_factor": round(fetch_factor, 6),
                    "write_factor": round(write_factor, 6)},
                "traffic_bytes_per_launch": round(traffic),
                "algorithmic_bytes_per_launch": nbytes,
                "traffic_over_algorithmic": round(traffic / nbytes, 5),
                "kernel_source_sha256": sha,
            }
            if "TCC_EA0_RDREQ_sum" in c:
                # every read request of these kernels is a 128-byte one (no 32-byte
                # requests; TCC_BUBBLE, which FETCH_SIZE prices at 128 bytes, reads 0)
                j["raw_ea_requests"] = {
                    "rdreq": round(c["TCC_EA0_RDREQ_sum"]),
                    "rdreq_32b": round(c.get("TCC_EA0_RDREQ_32B_sum", 0)),
                    "bubble": round(c.get("TCC_BUBBLE_sum", 0)),
                    "wrreq": round(c.get("TCC_EA0_WRREQ_sum", 0)),
                    "wrreq_64b": round(c.get("TCC_EA0_WRREQ_64B_sum", 0)),
                    "read_bytes_at_128_per_request": round(c["TCC_EA0_RDREQ_sum"] * 128),
                    "write_bytes_at_64_per_request": round(c.get("TCC_EA0_WRREQ_64B_sum", 0) * 64),
                }
            with open(os.path.join(PROFILES, f"{stem}_counters.json"), "w") as f:
                json.dump(j, f, indent=1)
                f.write("\n")
        with open(os.path.join(PROFILES, f"{stem}_kernel_trace.md"), "w") as f:
            f.write("\n".join(lines) + "\n")
        if "SQ_WAVES" in c and "TA_TA_BUSY_sum" in c:
            table.append((stem, kern, avg, c))
    if cal_trace and cal.get("SQ_WAVES"):
        table.append(("calibration copy (torch d2d, 774 MB)", CALIBRATION[0],
                      statistics.mean(cal_trace), cal))
    write_account(table)


def write_account(table):
    """The SQ / TA / TCP counters of each kernel, per wave and per CU cycle."""
    lines = [
        "# Where the cycles go: SQ, TA, TD and TCP counters per kernel", "",
        "Commands (from /tmp with TMPDIR=/tmp, on one MI355X; REPO is this repository, OUT any "
        "output folder), one counter pass per run, then "
        "`python3 REPO/summarize_profiles.py OUT`:", "", "```"]
    lines += [pmc_cmd(p) for p in ("sq1", "sq2", "tcp")]
    lines += ["```", "",
              "Each figure is the mean over the kernel's dispatches.  Cycles = GRBM_GUI_ACTIVE / 8 "
              "(the counter adds the 8 XCDs; divided by the trace's average duration it gives the "
              "clock below).  VALU busy = SQ_ACTIVE_INST_VALU x 4 / (1024 SIMDs x cycles): a "
              "wave64 VALU instruction holds a 16-lane SIMD for 4 cycles.  SALU, TA, TD busy and "
              "the TCP-to-TA data stall are per CU: the counter / (256 x cycles).", "",
              "| Kernel | Waves | VALU / wave | SALU / wave | SMEM / wave | VMEM rd + wr / wave "
              "| Clock (GHz) | VALU busy | SALU busy | TA busy | TD busy | TCP->TA data stall |",
              "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for stem, kern, avg_us, c in table:
        w = c["SQ_WAVES"]
        cyc = c["GRBM_GUI_ACTIVE"] / XCDS
        ghz = cyc / (avg_us * 1e3)
        lines.append(
            f"| {stem} (`{kern}`) | {w:,.0f} | {c['SQ_INSTS_VALU'] / w:.1f} | "
            f"{c['SQ_INSTS_SALU'] / w:.1f} | {c['SQ_INSTS_SMEM'] / w:.1f} | "
            f"{c['SQ_INSTS_VMEM_RD'] / w:.1f} + {c['SQ_INSTS_VMEM_WR'] / w:.1f} | {ghz:.2f} | "
            f"{100 * c['SQ_ACTIVE_INST_VALU'] * 4 / (SIMDS * cyc):.0f}% | "
            f"{100 * c['SQ_ACTIVE_INST_SCA'] / (CUS * cyc):.0f}% | "
            f"{100 * c['TA_TA_BUSY_sum'] / (CUS * cyc):.0f}% | "
            f"{100 * c['TD_TD_BUSY_sum'] / (CUS * cyc):.0f}% | "
            f"{100 * c.get('TCP_TCP_TA_DATA_STALL_CYCLES_sum', 0) / (CUS * cyc):.0f}% |")
    with open(os.path.join(PROFILES, "counters_by_kernel.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
