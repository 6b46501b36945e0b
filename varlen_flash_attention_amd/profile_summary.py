"""Turn rocprofv3 outputs of bench.py into the short summaries kept under profiles/.

Inputs (a directory written by the four commands below):
  <dir>/trace/bench_kernel_trace.csv, <dir>/trace/bench_kernel_stats.csv, <dir>/trace.log
  <dir>/FETCH_SIZE/bench_counter_collection.csv, <dir>/WRITE_SIZE/bench_counter_collection.csv
  <dir>/MFMA/bench_counter_collection.csv
Usage: python -m varlen_flash_attention_amd.profile_summary <dir> <profiles dir>
"""
import collections
import csv
import hashlib
import json
import os
import sys

TRACE_CMD = ("cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/trace -o bench -- "
             "python3 <repo>/bench.py --no-cpu > <dir>/trace.log")
PMC_CMD = ("cd /tmp && rocprofv3 --pmc {c} --output-format csv -d <dir>/{c} -o bench -- "
           "python3 <repo>/bench.py --no-cpu --steps 3 --warmup 1 --copy-calibration")
MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_INSTS_VALU "
                 "SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE")
MFMA_CMD = ("cd /tmp && rocprofv3 --pmc " + MFMA_COUNTERS + " --output-format csv -d <dir>/MFMA -o bench -- "
            "python3 <repo>/bench.py --no-cpu --steps 3 --warmup 1")
HEAD = "attn_fwd_overlap_kernelILi128ELb1EDF16b"   # the long-prefill kernel: D=128, causal, bf16 out
EMBED = "attn_fwd_short_kernelILi128ELb1EDF16b"   # short sequences: D=128, causal, bf16 out
SIMDS = 1024          # MI355X: 256 CUs x 4 SIMDs
XCCS = 8
MERGE = "attn_update_kernel<float, 128, 8, 1>"          # the merge config shape (one row per thread)
MERGE_BYTES = 9510912                                   # sp*bsh*(hd+1)*4 + bsh*(hd+1)*4 at sp=8, bsh=2048, hd=128
MERGE_GRID = 2048 * 32                                  # threads: 32 lanes per row at hd=128, fp32
FLUSH = ("reduce_kernel", "FillFunctor")               # the 1 GiB cache flush before each cold call
COPY = "__amd_rocclr_copyBuffer"
COPY_BYTES = 1 << 28


def short(name, n=100):
    return name if len(name) <= n else name[:n - 3] + "..."


def main(src, dst):
    repo = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    log = open(os.path.join(src, "trace.log")).read().splitlines()
    bench = json.loads([l for l in log if l.startswith("{")][-1])
    steps, warmup = bench["steps"], bench["warmup"]
    flops = bench["config"]["useful_gflop_per_step"] * 1e9
    event_ms = flops / (bench["roofline"]["achieved"] * 1e12) * 1e3

    stats = list(csv.DictReader(open(os.path.join(src, "trace", "bench_kernel_stats.csv"))))
    trace = list(csv.DictReader(open(os.path.join(src, "trace", "bench_kernel_trace.csv"))))
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    head_us = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in trace if HEAD in r["Kernel_Name"]]
    timed = head_us[warmup:warmup + steps]
    trace_avg = sum(timed) / len(timed)

    lines = ["# rocprofv3 kernel trace of bench.py: long-prefill causal headline and the extra workloads", "",
             "command (repository root copied to <repo>, TMPDIR=/tmp):", "  " + TRACE_CMD,
             "summarised by: python -m varlen_flash_attention_amd.profile_summary <dir> profiles", "",
             f"{'calls':>6} {'avg us':>10} {'min us':>10} {'max us':>10}  kernel"]
    for r in stats:
        lines.append(f"{int(r['Calls']):6d} {float(r['AverageNs'])/1e3:10.2f} {float(r['MinNs'])/1e3:10.2f} "
                     f"{float(r['MaxNs'])/1e3:10.2f}  {short(r['Name'])}")
    lines += ["",
              "kernel name key: attn_fwd_overlap_kernel<D, CAUSAL, OutT> (ILi128ELb1 = D 128, causal: the headline; "
              "ILi128ELb0 = the non-causal extra) runs after zero_tickets_kernel, which clears its work counters; "
              "attn_fwd_short_kernel<D, CAUSAL, OutT> (4 waves of 32 query columns, three workgroups per CU) "
              "serves the embedding prefill.",
              "  attn_decode_split_kernel<D, CAUSAL, PAGED, OutT>: ILi128ELb1ELb0 = contiguous decode (bench extra "
              "'decode'), ILi128ELb1ELb1 = paged decode (extras 'paged_decode_p16' and '_p128', one row for both).",
              "  gdn_prep_kernel<DK> then gdn_chunk_kernel<DK, DV>: one gated delta rule call (extra "
              "'gated_delta_rule', chunked form, Dk = Dv = 128).",
              f"headline kernel: {len(head_us)} launches = {warmup} warm-up + {steps} timed + the later extras' "
              "launches of the same kernel (none).",
              f"agreement: the {steps} timed launches average {trace_avg:.1f} us in this trace; bench.py's HIP events "
              f"on the launch stream gave {event_ms*1e3:.1f} us per launch in the same run "
              f"(roofline.achieved {bench['roofline']['achieved']} TFLOP/s, frac {bench['roofline']['frac']}).",
              "timed launch durations (us): " + ", ".join(f"{x:.0f}" for x in timed)]
    os.makedirs(dst, exist_ok=True)
    open(os.path.join(dst, "attn_fwd_long_prefill.kernel_stats.txt"), "w").write("\n".join(lines) + "\n")

    # Merge at the config shape: kernel durations, cold (right after the flush) and warm.
    cold, warm = [], []
    for prev, r in zip(trace, trace[1:]):
        if MERGE in r["Kernel_Name"] and int(r.get("Grid_Size_X", MERGE_GRID)) == MERGE_GRID:
            us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            (cold if any(f in prev["Kernel_Name"] for f in FLUSH) else warm).append(us)
    # Dispatch floors timed cold in the same case: the one-element fill and the
    # read-only sum over the merge's partials (a reduce much shorter than the
    # 1 GiB flush), each right after a flush.
    # A multi-block torch sum clears its own semaphore with a runtime fill
    # kernel first, so pairing skips those fills.
    fill_floor, sum_floor = [], []
    kernels = [r for r in trace if "__amd_rocclr_fillBuffer" not in r["Kernel_Name"]]
    for prev, r in zip(kernels, kernels[1:]):
        if not any(f in prev["Kernel_Name"] for f in FLUSH):
            continue
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        grid = int(r.get("Grid_Size", r.get("Grid_Size_X", 0)) or 0)
        if "FillFunctor<float>" in r["Kernel_Name"] and 0 < grid <= 1024:
            fill_floor.append(us)
        elif "reduce_kernel" in r["Kernel_Name"] and us < 60:
            sum_floor.append(us)
    if cold:
        def q(xs, f):
            ys = sorted(xs)
            return ys[min(len(ys) - 1, int(f * len(ys)))]
        ml = ["# rocprofv3 kernel durations of attn_update at the merge shape (sp=8, bsh=2048, hd=128, fp32)", "",
              "command: the kernel trace above (bench.py's merge case: cold calls follow a 1 GiB read that "
              "evicts L2 and the last-level cache; warm calls are queued back to back)",
              "summarised by: python -m varlen_flash_attention_amd.profile_summary <dir> profiles", "",
              f"algorithmic bytes per call: {MERGE_BYTES}", ""]
        for name, xs in (("cold", cold), ("warm", warm)):
            if not xs:
                continue
            med = q(xs, 0.5)
            ml.append(f"{name}: {len(xs)} calls, kernel median {med:.2f} us (p10 {q(xs, 0.1):.2f}, "
                      f"p90 {q(xs, 0.9):.2f}) -> {MERGE_BYTES / med / 1e3:.0f} GB/s, "
                      f"{MERGE_BYTES / med / 1e3 / 8000:.1%} of 8 TB/s")
        for name, xs in (("one-element fill (dispatch floor), cold", fill_floor),
                         ("read-only sum of the 8.4 MB of partials, cold", sum_floor)):
            if xs:
                ml.append(f"{name}: {len(xs)} calls, kernel median {q(xs, 0.5):.2f} us (p10 {q(xs, 0.1):.2f}, "
                          f"p90 {q(xs, 0.9):.2f})")
        ml += ["", f"70% of HBM peak at this size means a kernel of {MERGE_BYTES / 0.7 / 8e6:.2f} us, shorter than "
               "the one-element fill: a kernel that moves nothing already takes that long from start to end "
               "timestamp on this device, so the fill is the floor for any kernel here."]
        if fill_floor:
            f = q(fill_floor, 0.5)
            ml.append(f"attainable at this size: {MERGE_BYTES} B in {f:.2f} us = {MERGE_BYTES / f / 1e3:.0f} GB/s "
                      f"({MERGE_BYTES / f / 1e3 / 8000:.1%} of 8 TB/s); the cold merge reaches "
                      f"{f / q(cold, 0.5):.1%} of it.")
        if sum_floor:
            ml.append(f"torch's own read-only sum over the partials (no output to speak of) takes "
                      f"{q(sum_floor, 0.5) / q(cold, 0.5):.1f}x the merge's time.")
        open(os.path.join(dst, "attn_update_merge.kernel_durations.txt"), "w").write("\n".join(ml) + "\n")

    def counter(c):
        per = collections.defaultdict(list)
        for r in csv.DictReader(open(os.path.join(src, c, "bench_counter_collection.csv"))):
            per[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return per
    fetch, write = counter("FETCH_SIZE"), counter("WRITE_SIZE")
    copy_f, copy_w = max(fetch[COPY]), max(write[COPY])
    sf, sw = COPY_BYTES / (copy_f * 1024), COPY_BYTES / (copy_w * 1024)
    tl = ["# HBM traffic per dispatch from rocprofv3 FETCH_SIZE / WRITE_SIZE, bench.py with the extra workloads", "",
          "commands (one counter per run, repository root copied to <repo>, TMPDIR=/tmp):",
          "  " + PMC_CMD.format(c="FETCH_SIZE"), "  " + PMC_CMD.format(c="WRITE_SIZE"),
          "summarised by: python -m varlen_flash_attention_amd.profile_summary <dir> profiles", "",
          f"calibration: a 256 MiB device-to-device copy with cold caches reads FETCH_SIZE {copy_f:.1f} KiB and "
          f"WRITE_SIZE {copy_w:.1f} KiB; scales {sf:.4f} (fetch) and {sw:.4f} (write) convert the counters to bytes.",
          "", f"{'calls':>6} {'read MB':>10} {'write MB':>10}  kernel (mean per dispatch, calibrated)"]
    rec = None
    for name in sorted(fetch, key=lambda n: -sum(fetch[n]) / len(fetch[n])):
        if name not in write:
            continue
        f_b = sum(fetch[name]) / len(fetch[name]) * 1024 * sf
        w_b = sum(write[name]) / len(write[name]) * 1024 * sw
        tl.append(f"{len(fetch[name]):6d} {f_b/1e6:10.2f} {w_b/1e6:10.2f}  {short(name)}")
        if HEAD in name:
            rec = (sum(fetch[name]) / len(fetch[name]), sum(write[name]) / len(write[name]), f_b, w_b)
    tl += ["", "attn_update_kernel<float, 128, 8, 1> runs the 2048-row merge shape (cold and warm calls "
           "averaged, plus the 4x sweep point); <..., 2> the 16x and 64x sweep points (two rows per thread).",
           "gdn_prep_kernel writes the per-chunk T and M rows and decay factors (520 B per token and value head) and ranks the sequences by length; "
           "gdn_chunk_kernel reads them back with the chunk's K, Q and V and writes the output."]
    open(os.path.join(dst, "bench_kernels.hbm_traffic.txt"), "w").write("\n".join(tl) + "\n")

    sha = hashlib.sha256(open(os.path.join(repo, "varlen_flash_attention_amd", "csrc", "attn_fwd_overlap.hip"),
                              "rb").read()).hexdigest()
    mfma_summary(src, dst, bench, sha)
    out = {
        "kernel": "attn_fwd_overlap_kernel<128, causal, bf16> on the long-prefill workload (seed 3)",
        "kernel_source_sha256": sha,
        "fetch_size_kib_per_launch": round(rec[0], 1), "write_size_kib_per_launch": round(rec[1], 1),
        "copy_calibration": {"bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES, "fetch_size_kib": copy_f,
                             "write_size_kib": copy_w, "fetch_scale": round(sf, 4), "write_scale": round(sw, 4)},
        "hbm_read_bytes_per_launch": int(rec[2]), "hbm_write_bytes_per_launch": int(rec[3]),
        "hbm_bytes_per_launch": int(rec[2] + rec[3]),
        "commands": [PMC_CMD.format(c="FETCH_SIZE"), PMC_CMD.format(c="WRITE_SIZE")],
    }
    json.dump(out, open(os.path.join(dst, "attn_fwd_long_prefill_traffic.json"), "w"), indent=1)
    print("\n".join(lines[-4:-1]))
    print("\n".join(tl))


def mfma_summary(src, dst, bench, sha):
    """MFMA counters per dispatch of the two prefill kernels: issued bf16 MFMA FLOPs (MOPS x 512) against
    the useful FLOPs, the matrix unit's busy cycles per SIMD against the GPU's active cycles, and the clock
    those cycles imply over the dispatch's duration."""
    rows = list(csv.DictReader(open(os.path.join(src, "MFMA", "bench_counter_collection.csv"))))
    disp = collections.defaultdict(dict)
    for r in rows:
        d = disp[r["Dispatch_Id"]]
        d["name"] = r["Kernel_Name"]
        d["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    useful = {HEAD: bench["config"]["useful_gflop_per_step"] * 1e9,
              EMBED: bench["extra"]["embed_prefill_with_gather"]["useful_gflop"] * 1e9}
    lines = ["# rocprofv3 MFMA counters of the prefill kernels, per dispatch (bench.py with the extra workloads)", "",
             "command (repository root copied to <repo>, TMPDIR=/tmp):", "  " + MFMA_CMD,
             "summarised by: python -m varlen_flash_attention_amd.profile_summary <dir> profiles", "",
             "definitions (counters summed over the device by rocprofv3):",
             "  issued MFMA FLOPs      = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512",
             f"  cycles per XCD        = GRBM_GUI_ACTIVE / {XCCS}",
             f"  MFMA busy (per SIMD)  = SQ_VALU_MFMA_BUSY_CYCLES / ({SIMDS} SIMDs x cycles per XCD)",
             "  clock                 = cycles per XCD / dispatch duration",
             "  one busy cycle = 2 MOPS = 1024 FLOPs: a SIMD's bf16 peak per cycle (2.5 PFLOP/s = 1024 SIMDs x 1024 "
             "x 2.4 GHz)", ""]
    for key, label in ((HEAD, "long prefill, causal (headline kernel)"), (EMBED, "embedding prefill, causal")):
        ds = [d for d in disp.values() if key in d["name"]]
        if not ds:
            continue
        n = len(ds)
        mops = sum(d["SQ_INSTS_VALU_MFMA_MOPS_BF16"] for d in ds) / n
        busy = sum(d["SQ_VALU_MFMA_BUSY_CYCLES"] for d in ds) / n
        cyc = sum(d["GRBM_GUI_ACTIVE"] for d in ds) / n / XCCS
        ns = sum(d["ns"] for d in ds) / n
        valu = sum(d["SQ_INSTS_VALU"] for d in ds) / n
        mfma = sum(d["SQ_INSTS_MFMA"] for d in ds) / n
        clocks = sorted(d["GRBM_GUI_ACTIVE"] / XCCS / d["ns"] for d in ds)
        lines += [f"{label}: {short(ds[0]['name'])}",
                  f"  dispatches {n}; mean duration {ns / 1e3:.1f} us; cycles per XCD {cyc:.0f}; clock "
                  f"{cyc / ns:.2f} GHz (range {clocks[0]:.2f}-{clocks[-1]:.2f})",
                  f"  issued MFMA {mops * 512 / 1e9:.1f} GFLOP vs useful {useful[key] / 1e9:.1f} GFLOP: "
                  f"{mops * 512 / useful[key]:.3f}x (causal diagonal tiles and partial tiles)",
                  f"  MFMA busy per SIMD {busy / (SIMDS * cyc):.3f} of active cycles "
                  f"(= issued MFMA rate / (1024 FLOP/cycle x SIMDs x clock))",
                  f"  instructions: {mfma / 1e6:.1f} M MFMA, {valu / 1e6:.1f} M VALU ({valu / max(mfma, 1):.2f} VALU per MFMA)",
                  ""]
    lines.append(f"long-prefill kernel source sha256: {sha}")
    open(os.path.join(dst, "prefill_kernels.mfma_counters.txt"), "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main(sys.argv[1], sys.argv[2])
