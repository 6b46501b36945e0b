"""Turn rocprofv3 outputs of bench.py into the short summaries kept under profiles/.

Inputs (a directory written by the three commands below):
  <dir>/trace/bench_kernel_trace.csv, <dir>/trace/bench_kernel_stats.csv, <dir>/trace.log
  <dir>/FETCH_SIZE/bench_counter_collection.csv, <dir>/WRITE_SIZE/bench_counter_collection.csv
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
HEAD = "attn_fwd_bf16_kernelILi8ELi1ELi128ELb1EDF16b"   # 8 waves x 32 columns, D=128, causal, bf16 out
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
              "kernel name key: attn_fwd_bf16_kernel<WAVES, NQ, D, CAUSAL, OutT>; ILi8ELi1ELi128ELb1 = 8 waves of "
              "32 query columns, D=128, causal.",
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
    open(os.path.join(dst, "attn_fwd_bf16_long_prefill.kernel_stats.txt"), "w").write("\n".join(lines) + "\n")

    # Merge at the config shape: kernel durations, cold (right after the flush) and warm.
    cold, warm = [], []
    for prev, r in zip(trace, trace[1:]):
        if MERGE in r["Kernel_Name"] and int(r.get("Grid_Size_X", MERGE_GRID)) == MERGE_GRID:
            us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            (cold if any(f in prev["Kernel_Name"] for f in FLUSH) else warm).append(us)
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

    sha = hashlib.sha256(open(os.path.join(repo, "varlen_flash_attention_amd", "csrc", "attn_fwd_bf16.hip"),
                              "rb").read()).hexdigest()
    out = {
        "kernel": "attn_fwd_bf16_kernel<8, 1, 128, causal, bf16> on the long-prefill workload (seed 3)",
        "kernel_source_sha256": sha,
        "fetch_size_kib_per_launch": round(rec[0], 1), "write_size_kib_per_launch": round(rec[1], 1),
        "copy_calibration": {"bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES, "fetch_size_kib": copy_f,
                             "write_size_kib": copy_w, "fetch_scale": round(sf, 4), "write_scale": round(sw, 4)},
        "hbm_read_bytes_per_launch": int(rec[2]), "hbm_write_bytes_per_launch": int(rec[3]),
        "hbm_bytes_per_launch": int(rec[2] + rec[3]),
        "commands": [PMC_CMD.format(c="FETCH_SIZE"), PMC_CMD.format(c="WRITE_SIZE")],
    }
    json.dump(out, open(os.path.join(dst, "attn_fwd_bf16_long_prefill_traffic.json"), "w"), indent=1)
    print("\n".join(lines[-4:-1]))
    print("\n".join(tl))


if __name__ == "__main__":
    main(sys.argv[1], sys.argv[2])
