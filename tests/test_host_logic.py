"""CPU tests of the host-side logic: workload shapes, FLOP / byte accounting, the bf16
rounding the inputs go through, chunk bounds, bench.py's command line and the
rocprofv3 summariser."""
import csv
import json
import math
import os
import subprocess
import sys

import numpy as np
import pytest

from varlen_flash_attention_amd.workloads import (bf16_bits, chunk_bounds, make_custom, make_growing_scores,
                                                  make_workload, round_to_bf16)

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


# ------------------------------------------------------------------ workload shapes

def test_workload_shapes_match_their_descriptions():
    w = make_workload("tiny_fp32", values=False)
    assert w.lengths_q.tolist() == [17, 64, 5, 128] and w.total_q == 214
    assert (w.num_heads_q, w.num_heads_kv, w.head_dim, w.dtype, w.causal) == (4, 2, 64, "fp32", True)
    assert w.scale == pytest.approx(1 / 8)

    w = make_workload("embed_prefill", values=False)
    assert w.batch == 64 and w.lengths_q.min() >= 32 and w.lengths_q.max() <= 512
    assert (w.num_heads_q, w.num_heads_kv, w.head_dim, w.dtype, w.causal) == (16, 8, 128, "bf16", True)
    assert (w.lengths_q == w.lengths_k).all()

    for name, causal in (("long_prefill", True), ("long_prefill_full", False)):
        w = make_workload(name, values=False)
        assert w.batch == 16 and w.lengths_q.min() >= 256 and w.lengths_q.max() <= 8192
        assert (w.num_heads_q, w.num_heads_kv, w.head_dim, w.causal) == (32, 8, 128, causal)
    # both long-prefill variants draw the same lengths
    assert (make_workload("long_prefill", values=False).lengths_q
            == make_workload("long_prefill_full", values=False).lengths_q).all()

    w = make_workload("decode", values=False)
    assert w.batch == 64 and (w.lengths_q == 1).all()
    assert w.lengths_k.min() >= 1024 and w.lengths_k.max() <= 32768
    assert (w.num_heads_q, w.num_heads_kv, w.head_dim) == (32, 4, 128)


def test_cu_seqlens_are_prefix_sums():
    w = make_custom([3, 0, 5], [4, 2, 0], num_heads_q=2, num_heads_kv=1, head_dim=8)
    assert w.cu_seqlens_q.tolist() == [0, 3, 3, 8]
    assert w.cu_seqlens_k.tolist() == [0, 4, 6, 6]
    assert w.cu_seqlens_q.dtype == np.int32 and w.max_seqlen_q == 5 and w.max_seqlen_k == 4


def _brute_visible(lq, lk, causal):
    n = 0
    for a, b in zip(lq, lk):
        for i in range(a):
            for j in range(b):
                n += (not causal) or j <= i + b - a
    return n


@pytest.mark.parametrize("causal", [True, False])
def test_visible_pairs_and_flops_against_brute_force(causal):
    lq, lk = [7, 1, 0, 12, 5], [7, 9, 3, 4, 0]        # Lq = Lk, Lq < Lk, empty, Lq > Lk, no keys
    w = make_custom(lq, lk, num_heads_q=6, num_heads_kv=2, head_dim=16, causal=causal)
    assert w.visible_pairs() == _brute_visible(lq, lk, causal)
    assert w.useful_flops() == 4 * 16 * 6 * _brute_visible(lq, lk, causal)


def test_compulsory_bytes():
    w = make_custom([4, 6], [5, 7], num_heads_q=4, num_heads_kv=2, head_dim=8, dtype="bf16")
    tq, tk = 10, 12
    assert w.compulsory_bytes() == tq * 4 * 8 * 2 + 2 * tk * 2 * 8 * 2 + tq * 4 * 8 * 2 + tq * 4 * 4
    assert w.compulsory_bytes(4) == tq * 4 * 8 * 2 + 2 * tk * 2 * 8 * 2 + tq * 4 * 8 * 4 + tq * 4 * 4


def test_values_are_seeded_and_bf16_exact():
    a = make_custom([33, 2], num_heads_q=2, num_heads_kv=1, head_dim=16, dtype="bf16", seed=9)
    b = make_custom([33, 2], num_heads_q=2, num_heads_kv=1, head_dim=16, dtype="bf16", seed=9)
    c = make_custom([33, 2], num_heads_q=2, num_heads_kv=1, head_dim=16, dtype="bf16", seed=10)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.v, b.v) and not np.array_equal(a.q, c.q)
    bf16_bits(a.q)          # raises unless every value is bf16-exact
    assert abs(float(a.q.mean())) < 0.3 and 0.7 < float(a.q.std()) < 1.3


# ------------------------------------------------------------------ bf16 rounding

def test_growing_scores_workload():
    # seeded, bf16-exact, and the documented climb: a row's raw scores run from about 0 to about top_score
    a = make_growing_scores([300, 5], num_heads_q=4, num_heads_kv=2, head_dim=64, dtype="bf16", seed=3,
                            top_score=800.0)
    b = make_growing_scores([300, 5], num_heads_q=4, num_heads_kv=2, head_dim=64, dtype="bf16", seed=3,
                            top_score=800.0)
    assert all(np.array_equal(x, y) for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v)))
    bf16_bits(a.q), bf16_bits(a.k), bf16_bits(a.v)           # raises unless bf16-exact
    s = a.q[299, 0].astype(np.float64) @ a.k[:300, 0].astype(np.float64).T
    assert 0 < s[0] < 20 and 700 < s[-1] < 900
    assert np.all(np.diff(s[::30]) > 0)                      # climbs along the sequence
    assert a.lengths_q.tolist() == a.lengths_k.tolist() == [300, 5]


def test_round_to_bf16_ties_to_even_and_bits():
    one = 1.0
    ulp = 2.0 ** -7                                    # bf16 spacing in [1, 2)
    x = np.array([one, one + ulp / 2, one + 3 * ulp / 2, one + ulp / 4, -(one + 3 * ulp / 4), 3.0e38,
                  2.0 ** -130], dtype=np.float32)
    r = round_to_bf16(x)
    assert r[0] == 1.0
    assert r[1] == 1.0                                 # tie -> even (mantissa ...0)
    assert r[2] == np.float32(one + 2 * ulp)           # tie -> even (mantissa ...0 upward)
    assert r[3] == 1.0
    assert r[4] == np.float32(-(one + ulp))
    assert np.isfinite(r[5])
    assert r[6] == np.float32(2.0 ** -130)             # exactly representable subnormal
    bits = bf16_bits(r)
    assert bits.dtype == np.uint16 and bits[0] == 0x3F80
    with pytest.raises(ValueError):
        bf16_bits(np.array([one + ulp / 4], dtype=np.float32))


def test_round_to_bf16_matches_nearest_bf16_on_random_values():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(20000) * 10.0 ** rng.integers(-5, 5, 20000)).astype(np.float32)
    r = round_to_bf16(x).astype(np.float64)
    # the two bf16 neighbours of x: truncation and the next value up in magnitude
    u = x.view(np.uint32)
    lo = (u & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)
    hi = ((u & np.uint32(0xFFFF0000)) + np.uint32(0x10000)).view(np.float32).astype(np.float64)
    d_lo, d_hi = np.abs(x - lo), np.abs(x - hi)
    assert np.all(np.abs(x - r) <= np.minimum(d_lo, d_hi) + 0.0)
    assert np.all((r == lo) | (r == hi))


# ------------------------------------------------------------------ chunk bounds

@pytest.mark.parametrize("length,sp", [(0, 1), (1, 4), (4096, 8), (1000, 3), (17, 17), (5, 2)])
def test_chunk_bounds_partition(length, sp):
    b = chunk_bounds(length, sp)
    assert len(b) == sp and b[0][0] == 0 and b[-1][1] == length
    assert all(b[i][1] == b[i + 1][0] for i in range(sp - 1))
    sizes = [hi - lo for lo, hi in b]
    assert max(sizes) - min(sizes) <= 1


# ------------------------------------------------------------------ bench.py command line

def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(REPO, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


# ------------------------------------------------------------------ rocprofv3 summariser

HEAD = "_ZN3vfa12_GLOBAL__N_123attn_fwd_overlap_kernelILi128ELb1EDF16bEEvX"
EMBED = "_ZN3vfa12_GLOBAL__N_121attn_fwd_short_kernelILi128ELb1EDF16bEEvX"


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(header)
        w.writerows(rows)


def test_profile_summary_on_synthetic_counters(tmp_path):
    from varlen_flash_attention_amd import profile_summary
    src, dst = tmp_path / "prof", tmp_path / "out"
    steps, warmup = 3, 2
    bench = {"steps": steps, "warmup": warmup, "config": {"useful_gflop_per_step": 2000.0},
             "roofline": {"achieved": 1000.0, "frac": 0.4},
             "extra": {"embed_prefill_with_gather": {"useful_gflop": 20.0}}}
    os.makedirs(src, exist_ok=True)
    (src / "trace.log").write_text("[bench] noise\n" + json.dumps(bench) + "\n")
    # 5 launches of the headline kernel, 1000 ns apart, durations 2.0 .. 2.4 ms
    trace = [["KERNEL_DISPATCH", i, HEAD, 10_000_000 * i, 10_000_000 * i + 2_000_000 + 100_000 * i]
             for i in range(5)]
    _write_csv(str(src / "trace" / "bench_kernel_trace.csv"),
               ["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], trace)
    _write_csv(str(src / "trace" / "bench_kernel_stats.csv"), ["Name", "Calls", "AverageNs", "MinNs", "MaxNs"],
               [[HEAD, 5, 2.2e6, 2.0e6, 2.4e6]])
    # copy kernel: 256 MiB read counted as half (FETCH) and written in full (WRITE)
    for counter, copy_val, head_val in (("FETCH_SIZE", 131072.0, 1000.0), ("WRITE_SIZE", 262144.0, 500.0)):
        _write_csv(str(src / counter / "bench_counter_collection.csv"),
                   ["Kernel_Name", "Counter_Name", "Counter_Value"],
                   [["__amd_rocclr_copyBuffer", counter, copy_val], [HEAD, counter, head_val],
                    [HEAD, counter, head_val]])
    # MFMA counters: one dispatch of the headline kernel, 2 ms long, 8 XCCs x 3.6M active cycles (1.8 GHz);
    # 2100 GFLOP issued (4.1016e9 MOPS x 512) and busy cycles for 50% of 1024 SIMDs
    mf = []
    for name, val in (("SQ_INSTS_VALU_MFMA_MOPS_BF16", 2100e9 / 512), ("SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * 1024 * 3.6e6),
                      ("SQ_INSTS_MFMA", 64e6), ("SQ_INSTS_VALU", 256e6), ("SQ_BUSY_CU_CYCLES", 1.0),
                      ("GRBM_GUI_ACTIVE", 8 * 3.6e6)):
        mf.append([7, HEAD, name, val, 0, 2_000_000])
    _write_csv(str(src / "MFMA" / "bench_counter_collection.csv"),
               ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"], mf)
    profile_summary.main(str(src), str(dst))
    mtxt = (dst / "prefill_kernels.mfma_counters.txt").read_text()
    assert "clock 1.80 GHz" in mtxt
    assert "issued MFMA 2100.0 GFLOP vs useful 2000.0 GFLOP: 1.050x" in mtxt
    assert "MFMA busy per SIMD 0.500" in mtxt
    assert "4.00 VALU per MFMA" in mtxt
    rec = json.load(open(dst / "attn_fwd_long_prefill_traffic.json"))
    assert rec["copy_calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert rec["copy_calibration"]["write_scale"] == pytest.approx(1.0)
    assert rec["hbm_read_bytes_per_launch"] == 2 * 1000 * 1024
    assert rec["hbm_write_bytes_per_launch"] == 500 * 1024
    txt = (dst / "attn_fwd_long_prefill.kernel_stats.txt").read_text()
    # timed launches are dispatches 2, 3, 4 (after 2 warm-up): 2.2, 2.3, 2.4 ms -> 2300 us
    assert "average 2300.0 us" in txt
    assert f"gave {2000.0 / 1000.0 * 1e3:.1f} us" in txt
    assert math.isclose(rec["hbm_bytes_per_launch"], 2 * 1000 * 1024 + 500 * 1024)
