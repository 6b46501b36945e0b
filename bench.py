#!/usr/bin/env python3
"""Benchmark of the varlen attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extra]

A step is one varlen_attn_fwd call over the long-prefill workload (16
sequences, log-normal lengths with median 2048 clipped to [256, 8192],
Hq=32, Hkv=8, D=128, bf16, causal), inputs already resident in HBM. The
headline value is useful TFLOP/s: 4 * D FLOPs per visible (query row, query
head, key), masked pairs excluded. One JSON line is printed.

Extra fields (not the headline): the embedding-style prefill with the
last-token gather, the same long prefill without masking, decode against
long KV sets (contiguous, and paged with 16- and 128-key pages), the q/k
RMSNorm + rotary prologue on the long-prefill tokens, the gated delta rule
(linear attention) on the same lengths and one decode step of it (64
sequences of one token, state traffic in TB/s), and the attn_update merge of the
chunked-context config (sp=8, bsh=2048, hd=128, fp32) timed with caches
flushed before every rep. The embedding prefill is also timed cold (a 1 GiB
read before every rep: its 227 MB fit in the last-level cache), and the
fp64 oracle is timed on full inputs of the tiny, embedding, decode and merge
configs (`cpu_baseline_per_config`).

"roofline" is the attention kernel's achieved useful FLOP rate (per-launch
HIP-event durations on the launch stream) against the bf16 dense MFMA peak;
"cpu_baseline" is the fp64 CPU oracle timed on a bounded sample of the same
workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_long_prefill_traffic.json")
KERNEL_SOURCE = os.path.join(ROOT, "varlen_flash_attention_amd", "csrc", "attn_fwd_overlap.hip")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def device_inputs(w, torch):
    import numpy as np
    from varlen_flash_attention_amd.workloads import bf16_bits

    def dev(x):
        return torch.from_numpy(bf16_bits(x).view(np.int16)).cuda().view(torch.bfloat16)

    return dict(q=dev(w.q), k=dev(w.k), v=dev(w.v), cu_q=torch.from_numpy(w.cu_seqlens_q).cuda(),
                cu_k=torch.from_numpy(w.cu_seqlens_k).cuda())


def time_calls(fn, reps, warmup, torch, flush=None, queue_ahead=False):
    """Per-call durations (ms) from HIP events on the current stream.

    queue_ahead: hold the stream in a spin kernel while the host enqueues every
    call, so that a kernel shorter than its own host launch cost is timed back
    to back rather than as launch-bound gaps."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    if queue_ahead:
        torch.cuda._sleep(int(2.0e5 * reps))      # ~0.1 ms per queued call at 2 GHz
    ev = []
    for _ in range(reps):
        if flush is not None:
            flush()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        ev.append((s, e))
    torch.cuda.synchronize()
    return [s.elapsed_time(e) for s, e in ev]


def median(xs):
    ys = sorted(xs)
    n = len(ys)
    return ys[n // 2] if n % 2 else 0.5 * (ys[n // 2 - 1] + ys[n // 2])


def attn_case(vfa, torch, w, reps=20, warmup=3, gather=False, cold=False):
    """One workload's call timed by HIP events; with cold=True each rep follows a 1 GiB read of other
    data that evicts the inputs from L2 and the 256 MB last-level cache (it leaves them clean)."""
    d = device_inputs(w, torch)
    out = torch.empty((w.total_q, w.num_heads_q, w.head_dim), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.total_q, w.num_heads_q), dtype=torch.float32, device="cuda")
    ws_bytes = vfa.varlen_attn_fwd_workspace_size(w.batch, w.total_q, w.max_seqlen_q, w.max_seqlen_k,
                                                  w.num_heads_q, w.num_heads_kv, w.head_dim)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    last = torch.empty((w.batch, w.num_heads_q, w.head_dim), dtype=torch.bfloat16, device="cuda")

    def call():
        vfa.varlen_attn_fwd(d["q"], d["k"], d["v"], d["cu_q"], d["cu_k"], w.max_seqlen_q, w.max_seqlen_k,
                            softmax_scale=w.scale, causal=w.causal, out=out, lse=lse, workspace=ws)
        if gather:
            vfa.varlen_last_token_gather(out, d["cu_q"], out=last)

    ms = time_calls(call, reps, warmup, torch)
    res = attn_stats(w, ms)
    if cold:
        scratch = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        res["cold"] = attn_stats(w, time_calls(call, reps, warmup, torch, flush=lambda: scratch.sum()))
        del scratch
    del d, out, lse, ws, last
    torch.cuda.empty_cache()
    return res


def attn_stats(w, ms, extra_bytes=0):
    """Median / p10 / p90 of per-call times (ms), useful TFLOP/s and compulsory-byte GB/s."""
    t = median(ms)
    flops = w.useful_flops()
    byt = w.compulsory_bytes() + extra_bytes
    return {
        "ms_median": round(t, 4), "ms_p10": round(sorted(ms)[len(ms) // 10], 4),
        "ms_p90": round(sorted(ms)[(9 * len(ms)) // 10], 4),
        "useful_tflops": round(flops / t / 1e9, 2), "frac_bf16_peak": round(flops / t / 1e9 / PEAK_BF16_TFLOPS, 4),
        "compulsory_gb_per_s": round(byt / t / 1e6, 1), "frac_hbm_peak": round(byt / t / 1e6 / PEAK_HBM_GBPS, 4),
        "useful_gflop": round(flops / 1e9, 3), "compulsory_mb": round(byt / 1e6, 2),
        # time at the binding roofline, min(MFMA peak, HBM peak x intensity), over the measured time
        "frac_attainable_roofline": round(max(flops / (PEAK_BF16_TFLOPS * 1e9), byt / (PEAK_HBM_GBPS * 1e6)) / t, 4),
        "total_q": w.total_q, "total_k": w.total_k, "batch": w.batch, "seed": w.seed,
    }


def paged_case(vfa, torch, w, page_size, reps=20, warmup=3):
    """paged_attn_decode on workload w with its K/V in a paged cache (shuffled pages of page_size keys)."""
    import numpy as np
    from varlen_flash_attention_amd.workloads import bf16_bits, make_paged

    pc = make_paged(w, page_size, seed=7)

    def dev(x):
        return torch.from_numpy(bf16_bits(x).view(np.int16)).cuda().view(torch.bfloat16)

    q, kc, vc = dev(w.q), dev(pc.k_cache), dev(pc.v_cache)
    table = torch.from_numpy(pc.block_table).cuda()
    used = torch.from_numpy(pc.seqused_k).cuda()
    cu_q = torch.from_numpy(w.cu_seqlens_q).cuda()
    del pc
    out = torch.empty((w.total_q, w.num_heads_q, w.head_dim), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.total_q, w.num_heads_q), dtype=torch.float32, device="cuda")
    ws_bytes = vfa.paged_attn_decode_workspace_size(w.batch, w.total_q, w.max_seqlen_q, w.max_seqlen_k,
                                                    w.num_heads_q, w.num_heads_kv, w.head_dim)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")

    def call():
        vfa.paged_attn_decode(q, kc, vc, table, cu_q, used, w.max_seqlen_q, w.max_seqlen_k, softmax_scale=w.scale,
                              causal=w.causal, out=out, lse=lse, workspace=ws)

    ms = time_calls(call, reps, warmup, torch)
    # block-table entries the call reads, on top of Q, K, V, O and lse
    res = attn_stats(w, ms, extra_bytes=int(sum(-(-int(n) // page_size) for n in w.lengths_k)) * 4)
    res["page_size"] = page_size
    del q, kc, vc, table, used, cu_q, out, lse, ws
    torch.cuda.empty_cache()
    return res


def prologue_case(vfa, torch, lengths, reps=20, warmup=3):
    """qk_norm_rope on the long-prefill tokens (Hq=32, Hkv=8, D=128): q and k read and written once,
    one fp32 cos / sin row per token."""
    import numpy as np
    from varlen_flash_attention_amd.workloads import bf16_bits, make_prologue

    p = make_prologue(lengths, 32, 8, 128, seed=9)

    def dev(x):
        return torch.from_numpy(bf16_bits(x).view(np.int16)).cuda().view(torch.bfloat16)

    q, k, wq, wk = dev(p.q), dev(p.k), dev(p.q_weight), dev(p.k_weight)
    cos, sin = torch.from_numpy(p.cos).cuda(), torch.from_numpy(p.sin).cuda()
    qo, ko = torch.empty_like(q), torch.empty_like(k)

    def call():
        vfa.qk_norm_rope(q, k, wq, wk, cos, sin, eps=p.eps, q_out=qo, k_out=ko)

    ms = time_calls(call, reps, warmup, torch)
    t = median(ms)
    tokens = int(p.lengths.sum())
    qk_bytes = tokens * (32 + 8) * 128 * 2
    byt = 2 * qk_bytes + 2 * tokens * 128 * 4 + 2 * 128 * 2
    res = {"ms_median": round(t, 4), "ms_p10": round(sorted(ms)[len(ms) // 10], 4),
           "ms_p90": round(sorted(ms)[(9 * len(ms)) // 10], 4), "compulsory_mb": round(byt / 1e6, 2),
           "gb_per_s": round(byt / t / 1e6, 1), "frac_hbm_peak": round(byt / t / 1e6 / PEAK_HBM_GBPS, 4),
           "tokens": tokens}
    del q, k, wq, wk, cos, sin, qo, ko
    torch.cuda.empty_cache()
    return res


def gated_delta_case(vfa, torch, lengths, reps=5, warmup=1):
    """gated_delta_rule_fwd on the long-prefill lengths with 16 query/key and 32 value heads, D 128.
    Algorithmic FLOPs per (token, value head): 7 * Dk * Dv (S^T k, decay, rank-1 write, S^T q); compulsory
    bytes: q, k (bf16, shared by 2 value heads), v and out (bf16), g and beta (fp32). Neither HBM nor the
    matrix unit sets the time: the tokens of a sequence are sequential, and the chunked form runs the
    longest sequence as a chain of dependent 64-token chunks on one CU, so the time per chain chunk is
    reported beside the rates."""
    import numpy as np
    from varlen_flash_attention_amd.workloads import bf16_bits, make_gated_delta

    p = make_gated_delta(lengths, 16, 32, 128, 128, seed=93)

    def dev(x):
        return torch.from_numpy(bf16_bits(x).view(np.int16)).cuda().view(torch.bfloat16)

    q, k, v = dev(p.q), dev(p.k), dev(p.v)
    g, beta = torch.from_numpy(p.g).cuda(), torch.from_numpy(p.beta).cuda()
    cu = torch.from_numpy(p.cu_seqlens).cuda()
    out = torch.empty((int(p.lengths.sum()), 32, 128), dtype=torch.bfloat16, device="cuda")

    def call():
        vfa.gated_delta_rule_fwd(q, k, v, g, beta, cu, int(p.lengths.max()), scale=p.scale, out=out)

    ms = time_calls(call, reps, warmup, torch)
    t = median(ms)
    tokens = int(p.lengths.sum())
    flops = 7.0 * 128 * 128 * 32 * tokens
    byt = tokens * (2 * 16 * 128 * 2 + 2 * 32 * 128 * 2 + 2 * 32 * 4)
    chain = -(-int(p.lengths.max()) // 64)
    res = {"ms_median": round(t, 4), "ms_p10": round(sorted(ms)[len(ms) // 10], 4),
           "ms_p90": round(sorted(ms)[(9 * len(ms)) // 10], 4), "gflop": round(flops / 1e9, 2),
           "tflops": round(flops / t / 1e9, 2), "compulsory_mb": round(byt / 1e6, 1),
           "frac_hbm_peak": round(byt / t / 1e6 / PEAK_HBM_GBPS, 4), "bound": "chain of the longest sequence's chunks",
           "chain_chunks": chain, "us_per_chain_chunk": round(t * 1e3 / chain, 3),
           "tokens": tokens, "longest_sequence": int(p.lengths.max())}
    del q, k, v, g, beta, cu, out
    torch.cuda.empty_cache()
    return res


def gated_delta_decode_case(vfa, torch, reps=50, warmup=5):
    """One decode step of the gated delta rule: 64 sequences of one token, 16 q/k and 32 v heads, D 128,
    from given fp32 states to new ones (the token-by-token path). Algorithmic bytes: the states read and
    written, 2 * 64 * 32 * 128 * 128 * 4 = 268 MB (q, k, v, g, beta and the output add 0.6 MB)."""
    import numpy as np
    from varlen_flash_attention_amd.workloads import bf16_bits, make_gated_delta

    b, hqk, hv, d = 64, 16, 32, 128
    p = make_gated_delta([1] * b, hqk, hv, d, d, seed=94)

    def dev(x):
        return torch.from_numpy(bf16_bits(x).view(np.int16)).cuda().view(torch.bfloat16)

    q, k, v = dev(p.q), dev(p.k), dev(p.v)
    g, beta = torch.from_numpy(p.g).cuda(), torch.from_numpy(p.beta).cuda()
    cu = torch.from_numpy(p.cu_seqlens).cuda()
    s0 = torch.from_numpy(np.random.default_rng(95).standard_normal((b, hv, d, d)).astype(np.float32)).cuda()
    out = torch.empty((b, hv, d), dtype=torch.bfloat16, device="cuda")

    def call():
        vfa.gated_delta_rule_fwd(q, k, v, g, beta, cu, 1, scale=p.scale, initial_state=s0,
                                 output_final_state=True, out=out)

    ms = time_calls(call, reps, warmup, torch)
    t = median(ms)
    nbytes = 2 * b * hv * d * d * 4
    # Floor: a device-to-device copy of one state array moves the same bytes (read once, written once).
    dst = torch.empty_like(s0)
    tc = median(time_calls(lambda: dst.copy_(s0), reps, warmup, torch))
    res = {"ms_median": round(t, 4), "state_gb": round(nbytes / 1e9, 3), "tb_per_s": round(nbytes / t / 1e9, 3),
           "frac_hbm": round(nbytes / t / 1e6 / PEAK_HBM_GBPS, 4), "copy_floor_ms": round(tc, 4),
           "frac_of_copy_rate": round(tc / t, 4)}
    del q, k, v, g, beta, cu, s0, out, dst
    torch.cuda.empty_cache()
    return res


def merge_case(vfa, torch, reps=100, warmup=5):
    """attn_update on the chunked-context merge shape (sp 8, bsh 2048, hd 128) with seeded random fp32
    partials: lse ~ N(8, 2) and go ~ N(0, 1). The kernel reads every partial the same way whatever its
    values, so these stand in for the decode workload's chunk partials, which the parity tests use."""
    import numpy as np
    sp, bsh, hd = 8, 64 * 32, 128
    rng = np.random.default_rng(5)
    lse = torch.from_numpy(rng.normal(8.0, 2.0, (sp, bsh)).astype(np.float32)).cuda()
    go = torch.from_numpy(rng.standard_normal((sp, bsh, hd)).astype(np.float32)).cuda()
    out = torch.empty((bsh, hd), dtype=torch.float32, device="cuda")
    lse_out = torch.empty((bsh,), dtype=torch.float32, device="cuda")
    algo_bytes = sp * bsh * (hd + 1) * 4 + bsh * (hd + 1) * 4            # 9,510,912 B
    scratch = torch.ones(1 << 28, dtype=torch.float32, device="cuda")

    def flush():
        # Read 1 GiB of other data: evicts the inputs from L2 and the last-level
        # cache and leaves it clean. (A 1 GiB write would leave it full of dirty
        # lines, so the timed reads would first pay for their write-back.)
        scratch.sum()

    def call():
        vfa.attn_update(lse, go, 1, out=out, lse_out=lse_out)

    cold = time_calls(call, reps, warmup, torch, flush=flush)
    warm = time_calls(call, reps, warmup, torch, queue_ahead=True)
    # Floor for moving this many bytes at all: a device-to-device copy of half
    # of them (read + write = algo_bytes), cold, timed the same way.
    csrc = torch.empty(algo_bytes // 2, dtype=torch.uint8, device="cuda").fill_(7)
    cdst = torch.empty_like(csrc)
    copy_cold = time_calls(lambda: cdst.copy_(csrc), reps, warmup, torch, flush=flush)
    # Dispatch floors, cold like the merge: a one-element fill (a kernel that
    # moves nothing) and a read-only sum over the merge's 8.4 MB of partials.
    tiny = torch.empty(1, dtype=torch.float32, device="cuda")
    fill_cold = time_calls(lambda: tiny.fill_(1.0), reps, warmup, torch, flush=flush)
    read_cold = time_calls(lambda: go.sum(), reps, warmup, torch, flush=flush)
    res = {}
    for name, ms in (("cold", cold), ("warm", warm), ("copy_floor_cold", copy_cold),
                     ("one_element_fill_cold", fill_cold), ("read_only_sum_cold", read_cold)):
        t = median(ms)
        res[name] = {"us_median": round(t * 1e3, 3), "gb_per_s": round(algo_bytes / t / 1e6, 1),
                     "frac_hbm_peak": round(algo_bytes / t / 1e6 / PEAK_HBM_GBPS, 4)}
    res["algorithmic_bytes"] = algo_bytes
    res["shape"] = {"sp": sp, "bsh": bsh, "hd": hd, "dtype": "fp32"}
    del csrc, cdst, go, out, lse, lse_out, tiny
    torch.cuda.empty_cache()

    # The same kernel on 4x .. 64x the rows, cold: the bandwidth asymptote
    # once launch and first-byte latency amortise (64x is 608 MB, beyond the
    # last-level cache).
    sweep = {}
    for mult in (4, 16, 64):
        big = mult * bsh
        lse = torch.randn((sp, big), dtype=torch.float32, device="cuda")
        go = torch.randn((sp, big, hd), dtype=torch.float32, device="cuda")
        out = torch.empty((big, hd), dtype=torch.float32, device="cuda")
        lse_out = torch.empty((big,), dtype=torch.float32, device="cuda")
        big_bytes = sp * big * (hd + 1) * 4 + big * (hd + 1) * 4
        ms = time_calls(lambda: vfa.attn_update(lse, go, 1, out=out, lse_out=lse_out), 20, 3, torch, flush=flush)
        t = median(ms)
        sweep[f"rows_x{mult}"] = {"bsh": big, "algorithmic_bytes": big_bytes, "us_median": round(t * 1e3, 3),
                                  "gb_per_s": round(big_bytes / t / 1e6, 1),
                                  "frac_hbm_peak": round(big_bytes / t / 1e6 / PEAK_HBM_GBPS, 4)}
        del lse, go, out, lse_out
        torch.cuda.empty_cache()
    res["size_sweep_cold"] = sweep
    del scratch
    torch.cuda.empty_cache()
    return res


def cpu_baseline(w, budget_s=12.0):
    """The fp64 oracle on a bounded, seeded sample of query tokens of the same workload."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    rng = np.random.default_rng(123)
    order = rng.permutation(w.total_q)
    cu = w.cu_seqlens_q.astype(np.int64)
    seq_of = np.searchsorted(cu, order, side="right") - 1
    done, flops, t0 = 0, 0.0, time.perf_counter()
    while done < len(order) and time.perf_counter() - t0 < budget_s:
        toks = np.sort(order[done:done + 64])
        oracle.varlen_attention_rows(w.q, w.k, w.v, w.cu_seqlens_q, w.cu_seqlens_k, w.num_heads_kv, w.scale,
                                     w.causal, tokens=toks)
        for t, b in zip(order[done:done + 64], seq_of[done:done + 64]):
            i = int(t - cu[b])
            lq, lk = int(w.lengths_q[b]), int(w.lengths_k[b])
            vis = min(lk, max(0, i + 1 + lk - lq)) if w.causal else lk
            flops += 4.0 * w.head_dim * w.num_heads_q * vis
        done += len(toks)
    el = time.perf_counter() - t0
    return {"value": round(flops / el / 1e12, 6), "unit": "useful TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} of {w.total_q} query tokens (all {w.num_heads_q} heads), seeded random order, "
                      f"{el:.1f} s of fp64 numpy on {threads} BLAS threads; host has "
                      f"{len(os.sched_getaffinity(0))} usable cores"}


def cpu_baselines():
    """The fp64 oracle on the other configs: full inputs of the tiny fp32 config, the embedding prefill
    with its gather and the chunked-context merge, and two of the decode config's 64 sequences (the
    long-prefill oracle is the sampled `cpu_baseline`). Each is timed once with time.perf_counter on the host's BLAS threads and
    reported on the same useful-FLOP (or algorithmic-byte) count as the GPU."""
    import numpy as np
    import oracle
    from varlen_flash_attention_amd.workloads import make_workload
    try:
        from threadpoolctl import threadpool_info
        threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    res = {"cores": len(os.sched_getaffinity(0)), "blas_threads": threads, "kind": "oracle"}
    for name in ("tiny_fp32", "embed_prefill"):
        w = make_workload(name)
        t0 = time.perf_counter()
        o, _ = oracle.varlen_attention(w.q, w.k, w.v, w.cu_seqlens_q, w.cu_seqlens_k, w.num_heads_kv, w.scale,
                                       w.causal)
        if name == "embed_prefill":
            oracle.last_token_gather(o, w.cu_seqlens_q)
        el = time.perf_counter() - t0
        res[name] = {"s": round(el, 3), "useful_gflop": round(w.useful_flops() / 1e9, 3),
                     "useful_tflops": round(w.useful_flops() / el / 1e12, 6), "sample": "full inputs"}
    # Decode: the oracle walks each (sequence, head) over strided K/V rows, minutes for all 64 sequences,
    # so it runs on the first two sequences of the same workload (same values) and reports that rate.
    w = make_workload("decode")
    ck = w.cu_seqlens_k.astype(np.int64)
    sub = 2
    cu_q = w.cu_seqlens_q[:sub + 1]
    cu_k = w.cu_seqlens_k[:sub + 1]
    t0 = time.perf_counter()
    oracle.varlen_attention(w.q[:sub], w.k[:ck[sub]], w.v[:ck[sub]], cu_q, cu_k, w.num_heads_kv, w.scale, w.causal)
    el = time.perf_counter() - t0
    fl = 4.0 * w.head_dim * w.num_heads_q * float(ck[sub])
    res["decode"] = {"s": round(el, 3), "useful_gflop": round(fl / 1e9, 3), "useful_tflops": round(fl / el / 1e12, 6),
                     "sample": f"sequences 0-{sub - 1} of {w.batch} ({int(ck[sub])} of {w.total_k} keys)"}
    rng = np.random.default_rng(5)
    sp, bsh, hd = 8, 64 * 32, 128
    lse = rng.normal(8.0, 2.0, (sp, bsh)).astype(np.float32)
    go = rng.standard_normal((sp, bsh, hd)).astype(np.float32)
    t0 = time.perf_counter()
    oracle.attn_update(lse, go, 1)
    el = time.perf_counter() - t0
    nbytes = sp * bsh * (hd + 1) * 4 + bsh * (hd + 1) * 4
    res["merge"] = {"s": round(el, 4), "algorithmic_bytes": nbytes, "gb_per_s": round(nbytes / el / 1e9, 3)}
    return res


def traffic_record():
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it matches the kernel source."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
        with open(KERNEL_SOURCE, "rb") as fh:
            sha = hashlib.sha256(fh.read()).hexdigest()
        if rec.get("kernel_source_sha256") != sha:
            return None
        return int(rec["hbm_bytes_per_launch"])
    except Exception:  # noqa: BLE001
        return None


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the extra workloads")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed region, copy 256 MiB device-to-device with cold caches: a kernel of "
                         "known traffic against which rocprofv3 FETCH_SIZE / WRITE_SIZE readings are scaled")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library's hot path runs on a single device "
              "(sequences and heads would shard across GPUs, each running this path on its share); "
              "run with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    import varlen_flash_attention_amd as vfa
    from varlen_flash_attention_amd.workloads import make_workload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    vfa.load_library()

    w = make_workload("long_prefill")
    log(f"[bench] long_prefill causal: B={w.batch} lengths={w.lengths_q.tolist()} T={w.total_q}")
    d = device_inputs(w, torch)
    out = torch.empty((w.total_q, w.num_heads_q, w.head_dim), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.total_q, w.num_heads_q), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, vfa.varlen_attn_fwd_workspace_size(w.batch, w.total_q, w.max_seqlen_q, w.max_seqlen_k,
                                                                w.num_heads_q, w.num_heads_kv, w.head_dim)),
                     dtype=torch.uint8, device="cuda")

    def step():
        vfa.varlen_attn_fwd(d["q"], d["k"], d["v"], d["cu_q"], d["cu_k"], w.max_seqlen_q, w.max_seqlen_k,
                            softmax_scale=w.scale, causal=True, out=out, lse=lse, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        step()
        e.record(stream)
        evs.append((s, e))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [s.elapsed_time(e) for s, e in evs]
    avg_launch = sum(launch_ms) / len(launch_ms)
    flops = w.useful_flops()
    value = flops * args.steps / wall / 1e12
    achieved = flops / (avg_launch * 1e-3) / 1e12
    log(f"[bench] {args.steps} steps in {wall * 1e3:.1f} ms; avg launch {avg_launch:.3f} ms; "
        f"{achieved:.1f} TFLOP/s useful")
    del d, out, lse, ws
    torch.cuda.empty_cache()

    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.uint8, device="cuda").fill_(7)
        dst = torch.empty_like(src)
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)   # evict src from L2 / MALL
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 268435456 bytes read, 268435456 bytes written")
        del src, dst, scratch
        torch.cuda.empty_cache()

    extra = {}
    if not args.no_extra:
        log("[bench] extra: embed_prefill")
        extra["embed_prefill_with_gather"] = attn_case(vfa, torch, make_workload("embed_prefill"), gather=True,
                                                       cold=True)
        log("[bench] extra: long_prefill non-causal")
        extra["long_prefill_full"] = attn_case(vfa, torch, make_workload("long_prefill_full"))
        log("[bench] extra: decode")
        wd = make_workload("decode")
        extra["decode"] = attn_case(vfa, torch, wd)
        for page in (16, 128):
            log(f"[bench] extra: paged decode, {page}-key pages")
            extra[f"paged_decode_p{page}"] = paged_case(vfa, torch, wd, page)
        del wd
        log("[bench] extra: q/k RMSNorm + rotary prologue")
        extra["qk_norm_rope"] = prologue_case(vfa, torch, w.lengths_q)
        log("[bench] extra: gated delta rule (linear attention)")
        extra["gated_delta_rule"] = gated_delta_case(vfa, torch, w.lengths_q)
        log("[bench] extra: gated delta rule decode step")
        extra["gated_delta_decode_step"] = gated_delta_decode_case(vfa, torch)
        log("[bench] extra: attn_update merge")
        extra["attn_update_merge"] = merge_case(vfa, torch)

    cpu = None
    if not args.no_cpu:
        log("[bench] cpu baseline (oracle)")
        cpu = cpu_baseline(w)
        log("[bench] cpu baselines of the other configs, full inputs")
        extra["cpu_baseline_per_config"] = cpu_baselines()

    result = {
        "metric": "varlen attn useful TFLOP/s (% bf16 MFMA peak)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "long_prefill causal: 16 sequences, log-normal lengths (median 2048, sigma 1, clipped "
                        "to [256, 8192]), TND, Hq=32 Hkv=8 D=128, bf16 in/out, fp32 accumulation, seed 3",
            "total_tokens": w.total_q, "lengths": w.lengths_q.tolist(), "useful_gflop_per_step": round(flops / 1e9, 3),
        },
        "roofline": {
            "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic_record(),
        },
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
