"""GPU parity on seeded random shapes: varlen_attn_fwd against the fp64 oracle, every row.

Each case draws its own batch, ragged lengths (empty, single-token, short, medium and long
sequences), unequal query and key counts, head counts (Hkv 1-8, G 1-16 including group sizes that
do not divide the 256-column tile), head dim 64 or 128, causal or full masking, bf16 or fp32 inputs
and bf16 or fp32 output. The case mix reaches all three routes of the entry point (the short-sequence
kernel, the persistent long-prefill kernel and split-KV decode); test_route_mix checks that it does.
Lengths are capped so that the oracle of one case stays near a few GFLOP.
"""
import numpy as np
import pytest

import oracle
import varlen_flash_attention_amd as vfa
from varlen_flash_attention_amd.workloads import make_custom
from tests.gpu_util import check, host64, need_gpu, to_device

N_CASES = 48
ORACLE_FLOP_CAP = 3e9


def _oracle_flops(lq, lk, hq, d):
    return float(np.sum(lq.astype(np.float64) * lk)) * hq * d * 4


def draw_case(i):
    """Shape parameters of case i (seeded by i alone)."""
    rng = np.random.default_rng(9100 + i)
    kind = ("short", "short", "long", "decode")[i % 4]
    d = int(rng.choice([64, 128]))
    causal = bool(rng.integers(2))
    if kind == "long":
        hkv = int(rng.choice([1, 2]))
        g = int(rng.choice([1, 2, 3, 4, 6, 8, 16]))
    else:
        hkv = int(rng.choice([1, 2, 4, 8]))
        g = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
    hq = hkv * g
    dtype = "fp32" if kind == "short" and rng.random() < 0.25 else "bf16"
    out_dtype = "fp32" if dtype == "bf16" and rng.random() < 0.2 else None
    if kind == "decode":
        b = int(rng.integers(1, 9))
        lq = rng.integers(1, 5, b)
        lk = rng.integers(300, 9000, b)
        lk[rng.random(b) < 0.1] = 0
    elif kind == "long":
        need = 8 * (256 // g)                          # mean query tokens per sequence for the long kernel
        b = int(rng.integers(1, 5))
        lq = rng.integers(need, 2 * need, b)
        if b > 1 and rng.random() < 0.5:
            lq[rng.integers(b)] = int(rng.integers(0, 40))   # a short or empty sequence among long ones
        lk = lq.copy()
        if rng.random() < 0.3:
            lk = np.maximum(0, lq + rng.integers(-need // 2, need // 2, b))
    else:
        b = int(rng.integers(1, 13))
        pick = rng.random(b)
        lq = np.where(pick < 0.08, 0, np.where(pick < 0.16, 1, np.where(pick < 0.6, rng.integers(2, 65, b),
                                                                          rng.integers(65, 700, b))))
        lk = lq.copy()
        if rng.random() < 0.4:
            lk = np.maximum(0, lq + rng.integers(-30, 200, b))
    lq = np.asarray(lq, dtype=np.int64)
    lk = np.asarray(lk, dtype=np.int64)
    while _oracle_flops(lq, lk, hq, d) > ORACLE_FLOP_CAP and hq > hkv:
        g = max(1, g // 2)
        hq = hkv * g
    if kind == "long":   # keep the long-kernel mean after any change of G
        need = 8 * (256 // g)
        if lq.sum() // len(lq) < need:
            lq = lq + (need - lq.sum() // len(lq))
            lk = np.where(lk > 0, lk + (lq - lk).clip(min=0), lk)
    while _oracle_flops(lq, lk, hq, d) > ORACLE_FLOP_CAP:
        lq, lk = (lq * 3) // 4, (lk * 3) // 4
    return dict(lq=lq, lk=lk, hq=hq, hkv=hkv, d=d, causal=causal, dtype=dtype, out_dtype=out_dtype, seed=9200 + i)


def route(p):
    b, tq = len(p["lq"]), int(p["lq"].sum())
    wide = tq // b >= 8 * (256 // (p["hq"] // p["hkv"]))
    if wide and (int(p["lk"].max()) + 256) * p["hkv"] * p["d"] * 2 < 2 ** 32:
        return "long"
    ws = vfa.varlen_attn_fwd_workspace_size(b, tq, int(p["lq"].max()), int(p["lk"].max()), p["hq"], p["hkv"], p["d"])
    return "decode" if ws > 0 else "short"


def test_route_mix():
    routes = [route(draw_case(i)) for i in range(N_CASES)]
    assert {"short", "long", "decode"} <= set(routes), routes


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(i):
    torch = need_gpu()
    p = draw_case(i)
    name = (f"random case {i}: seed={p['seed']} route={route(p)} B={len(p['lq'])} Lq={p['lq'].tolist()} "
            f"Lk={p['lk'].tolist()} Hq={p['hq']} Hkv={p['hkv']} D={p['d']} {p['dtype']} "
            f"out={p['out_dtype'] or p['dtype']} causal={p['causal']}")
    print(f"[case] {name}", flush=True)
    w = make_custom(p["lq"], p["lk"], num_heads_q=p["hq"], num_heads_kv=p["hkv"], head_dim=p["d"], dtype=p["dtype"],
                    causal=p["causal"], seed=p["seed"], name=f"random{i}")
    dv = to_device(w)
    odt = None if p["out_dtype"] is None else torch.float32
    out, lse = vfa.varlen_attn_fwd(dv["q"], dv["k"], dv["v"], dv["cu_q"], dv["cu_k"], w.max_seqlen_q, w.max_seqlen_k,
                                   softmax_scale=w.scale, causal=w.causal, out_dtype=odt)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.varlen_attention(w.q, w.k, w.v, w.cu_seqlens_q, w.cu_seqlens_k, w.num_heads_kv, w.scale,
                                           w.causal)
    check(name, host64(out), host64(lse), o_ref, l_ref, w.dtype)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(0, N_CASES, 2))
def test_random_shape_causal_offset(i):
    # the same shapes through the explicit-alignment entry point, causal, with per-sequence offsets of every
    # kind (bottom-right, top-left, chunk-style negative, past every key, below every row, random)
    from tests.test_gpu_causal_offset import offsets_for
    torch = need_gpu()
    p = draw_case(i)
    offs = offsets_for(p["lq"].tolist(), p["lk"].tolist(), np.random.default_rng(p["seed"] + 5))
    name = (f"random offset case {i}: seed={p['seed']} route={route(p)} Lq={p['lq'].tolist()} Lk={p['lk'].tolist()} "
            f"offsets={offs} Hq={p['hq']} Hkv={p['hkv']} D={p['d']} {p['dtype']}")
    print(f"[case] {name}", flush=True)
    w = make_custom(p["lq"], p["lk"], num_heads_q=p["hq"], num_heads_kv=p["hkv"], head_dim=p["d"], dtype=p["dtype"],
                    causal=True, seed=p["seed"], name=f"random_offset{i}")
    dv = to_device(w)
    off = torch.tensor(np.asarray(offs, dtype=np.int32), device="cuda")
    out, lse = vfa.varlen_attn_fwd(dv["q"], dv["k"], dv["v"], dv["cu_q"], dv["cu_k"], w.max_seqlen_q, w.max_seqlen_k,
                                   softmax_scale=w.scale, causal=True, causal_offset=off)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.varlen_attention(w.q, w.k, w.v, w.cu_seqlens_q, w.cu_seqlens_k, w.num_heads_kv, w.scale,
                                           True, causal_offset=offs)
    check(name, host64(out), host64(lse), o_ref, l_ref, w.dtype)
