"""GPU parity: varlen_attn_fwd (through the C ABI) against the fp64 CPU oracle.

Every test draws seeded inputs from varlen_flash_attention_amd.workloads,
gives the same values to the GPU and to the oracle, and applies the
tolerance rule in tests/gpu_util.py element by element.
"""
import numpy as np
import pytest

import oracle
import varlen_flash_attention_amd as vfa
from varlen_flash_attention_amd.workloads import make_custom, make_growing_scores, make_workload
from tests.gpu_util import check, host64, need_gpu, tile_tokens, to_device

pytestmark = pytest.mark.gpu


def run_gpu(w, out_dtype=None, max_q=None, max_k=None, causal=None):
    torch = need_gpu()
    d = to_device(w)
    odt = None if out_dtype is None else {"fp32": torch.float32, "bf16": torch.bfloat16}[out_dtype]
    out, lse = vfa.varlen_attn_fwd(d["q"], d["k"], d["v"], d["cu_q"], d["cu_k"],
                                   w.max_seqlen_q if max_q is None else max_q,
                                   w.max_seqlen_k if max_k is None else max_k,
                                   softmax_scale=w.scale, causal=w.causal if causal is None else causal,
                                   out_dtype=odt)
    torch.cuda.synchronize()
    return out, lse


def run_oracle(w, tokens=None):
    return oracle.varlen_attention_rows(w.q, w.k, w.v, w.cu_seqlens_q, w.cu_seqlens_k, w.num_heads_kv,
                                       w.scale, w.causal, tokens=tokens)


def full_check(name, w, **kw):
    print(f"[case] {name}: B={w.batch} Tq={w.total_q} Tk={w.total_k} Hq={w.num_heads_q} "
          f"Hkv={w.num_heads_kv} D={w.head_dim} {w.dtype} causal={w.causal}", flush=True)
    out, lse = run_gpu(w, **kw)
    o_ref, l_ref = run_oracle(w)
    return check(name, host64(out), host64(lse), o_ref, l_ref, w.dtype)


# ------------------------------------------------------------------ configs

def test_tiny_fp32():
    w = make_workload("tiny_fp32")
    full_check("tiny_fp32", w)


def test_embed_prefill_small():
    w = make_custom(np.random.default_rng(20).integers(32, 513, 8), num_heads_q=16, num_heads_kv=8,
                    head_dim=128, dtype="bf16", causal=True, seed=21, name="embed_small")
    full_check("embed_prefill_small", w)


def test_embed_prefill_full_with_gather():
    torch = need_gpu()
    w = make_workload("embed_prefill")
    print(f"[case] embed_prefill full: Tq={w.total_q}", flush=True)
    d = to_device(w)
    out, lse = vfa.varlen_attn_fwd(d["q"], d["k"], d["v"], d["cu_q"], d["cu_k"], w.max_seqlen_q,
                                   w.max_seqlen_k, softmax_scale=w.scale, causal=True)
    last = vfa.varlen_last_token_gather(out, d["cu_q"])
    last_lse = vfa.varlen_last_token_gather(lse, d["cu_q"])
    torch.cuda.synchronize()
    o_ref, l_ref = run_oracle(w)
    check("embed_prefill", host64(out), host64(lse), o_ref, l_ref, "bf16")
    # the gather is a copy: bit-exact against the GPU's own rows, and within tolerance of the oracle's
    idx = w.cu_seqlens_q[1:].astype(np.int64) - 1
    assert torch.equal(last, out[torch.from_numpy(idx).cuda()])
    assert torch.equal(last_lse, lse[torch.from_numpy(idx).cuda()])
    check("embed_prefill_gather", host64(last), host64(last_lse), oracle.last_token_gather(o_ref, w.cu_seqlens_q),
          oracle.last_token_gather(l_ref, w.cu_seqlens_q), "bf16")
    assert tuple(last.shape) == (64, 16, 128)


# The launcher takes 256-column workgroups (eight waves) once sequences average
# at least eight of their query tiles, i.e. mean Lq >= 8 * 256 / G tokens, and
# 128-column workgroups (four waves) below that.
def wide_shape(w):
    return w.total_q // w.batch >= 8 * (256 // (w.num_heads_q // w.num_heads_kv))


@pytest.mark.parametrize("causal", [True, False])
def test_long_prefill_small_four_wave(causal):
    w = make_custom([300, 513, 1029, 77], num_heads_q=32, num_heads_kv=8, head_dim=128, dtype="bf16",
                    causal=causal, seed=31, name="long_small")
    assert not wide_shape(w)
    full_check(f"long_prefill_small (4-wave shape) causal={causal}", w)


@pytest.mark.parametrize("causal", [True, False])
def test_long_prefill_small_eight_wave(causal):
    # The headline shape (Hq 32, Hkv 8, D 128, bf16) with ragged tails, on the eight-wave kernel.
    w = make_custom([1300, 513, 1029, 77, 700, 1500], num_heads_q=32, num_heads_kv=8, head_dim=128, dtype="bf16",
                    causal=causal, seed=32, name="long_small_wide")
    assert wide_shape(w)
    full_check(f"long_prefill_small (8-wave shape) causal={causal}", w)


@pytest.mark.parametrize("name", ["long_prefill", "long_prefill_full"])
def test_long_prefill_full_size_every_tile(name):
    # Full size, in the launch configuration the benchmark times: one token from every 64-token query
    # tile (256 columns / G = 4 heads, one workgroup per tile and kv head) plus each sequence's first
    # and last token, all 32 heads, element by element against the oracle.
    w = make_workload(name)
    assert wide_shape(w)
    print(f"[case] {name} full size: lengths={w.lengths_q.tolist()} Tq={w.total_q}", flush=True)
    out, lse = run_gpu(w)
    toks = tile_tokens(w, 64, seed=3)
    o_ref, l_ref = run_oracle(w, tokens=toks)
    check(f"{name} ({len(toks)} tokens, every query tile)", host64(out)[toks], host64(lse)[toks], o_ref, l_ref,
          "bf16")


@pytest.mark.parametrize("causal", [True, False])
def test_decode_small(causal):
    rng = np.random.default_rng(40)
    lk = rng.integers(1024, 4097, 8)
    w = make_custom(np.ones(8, dtype=np.int64), lk, num_heads_q=32, num_heads_kv=4, head_dim=128,
                    dtype="bf16", causal=causal, seed=41, name="decode_small")
    full_check(f"decode_small causal={causal}", w)


@pytest.mark.parametrize("causal", [True, False])
def test_decode_full_size(causal):
    w = make_workload("decode").with_causal(causal)
    print(f"[case] decode full size causal={causal}: Tk={w.total_k}", flush=True)
    out, lse = run_gpu(w)
    o_ref, l_ref = run_oracle(w)
    check(f"decode causal={causal}", host64(out), host64(lse), o_ref, l_ref, "bf16")


# ------------------------------------------------------------------ edge cases

@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("causal", [True, False])
def test_empty_and_ragged(dtype, causal):
    # empty query sets, empty key sets, Lk < Lq (fully masked causal rows), single tokens, ragged tails
    lq = [0, 5, 1, 0, 37, 3, 70, 1]
    lk = [0, 5, 9, 4, 37, 0, 65, 1]
    w = make_custom(lq, lk, num_heads_q=8, num_heads_kv=2, head_dim=64, dtype=dtype, causal=causal, seed=50)
    full_check(f"empty_and_ragged {dtype} causal={causal}", w)


@pytest.mark.parametrize("hq,hkv,d", [(4, 4, 128), (8, 1, 64), (6, 2, 128), (16, 2, 128), (64, 2, 64),
                                      (12, 4, 64), (32, 8, 64)])
@pytest.mark.parametrize("causal", [True, False])
def test_gqa_shapes(hq, hkv, d, causal):
    w = make_custom([130, 64, 1, 257, 33], num_heads_q=hq, num_heads_kv=hkv, head_dim=d, dtype="bf16",
                    causal=causal, seed=60 + hq + hkv + d)
    full_check(f"gqa Hq={hq} Hkv={hkv} D={d} causal={causal}", w)


@pytest.mark.parametrize("batch,hq,hkv,d,out_dtype,causal", [(257, 8, 2, 64, None, True),
                                                            (257, 8, 2, 64, None, False),
                                                            (1000, 6, 3, 128, "fp32", True)])
def test_many_sequences(batch, hq, hkv, d, out_dtype, causal):
    # hundreds of short sequences: many (sequence, kv head) pairs per XCD, a pair count that is not a
    # multiple of the 8 XCDs, and query tiles past most sequences' ends
    lengths = np.random.default_rng(batch + d).integers(1, 160, batch)
    w = make_custom(lengths, num_heads_q=hq, num_heads_kv=hkv, head_dim=d, dtype="bf16", causal=causal,
                    seed=batch + hq + d)
    assert not wide_shape(w)
    full_check(f"many_sequences B={batch} Hq={hq} Hkv={hkv} D={d} causal={causal}", w, out_dtype=out_dtype)


@pytest.mark.parametrize("lengths,hq,hkv,dtype,causal,wide", [
    ([200, 513, 37, 300], 8, 2, "bf16", True, False),
    ([200, 513, 37, 300], 8, 2, "bf16", False, False),
    ([1300, 513, 1029, 700, 1500], 32, 8, "bf16", True, True),
    ([1300, 513, 1029, 700, 1500], 32, 8, "bf16", False, True),
])
def test_growing_scores_move_the_reference(lengths, hq, hkv, dtype, causal, wide):
    # Scores that climb by about 8 log2 units per 32 keys: the bf16 kernels' running sum against their lazy
    # softmax reference passes 2^32 every few sub-blocks, so the rescale path runs many times per row (both
    # the short-sequence and the long-sequence kernel). The fp32 kernel has no lazy reference (it rescales
    # whenever the max grows) and is not run here: at raw scores near 1000, fp32 rounding of q . k alone
    # moves lse by about two fp32 ulps of its value (~88), past the fp32 tolerance of 1e-5.
    w = make_growing_scores(lengths, num_heads_q=hq, num_heads_kv=hkv, head_dim=128, dtype=dtype, causal=causal,
                            seed=sum(lengths) + hq)
    assert wide_shape(w) == wide
    full_check(f"growing_scores {dtype} Hq={hq} causal={causal} wide={wide}", w)


@pytest.mark.parametrize("lengths,hq,hkv", [([2500, 3000, 900], 4, 4),      # G = 1: 256-token tiles
                                             ([1500, 1200, 700], 4, 2),      # G = 2: 128-token tiles
                                             ([900, 700, 503], 12, 4),       # G = 3: 85 tokens, one column idle
                                             ([700, 400, 333], 12, 2),       # G = 6: 42 tokens, four columns idle
                                             ([600, 333, 290], 16, 2),       # G = 8: 32 tokens, a head per wave
                                             ([300, 150, 77], 32, 2),        # G = 16: 16-token tiles
                                             ([150, 97, 40], 32, 1)])        # G = 32: 8 tokens, four heads per wave
@pytest.mark.parametrize("causal", [True, False])
def test_long_prefill_group_sizes(lengths, hq, hkv, causal):
    w = make_custom(lengths, num_heads_q=hq, num_heads_kv=hkv, head_dim=128, dtype="bf16", causal=causal,
                    seed=128 + hq)
    assert wide_shape(w)
    full_check(f"long_prefill G={hq // hkv} causal={causal}", w)


@pytest.mark.parametrize("causal", [True, False])
def test_long_prefill_head_dim_64(causal):
    # the persistent long-sequence kernel's D = 64 instance, with ragged tails
    w = make_custom([1100, 600, 901, 33], num_heads_q=16, num_heads_kv=4, head_dim=64, dtype="bf16",
                    causal=causal, seed=127)
    assert wide_shape(w)
    full_check(f"long_prefill_d64 causal={causal}", w)


@pytest.mark.parametrize("causal", [True, False])
def test_long_prefill_unequal_and_empty_keys(causal):
    # the persistent long-sequence kernel through the plain entry point with Lk < Lq (bottom-right causal
    # alignment leaves the first Lq - Lk rows without a visible key), Lk > Lq and empty key sets
    lq = [1300, 513, 1029, 77, 700, 1500]
    lk = [900, 513, 0, 300, 1400, 40]
    w = make_custom(lq, lk, num_heads_q=32, num_heads_kv=8, head_dim=128, dtype="bf16", causal=causal, seed=126)
    assert wide_shape(w)
    full_check(f"long_prefill_unequal causal={causal}", w)


def test_unequal_lengths_bottom_right():
    # prefill-shaped with Lq != Lk (chunked prefill against a longer cache, and the reverse)
    w = make_custom([100, 7, 64, 200], [300, 7, 20, 129], num_heads_q=8, num_heads_kv=4, head_dim=128,
                    dtype="bf16", causal=True, seed=70)
    full_check("unequal_lengths causal", w)


@pytest.mark.parametrize("lengths,wide", [([77, 256, 3], False), ([1300, 513, 1029, 70], True)])
def test_bf16_in_fp32_out(lengths, wide):
    w = make_custom(lengths, num_heads_q=8, num_heads_kv=2, head_dim=128, dtype="bf16", causal=True, seed=80)
    assert wide_shape(w) == wide
    print(f"[case] bf16 in, fp32 out, wide={wide}", flush=True)
    out, lse = run_gpu(w, out_dtype="fp32")
    assert str(out.dtype) == "torch.float32"
    o_ref, l_ref = run_oracle(w)
    check(f"bf16_in_fp32_out wide={wide}", host64(out), host64(lse), o_ref, l_ref, "bf16")


@pytest.mark.parametrize("hq,hkv,lq,d,causal", [
    (32, 2, 1, 128, True),    # G = 16
    (32, 4, 1, 64, False),
    (16, 2, 2, 128, True),    # 2 query tokens x 8 heads fill the 16 columns; the causal mask bites
    (8, 8, 1, 128, True),     # G = 1
    (12, 4, 5, 128, True),    # G = 3 with 5 tokens: 15 of 16 columns
    (8, 1, 1, 128, True),     # one kv head: one head per workgroup, four waves split its keys
    (24, 3, 1, 64, False),    # odd kv head count: one head per workgroup
])
def test_decode_variants(hq, hkv, lq, d, causal):
    lk = [1500, 600, 4099, 0, 513, 2048]
    lqs = [min(lq, x) if x > 0 else lq for x in lk]
    w = make_custom(lqs, lk, num_heads_q=hq, num_heads_kv=hkv, head_dim=d, dtype="bf16", causal=causal,
                    seed=90 + hq + lq)
    full_check(f"decode Hq={hq} Hkv={hkv} Lq={lq} D={d} causal={causal}", w)


@pytest.mark.parametrize("lk,hq,hkv", [
    ([12800, 300, 9000], 16, 2),       # 50 splits of 256 keys: the combine's 64-partial register path
    ([70000, 17, 40000], 8, 1),        # 274 splits: the combine's streaming loop
])
def test_decode_many_splits(lk, hq, hkv):
    w = make_custom([1] * len(lk), lk, num_heads_q=hq, num_heads_kv=hkv, head_dim=128, dtype="bf16", causal=True,
                    seed=110 + len(lk) + hkv)
    ws = vfa.varlen_attn_fwd_workspace_size(w.batch, w.total_q, w.max_seqlen_q, w.max_seqlen_k, hq, hkv, 128)
    print(f"[case] decode many splits lk={lk} workspace={ws}", flush=True)
    full_check(f"decode_many_splits lk={lk}", w)


@pytest.mark.parametrize("lengths,wide", [([40, 129, 7], False), ([1300, 513, 1029, 70], True)])
def test_loose_max_seqlen_bounds(lengths, wide):
    # bounds far above the real lengths only add empty query tiles (the persistent kernel's ticket slots
    # past a sequence's end are skipped): the results are bit-identical
    w = make_custom(lengths, num_heads_q=8, num_heads_kv=2, head_dim=128, dtype="bf16", causal=True, seed=100)
    assert wide_shape(w) == wide
    print(f"[case] loose max_seqlen bounds, wide={wide}", flush=True)
    out_a, lse_a = run_gpu(w)
    out_b, lse_b = run_gpu(w, max_q=w.total_q, max_k=w.total_k)
    assert (out_a.float() - out_b.float()).abs().max().item() == 0
    assert (lse_a - lse_b).abs().max().item() == 0


@pytest.mark.parametrize("lengths,wide", [([300, 5, 130, 64], False), ([1300, 600, 900], True)])
def test_deterministic_and_packing_invariant(lengths, wide):
    # Repeated calls are bit-identical (the persistent kernel hands its tiles to whichever workgroup draws
    # them first, so its tiles land on different workgroups from call to call), and a sequence computed
    # alone equals its rows in the packed call. In the long-sequence case every sequence is long enough
    # to take the same kernel alone.
    torch = need_gpu()
    w = make_custom(lengths, num_heads_q=16, num_heads_kv=4, head_dim=128, dtype="bf16", causal=True, seed=110)
    assert wide_shape(w) == wide
    print(f"[case] determinism + packed == per-sequence, wide={wide}", flush=True)
    o1, l1 = run_gpu(w)
    for _ in range(2):
        o2, l2 = run_gpu(w)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), "two identical calls differ"
    cq = w.cu_seqlens_q
    for b in range(w.batch):
        sub = make_custom([w.lengths_q[b]], num_heads_q=16, num_heads_kv=4, head_dim=128, dtype="bf16",
                          causal=True, seed=0)
        sub.q = w.q[cq[b]:cq[b + 1]]
        sub.k = w.k[cq[b]:cq[b + 1]]
        sub.v = w.v[cq[b]:cq[b + 1]]
        if wide:
            assert wide_shape(sub)
        ob, lb = run_gpu(sub)
        assert torch.equal(ob, o1[cq[b]:cq[b + 1]]), f"sequence {b}: packed and alone differ"
        assert torch.equal(lb, l1[cq[b]:cq[b + 1]])
