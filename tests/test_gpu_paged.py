"""GPU parity: paged_attn_decode (through the C ABI) against the fp64 CPU oracle.

K/V are written into a paged cache by varlen_flash_attention_amd.workloads.make_paged
(shuffled physical pages, spare pages and unused slots holding other values);
the GPU reads them through the block table and the oracle gathers them with
its own paged_gather. Tolerances are those of tests/gpu_util.py.
"""
import os

import numpy as np
import pytest

import oracle
import varlen_flash_attention_amd as vfa
from varlen_flash_attention_amd.workloads import make_custom, make_paged, make_workload
from tests.gpu_util import check, dev_array, host64, need_gpu, sample_tokens

pytestmark = pytest.mark.gpu


def dev_paged(w, pc):
    torch = need_gpu()
    return dict(q=dev_array(w.q, w.dtype), kc=dev_array(pc.k_cache, w.dtype), vc=dev_array(pc.v_cache, w.dtype),
                table=torch.from_numpy(pc.block_table).cuda(), used=torch.from_numpy(pc.seqused_k).cuda(),
                cu_q=torch.from_numpy(w.cu_seqlens_q).cuda())


def run_paged(w, pc, d=None, out_dtype=None, workspace=None, max_q=None, max_k=None):
    torch = need_gpu()
    d = dev_paged(w, pc) if d is None else d
    odt = None if out_dtype is None else {"fp32": torch.float32, "bf16": torch.bfloat16}[out_dtype]
    out, lse = vfa.paged_attn_decode(d["q"], d["kc"], d["vc"], d["table"], d["cu_q"], d["used"],
                                     w.max_seqlen_q if max_q is None else max_q,
                                     w.max_seqlen_k if max_k is None else max_k,
                                     softmax_scale=w.scale, causal=w.causal, out_dtype=odt, workspace=workspace)
    torch.cuda.synchronize()
    return out, lse


def run_oracle(w, pc, tokens=None):
    return oracle.paged_attention_rows(w.q, pc.k_cache, pc.v_cache, pc.block_table, pc.seqused_k,
                                       w.cu_seqlens_q, w.num_heads_kv, w.scale, w.causal, tokens=tokens)


def describe(name, w, pc):
    print(f"[case] {name}: B={w.batch} lq={w.lengths_q.tolist()[:8]} lk={w.lengths_k.tolist()[:8]} "
          f"Hq={w.num_heads_q} Hkv={w.num_heads_kv} D={w.head_dim} page={pc.page_size} pages={pc.num_pages} "
          f"causal={w.causal} ws={vfa.paged_attn_decode_workspace_size(w.batch, w.total_q, w.max_seqlen_q, w.max_seqlen_k, w.num_heads_q, w.num_heads_kv, w.head_dim)}",
          flush=True)


CASES = {
    # name: (page, lengths_q, lengths_k, Hq, Hkv, D, causal)
    "p16_decode_many_splits": (16, [1] * 6, [1, 15, 16, 17, 300, 5000], 32, 4, 128, True),
    "p32_mha_full": (32, [1] * 5, [33, 64, 1000, 2049, 4097], 8, 8, 64, False),
    "p64_two_groups": (64, [2, 3, 1], [100, 2000, 1], 16, 2, 128, True),
    "p128_g32_six_groups": (128, [3, 4], [3, 4500], 32, 1, 64, True),
    "p256_g3_rows_without_keys": (256, [7, 1], [5, 3000], 6, 2, 128, True),
    "p4096_page_above_split": (4096, [1, 1], [4096, 4095], 32, 4, 128, False),
    "p16_empty_sequences": (16, [1, 1, 1, 2], [0, 20, 0, 0], 32, 4, 128, True),
    "p16_spec_tokens_full": (16, [4, 4, 4], [700, 1, 2600], 16, 4, 128, False),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_paged_parity(name):
    need_gpu()
    page, lq, lk, hq, hkv, d, causal = CASES[name]
    w = make_custom(lq, lk, num_heads_q=hq, num_heads_kv=hkv, head_dim=d, dtype="bf16", causal=causal,
                    seed=sum(lk) % 997)
    pc = make_paged(w, page, seed=5)
    describe(name, w, pc)
    out, lse = run_paged(w, pc)
    o_ref, l_ref = run_oracle(w, pc)
    check(name, host64(out), host64(lse), o_ref, l_ref, "bf16")


def test_paged_fp32_out():
    need_gpu()
    w = make_custom([1, 2, 1], [1500, 77, 6000], num_heads_q=32, num_heads_kv=4, head_dim=128, dtype="bf16",
                    causal=True, seed=31)
    pc = make_paged(w, 32, seed=6)
    describe("paged_fp32_out", w, pc)
    out, lse = run_paged(w, pc, out_dtype="fp32")
    o_ref, l_ref = run_oracle(w, pc)
    check("paged_fp32_out", host64(out), host64(lse), o_ref, l_ref, "bf16")


@pytest.mark.parametrize("page", [16])
def test_paged_decode_full_size(page):
    """The decode workload (64 sequences, 1 query, 1024-32768 keys, 32/4 heads, D 128) in a paged cache."""
    need_gpu()
    w = make_workload("decode")
    pc = make_paged(w, page, seed=7)
    describe(f"paged_decode_full_p{page}", w, pc)
    out, lse = run_paged(w, pc)
    o_ref, l_ref = run_oracle(w, pc)
    check(f"paged_decode_full_p{page}", host64(out), host64(lse), o_ref, l_ref, "bf16")


def test_paged_workspace_reuse():
    """One workspace, filled with junk first, serves a larger then a smaller call; each matches a
    call with a fresh workspace bit for bit."""
    torch = need_gpu()
    big = make_custom([1] * 8, [9000, 1, 4097, 300, 8192, 33, 5000, 12000], num_heads_q=32, num_heads_kv=4,
                      head_dim=128, dtype="bf16", causal=True, seed=41)
    small = make_custom([2, 1, 1], [3000, 5000, 2], num_heads_q=16, num_heads_kv=2, head_dim=64, dtype="bf16",
                        causal=True, seed=42)
    sizes = [vfa.paged_attn_decode_workspace_size(w.batch, w.total_q, w.max_seqlen_q, w.max_seqlen_k,
                                                  w.num_heads_q, w.num_heads_kv, w.head_dim) for w in (big, small)]
    assert sizes[0] > 0 and sizes[1] > 0
    ws = torch.full((max(sizes),), 0x5A, dtype=torch.uint8, device="cuda")
    for name, w, seed in (("reuse_big", big, 8), ("reuse_small", small, 9)):
        pc = make_paged(w, 16, seed=seed)
        describe(name, w, pc)
        d = dev_paged(w, pc)
        o_shared, l_shared = run_paged(w, pc, d=d, workspace=ws)
        o_fresh, l_fresh = run_paged(w, pc, d=d)
        assert torch.equal(o_shared, o_fresh) and torch.equal(l_shared, l_fresh), name
        o_ref, l_ref = run_oracle(w, pc)
        check(name, host64(o_shared), host64(l_shared), o_ref, l_ref, "bf16")


def test_paged_deterministic():
    torch = need_gpu()
    w = make_custom([1] * 4, [20000, 3, 9000, 4100], num_heads_q=32, num_heads_kv=4, head_dim=128, dtype="bf16",
                    causal=True, seed=43)
    pc = make_paged(w, 64, seed=10)
    describe("paged_deterministic", w, pc)
    d = dev_paged(w, pc)
    a = run_paged(w, pc, d=d)
    b = run_paged(w, pc, d=d)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    # 79 splits of 256 keys: the combine's streaming loop, against the oracle too
    o_ref, l_ref = run_oracle(w, pc)
    check("paged_deterministic", host64(a[0]), host64(a[1]), o_ref, l_ref, "bf16")


def test_paged_debug_check(monkeypatch):
    """VFA_DEBUG: a block-table entry outside the cache or a key count above the bound is reported
    before anything else is launched; a valid call gives the normal result."""
    torch = need_gpu()
    w = make_custom([1, 1], [100, 40], num_heads_q=8, num_heads_kv=2, head_dim=64, dtype="bf16", causal=True,
                    seed=44)
    pc = make_paged(w, 16, seed=11)
    describe("paged_debug_check", w, pc)
    d = dev_paged(w, pc)
    ref = run_paged(w, pc, d=d)
    monkeypatch.setenv("VFA_DEBUG", "1")
    got = run_paged(w, pc, d=d)
    assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1])
    bad_table = d["table"].clone()
    bad_table[1, 2] = pc.num_pages              # third page of sequence 1 (keys 32..39): out of the cache
    with pytest.raises(vfa.VfaError) as e:
        run_paged(w, pc, d={**d, "table": bad_table})
    assert e.value.status == 2
    bad_used = d["used"].clone()
    bad_used[0] = 101                           # above max_seqlen_k = 100
    with pytest.raises(vfa.VfaError) as e:
        run_paged(w, pc, d={**d, "used": bad_used})
    assert e.value.status == 2
    monkeypatch.delenv("VFA_DEBUG")


def draw_paged_case(i):
    """Seeded random paged-decode shape: batch 1-8, 1-7 query tokens per sequence, 0-6000 keys, pages of
    16-256 keys (powers of two), Hkv 1-8 with G 1-8, D 64 or 128, either mask, bf16 or fp32 output."""
    rng = np.random.default_rng(6100 + i)
    b = int(rng.integers(1, 9))
    lq = rng.integers(1, 8, b) if rng.random() < 0.3 else np.ones(b, dtype=np.int64)
    lk = rng.integers(0, 6001, b)
    lk[rng.random(b) < 0.15] = 0
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 3, 4, 8]))
    return dict(page=int(rng.choice([16, 32, 64, 128, 256])), lq=[int(x) for x in lq], lk=[int(x) for x in lk],
                hq=hkv * g, hkv=hkv, d=int(rng.choice([64, 128])), causal=bool(rng.integers(2)),
                out_dtype="fp32" if rng.random() < 0.25 else None, seed=6200 + i)


@pytest.mark.parametrize("i", range(16))
def test_paged_random_shape(i):
    need_gpu()
    c = draw_paged_case(i)
    w = make_custom(c["lq"], c["lk"], num_heads_q=c["hq"], num_heads_kv=c["hkv"], head_dim=c["d"], dtype="bf16",
                    causal=c["causal"], seed=c["seed"])
    pc = make_paged(w, c["page"], seed=c["seed"] + 1)
    describe(f"paged random case {i} (seed {c['seed']}, out {c['out_dtype'] or 'bf16'})", w, pc)
    out, lse = run_paged(w, pc, out_dtype=c["out_dtype"])
    o_ref, l_ref = run_oracle(w, pc)
    check(f"paged random case {i}", host64(out), host64(lse), o_ref, l_ref, "bf16")
