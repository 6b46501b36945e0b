"""GPU parity: varlen_attn_fwd_offset (explicit causal alignment per sequence) against the oracle,
and the context-parallel use it exists for: each key chunk's partial from one call with offset -a,
merged by attn_update, against unchunked attention.

The offset of sequence b is the position of its first query minus that of its first key; query i
sees key j iff j <= i + offset[b]. Tolerances are those of tests/gpu_util.py.
"""
import numpy as np
import pytest

import oracle
import varlen_flash_attention_amd as vfa
from varlen_flash_attention_amd.workloads import chunk_bounds, make_custom
from tests.gpu_util import check, dev_array, host64, need_gpu, to_device

pytestmark = pytest.mark.gpu


def run_offset(w, offsets, out_dtype=None, max_q=None, max_k=None):
    torch = need_gpu()
    d = to_device(w)
    off = torch.tensor(np.asarray(offsets, dtype=np.int32), device="cuda")
    odt = None if out_dtype is None else {"fp32": torch.float32, "bf16": torch.bfloat16}[out_dtype]
    out, lse = vfa.varlen_attn_fwd(d["q"], d["k"], d["v"], d["cu_q"], d["cu_k"],
                                   w.max_seqlen_q if max_q is None else max_q,
                                   w.max_seqlen_k if max_k is None else max_k,
                                   softmax_scale=w.scale, causal=True, out_dtype=odt, causal_offset=off)
    torch.cuda.synchronize()
    return out, lse


def offsets_for(lq, lk, rng):
    """Per sequence: bottom-right, top-left, a chunk-style negative offset, beyond every key, below every row."""
    kinds = []
    for a, b in zip(lq, lk):
        kinds.append(int(rng.choice([b - a, 0, -int(rng.integers(0, b + 1)), b + 7, -a - 9,
                                     int(rng.integers(-a, b + 1))])))
    return kinds


CASES = {
    # name: (lengths_q, lengths_k, Hq, Hkv, D, dtype)
    # mean 853 query rows >= 8 tiles of 64 tokens: the 8-wave (256-column) prefill shape
    "prefill_wide": ([1300, 513, 1029, 77, 700, 1500], [1300, 900, 1029, 300, 700, 1], 32, 8, 128, "bf16"),
    # mean 97 rows: the 4-wave (128-column) shape
    "prefill_narrow": ([40, 130, 1, 64, 250], [40, 60, 500, 64, 250], 16, 8, 64, "bf16"),
    "tiny_fp32": ([17, 64, 5, 128], [17, 80, 5, 100], 4, 2, 64, "fp32"),
    "decode_split": ([1, 2, 1, 1], [5000, 9000, 700, 12000], 32, 4, 128, "bf16"),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_causal_offset_parity(name):
    need_gpu()
    lq, lk, hq, hkv, d, dtype = CASES[name]
    w = make_custom(lq, lk, num_heads_q=hq, num_heads_kv=hkv, head_dim=d, dtype=dtype, causal=True,
                    seed=len(name) * 7)
    offs = offsets_for(lq, lk, np.random.default_rng(len(name)))
    print(f"[case] causal_offset {name}: lq={lq} lk={lk} offsets={offs} {dtype}", flush=True)
    out, lse = run_offset(w, offs)
    o_ref, l_ref = oracle.varlen_attention(w.q, w.k, w.v, w.cu_seqlens_q, w.cu_seqlens_k, hkv, w.scale, True,
                                           causal_offset=offs)
    check(f"causal_offset_{name}", host64(out), host64(lse), o_ref, l_ref, dtype)


def test_offset_equal_to_bottom_right_matches_plain_call():
    torch = need_gpu()
    w = make_custom([300, 7, 1000], [400, 7, 1000], num_heads_q=32, num_heads_kv=8, head_dim=128, dtype="bf16",
                    causal=True, seed=61)
    print("[case] offset == Lk - Lq vs varlen_attn_fwd", flush=True)
    a = run_offset(w, (w.lengths_k - w.lengths_q).tolist())
    d = to_device(w)
    b = vfa.varlen_attn_fwd(d["q"], d["k"], d["v"], d["cu_q"], d["cu_k"], w.max_seqlen_q, w.max_seqlen_k,
                            softmax_scale=w.scale, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("sp", [2, 4])
def test_context_parallel_chunks_merged(sp):
    """One GPU's share of context parallelism over keys: chunk c of every sequence is packed alone and
    computed against all queries with offset -a_c (fp32 partials); attn_update merges the sp partials.
    The result must match unchunked causal attention, and each partial the oracle's chunk partial."""
    torch = need_gpu()
    lens = [1500, 333, 2048, 1]
    w = make_custom(lens, num_heads_q=32, num_heads_kv=8, head_dim=128, dtype="bf16", causal=True, seed=62)
    print(f"[case] context-parallel chunks sp={sp} lengths={lens}", flush=True)
    cu = w.cu_seqlens_k.astype(np.int64)
    q = dev_array(w.q, "bf16")
    cu_q = torch.from_numpy(w.cu_seqlens_q).cuda()
    rows = w.total_q * w.num_heads_q
    lse_parts = torch.empty((sp, rows), dtype=torch.float32, device="cuda")
    go_parts = torch.empty((sp, rows, w.head_dim), dtype=torch.float32, device="cuda")
    lse_o, go_o = oracle.chunked_partials(w.q, w.k, w.v, w.cu_seqlens_q, w.cu_seqlens_k, w.num_heads_kv,
                                          w.scale, True, sp)
    for c in range(sp):
        bounds = [chunk_bounds(int(n), sp)[c] for n in lens]
        kc = np.concatenate([w.k[cu[b] + lo:cu[b] + hi] for b, (lo, hi) in enumerate(bounds)])
        vc = np.concatenate([w.v[cu[b] + lo:cu[b] + hi] for b, (lo, hi) in enumerate(bounds)])
        clen = [hi - lo for lo, hi in bounds]
        cu_k = torch.from_numpy(np.concatenate([[0], np.cumsum(clen)]).astype(np.int32)).cuda()
        off = torch.tensor([-lo for lo, _ in bounds], dtype=torch.int32, device="cuda")
        o, l = vfa.varlen_attn_fwd(q, dev_array(kc, "bf16"), dev_array(vc, "bf16"), cu_q, cu_k, w.max_seqlen_q,
                                   max(max(clen), 1), softmax_scale=w.scale, causal=True, out_dtype=torch.float32,
                                   causal_offset=off)
        torch.cuda.synchronize()
        check(f"cp_sp{sp}_chunk{c}", host64(o).reshape(rows, -1), host64(l).reshape(rows), go_o[c], lse_o[c],
              "bf16")
        go_parts[c] = o.reshape(rows, -1)
        lse_parts[c] = l.reshape(rows)
    out, lse_m = vfa.attn_update(lse_parts, go_parts, update_type=1)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.varlen_attention(w.q, w.k, w.v, w.cu_seqlens_q, w.cu_seqlens_k, w.num_heads_kv,
                                           w.scale, True)
    check(f"cp_sp{sp}_merged", host64(out).reshape(w.total_q, w.num_heads_q, -1),
          host64(lse_m).reshape(w.total_q, w.num_heads_q), o_ref, l_ref, "bf16")
