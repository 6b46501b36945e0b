"""GPU parity: attn_update, chunked attention merged on the GPU, and the last-token gather."""
import numpy as np
import pytest

import oracle
import varlen_flash_attention_amd as vfa
from varlen_flash_attention_amd.workloads import chunk_bounds, make_workload
from tests.gpu_util import check, dev_array, host64, need_gpu, to_device

pytestmark = pytest.mark.gpu


def _random_partials(rng, sp, bsh, hd, dead_frac=0.1):
    lse = rng.normal(0.0, 3.0, (sp, bsh)).astype(np.float32)
    lse[rng.random((sp, bsh)) < dead_frac] = -np.inf          # empty chunks
    lse[:, :3] = -np.inf                                         # rows with no live chunk at all
    go = rng.standard_normal((sp, bsh, hd)).astype(np.float32)
    return lse, go


@pytest.mark.parametrize("sp", [1, 2, 3, 5, 8, 16, 17, 33])
@pytest.mark.parametrize("hd", [64, 128])
@pytest.mark.parametrize("go_dtype", ["fp32", "bf16"])
def test_attn_update_random(sp, hd, go_dtype):
    torch = need_gpu()
    rng = np.random.default_rng(1000 + sp * 7 + hd)
    bsh = 1000 + sp                      # not a multiple of the rows per block
    lse, go = _random_partials(rng, sp, bsh, hd)
    if go_dtype == "bf16":
        from varlen_flash_attention_amd.workloads import round_to_bf16
        go = round_to_bf16(go)
    print(f"[case] attn_update sp={sp} hd={hd} go={go_dtype} bsh={bsh}", flush=True)
    lse_d = torch.from_numpy(lse).cuda()
    go_d = dev_array(go, go_dtype)
    out, lse_out = vfa.attn_update(lse_d, go_d, 1)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attn_update(lse, go, 1)
    # fp32 partials: fp32 tolerance; bf16 partials: the output is rounded to bf16
    check(f"attn_update sp={sp} hd={hd} {go_dtype}", host64(out), host64(lse_out), ref_o, ref_l,
          "fp32" if go_dtype == "fp32" else "bf16")


@pytest.mark.parametrize("go_dtype,sp,bsh,hd", [
    ("fp32", 8, 20003, 128),    # 2501 workgroups: one row per thread
    ("fp32", 8, 40003, 128),    # 5001 workgroups: two rows per thread, ragged last pair
    ("bf16", 2, 65537, 128),    # two rows per thread, one row past the last full pair
    ("bf16", 3, 140003, 64),    # hd = 64, two rows per thread
])
def test_attn_update_large(go_dtype, sp, bsh, hd):
    """Large merges (at least 4096 workgroups of rows) take the two-rows-per-thread variant."""
    torch = need_gpu()
    rng = np.random.default_rng(bsh + sp)
    lse, go = _random_partials(rng, sp, bsh, hd)
    if go_dtype == "bf16":
        from varlen_flash_attention_amd.workloads import round_to_bf16
        go = round_to_bf16(go)
    print(f"[case] attn_update large sp={sp} hd={hd} go={go_dtype} bsh={bsh}", flush=True)
    out, lse_out = vfa.attn_update(torch.from_numpy(lse).cuda(), dev_array(go, go_dtype), 1)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attn_update(lse, go, 1)
    check(f"attn_update large {go_dtype} sp={sp} bsh={bsh}", host64(out), host64(lse_out), ref_o, ref_l,
          "fp32" if go_dtype == "fp32" else "bf16")


def test_attn_update_type0_leaves_lse_out():
    torch = need_gpu()
    rng = np.random.default_rng(7)
    lse, go = _random_partials(rng, 4, 300, 128)
    sentinel = torch.full((300,), 123.0, device="cuda")
    out, none = vfa.attn_update(torch.from_numpy(lse).cuda(), torch.from_numpy(go).cuda(), 0, lse_out=sentinel)
    torch.cuda.synchronize()
    assert none is None
    assert (sentinel == 123.0).all()
    ref_o, _ = oracle.attn_update(lse, go, 0)
    check("attn_update type 0", host64(out), np.zeros(300), ref_o, np.zeros(300), "fp32")


def test_attn_update_merge_config_oracle_partials():
    """Chunked-context merge shape: sp=8, bsh=64*32, hd=128, fp32 partials from the oracle."""
    torch = need_gpu()
    w = make_workload("decode")
    print("[case] merge config with oracle partials (sp=8, bsh=2048, hd=128)", flush=True)
    lse_c, go_c = oracle.chunked_partials(w.q, w.k, w.v, w.cu_seqlens_q, w.cu_seqlens_k, w.num_heads_kv,
                                          w.scale, True, 8)
    lse32, go32 = lse_c.astype(np.float32), go_c.astype(np.float32)
    out, lse_m = vfa.attn_update(torch.from_numpy(lse32).cuda(), torch.from_numpy(go32).cuda(), 1)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (2048, 128) and tuple(lse_m.shape) == (2048,)
    ref_o, ref_l = oracle.attn_update(lse32, go32, 1)       # fp64 merge of the same fp32 partials
    check("merge of fp32 oracle partials", host64(out), host64(lse_m), ref_o, ref_l, "fp32")


def _chunk_pack(w, sp, c):
    """K/V rows of chunk c of every sequence, packed, with their cu_seqlens_k."""
    cu = w.cu_seqlens_k.astype(np.int64)
    idx, lens = [], []
    for b in range(w.batch):
        lo, hi = chunk_bounds(int(w.lengths_k[b]), sp)[c]
        idx.append(np.arange(cu[b] + lo, cu[b] + hi))
        lens.append(hi - lo)
    idx = np.concatenate(idx).astype(np.int64)
    cuk = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return idx, cuk, max(lens)


def test_chunked_decode_merged_on_gpu():
    """Chunked-context merge end to end: per-chunk GPU attention (fp32 partials) -> attn_update."""
    torch = need_gpu()
    w = make_workload("decode")
    print("[case] decode split into 8 key chunks, GPU partials + GPU merge", flush=True)
    d = to_device(w)
    lses, gos = [], []
    for c in range(8):
        idx, cuk, maxk = _chunk_pack(w, 8, c)
        ii = torch.from_numpy(idx).cuda()
        o_c, l_c = vfa.varlen_attn_fwd(d["q"], d["k"][ii].contiguous(), d["v"][ii].contiguous(), d["cu_q"],
                                       torch.from_numpy(cuk).cuda(), 1, maxk, softmax_scale=w.scale,
                                       causal=True, out_dtype=torch.float32)
        lses.append(l_c.reshape(-1))
        gos.append(o_c.reshape(-1, 128))
    lse = torch.stack(lses).contiguous()
    go = torch.stack(gos).contiguous()
    out, lse_m = vfa.attn_update(lse, go, 1)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.varlen_attention(w.q, w.k, w.v, w.cu_seqlens_q, w.cu_seqlens_k, w.num_heads_kv,
                                           w.scale, True)
    check("chunked decode merged", host64(out), host64(lse_m), o_ref.reshape(-1, 128), l_ref.reshape(-1), "bf16")


def test_tiny_causal_sp2_merged_on_gpu():
    """Tiny fp32 config: keys split into 2 chunks with causal masking on absolute positions.

    For chunk [a, b) of a sequence with Lq = Lk = L, queries [a, b) see chunk keys
    causally (a square causal problem), queries [b, L) see the whole chunk (full
    mask) and queries [0, a) see nothing (lse = -inf, O = 0).
    """
    torch = need_gpu()
    w = make_workload("tiny_fp32")
    print("[case] tiny fp32 causal, sp=2 chunks merged on the GPU", flush=True)
    hq, dd = w.num_heads_q, w.head_dim
    T = w.total_q
    cu = w.cu_seqlens_q.astype(np.int64)
    lse_parts = np.full((2, T, hq), -np.inf, dtype=np.float32)
    go_parts = np.zeros((2, T, hq, dd), dtype=np.float32)
    for c in range(2):
        for causal in (True, False):
            qi, ki, lq, lk = [], [], [], []
            for b in range(w.batch):
                L = int(w.lengths_q[b])
                a, e = chunk_bounds(L, 2)[c]
                qr = np.arange(a, e) if causal else np.arange(e, L)
                qi.append(cu[b] + qr)
                ki.append(cu[b] + np.arange(a, e))
                lq.append(len(qr))
                lk.append(e - a)
            qi = np.concatenate(qi).astype(np.int64)
            ki = np.concatenate(ki).astype(np.int64)
            if len(qi) == 0:
                continue
            q = torch.from_numpy(np.ascontiguousarray(w.q[qi])).cuda()
            k = torch.from_numpy(np.ascontiguousarray(w.k[ki])).cuda()
            v = torch.from_numpy(np.ascontiguousarray(w.v[ki])).cuda()
            cuq = torch.from_numpy(np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)).cuda()
            cuk = torch.from_numpy(np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)).cuda()
            o, l = vfa.varlen_attn_fwd(q, k, v, cuq, cuk, max(lq), max(lk), softmax_scale=w.scale, causal=causal)
            torch.cuda.synchronize()
            go_parts[c, qi] = o.cpu().numpy()
            lse_parts[c, qi] = l.cpu().numpy()
    lse_d = torch.from_numpy(lse_parts.reshape(2, T * hq)).cuda()
    go_d = torch.from_numpy(go_parts.reshape(2, T * hq, dd)).cuda()
    out, lse_m = vfa.attn_update(lse_d, go_d, 1)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.varlen_attention(w.q, w.k, w.v, w.cu_seqlens_q, w.cu_seqlens_k, w.num_heads_kv,
                                           w.scale, True)
    check("tiny sp=2 merged", host64(out), host64(lse_m), o_ref.reshape(-1, dd), l_ref.reshape(-1), "fp32")


@pytest.mark.parametrize("dtype,shape", [("fp32", (7, 3)), ("bf16", (5, 16, 128)), ("bf16", (3,)),
                                         ("fp32", (4, 32))])
def test_last_token_gather_edges(dtype, shape):
    torch = need_gpu()
    lengths = np.array([3, 0, 1, 9, 0, 2], dtype=np.int64)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((int(cu[-1]), *shape[1:])).astype(np.float32)
    if dtype == "bf16":
        from varlen_flash_attention_amd.workloads import round_to_bf16
        x = round_to_bf16(x)
    print(f"[case] gather {dtype} row shape {shape[1:]}", flush=True)
    got = vfa.varlen_last_token_gather(dev_array(x, dtype), torch.from_numpy(cu).cuda())
    torch.cuda.synchronize()
    got = host64(got)
    for b in range(len(lengths)):
        if lengths[b] == 0:
            assert (got[b] == 0).all()
        else:
            assert np.array_equal(got[b], x[cu[b + 1] - 1].astype(np.float64))
