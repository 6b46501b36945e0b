"""GPU parity for a sequence whose keys span more than 4 GiB.

The prefill kernels read K and V through buffer resources with 32-bit byte
offsets. Here one sequence holds 2,100,001 keys of 8 kv heads x 128 dims in
bf16: 4.30e9 bytes per tensor, past 2^32. Its query lengths would select the
persistent long-prefill kernel, which addresses a whole sequence from one
buffer, so the launcher hands it to the 128-column kernel, which rebases its
buffers on every 32-key sub-block. The first sequence is short and sits in
front, so the long one starts at a nonzero key offset.

Sampled rows (first, middle and last query of each sequence) of two kv
heads are compared with the fp64 oracle, called on those heads' slices only
(heads are independent: query head h reads kv head h / G).
"""
import numpy as np
import pytest

import oracle
import varlen_flash_attention_amd as vfa
from varlen_flash_attention_amd.workloads import make_custom
from tests.gpu_util import check, host64, need_gpu, to_device

pytestmark = pytest.mark.gpu

HQ, HKV, D = 64, 8, 128
LQ = [512, 300]
LK = [1000, 2_100_001]


def test_causal_prefill_keys_past_4gib():
    torch = need_gpu()
    assert LK[1] * HKV * D * 2 > 2**32
    print(f"[case] keys_4gib: Lq={LQ} Lk={LK} Hq={HQ} Hkv={HKV} D={D} bf16 causal", flush=True)
    w = make_custom(LQ, LK, num_heads_q=HQ, num_heads_kv=HKV, head_dim=D, dtype="bf16", causal=True, seed=43,
                    name="keys_4gib")
    grp = HQ // HKV
    assert w.total_q // w.batch >= 8 * (256 // grp)      # long-prefill by its query lengths
    assert vfa.varlen_attn_fwd_workspace_size(w.batch, w.total_q, w.max_seqlen_q, w.max_seqlen_k, HQ, HKV, D) == 0
    d = to_device(w)
    print("[step] inputs on the device", flush=True)
    out, lse = vfa.varlen_attn_fwd(d["q"], d["k"], d["v"], d["cu_q"], d["cu_k"], w.max_seqlen_q, w.max_seqlen_k,
                                   softmax_scale=w.scale, causal=True)
    torch.cuda.synchronize()
    del d
    print("[step] kernel done", flush=True)
    tokens = np.array([0, LQ[0] // 2, LQ[0] - 1, LQ[0], LQ[0] + LQ[1] // 2, LQ[0] + LQ[1] - 1], dtype=np.int64)
    idx = torch.from_numpy(tokens).to(out.device)
    o_sel, l_sel = host64(out[idx]), host64(lse[idx])
    for g in (0, HKV - 1):
        heads = slice(g * grp, (g + 1) * grp)
        o_ref, l_ref = oracle.varlen_attention_rows(w.q[:, heads], w.k[:, g:g + 1], w.v[:, g:g + 1],
                                                    w.cu_seqlens_q, w.cu_seqlens_k, 1, w.scale, True,
                                                    tokens=tokens)
        check(f"keys_4gib kv head {g}", o_sel[:, heads], l_sel[:, heads], o_ref, l_ref, "bf16")
