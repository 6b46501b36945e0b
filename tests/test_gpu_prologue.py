"""GPU parity: qk_norm_rope (per-head q/k RMSNorm, then the rotary embedding) against the fp64 oracle.

The kernel computes in fp32 and rounds once to bf16, so each output must lie within one bf16 unit in
the last place of the exact value: |out - ref| <= 2^-7 |ref| + 1e-6 (2^-7 |ref| bounds one bf16 ulp;
the 1e-6 covers fp32 arithmetic on values near 0).
"""
import numpy as np
import pytest

import oracle
import varlen_flash_attention_amd as vfa
from varlen_flash_attention_amd.workloads import make_prologue
from tests.gpu_util import dev_array, host64, need_gpu

pytestmark = pytest.mark.gpu


def dev_inputs(p):
    torch = need_gpu()
    return dict(q=dev_array(p.q, "bf16"), k=dev_array(p.k, "bf16"), wq=dev_array(p.q_weight, "bf16"),
                wk=dev_array(p.k_weight, "bf16"), cos=torch.from_numpy(p.cos).cuda(),
                sin=torch.from_numpy(p.sin).cuda())


def check_ulp(name, got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape and not np.isnan(got).any()
    bound = 2.0 ** -7 * np.abs(ref) + 1e-6
    err = np.abs(got - ref)
    worst = float((err / bound).max())
    print(f"[parity] {name}: worst err/bound {worst:.3f}", flush=True)
    assert (err <= bound).all(), f"{name}: {(err > bound).sum()} values beyond one bf16 ulp (worst {worst:.3f})"


CASES = {
    # name: (lengths, Hq, Hkv, D, eps)
    "d128_gqa": ([1, 17, 300, 1000, 64], 32, 8, 128, 1e-6),
    "d64_mha": ([5, 129, 33], 16, 16, 64, 1e-6),
    "d128_wide_group": ([700, 2], 64, 4, 128, 1e-5),
    "d64_large_eps": ([50, 50], 8, 2, 64, 0.5),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_qk_norm_rope_parity(name):
    torch = need_gpu()
    lens, hq, hkv, d, eps = CASES[name]
    p = make_prologue(lens, hq, hkv, d, eps=eps, seed=len(name))
    print(f"[case] qk_norm_rope {name}: lengths={lens} Hq={hq} Hkv={hkv} D={d} eps={eps}", flush=True)
    x = dev_inputs(p)
    qo, ko = vfa.qk_norm_rope(x["q"], x["k"], x["wq"], x["wk"], x["cos"], x["sin"], eps=eps)
    torch.cuda.synchronize()
    q_ref, k_ref = oracle.qk_norm_rope(p.q, p.k, p.q_weight, p.k_weight, p.cos, p.sin, eps)
    check_ulp(f"{name}_q", host64(qo), q_ref)
    check_ulp(f"{name}_k", host64(ko), k_ref)


def test_qk_norm_rope_in_place_matches():
    torch = need_gpu()
    p = make_prologue([3, 400, 77], 32, 8, 128, seed=71)
    print("[case] qk_norm_rope in place", flush=True)
    x = dev_inputs(p)
    qo, ko = vfa.qk_norm_rope(x["q"], x["k"], x["wq"], x["wk"], x["cos"], x["sin"], eps=p.eps)
    qi, ki = x["q"].clone(), x["k"].clone()
    vfa.qk_norm_rope(qi, ki, x["wq"], x["wk"], x["cos"], x["sin"], eps=p.eps, q_out=qi, k_out=ki)
    torch.cuda.synchronize()
    assert torch.equal(qi, qo) and torch.equal(ki, ko)


def test_qk_norm_rope_long_prefill_shape_sampled():
    """The long-prefill token count (35 324 tokens, 32/8 heads, D 128), checked on sampled tokens."""
    torch = need_gpu()
    from varlen_flash_attention_amd.workloads import make_workload
    lens = make_workload("long_prefill", values=False).lengths_q
    p = make_prologue(lens, 32, 8, 128, seed=72)
    print(f"[case] qk_norm_rope long-prefill shape T={int(lens.sum())}", flush=True)
    x = dev_inputs(p)
    qo, ko = vfa.qk_norm_rope(x["q"], x["k"], x["wq"], x["wk"], x["cos"], x["sin"], eps=p.eps)
    torch.cuda.synchronize()
    toks = np.unique(np.concatenate([np.random.default_rng(0).integers(0, int(lens.sum()), 3000),
                                     p.cu_seqlens[:-1], p.cu_seqlens[1:] - 1]))
    q_ref, k_ref = oracle.qk_norm_rope(p.q[toks], p.k[toks], p.q_weight, p.k_weight, p.cos[toks], p.sin[toks],
                                       p.eps)
    idx = torch.from_numpy(toks).cuda()
    check_ulp("long_prefill_q", host64(qo[idx]), q_ref)
    check_ulp("long_prefill_k", host64(ko[idx]), k_ref)
