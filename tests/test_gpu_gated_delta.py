"""GPU parity: gated_delta_rule_fwd (varlen gated delta rule, fp32 state) against the fp64 oracle.

Tolerances: out is one bf16 rounding of an fp32 result, |out - ref| <= 2^-7 |ref| + 1e-4; the fp32 final
state, |S - ref| <= 1e-4 + 1e-4 |ref| (fp32 arithmetic over the sequence against fp64 on the same
bf16-exact inputs)."""
import numpy as np
import pytest

import oracle
import varlen_flash_attention_amd as vfa
from varlen_flash_attention_amd.workloads import make_gated_delta, make_workload
from tests.gpu_util import dev_array, host64, need_gpu

pytestmark = pytest.mark.gpu


def dev_inputs(p):
    torch = need_gpu()
    return dict(q=dev_array(p.q, "bf16"), k=dev_array(p.k, "bf16"), v=dev_array(p.v, "bf16"),
                g=torch.from_numpy(p.g).cuda(), beta=torch.from_numpy(p.beta).cuda(),
                cu=torch.from_numpy(p.cu_seqlens).cuda())


def check_close(name, got, ref, rtol, atol):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape and not np.isnan(got).any()
    bound = rtol * np.abs(ref) + atol
    err = np.abs(got - ref)
    worst = float((err / bound).max()) if err.size else 0.0
    print(f"[parity] {name}: worst err/bound {worst:.3f}", flush=True)
    assert (err <= bound).all(), f"{name}: {(err > bound).sum()} values out of tolerance (worst {worst:.3f})"


CASES = {
    # name: (lengths, Hqk, Hv, Dk, Dv, with initial state)
    "d128_gva": ([1, 17, 64, 200, 33, 0], 2, 4, 128, 128, False),
    "d64_mh": ([40, 3, 130], 3, 3, 64, 64, True),
    "dk128_dv64": ([70, 129], 1, 2, 128, 64, True),
    "dk64_dv128": ([31, 96, 5], 2, 2, 64, 128, False),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_gated_delta_parity(name):
    torch = need_gpu()
    lens, hqk, hv, dk, dv, with_init = CASES[name]
    p = make_gated_delta(lens, hqk, hv, dk, dv, seed=len(name))
    print(f"[case] gated_delta {name}: lengths={lens} Hqk={hqk} Hv={hv} Dk={dk} Dv={dv} init={with_init}", flush=True)
    x = dev_inputs(p)
    s0 = None
    s0_dev = None
    if with_init:
        s0 = np.random.default_rng(7).standard_normal((len(lens), hv, dk, dv)).astype(np.float32) * 0.5
        s0_dev = torch.from_numpy(s0).cuda()
    out, fin = vfa.gated_delta_rule_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu"], scale=p.scale,
                                        initial_state=s0_dev, output_final_state=True)
    torch.cuda.synchronize()
    o_ref, f_ref = oracle.gated_delta_rule(p.q, p.k, p.v, p.g, p.beta, p.cu_seqlens, p.scale, initial_state=s0)
    check_close(f"{name}_out", host64(out), o_ref, 2.0 ** -7, 1e-4)
    check_close(f"{name}_state", host64(fin), f_ref, 1e-4, 1e-4)


def test_gated_delta_continuation_is_exact():
    """Two calls, the second starting from the first's final state, give bit for bit the outputs and
    state of one call over the whole sequences (the kernel keeps the state in fp32 between tokens)."""
    torch = need_gpu()
    a = make_gated_delta([100, 37], 2, 4, 128, 128, seed=91)
    print("[case] gated_delta continuation", flush=True)
    x = dev_inputs(a)
    whole, fin = vfa.gated_delta_rule_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu"], scale=a.scale,
                                          output_final_state=True)
    cu1 = np.array([0, 60, 60 + 20], dtype=np.int32)            # first 60 and 20 tokens of each sequence
    idx1 = np.r_[0:60, 100:120]
    idx2 = np.r_[60:100, 120:137]
    cu2 = np.array([0, 40, 57], dtype=np.int32)

    def part(idx, cu, init):
        ii = torch.from_numpy(idx).cuda()
        return vfa.gated_delta_rule_fwd(x["q"][ii].contiguous(), x["k"][ii].contiguous(), x["v"][ii].contiguous(),
                                        x["g"][ii].contiguous(), x["beta"][ii].contiguous(),
                                        torch.from_numpy(cu).cuda(), scale=a.scale, initial_state=init,
                                        output_final_state=True)
    o1, f1 = part(idx1, cu1, None)
    o2, f2 = part(idx2, cu2, f1)
    torch.cuda.synchronize()
    assert torch.equal(o1, whole[torch.from_numpy(idx1).cuda()])
    assert torch.equal(o2, whole[torch.from_numpy(idx2).cuda()])
    assert torch.equal(f2, fin)


def test_gated_delta_long_prefill_shape_sampled():
    """The long-prefill lengths (16 sequences, 35 324 tokens) with 16 query/key and 32 value heads,
    D 128: three whole (sequence, value head) chains, the longest sequence among them, against the oracle."""
    torch = need_gpu()
    lens = make_workload("long_prefill", values=False).lengths_q
    p = make_gated_delta(lens, 16, 32, 128, 128, seed=92)
    print(f"[case] gated_delta long-prefill shape T={int(lens.sum())}", flush=True)
    x = dev_inputs(p)
    out, fin = vfa.gated_delta_rule_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu"], scale=p.scale,
                                        output_final_state=True)
    torch.cuda.synchronize()
    cu = p.cu_seqlens
    longest = int(np.argmax(lens))
    for b, h in ((longest, 31), (1, 0), (len(lens) - 1, 17)):
        lo, hi = int(cu[b]), int(cu[b + 1])
        hk = h // 2
        o_ref, f_ref = oracle.gated_delta_rule(p.q[lo:hi, hk:hk + 1], p.k[lo:hi, hk:hk + 1], p.v[lo:hi, h:h + 1],
                                               p.g[lo:hi, h:h + 1], p.beta[lo:hi, h:h + 1], [0, hi - lo], p.scale)
        check_close(f"long_b{b}_h{h}_out", host64(out[lo:hi, h:h + 1]), o_ref, 2.0 ** -7, 1e-4)
        check_close(f"long_b{b}_h{h}_state", host64(fin[b, h]), f_ref[0, 0], 1e-4, 1e-4)
