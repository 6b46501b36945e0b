"""GPU parity: gated_delta_rule_fwd (varlen gated delta rule, fp32 state) against the fp64 oracle.

Both paths are covered: max_seqlen up to 16 runs the token-by-token recurrence, above it the chunked form
(64-token chunks; T = (I + A)^-1 and M per chunk, bf16 hi / lo products on MFMA).

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
    # name: (lengths, Hqk, Hv, Dk, Dv, with initial state, max_seqlen or None for max(lengths))
    "d128_gva": ([1, 17, 64, 200, 33, 0], 2, 4, 128, 128, False, None),
    "d64_mh": ([40, 3, 130], 3, 3, 64, 64, True, None),
    "dk128_dv64": ([70, 129], 1, 2, 128, 64, True, None),
    "dk64_dv128": ([31, 96, 5], 2, 2, 64, 128, False, None),
    "chunk_edges": ([63, 64, 65, 127, 128, 129, 1, 191], 1, 2, 128, 128, True, None),
    "recurrent_short": ([1, 16, 5, 0, 9, 16], 2, 4, 128, 128, True, None),
    "recurrent_d64": ([7, 12, 3], 1, 1, 64, 64, False, None),
    "chunked_loose_bound": ([1, 16, 5, 0, 9, 16], 2, 4, 128, 128, True, 300),
    "all_empty": ([0, 0, 0], 1, 2, 64, 128, True, None),
    "gva4": ([150, 70], 2, 8, 128, 128, True, None),
    "single_head": ([300], 1, 1, 128, 64, True, None),
    # 100 sequences of 1..80 tokens: many partial chunks, grid sizes not divisible by 8
    "many_short": ([int(x) for x in np.random.default_rng(97).integers(1, 81, 100)], 2, 4, 64, 64, False, None),
    # one serving decode step: 128 sequences of one token each from their states
    "decode_step": ([1] * 128, 4, 8, 128, 128, True, None),
    # the chunked path ranks up to 4096 sequences by length (ties by index) for its second kernel and
    # keeps larger batches in index order: both sides of that limit, lengths 17..19 (many ties)
    "ranked_4096": ([int(x) for x in np.random.default_rng(5).integers(17, 20, 4096)], 1, 1, 64, 64, False, None),
    "unranked_4097": ([int(x) for x in np.random.default_rng(6).integers(17, 20, 4097)], 1, 1, 64, 64, True,
                      None),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_gated_delta_parity(name):
    torch = need_gpu()
    lens, hqk, hv, dk, dv, with_init, bound = CASES[name]
    p = make_gated_delta(lens, hqk, hv, dk, dv, seed=len(name))
    ms = max(lens) if bound is None else bound
    print(f"[case] gated_delta {name}: lengths={lens} Hqk={hqk} Hv={hv} Dk={dk} Dv={dv} init={with_init} "
          f"max_seqlen={ms}", flush=True)
    x = dev_inputs(p)
    s0 = None
    s0_dev = None
    if with_init:
        s0 = np.random.default_rng(7).standard_normal((len(lens), hv, dk, dv)).astype(np.float32) * 0.5
        s0_dev = torch.from_numpy(s0).cuda()
    out, fin = vfa.gated_delta_rule_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu"], ms, scale=p.scale,
                                        initial_state=s0_dev, output_final_state=True)
    torch.cuda.synchronize()
    o_ref, f_ref = oracle.gated_delta_rule(p.q, p.k, p.v, p.g, p.beta, p.cu_seqlens, p.scale, initial_state=s0)
    check_close(f"{name}_out", host64(out), o_ref, 2.0 ** -7, 1e-4)
    check_close(f"{name}_state", host64(fin), f_ref, 1e-4, 1e-4)


GATE_CASES = {
    # name: how g and beta are replaced (the rest as make_gated_delta draws it)
    "strong_decay": "g uniform in [-8, 0): e^gamma underflows to 0 inside a 64-token chunk",
    "no_decay": "g = 0: the plain delta rule",
    "beta_extremes": "beta exactly 0 or 1, alternating per token",
}


@pytest.mark.parametrize("name", sorted(GATE_CASES))
def test_gated_delta_gate_extremes(name):
    """Both paths against the oracle with gates the default draw never makes. The chunked path takes
    decay factors from fp64 differences of the cumulative log decay, so factors that underflow in fp32
    stay exact zeros rather than 0/0."""
    torch = need_gpu()
    lens = [200, 13, 64, 1]
    p = make_gated_delta(lens, 2, 4, 128, 128, seed=95)
    rng = np.random.default_rng(96)
    if name == "strong_decay":
        p.g[:] = (-8.0 * rng.random(p.g.shape)).astype(np.float32)
    elif name == "no_decay":
        p.g[:] = 0.0
    else:
        p.beta[:] = (np.arange(p.beta.shape[0])[:, None] % 2).astype(np.float32)
    s0 = rng.standard_normal((len(lens), 4, 128, 128)).astype(np.float32) * 0.5
    print(f"[case] gated_delta gates {name}: {GATE_CASES[name]}", flush=True)
    x = dev_inputs(p)
    o_ref, f_ref = oracle.gated_delta_rule(p.q, p.k, p.v, p.g, p.beta, p.cu_seqlens, p.scale, initial_state=s0)
    for ms in (max(lens), 16):                       # chunked path, then token by token on the short ones
        if ms == 16:
            keep = [b for b, n in enumerate(lens) if n <= 16]
            idx = np.concatenate([np.arange(p.cu_seqlens[b], p.cu_seqlens[b + 1]) for b in keep])
            ii = torch.from_numpy(idx).cuda()
            cu = torch.from_numpy(np.r_[0, np.cumsum([lens[b] for b in keep])].astype(np.int32)).cuda()
            sub = {name: x[name][ii].contiguous() for name in ("q", "k", "v", "g", "beta")}
            out, fin = vfa.gated_delta_rule_fwd(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], cu, 16,
                                                scale=p.scale, initial_state=torch.from_numpy(s0[keep]).cuda(),
                                                output_final_state=True)
            want_o, want_f = o_ref[idx], f_ref[keep]
        else:
            out, fin = vfa.gated_delta_rule_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu"], ms, scale=p.scale,
                                                initial_state=torch.from_numpy(s0).cuda(), output_final_state=True)
            want_o, want_f = o_ref, f_ref
        torch.cuda.synchronize()
        check_close(f"{name}_ms{ms}_out", host64(out), want_o, 2.0 ** -7, 1e-4)
        check_close(f"{name}_ms{ms}_state", host64(fin), want_f, 1e-4, 1e-4)


def _continuation(lengths, split, seed):
    """Runs the packed sequences whole, then as two calls (the first `split[b]` tokens of each sequence,
    then the rest from the first call's final state); returns both outputs and final states."""
    torch = need_gpu()
    a = make_gated_delta(lengths, 2, 4, 128, 128, seed=seed)
    x = dev_inputs(a)
    whole, fin = vfa.gated_delta_rule_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu"], max(lengths),
                                          scale=a.scale, output_final_state=True)
    starts = np.r_[0, np.cumsum(lengths)[:-1]]
    idx1 = np.concatenate([np.arange(s0, s0 + m) for s0, m in zip(starts, split)])
    idx2 = np.concatenate([np.arange(s0 + m, s0 + n) for s0, m, n in zip(starts, split, lengths)])
    rest = [n - m for n, m in zip(lengths, split)]

    def part(idx, lens, init):
        ii = torch.from_numpy(idx).cuda()
        cu = torch.from_numpy(np.r_[0, np.cumsum(lens)].astype(np.int32)).cuda()
        return vfa.gated_delta_rule_fwd(x["q"][ii].contiguous(), x["k"][ii].contiguous(), x["v"][ii].contiguous(),
                                        x["g"][ii].contiguous(), x["beta"][ii].contiguous(), cu, max(lens),
                                        scale=a.scale, initial_state=init, output_final_state=True)
    o1, f1 = part(idx1, split, None)
    o2, f2 = part(idx2, rest, f1)
    torch.cuda.synchronize()
    return (whole[torch.from_numpy(idx1).cuda()], o1), (whole[torch.from_numpy(idx2).cuda()], o2), (fin, f2)


def test_gated_delta_continuation_is_exact_chunked():
    """Split at 64-token chunk boundaries, two chunked calls (the second from the first's fp32 final
    state) repeat one whole call's chunks exactly: outputs and state bit for bit."""
    torch = need_gpu()
    print("[case] gated_delta continuation, chunked", flush=True)
    for want, got in _continuation([100, 137], [64, 128], seed=91):
        assert torch.equal(got, want)


def test_gated_delta_continuation_is_exact_recurrent():
    """The token-by-token path (lengths up to 16) keeps the state in fp32 between tokens, so a split
    anywhere gives the whole call's outputs and state bit for bit."""
    torch = need_gpu()
    print("[case] gated_delta continuation, recurrent", flush=True)
    for want, got in _continuation([10, 15, 7], [4, 9, 1], seed=92):
        assert torch.equal(got, want)


def test_gated_delta_paths_agree():
    """The same short sequences through both paths (max_seqlen 16, then a loose bound of 17): each is
    within the oracle bound, so they differ by at most the sum of the two bounds."""
    torch = need_gpu()
    lens = [16, 3, 11, 1]
    p = make_gated_delta(lens, 2, 4, 128, 128, seed=94)
    print("[case] gated_delta paths agree", flush=True)
    x = dev_inputs(p)
    outs = [vfa.gated_delta_rule_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu"], ms, scale=p.scale,
                                     output_final_state=True) for ms in (16, 17)]
    torch.cuda.synchronize()
    (o_r, f_r), (o_c, f_c) = ((host64(o), host64(f)) for o, f in outs)
    ref_o, ref_f = oracle.gated_delta_rule(p.q, p.k, p.v, p.g, p.beta, p.cu_seqlens, p.scale)
    # |o_r| is within 2^-7 of |ref|, so two oracle bounds fit inside 2.1 * 2^-7 |o_r| + 2e-4.
    check_close("paths_out", o_c, o_r, 2.1 * 2.0 ** -7, 2e-4)
    check_close("paths_state", f_c, f_r, 2.1e-4, 2e-4)
    check_close("recurrent_vs_oracle", o_r, ref_o, 2.0 ** -7, 1e-4)
    check_close("chunked_vs_oracle", o_c, ref_o, 2.0 ** -7, 1e-4)
    check_close("recurrent_state_vs_oracle", f_r, ref_f, 1e-4, 1e-4)
    check_close("chunked_state_vs_oracle", f_c, ref_f, 1e-4, 1e-4)


def test_gated_delta_long_prefill_shape_sampled():
    """The long-prefill lengths (16 sequences, 35 324 tokens) with 16 query/key and 32 value heads,
    D 128: three whole (sequence, value head) chains, the longest sequence among them, against the oracle."""
    torch = need_gpu()
    lens = make_workload("long_prefill", values=False).lengths_q
    p = make_gated_delta(lens, 16, 32, 128, 128, seed=92)
    print(f"[case] gated_delta long-prefill shape T={int(lens.sum())}", flush=True)
    x = dev_inputs(p)
    out, fin = vfa.gated_delta_rule_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu"], int(lens.max()),
                                        scale=p.scale, output_final_state=True)
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
