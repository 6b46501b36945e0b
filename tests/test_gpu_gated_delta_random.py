"""GPU parity of gated_delta_rule_fwd on seeded random shapes against the fp64 recurrence.

Each case draws a batch of 1-10 sequences (empty, decode-like, one-chunk, several-chunk and ragged
lengths up to 400 tokens), Hqk 1-4 with Hv = Hqk times 1, 2 or 4, Dk and Dv each 64 or 128, with or without
an initial state, and sometimes a max_seqlen above the longest sequence (which sends batches of short
sequences to the chunked form). Both paths are reached; test_path_mix checks that they are. Tolerances as in
test_gpu_gated_delta: out |err| <= 2^-7 |ref| + 1e-4, final state |err| <= 1e-4 + 1e-4 |ref|.
"""
import numpy as np
import pytest

import oracle
import varlen_flash_attention_amd as vfa
from varlen_flash_attention_amd.workloads import make_gated_delta
from tests.gpu_util import dev_array, host64, need_gpu
from tests.test_gpu_gated_delta import check_close

N_CASES = 24
TOKEN_BY_TOKEN_MAX = 16   # max_seqlen up to which the entry point runs the token-by-token kernel


def draw_case(i):
    rng = np.random.default_rng(7300 + i)
    b = int(rng.integers(1, 11))
    pick = rng.random(b)
    lens = np.where(pick < 0.1, 0, np.where(pick < 0.4, rng.integers(1, 17, b),
                                            np.where(pick < 0.9, rng.integers(17, 201, b), rng.integers(201, 401, b))))
    if i % 3 == 0:   # a decode-like batch: every sequence within the token-by-token limit
        lens = rng.integers(0, 17, b)
    lens = [int(x) for x in lens]
    hqk = int(rng.integers(1, 5))
    hv = hqk * int(rng.choice([1, 2, 4]))
    dk = int(rng.choice([64, 128]))
    dv = int(rng.choice([64, 128]))
    with_init = bool(rng.integers(2))
    ms = max(lens) if lens else 0
    if rng.random() < 0.2:
        ms += int(rng.integers(1, 300))
    return dict(lens=lens, hqk=hqk, hv=hv, dk=dk, dv=dv, with_init=with_init, max_seqlen=ms, seed=7400 + i)


def test_path_mix():
    paths = {"token" if draw_case(i)["max_seqlen"] <= TOKEN_BY_TOKEN_MAX else "chunked" for i in range(N_CASES)}
    assert paths == {"token", "chunked"}, paths


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES))
def test_gated_delta_random_shape(i):
    torch = need_gpu()
    c = draw_case(i)
    name = (f"gated_delta random case {i}: seed={c['seed']} lengths={c['lens']} Hqk={c['hqk']} Hv={c['hv']} "
            f"Dk={c['dk']} Dv={c['dv']} init={c['with_init']} max_seqlen={c['max_seqlen']}")
    print(f"[case] {name}", flush=True)
    p = make_gated_delta(c["lens"], c["hqk"], c["hv"], c["dk"], c["dv"], seed=c["seed"])
    x = dict(q=dev_array(p.q, "bf16"), k=dev_array(p.k, "bf16"), v=dev_array(p.v, "bf16"),
             g=torch.from_numpy(p.g).cuda(), beta=torch.from_numpy(p.beta).cuda(),
             cu=torch.from_numpy(p.cu_seqlens).cuda())
    s0 = s0_dev = None
    if c["with_init"]:
        s0 = (np.random.default_rng(c["seed"] + 1).standard_normal((len(c["lens"]), c["hv"], c["dk"], c["dv"]))
              .astype(np.float32) * 0.5)
        s0_dev = torch.from_numpy(s0).cuda()
    out, fin = vfa.gated_delta_rule_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu"], c["max_seqlen"],
                                        scale=p.scale, initial_state=s0_dev, output_final_state=True)
    torch.cuda.synchronize()
    o_ref, f_ref = oracle.gated_delta_rule(p.q, p.k, p.v, p.g, p.beta, p.cu_seqlens, p.scale, initial_state=s0)
    check_close(f"random{i}_out", host64(out), o_ref, 2.0 ** -7, 1e-4)
    check_close(f"random{i}_state", host64(fin), f_ref, 1e-4, 1e-4)
