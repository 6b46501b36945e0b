"""GPU: the VFA_DEBUG device check of the cu_seqlens contract (TND layout: "From GPU to NPU:
Qwen3-Embedding on Ascend", core optimisation 1). Every case below only makes the check kernel
read cu_seqlens; a violation must be reported before any attention kernel is launched."""
import numpy as np
import pytest

import varlen_flash_attention_amd as vfa
from tests.gpu_util import need_gpu

pytestmark = pytest.mark.gpu


def _inputs(torch, total, hq=4, hkv=2, d=64):
    g = torch.Generator(device="cuda").manual_seed(0)
    q = torch.randn((total, hq, d), device="cuda", generator=g).to(torch.bfloat16)
    k = torch.randn((total, hkv, d), device="cuda", generator=g).to(torch.bfloat16)
    v = torch.randn((total, hkv, d), device="cuda", generator=g).to(torch.bfloat16)
    return q, k, v


def _cu(torch, xs):
    return torch.tensor(xs, dtype=torch.int32, device="cuda")


def test_debug_check_passes_a_valid_call(monkeypatch):
    torch = need_gpu()
    q, k, v = _inputs(torch, 20)
    cu = _cu(torch, [0, 12, 20])
    print("[case] VFA_DEBUG valid call", flush=True)
    ref_o, ref_l = vfa.varlen_attn_fwd(q, k, v, cu, cu, 12, 12)
    monkeypatch.setenv("VFA_DEBUG", "1")
    o, l = vfa.varlen_attn_fwd(q, k, v, cu, cu, 12, 12)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l)


@pytest.mark.parametrize("cu_q,max_q,why", [
    ([1, 12, 20], 12, "cu[0] != 0"),
    ([0, 14, 12, 20], 14, "decreasing entries"),
    ([0, 12, 19], 12, "cu[batch] != total_q"),
    ([0, 14, 20], 12, "a length above max_seqlen_q"),
])
def test_debug_check_rejects_contract_violations(monkeypatch, cu_q, max_q, why):
    torch = need_gpu()
    q, k, v = _inputs(torch, 20)
    cu_k = _cu(torch, [0, 12, 20] if len(cu_q) == 3 else [0, 6, 12, 20])
    monkeypatch.setenv("VFA_DEBUG", "1")
    out = torch.full((20, 4, 64), 7.0, device="cuda").to(torch.bfloat16)
    print(f"[case] VFA_DEBUG rejects {why}", flush=True)
    with pytest.raises(vfa.VfaError) as e:
        vfa.varlen_attn_fwd(q, k, v, _cu(torch, cu_q), cu_k, max_q, 14, out=out)
    assert e.value.status == 2
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())            # nothing was launched


def test_debug_check_gather(monkeypatch):
    torch = need_gpu()
    x = torch.randn((20, 8), device="cuda")
    monkeypatch.setenv("VFA_DEBUG", "1")
    print("[case] VFA_DEBUG gather", flush=True)
    got = vfa.varlen_last_token_gather(x, _cu(torch, [0, 5, 20]))
    torch.cuda.synchronize()
    assert torch.equal(got, x[[4, 19]])
    with pytest.raises(vfa.VfaError) as e:
        vfa.varlen_last_token_gather(x, _cu(torch, [0, 9, 5]))
    assert e.value.status == 2


def test_debug_check_refused_under_graph_capture(monkeypatch):
    # The check synchronises its stream, which graph capture forbids: a checked call on a capturing
    # stream returns VFA_ERR_UNSUPPORTED before touching the stream, and the capture stays usable.
    torch = need_gpu()
    q, k, v = _inputs(torch, 20)
    cu = _cu(torch, [0, 12, 20])
    out = torch.empty((20, 4, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((20, 4), dtype=torch.float32, device="cuda")
    ref_o, ref_l = vfa.varlen_attn_fwd(q, k, v, cu, cu, 12, 12)
    torch.cuda.synchronize()
    print("[case] VFA_DEBUG under graph capture", flush=True)
    monkeypatch.setenv("VFA_DEBUG", "1")
    g = torch.cuda.CUDAGraph()
    status = None
    with torch.cuda.graph(g):
        try:
            vfa.varlen_attn_fwd(q, k, v, cu, cu, 12, 12, out=out, lse=lse)
        except vfa.VfaError as e:
            status = e.status
        monkeypatch.setenv("VFA_DEBUG", "0")
        vfa.varlen_attn_fwd(q, k, v, cu, cu, 12, 12, out=out, lse=lse)   # unchecked: captured as usual
    assert status == 3
    out.zero_()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
