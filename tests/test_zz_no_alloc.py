"""GPU: varlen_attn_fwd_noalloc (through the C ABI) against varlen_attn_fwd with a caller workspace.

The allocation-free entry point runs the same kernels, with the split-KV partials in the library's
static per-device array instead of a workspace. Two calls in a row share that array: the first on the
full decode workload (8.5 MB of partials), the second on a smaller decode input, so the second runs on
what the first left behind. Each must equal the workspace entry point's result bit for bit (a stronger
bar than the oracle tolerance), and the smaller one is also checked against the fp64 oracle. A prefill
call (no split, no scratch) goes through the same entry point.
"""
import numpy as np
import pytest

import oracle
import varlen_flash_attention_amd as vfa
from varlen_flash_attention_amd.workloads import make_custom, make_workload
from tests.gpu_util import check, host64, need_gpu, to_device

pytestmark = pytest.mark.gpu


def _both(w):
    torch = need_gpu()
    d = to_device(w)
    tq, hq, dd = w.total_q, w.num_heads_q, w.head_dim
    need = vfa.varlen_attn_fwd_workspace_size(w.batch, tq, w.max_seqlen_q, w.max_seqlen_k, hq, w.num_heads_kv, dd)
    assert need <= vfa.STATIC_SCRATCH_BYTES
    # the workspace entry point, with a junk-filled workspace of exactly the planned size
    ws = torch.full((max(need, 1),), 0x5A, dtype=torch.uint8, device="cuda")
    o_ref, l_ref = vfa.varlen_attn_fwd(d["q"], d["k"], d["v"], d["cu_q"], d["cu_k"], w.max_seqlen_q,
                                       w.max_seqlen_k, softmax_scale=w.scale, causal=w.causal, workspace=ws)
    out = torch.full((tq, hq, dd), 3.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((tq, hq), 3.0, dtype=torch.float32, device="cuda")
    vfa.varlen_attn_fwd_noalloc(d["q"], d["k"], d["v"], d["cu_q"], d["cu_k"], w.max_seqlen_q, w.max_seqlen_k,
                                out, lse, softmax_scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    return need, out, lse, o_ref, l_ref


def test_noalloc_matches_workspace_entry_point_twice():
    torch = need_gpu()
    big = make_workload("decode")
    print(f"[case] noalloc call 1: decode workload B={big.batch} Tk={big.total_k}", flush=True)
    need, out, lse, o_ref, l_ref = _both(big)
    assert need > 0
    assert torch.equal(out, o_ref) and torch.equal(lse, l_ref), "call 1: noalloc differs from varlen_attn_fwd"

    rng = np.random.default_rng(7)
    small = make_custom(np.ones(8, dtype=np.int64), rng.integers(600, 5000, 8), num_heads_q=32, num_heads_kv=4,
                        head_dim=128, dtype="bf16", causal=True, seed=8, name="decode_small_noalloc")
    print(f"[case] noalloc call 2: smaller decode B={small.batch} Tk={small.total_k}", flush=True)
    need2, out2, lse2, o_ref2, l_ref2 = _both(small)
    assert 0 < need2 < need
    assert torch.equal(out2, o_ref2) and torch.equal(lse2, l_ref2), "call 2: noalloc differs from varlen_attn_fwd"
    o_or, l_or = oracle.varlen_attention_rows(small.q, small.k, small.v, small.cu_seqlens_q, small.cu_seqlens_k,
                                              small.num_heads_kv, small.scale, True)
    check("noalloc small decode vs oracle", host64(out2), host64(lse2), o_or, l_or, "bf16")


def test_noalloc_prefill():
    torch = need_gpu()
    w = make_custom([130, 64, 1, 257], num_heads_q=8, num_heads_kv=2, head_dim=128, dtype="bf16", causal=True,
                    seed=9)
    print("[case] noalloc prefill (no scratch)", flush=True)
    need, out, lse, o_ref, l_ref = _both(w)
    assert need == 0
    assert torch.equal(out, o_ref) and torch.equal(lse, l_ref)


def test_noalloc_long_prefill_counters_twice():
    """Long-sequence prefill keeps its 1 KB of work counters in the static array: two calls in a row (the
    second smaller, on the counters the first left behind) must each equal the workspace entry point."""
    torch = need_gpu()
    for name, lengths, seed in (("call 1", [1300, 513, 1029, 77, 700, 1500], 31), ("call 2", [900, 640, 33], 32)):
        w = make_custom(lengths, num_heads_q=32, num_heads_kv=8, head_dim=128, dtype="bf16", causal=True, seed=seed)
        assert w.total_q // w.batch >= 8 * (256 // 4)    # the persistent long-prefill kernel
        print(f"[case] noalloc long prefill {name}: lengths {lengths}", flush=True)
        need, out, lse, o_ref, l_ref = _both(w)
        assert need == 1024
        assert torch.equal(out, o_ref) and torch.equal(lse, l_ref), f"{name}: noalloc differs from varlen_attn_fwd"


def test_noalloc_under_graph_capture():
    """The callers this entry point is for: a decode call (partials in the static array) and a long-prefill call
    (work counters in it) captured into one HIP graph; three replays, with eager work on the outputs and elsewhere
    between them, each equal the eager result bit for bit."""
    torch = need_gpu()
    print("[case] noalloc under graph capture: decode workload and long prefill", flush=True)
    wd = make_workload("decode")
    wl = make_custom([1300, 513, 1029, 77, 700, 1500], num_heads_q=32, num_heads_kv=8, head_dim=128, dtype="bf16",
                     causal=True, seed=33)
    calls = []
    for w in (wd, wl):
        d = to_device(w)
        out = torch.empty((w.total_q, w.num_heads_q, w.head_dim), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((w.total_q, w.num_heads_q), dtype=torch.float32, device="cuda")
        calls.append((w, d, out, lse))

    def run_all():
        for w, d, out, lse in calls:
            vfa.varlen_attn_fwd_noalloc(d["q"], d["k"], d["v"], d["cu_q"], d["cu_k"], w.max_seqlen_q,
                                        w.max_seqlen_k, out, lse, softmax_scale=w.scale, causal=w.causal)

    run_all()
    torch.cuda.synchronize()
    ref = [(out.clone(), lse.clone()) for _, _, out, lse in calls]
    side = torch.cuda.Stream()                                 # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_all()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_all()
    for rep in range(3):
        for _, _, out, lse in calls:
            out.zero_()
            lse.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert float(junk) == float(junk)
        for i, ((_, _, out, lse), (o_ref, l_ref)) in enumerate(zip(calls, ref)):
            assert torch.equal(out, o_ref) and torch.equal(lse, l_ref), f"replay {rep}: call {i} differs"
