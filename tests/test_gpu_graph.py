"""HIP graph capture: the entry points launch kernels only (no allocation, host synchronisation or
memset inside the library), so a caller can capture them into a graph and replay it.

One graph holds a prefill call, a split-KV decode call (split + combine kernels), an attn_update merge,
a paged decode call, the q/k RMSNorm + rotary prologue and two gated delta rule calls (the chunked form's
two kernels, and the token-by-token kernel). It is replayed three times with unrelated
eager work in between, and every replay must equal the eager results bit for bit (the kernels are
deterministic)."""
import numpy as np
import pytest

import varlen_flash_attention_amd as vfa
from varlen_flash_attention_amd.workloads import make_custom, make_gated_delta, make_paged, make_prologue
from tests.gpu_util import dev_array, need_gpu, to_device

pytestmark = pytest.mark.gpu


def test_graph_capture_and_replay(monkeypatch):
    torch = need_gpu()
    monkeypatch.delenv("VFA_DEBUG", raising=False)          # the debug check synchronises: not capturable
    print("[case] graph capture of short and long prefill, decode, merge, paged decode, prologue and gated delta rule",
          flush=True)
    wp = make_custom([300, 77, 513], num_heads_q=32, num_heads_kv=8, head_dim=128, dtype="bf16", causal=True, seed=120)
    # long-sequence prefill: the persistent kernel, whose work counters a kernel (not a memset) clears per call
    wl = make_custom([1300, 513, 1029, 77, 700, 1500], num_heads_q=32, num_heads_kv=8, head_dim=128, dtype="bf16",
                     causal=True, seed=125)
    assert wl.total_q // wl.batch >= 8 * (256 // 4)
    wd = make_custom([1] * 4, [5000, 300, 9000, 70], num_heads_q=32, num_heads_kv=4, head_dim=128, dtype="bf16",
                     causal=True, seed=121)
    pc = make_paged(wd, 16, seed=12)
    pro = make_prologue([50, 300], 32, 8, 128, seed=122)
    dp, dd, dl = to_device(wp), to_device(wd), to_device(wl)
    kc, vc = dev_array(pc.k_cache, "bf16"), dev_array(pc.v_cache, "bf16")
    table, used = torch.from_numpy(pc.block_table).cuda(), torch.from_numpy(pc.seqused_k).cuda()
    rng = np.random.default_rng(123)
    lse_p = torch.from_numpy(rng.normal(0, 2, (4, 512)).astype(np.float32)).cuda()
    go = torch.from_numpy(rng.standard_normal((4, 512, 128)).astype(np.float32)).cuda()
    pq, pk = dev_array(pro.q, "bf16"), dev_array(pro.k, "bf16")
    pwq, pwk = dev_array(pro.q_weight, "bf16"), dev_array(pro.k_weight, "bf16")
    cos, sin = torch.from_numpy(pro.cos).cuda(), torch.from_numpy(pro.sin).cuda()
    gd = make_gated_delta([130, 9, 64], 2, 4, 128, 128, seed=124)
    gx = dict(q=dev_array(gd.q, "bf16"), k=dev_array(gd.k, "bf16"), v=dev_array(gd.v, "bf16"),
              g=torch.from_numpy(gd.g).cuda(), beta=torch.from_numpy(gd.beta).cuda(),
              cu=torch.from_numpy(gd.cu_seqlens).cuda())
    gs0 = torch.from_numpy(rng.standard_normal((3, 4, 128, 128)).astype(np.float32)).cuda()
    short = torch.arange(130, 139, device="cuda")                 # the 9-token sequence alone
    gshort = {n: gx[n][short].contiguous() for n in ("q", "k", "v", "g", "beta")}
    gcu_short = torch.tensor([0, 9], dtype=torch.int32, device="cuda")

    def run_all():
        return (
            *vfa.varlen_attn_fwd(dp["q"], dp["k"], dp["v"], dp["cu_q"], dp["cu_k"], wp.max_seqlen_q, wp.max_seqlen_k,
                                 softmax_scale=wp.scale, causal=True),
            *vfa.varlen_attn_fwd(dd["q"], dd["k"], dd["v"], dd["cu_q"], dd["cu_k"], wd.max_seqlen_q, wd.max_seqlen_k,
                                 softmax_scale=wd.scale, causal=True),
            *vfa.varlen_attn_fwd(dl["q"], dl["k"], dl["v"], dl["cu_q"], dl["cu_k"], wl.max_seqlen_q, wl.max_seqlen_k,
                                 softmax_scale=wl.scale, causal=True),
            *vfa.attn_update(lse_p, go, update_type=1),
            *vfa.paged_attn_decode(dd["q"], kc, vc, table, dd["cu_q"], used, wd.max_seqlen_q, wd.max_seqlen_k,
                                   softmax_scale=wd.scale, causal=True),
            *vfa.qk_norm_rope(pq, pk, pwq, pwk, cos, sin, eps=pro.eps),
            *vfa.gated_delta_rule_fwd(gx["q"], gx["k"], gx["v"], gx["g"], gx["beta"], gx["cu"], 130,
                                      scale=gd.scale, initial_state=gs0, output_final_state=True),
            *vfa.gated_delta_rule_fwd(gshort["q"], gshort["k"], gshort["v"], gshort["g"], gshort["beta"], gcu_short,
                                      9, scale=gd.scale, initial_state=gs0[1:2].contiguous(),
                                      output_final_state=True),
        )

    ref = [t.clone() for t in run_all()]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()                               # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_all()                                            # warm-up on the side stream, as torch recommends
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = run_all()
    for rep in range(3):
        for t in outs:
            t.zero_()                                        # eager work between replays, on the graph's outputs
        junk = torch.randn(1 << 20, device="cuda").sum()     # and unrelated eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert float(junk) == float(junk)
        for i, (a, b) in enumerate(zip(outs, ref)):
            assert torch.equal(a, b), f"replay {rep}: output {i} differs from the eager result"
    print("[graph] 3 replays equal the eager results", flush=True)
