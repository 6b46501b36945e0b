"""The Python binding rejects caller-supplied outputs of the wrong shape or dtype, and weights of the
wrong length, before any launch (the kernels touch exactly the shapes they are given pointers for)."""
import numpy as np
import pytest

import varlen_flash_attention_amd as vfa
from tests.gpu_util import need_gpu

pytestmark = pytest.mark.gpu


def test_outputs_of_wrong_shape_or_dtype_are_rejected():
    torch = need_gpu()
    dev = "cuda"
    bf, f32 = torch.bfloat16, torch.float32
    cu = torch.tensor([0, 3, 8], dtype=torch.int32, device=dev)
    q = torch.zeros((8, 4, 128), dtype=bf, device=dev)
    kv = torch.zeros((8, 2, 128), dtype=bf, device=dev)
    with pytest.raises(ValueError):
        vfa.varlen_attn_fwd(q, kv, kv, cu, cu, 5, 5, out=torch.empty((7, 4, 128), dtype=bf, device=dev))
    with pytest.raises(TypeError):
        vfa.varlen_attn_fwd(q, kv, kv, cu, cu, 5, 5, lse=torch.empty((8, 4), dtype=bf, device=dev))
    with pytest.raises(ValueError):
        vfa.varlen_attn_fwd(q, kv, kv, cu, cu, 5, 5, lse=torch.empty((8, 3), dtype=f32, device=dev))
    lse = torch.zeros((2, 16), dtype=f32, device=dev)
    go = torch.zeros((2, 16, 128), dtype=f32, device=dev)
    with pytest.raises(ValueError):
        vfa.attn_update(lse, go, out=torch.empty((16, 64), dtype=f32, device=dev))
    with pytest.raises(TypeError):
        vfa.attn_update(lse, go, out=torch.empty((16, 128), dtype=bf, device=dev))
    with pytest.raises(ValueError):
        vfa.attn_update(lse, go, lse_out=torch.empty((15,), dtype=f32, device=dev))
    with pytest.raises(ValueError):
        vfa.varlen_last_token_gather(q, cu, out=torch.empty((3, 4, 128), dtype=bf, device=dev))
    w = torch.ones((128,), dtype=bf, device=dev)
    cs = torch.zeros((8, 128), dtype=f32, device=dev)
    with pytest.raises(ValueError):
        vfa.qk_norm_rope(q, kv, w, w, cs, cs, q_out=torch.empty((8, 2, 128), dtype=bf, device=dev))
    with pytest.raises(ValueError):
        vfa.qk_norm_rope(q, kv, w[:64], w, cs, cs)
    g = torch.zeros((8, 4), dtype=f32, device=dev)
    gk = torch.zeros((8, 2, 128), dtype=bf, device=dev)
    with pytest.raises(ValueError):
        vfa.gated_delta_rule_fwd(gk, gk, q, g, g, cu, 5, out=torch.empty((8, 4, 64), dtype=bf, device=dev))
    with pytest.raises(TypeError):
        vfa.gated_delta_rule_fwd(gk, gk, q, g, g, cu, 5, out=torch.empty((8, 4, 128), dtype=f32, device=dev))
    torch.cuda.synchronize()


def test_bad_workspaces_are_rejected():
    # The split kernels write the whole planned workspace through its pointer, so a caller's workspace
    # must be a contiguous 1-D uint8 tensor on the call's GPU that holds the planned bytes.
    torch = need_gpu()
    dev = "cuda"
    bf = torch.bfloat16
    q = torch.zeros((2, 8, 128), dtype=bf, device=dev)
    kv = torch.zeros((1200, 2, 128), dtype=bf, device=dev)
    cu_q = torch.tensor([0, 1, 2], dtype=torch.int32, device=dev)
    cu_k = torch.tensor([0, 600, 1200], dtype=torch.int32, device=dev)
    need = vfa.varlen_attn_fwd_workspace_size(2, 2, 1, 600, 8, 2, 128)
    assert need > 0
    bad = [
        (torch.empty(need, dtype=torch.uint8), ValueError),                          # host memory
        (torch.empty(need // 4 + 1, dtype=torch.float32, device=dev), TypeError),    # not bytes
        (torch.empty(1, dtype=torch.uint8, device=dev).expand(need), ValueError),    # one byte, viewed as many
        (torch.empty((2, need), dtype=torch.uint8, device=dev), ValueError),         # not 1-D
        (torch.empty(need - 1, dtype=torch.uint8, device=dev), ValueError),          # too small
    ]
    for ws, exc in bad:
        with pytest.raises(exc):
            vfa.varlen_attn_fwd(q, kv, kv, cu_q, cu_k, 1, 600, workspace=ws)
    # paged: 16-key pages, 2 x 38 pages; 600 keys split in several parts need a workspace too
    cache = torch.zeros((80, 16, 2, 128), dtype=bf, device=dev)
    table = torch.arange(80, dtype=torch.int32, device=dev).reshape(2, 40)
    used = torch.tensor([600, 600], dtype=torch.int32, device=dev)
    need_p = vfa.paged_attn_decode_workspace_size(2, 2, 1, 600, 8, 2, 128)
    assert need_p > 0
    for ws, exc in ((torch.empty(need_p, dtype=torch.uint8), ValueError),
                    (torch.empty(need_p - 1, dtype=torch.uint8, device=dev), ValueError)):
        with pytest.raises(exc):
            vfa.paged_attn_decode(q, cache, cache, table, cu_q, used, 1, 600, workspace=ws)
    # a valid caller workspace is used as given
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    vfa.varlen_attn_fwd(q, kv, kv, cu_q, cu_k, 1, 600, workspace=ws)
    torch.cuda.synchronize()


def test_tensors_on_the_host_are_rejected():
    torch = need_gpu()
    bf = torch.bfloat16
    q = torch.zeros((8, 4, 128), dtype=bf, device="cuda")
    kv = torch.zeros((8, 2, 128), dtype=bf, device="cuda")
    cu = torch.tensor([0, 3, 8], dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        vfa.varlen_attn_fwd(q, kv.cpu(), kv, cu, cu, 5, 5)
    with pytest.raises(ValueError):
        vfa.varlen_attn_fwd(q, kv, kv, cu.cpu(), cu, 5, 5)
    with pytest.raises(ValueError):
        vfa.varlen_attn_fwd(q, kv, kv, cu, cu, 5, 5, lse=torch.empty((8, 4), dtype=torch.float32))
    lse = torch.zeros((2, 16), dtype=torch.float32, device="cuda")
    go = torch.zeros((2, 16, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        vfa.attn_update(lse.cpu(), go)
