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
