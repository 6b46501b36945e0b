"""varlen_flash_attention_amd -- varlen attention and the AttentionUpdate merge on MI355X.

A thin ctypes binding over libvfa.so, the C-ABI library built from csrc/
(HIP kernels for gfx950). The functions here only marshal arguments: they
check that tensors are on the GPU, contiguous and of a supported dtype,
allocate outputs (and workspace) with torch on the tensors' device, pass the
current HIP stream, and raise VfaError on a non-zero status. Every step of
the computation runs in the library's kernels; there is no CPU fallback. If
the library has not been built the first call raises.

Entry points (same names as the C ABI in include/vfa.h):
  varlen_attn_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                  softmax_scale=None, causal=True, out_dtype=None, causal_offset=None) -> (out, lse)
      (with causal_offset given: the C entry point varlen_attn_fwd_offset)
  varlen_attn_fwd_noalloc(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, out, lse,
                          softmax_scale=None, causal=True) -> (out, lse)
      (no workspace: split-KV partials in the library's static per-device array)
  attn_update(lse, go, update_type=1) -> (out, lse_out or None)
  varlen_last_token_gather(x, cu_seqlens) -> x[cu_seqlens[1:] - 1]
  varlen_attn_fwd_workspace_size(...) -> bytes
  paged_attn_decode(q, k_cache, v_cache, block_table, cu_seqlens_q, seqused_k, max_seqlen_q,
                    max_seqlen_k, softmax_scale=None, causal=True, out_dtype=None) -> (out, lse)
  paged_attn_decode_workspace_size(...) -> bytes
  qk_norm_rope(q, k, q_weight, k_weight, cos, sin, eps=1e-6, q_out=None, k_out=None) -> (q_out, k_out)
  gated_delta_rule_fwd(q, k, v, g, beta, cu_seqlens, max_seqlen, scale=None, initial_state=None,
                       output_final_state=False, out=None) -> (out, final_state or None)
  gated_delta_rule_fwd_workspace_size(total_tokens, num_heads_v, max_seqlen) -> bytes
"""
from __future__ import annotations

import ctypes
import math
import os
import re

__all__ = [
    "VfaError",
    "library_path",
    "load_library",
    "abi_version",
    "status_string",
    "varlen_attn_fwd",
    "varlen_attn_fwd_workspace_size",
    "varlen_attn_fwd_noalloc",
    "STATIC_SCRATCH_BYTES",
    "attn_update",
    "varlen_last_token_gather",
    "paged_attn_decode",
    "paged_attn_decode_workspace_size",
    "qk_norm_rope",
    "gated_delta_rule_fwd",
    "gated_delta_rule_fwd_workspace_size",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_HEADER = os.path.join(os.path.dirname(_PKG), "include", "vfa.h")
_LIB = None

VFA_F32 = 0
VFA_BF16 = 1


class VfaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = int(status)
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def library_path() -> str:
    return os.path.join(_PKG, "libvfa.so")


def _header_abi_version() -> int:
    with open(_HEADER) as fh:
        m = re.search(r"#define\s+VFA_ABI_VERSION\s+(\d+)", fh.read())
    if not m:
        raise RuntimeError("VFA_ABI_VERSION not found in include/vfa.h")
    return int(m.group(1))


def load_library() -> ctypes.CDLL:
    """Load libvfa.so by absolute path and check its ABI version against the header."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m varlen_flash_attention_amd.build`")
    lib = ctypes.CDLL(path)
    c = ctypes
    lib.vfa_abi_version.restype = c.c_int32
    lib.vfa_abi_version.argtypes = []
    lib.vfa_status_string.restype = c.c_char_p
    lib.vfa_status_string.argtypes = [c.c_int32]
    lib.varlen_attn_fwd_workspace_size.restype = c.c_size_t
    lib.varlen_attn_fwd_workspace_size.argtypes = [c.c_int32] * 7
    lib.varlen_attn_fwd.restype = c.c_int32
    lib.varlen_attn_fwd.argtypes = [
        c.c_void_p, c.c_void_p, c.c_void_p, c.c_int32,          # q k v in_dtype
        c.c_void_p, c.c_void_p,                                 # cu_q cu_k
        c.c_int32, c.c_int32, c.c_int32, c.c_int32, c.c_int32,  # batch total_q total_k max_q max_k
        c.c_int32, c.c_int32, c.c_int32,                        # hq hkv d
        c.c_float, c.c_int32,                                   # scale causal
        c.c_void_p, c.c_int32, c.c_void_p,                      # out out_dtype lse
        c.c_void_p, c.c_size_t, c.c_void_p,                     # workspace bytes stream
    ]
    lib.varlen_attn_fwd_offset.restype = c.c_int32
    lib.varlen_attn_fwd_offset.argtypes = [
        c.c_void_p, c.c_void_p, c.c_void_p, c.c_int32,          # q k v in_dtype
        c.c_void_p, c.c_void_p, c.c_void_p,                     # cu_q cu_k causal_offset
        c.c_int32, c.c_int32, c.c_int32, c.c_int32, c.c_int32,  # batch total_q total_k max_q max_k
        c.c_int32, c.c_int32, c.c_int32,                        # hq hkv d
        c.c_float, c.c_int32,                                   # scale causal
        c.c_void_p, c.c_int32, c.c_void_p,                      # out out_dtype lse
        c.c_void_p, c.c_size_t, c.c_void_p,                     # workspace bytes stream
    ]
    lib.varlen_attn_fwd_noalloc.restype = c.c_int32
    lib.varlen_attn_fwd_noalloc.argtypes = [
        c.c_void_p, c.c_void_p, c.c_void_p, c.c_int32,          # q k v in_dtype
        c.c_void_p, c.c_void_p,                                 # cu_q cu_k
        c.c_int32, c.c_int32, c.c_int32, c.c_int32, c.c_int32,  # batch total_q total_k max_q max_k
        c.c_int32, c.c_int32, c.c_int32,                        # hq hkv d
        c.c_float, c.c_int32,                                   # scale causal
        c.c_void_p, c.c_int32, c.c_void_p,                      # out out_dtype lse
        c.c_void_p,                                             # stream
    ]
    lib.attn_update.restype = c.c_int32
    lib.attn_update.argtypes = [c.c_void_p, c.c_void_p, c.c_int32, c.c_int32, c.c_int64, c.c_int32,
                                c.c_int32, c.c_void_p, c.c_void_p, c.c_void_p]
    lib.varlen_last_token_gather.restype = c.c_int32
    lib.varlen_last_token_gather.argtypes = [c.c_void_p, c.c_int32, c.c_void_p, c.c_int32, c.c_int64,
                                             c.c_void_p, c.c_void_p]
    lib.paged_attn_decode_workspace_size.restype = c.c_size_t
    lib.paged_attn_decode_workspace_size.argtypes = [c.c_int32] * 7
    lib.paged_attn_decode.restype = c.c_int32
    lib.paged_attn_decode.argtypes = [
        c.c_void_p, c.c_int32, c.c_void_p, c.c_void_p,          # q in_dtype k_cache v_cache
        c.c_void_p, c.c_int32, c.c_int32, c.c_int32,            # block_table max_pages num_pages page_size
        c.c_void_p, c.c_void_p,                                 # cu_q seqused_k
        c.c_int32, c.c_int32, c.c_int32, c.c_int32,             # batch total_q max_q max_k
        c.c_int32, c.c_int32, c.c_int32,                        # hq hkv d
        c.c_float, c.c_int32,                                   # scale causal
        c.c_void_p, c.c_int32, c.c_void_p,                      # out out_dtype lse
        c.c_void_p, c.c_size_t, c.c_void_p,                     # workspace bytes stream
    ]
    lib.qk_norm_rope.restype = c.c_int32
    lib.qk_norm_rope.argtypes = [c.c_void_p, c.c_void_p, c.c_int32, c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p,
                                 c.c_int32, c.c_int32, c.c_int32, c.c_int32, c.c_float, c.c_void_p, c.c_void_p,
                                 c.c_void_p]
    lib.gated_delta_rule_fwd.restype = c.c_int32
    lib.gated_delta_rule_fwd.argtypes = [c.c_void_p, c.c_void_p, c.c_void_p, c.c_int32, c.c_void_p, c.c_void_p,
                                         c.c_void_p, c.c_int32, c.c_int32, c.c_int32, c.c_int32, c.c_int32,
                                         c.c_int32, c.c_int32, c.c_float, c.c_void_p, c.c_void_p, c.c_void_p,
                                         c.c_void_p, c.c_int64, c.c_void_p]
    lib.gated_delta_rule_fwd_workspace_size.restype = c.c_int64
    lib.gated_delta_rule_fwd_workspace_size.argtypes = [c.c_int32, c.c_int32, c.c_int32]
    got, want = lib.vfa_abi_version(), _header_abi_version()
    if got != want:
        raise RuntimeError(f"{path} has ABI version {got}, include/vfa.h expects {want}: stale library")
    _LIB = lib
    return lib


def abi_version() -> int:
    return int(load_library().vfa_abi_version())


def status_string(status: int) -> str:
    try:
        return load_library().vfa_status_string(int(status)).decode()
    except Exception:  # noqa: BLE001 - used while formatting an error
        return "status"


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return VFA_F32
    if t.dtype == torch.bfloat16:
        return VFA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16")


def _check_gpu(name, t, ndim=None, device=None):
    """A tensor the kernels read or write: on the GPU (on `device` when given: one call runs on one
    device), contiguous, and of `ndim` dimensions when given."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (libvfa has no CPU path)")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the call runs on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {t.dim()}")


def _check_out(name, t, shape, dtype=None, device=None):
    """A caller-supplied output: on the call's GPU, contiguous, of exactly the shape (and dtype) the
    kernel writes, so that no launch writes past its end."""
    _check_gpu(name, t, len(shape), device)
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _workspace(workspace, need: int, device):
    """The split kernels' partials buffer: None when the call needs none; a fresh uint8 buffer when the
    caller gives none; else the caller's, which must be a contiguous 1-D uint8 tensor on the call's
    device holding at least `need` bytes (the kernels write up to `need` bytes through its pointer)."""
    torch = _torch()
    if need <= 0:
        return None
    if workspace is None:
        return torch.empty(need, dtype=torch.uint8, device=device)
    _check_gpu("workspace", workspace, 1, device)
    if workspace.dtype != torch.uint8:
        raise TypeError(f"workspace must be uint8, got {workspace.dtype}")
    if workspace.numel() < need:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, the call needs {need}")
    return workspace


def _stream_ptr(device) -> int:
    torch = _torch()
    return int(torch.cuda.current_stream(device).cuda_stream)


def varlen_attn_fwd_workspace_size(batch, total_q, max_seqlen_q, max_seqlen_k, num_heads_q, num_heads_kv,
                                   head_dim) -> int:
    return int(load_library().varlen_attn_fwd_workspace_size(int(batch), int(total_q), int(max_seqlen_q),
                                                             int(max_seqlen_k), int(num_heads_q),
                                                             int(num_heads_kv), int(head_dim)))


def varlen_attn_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                    softmax_scale: float | None = None, causal: bool = True, out_dtype=None,
                    out=None, lse=None, workspace=None, causal_offset=None):
    """Attention over packed sequences (TND). Returns (out [Tq,Hq,D], lse [Tq,Hq] fp32).

    q [Tq, Hq, D], k / v [Tk, Hkv, D] (bf16 or fp32, same dtype); cu_seqlens_*
    int32 [B+1] on the GPU. max_seqlen_* are host upper bounds of the lengths.
    Default scale 1/sqrt(D); default out dtype = input dtype. causal_offset
    (int32 [B] on the GPU): query i of sequence b sees key j iff
    j <= i + causal_offset[b] (default Lk - Lq, bottom-right).
    """
    torch = _torch()
    lib = load_library()
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_gpu(name, t, 3, dev)
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        _check_gpu(name, t, 1, dev)
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    if q.shape[2] != k.shape[2]:
        raise ValueError("q and k must have the same head_dim")
    tq, hq, d = (int(x) for x in q.shape)
    tk, hkv = int(k.shape[0]), int(k.shape[1])
    batch = int(cu_seqlens_q.shape[0]) - 1
    if int(cu_seqlens_k.shape[0]) != batch + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    in_code = _dtype_code(q)
    odt = q.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((tq, hq, d), dtype=odt, device=q.device)
    _check_out("out", out, (tq, hq, d), None if out_dtype is None else odt, dev)
    out_code = _dtype_code(out)
    if lse is None:
        lse = torch.empty((tq, hq), dtype=torch.float32, device=q.device)
    _check_out("lse", lse, (tq, hq), torch.float32, dev)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    ws_bytes = varlen_attn_fwd_workspace_size(batch, tq, max_seqlen_q, max_seqlen_k, hq, hkv, d)
    workspace = _workspace(workspace, ws_bytes, dev)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    if causal_offset is None:
        st = lib.varlen_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), in_code,
                                 cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(),
                                 batch, tq, tk, int(max_seqlen_q), int(max_seqlen_k), hq, hkv, d,
                                 scale, 1 if causal else 0, out.data_ptr(), out_code, lse.data_ptr(),
                                 ws_ptr, ws_bytes, _stream_ptr(q.device))
        if st != 0:
            raise VfaError(st, "varlen_attn_fwd")
        return out, lse
    _check_gpu("causal_offset", causal_offset, 1, dev)
    if causal_offset.dtype != torch.int32 or int(causal_offset.shape[0]) != batch:
        raise ValueError("causal_offset must be int32 with one entry per sequence")
    st = lib.varlen_attn_fwd_offset(q.data_ptr(), k.data_ptr(), v.data_ptr(), in_code,
                                    cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), causal_offset.data_ptr(),
                                    batch, tq, tk, int(max_seqlen_q), int(max_seqlen_k), hq, hkv, d,
                                    scale, 1 if causal else 0, out.data_ptr(), out_code, lse.data_ptr(),
                                    ws_ptr, ws_bytes, _stream_ptr(q.device))
    if st != 0:
        raise VfaError(st, "varlen_attn_fwd_offset")
    return out, lse


STATIC_SCRATCH_BYTES = 16 << 20   # VFA_STATIC_SCRATCH_BYTES in include/vfa.h


def varlen_attn_fwd_noalloc(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int, out, lse,
                            softmax_scale: float | None = None, causal: bool = True):
    """varlen_attn_fwd for callers that cannot allocate: the caller passes out [Tq,Hq,D] and lse [Tq,Hq]
    fp32, and the split-KV partials of decode-shaped calls go to the library's static per-device array
    (STATIC_SCRATCH_BYTES), so nothing is allocated on the call. Calls that need more split-KV storage than
    the array holds raise VfaError (VFA_ERR_WORKSPACE); calls that overlap on one device race on the array."""
    torch = _torch()
    lib = load_library()
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_gpu(name, t, 3, dev)
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        _check_gpu(name, t, 1, dev)
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    if k.shape != v.shape or q.shape[2] != k.shape[2]:
        raise ValueError("k and v must have one shape, with q's head_dim")
    tq, hq, d = (int(x) for x in q.shape)
    tk, hkv = int(k.shape[0]), int(k.shape[1])
    batch = int(cu_seqlens_q.shape[0]) - 1
    if int(cu_seqlens_k.shape[0]) != batch + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    _check_out("out", out, (tq, hq, d), None, dev)
    _check_out("lse", lse, (tq, hq), torch.float32, dev)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    st = lib.varlen_attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q),
                                     cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(),
                                     batch, tq, tk, int(max_seqlen_q), int(max_seqlen_k), hq, hkv, d,
                                     scale, 1 if causal else 0, out.data_ptr(), _dtype_code(out), lse.data_ptr(),
                                     _stream_ptr(dev))
    if st != 0:
        raise VfaError(st, "varlen_attn_fwd_noalloc")
    return out, lse


def attn_update(lse, go, update_type: int = 1, out=None, lse_out=None):
    """Merge sp partials: lse [sp, bsh] fp32, go [sp, bsh, hd] -> (out [bsh, hd], lse_out [bsh] | None)."""
    torch = _torch()
    lib = load_library()
    _check_gpu("go", go, 3)
    _check_gpu("lse", lse, 2, go.device)
    if lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    sp, bsh = int(lse.shape[0]), int(lse.shape[1])
    if tuple(go.shape[:2]) != (sp, bsh):
        raise ValueError(f"go must be [sp, bsh, hd] = [{sp}, {bsh}, hd], got {tuple(go.shape)}")
    hd = int(go.shape[2])
    code = _dtype_code(go)
    if out is None:
        out = torch.empty((bsh, hd), dtype=go.dtype, device=go.device)
    _check_out("out", out, (bsh, hd), go.dtype, go.device)
    if update_type == 1 and lse_out is None:
        lse_out = torch.empty((bsh,), dtype=torch.float32, device=go.device)
    if update_type == 1:
        _check_out("lse_out", lse_out, (bsh,), torch.float32, go.device)
    st = lib.attn_update(lse.data_ptr(), go.data_ptr(), code, sp, bsh, hd, int(update_type), out.data_ptr(),
                         lse_out.data_ptr() if (update_type == 1 and lse_out is not None) else None,
                         _stream_ptr(go.device))
    if st != 0:
        raise VfaError(st, "attn_update")
    return out, (lse_out if update_type == 1 else None)


def varlen_last_token_gather(x, cu_seqlens, out=None):
    """x[cu_seqlens[1:] - 1] along dim 0 of a packed-token tensor (rows of empty sequences: zeros)."""
    torch = _torch()
    lib = load_library()
    _check_gpu("x", x)
    _check_gpu("cu_seqlens", cu_seqlens, 1, x.device)
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    batch = int(cu_seqlens.shape[0]) - 1
    row = 1
    for s in x.shape[1:]:
        row *= int(s)
    if out is None:
        out = torch.empty((batch, *x.shape[1:]), dtype=x.dtype, device=x.device)
    _check_out("out", out, (batch, *x.shape[1:]), x.dtype, x.device)
    st = lib.varlen_last_token_gather(x.data_ptr(), _dtype_code(x), cu_seqlens.data_ptr(), batch, row,
                                      out.data_ptr(), _stream_ptr(x.device))
    if st != 0:
        raise VfaError(st, "varlen_last_token_gather")
    return out


def paged_attn_decode_workspace_size(batch, total_q, max_seqlen_q, max_seqlen_k, num_heads_q, num_heads_kv,
                                     head_dim) -> int:
    return int(load_library().paged_attn_decode_workspace_size(int(batch), int(total_q), int(max_seqlen_q),
                                                               int(max_seqlen_k), int(num_heads_q),
                                                               int(num_heads_kv), int(head_dim)))


def paged_attn_decode(q, k_cache, v_cache, block_table, cu_seqlens_q, seqused_k, max_seqlen_q: int,
                      max_seqlen_k: int, softmax_scale: float | None = None, causal: bool = True,
                      out_dtype=None, out=None, lse=None, workspace=None):
    """Attention of packed queries against a paged K/V cache. Returns (out [Tq,Hq,D], lse [Tq,Hq] fp32).

    q [Tq, Hq, D] bf16; k_cache / v_cache [num_pages, page_size, Hkv, D] bf16;
    block_table int32 [B, max_pages]; cu_seqlens_q int32 [B+1]; seqused_k int32
    [B] (keys of each sequence). max_seqlen_* are host upper bounds. Default
    scale 1/sqrt(D); default out dtype = bf16.
    """
    torch = _torch()
    lib = load_library()
    dev = q.device
    _check_gpu("q", q, 3)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _check_gpu(name, t, 4, dev)
    _check_gpu("block_table", block_table, 2, dev)
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("seqused_k", seqused_k)):
        _check_gpu(name, t, 1, dev)
    for name, t in (("block_table", block_table), ("cu_seqlens_q", cu_seqlens_q), ("seqused_k", seqused_k)):
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q, k_cache and v_cache must share one dtype")
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    if q.shape[2] != k_cache.shape[3]:
        raise ValueError("q and k_cache must have the same head_dim")
    tq, hq, d = (int(x) for x in q.shape)
    num_pages, page_size, hkv = (int(x) for x in k_cache.shape[:3])
    batch = int(cu_seqlens_q.shape[0]) - 1
    if int(seqused_k.shape[0]) != batch or int(block_table.shape[0]) != batch:
        raise ValueError("seqused_k and block_table must have one entry / row per sequence")
    max_pages = int(block_table.shape[1])
    in_code = _dtype_code(q)
    odt = q.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((tq, hq, d), dtype=odt, device=q.device)
    _check_out("out", out, (tq, hq, d), None if out_dtype is None else odt, dev)
    if lse is None:
        lse = torch.empty((tq, hq), dtype=torch.float32, device=q.device)
    _check_out("lse", lse, (tq, hq), torch.float32, dev)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    ws_bytes = paged_attn_decode_workspace_size(batch, tq, max_seqlen_q, max_seqlen_k, hq, hkv, d)
    workspace = _workspace(workspace, ws_bytes, dev)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    st = lib.paged_attn_decode(q.data_ptr(), in_code, k_cache.data_ptr(), v_cache.data_ptr(),
                               block_table.data_ptr(), max_pages, num_pages, page_size,
                               cu_seqlens_q.data_ptr(), seqused_k.data_ptr(),
                               batch, tq, int(max_seqlen_q), int(max_seqlen_k), hq, hkv, d,
                               scale, 1 if causal else 0, out.data_ptr(), _dtype_code(out), lse.data_ptr(),
                               ws_ptr, ws_bytes, _stream_ptr(q.device))
    if st != 0:
        raise VfaError(st, "paged_attn_decode")
    return out, lse


def qk_norm_rope(q, k, q_weight, k_weight, cos, sin, eps: float = 1e-6, q_out=None, k_out=None):
    """Per-head RMSNorm of q [T, Hq, D] and k [T, Hkv, D] (bf16) with bf16 weights [D], then the rotary
    embedding with fp32 cos / sin [T, D]. Returns (q_out, k_out); pass q_out=q, k_out=k to work in place."""
    torch = _torch()
    lib = load_library()
    dev = q.device
    _check_gpu("q", q, 3)
    _check_gpu("k", k, 3, dev)
    for name, t in (("q_weight", q_weight), ("k_weight", k_weight)):
        _check_gpu(name, t, 1, dev)
    for name, t in (("cos", cos), ("sin", sin)):
        _check_gpu(name, t, 2, dev)
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16:
        raise TypeError("q and k must be bfloat16")
    if q_weight.dtype != torch.bfloat16 or k_weight.dtype != torch.bfloat16:
        raise TypeError("q_weight and k_weight must be bfloat16")
    t, hq, d = (int(x) for x in q.shape)
    if int(k.shape[0]) != t or int(k.shape[2]) != d:
        raise ValueError("q and k must share the token count and head_dim")
    if tuple(cos.shape) != (t, d) or tuple(sin.shape) != (t, d):
        raise ValueError(f"cos and sin must be [{t}, {d}]")
    if int(q_weight.shape[0]) != d or int(k_weight.shape[0]) != d:
        raise ValueError(f"q_weight and k_weight must have {d} entries")
    if q_out is None:
        q_out = torch.empty_like(q)
    if k_out is None:
        k_out = torch.empty_like(k)
    _check_out("q_out", q_out, tuple(q.shape), q.dtype, dev)
    _check_out("k_out", k_out, tuple(k.shape), k.dtype, dev)
    st = lib.qk_norm_rope(q.data_ptr(), k.data_ptr(), VFA_BF16, q_weight.data_ptr(), k_weight.data_ptr(),
                          cos.data_ptr(), sin.data_ptr(), t, hq, int(k.shape[1]), d, float(eps), q_out.data_ptr(),
                          k_out.data_ptr(), _stream_ptr(q.device))
    if st != 0:
        raise VfaError(st, "qk_norm_rope")
    return q_out, k_out


def gated_delta_rule_fwd_workspace_size(total_tokens: int, num_heads_v: int, max_seqlen: int) -> int:
    return int(load_library().gated_delta_rule_fwd_workspace_size(int(total_tokens), int(num_heads_v),
                                                                  int(max_seqlen)))


def gated_delta_rule_fwd(q, k, v, g, beta, cu_seqlens, max_seqlen: int, scale: float | None = None,
                         initial_state=None, output_final_state: bool = False, out=None):
    """Varlen gated delta rule forward. q, k [T, Hqk, Dk] and v [T, Hv, Dv] bf16; g, beta [T, Hv] fp32;
    cu_seqlens int32 [B+1] on the GPU; max_seqlen a host upper bound of the lengths (it also picks the
    token-by-token path up to 16 and the chunked one above); initial_state [B, Hv, Dk, Dv] fp32 or None.
    Default scale 1/sqrt(Dk). Returns (out [T, Hv, Dv] bf16, final_state [B, Hv, Dk, Dv] fp32 or None)."""
    torch = _torch()
    lib = load_library()
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_gpu(name, t, 3, dev)
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16")
    for name, t in (("g", g), ("beta", beta)):
        _check_gpu(name, t, 2, dev)
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    _check_gpu("cu_seqlens", cu_seqlens, 1, dev)
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    tt, hqk, dk = (int(x) for x in q.shape)
    hv, dv = int(v.shape[1]), int(v.shape[2])
    if tuple(k.shape) != tuple(q.shape) or int(v.shape[0]) != tt:
        raise ValueError("q and k must match, and v must have the same token count")
    if tuple(g.shape) != (tt, hv) or tuple(beta.shape) != (tt, hv):
        raise ValueError(f"g and beta must be [{tt}, {hv}]")
    batch = int(cu_seqlens.shape[0]) - 1
    if initial_state is not None:
        _check_gpu("initial_state", initial_state, 4, dev)
        if initial_state.dtype != torch.float32 or tuple(initial_state.shape) != (batch, hv, dk, dv):
            raise ValueError(f"initial_state must be float32 [{batch}, {hv}, {dk}, {dv}]")
    if out is None:
        out = torch.empty((tt, hv, dv), dtype=torch.bfloat16, device=q.device)
    _check_out("out", out, (tt, hv, dv), torch.bfloat16, dev)
    final = torch.empty((batch, hv, dk, dv), dtype=torch.float32, device=q.device) if output_final_state else None
    sc = 1.0 / math.sqrt(dk) if scale is None else float(scale)
    ws_bytes = gated_delta_rule_fwd_workspace_size(tt, hv, max_seqlen)
    workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device) if ws_bytes > 0 else None
    st = lib.gated_delta_rule_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), VFA_BF16, g.data_ptr(), beta.data_ptr(),
                                  cu_seqlens.data_ptr(), batch, tt, int(max_seqlen), hqk, hv, dk, dv, sc,
                                  initial_state.data_ptr() if initial_state is not None else None, out.data_ptr(),
                                  final.data_ptr() if final is not None else None,
                                  workspace.data_ptr() if workspace is not None else None, ws_bytes,
                                  _stream_ptr(q.device))
    if st != 0:
        raise VfaError(st, "gated_delta_rule_fwd")
    return out, final
