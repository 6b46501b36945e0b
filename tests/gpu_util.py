"""Helpers for GPU parity tests: device copies of workloads and the tolerance rule.

Tolerances (element by element):
  bf16 inputs:  |O - ref| <= 2e-2 + 2e-2 |ref|,  |lse - ref| <= 1e-3
  fp32 inputs:  |O - ref| <= 1e-5 + 1e-5 |ref|,  |lse - ref| <= 1e-5
Rows whose reference lse is -inf must come back with lse exactly -inf and
O exactly 0. No NaN anywhere.
"""
from __future__ import annotations

import numpy as np
import pytest

from varlen_flash_attention_amd.workloads import bf16_bits

TOL = {"bf16": (2e-2, 2e-2, 1e-3), "fp32": (1e-5, 1e-5, 1e-5)}


def torch_mod():
    import torch
    return torch


def need_gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def dev_array(x: np.ndarray, dtype: str, device="cuda"):
    torch = torch_mod()
    if dtype == "bf16":
        bits = bf16_bits(x).view(np.int16)
        return torch.from_numpy(np.ascontiguousarray(bits)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def to_device(w, device="cuda"):
    torch = torch_mod()
    return dict(
        q=dev_array(w.q, w.dtype, device), k=dev_array(w.k, w.dtype, device), v=dev_array(w.v, w.dtype, device),
        cu_q=torch.from_numpy(w.cu_seqlens_q).to(device), cu_k=torch.from_numpy(w.cu_seqlens_k).to(device),
    )


def host64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check(name, o_gpu, lse_gpu, o_ref, lse_ref, dtype):
    """Assert the tolerance rule; return the worst err/bound ratios for reporting."""
    a_o, r_o, a_l = TOL[dtype]
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    lse_ref = np.asarray(lse_ref, dtype=np.float64)
    assert o_gpu.shape == o_ref.shape, (name, o_gpu.shape, o_ref.shape)
    assert lse_gpu.shape == lse_ref.shape, (name, lse_gpu.shape, lse_ref.shape)
    assert not np.isnan(o_gpu).any(), f"{name}: NaN in O"
    assert not np.isnan(lse_gpu).any(), f"{name}: NaN in lse"
    dead = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_gpu), dead), f"{name}: -inf rows differ ({np.isneginf(lse_gpu).sum()} vs {dead.sum()})"
    assert not np.isinf(lse_gpu[~dead]).any(), f"{name}: inf lse on a live row"
    if dead.any():
        assert (o_gpu[dead] == 0).all(), f"{name}: fully masked rows must have O = 0"
    err_o = np.abs(o_gpu - o_ref)
    bound_o = a_o + r_o * np.abs(o_ref)
    err_l = np.abs(lse_gpu[~dead] - lse_ref[~dead])
    worst_o = float((err_o / bound_o).max()) if err_o.size else 0.0
    worst_l = float((err_l / a_l).max()) if err_l.size else 0.0
    bad_o = int((err_o > bound_o).sum())
    bad_l = int((err_l > a_l).sum())
    print(f"[parity] {name}: worst O err/bound {worst_o:.3f}, worst lse err/bound {worst_l:.3f}, "
          f"violations {bad_o + bad_l}", flush=True)
    assert bad_o == 0, f"{name}: {bad_o} O elements out of tolerance (worst ratio {worst_o:.3f})"
    assert bad_l == 0, f"{name}: {bad_l} lse elements out of tolerance (worst ratio {worst_l:.3f})"
    return worst_o, worst_l


def sample_tokens(w, per_seq=4, seed=0, limit=None):
    """First, last and a few random tokens of each sequence (sorted, unique)."""
    rng = np.random.default_rng(seed)
    cu = w.cu_seqlens_q.astype(np.int64)
    toks = []
    for b in range(w.batch):
        lo, hi = int(cu[b]), int(cu[b + 1])
        if hi <= lo:
            continue
        toks += [lo, hi - 1]
        toks += list(rng.integers(lo, hi, per_seq))
    toks = np.unique(np.array(toks, dtype=np.int64))
    if limit is not None and len(toks) > limit:
        toks = np.sort(rng.choice(toks, limit, replace=False))
    return toks


def tile_tokens(w, tile, seed=0):
    """One seeded token from every `tile`-token query tile of every sequence, plus each sequence's first
    and last token (sorted, unique): with `tile` the kernel's tokens per workgroup, every workgroup of
    the call has a row in the sample."""
    rng = np.random.default_rng(seed)
    cu = w.cu_seqlens_q.astype(np.int64)
    toks = []
    for b in range(w.batch):
        lo, hi = int(cu[b]), int(cu[b + 1])
        if hi <= lo:
            continue
        toks += [lo, hi - 1]
        for t0 in range(lo, hi, tile):
            toks.append(int(rng.integers(t0, min(hi, t0 + tile))))
    return np.unique(np.array(toks, dtype=np.int64))
