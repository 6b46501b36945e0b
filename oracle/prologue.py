"""fp64 CPU oracle for the attention prologue: per-head RMSNorm of q and k, then rotary embedding.

TEST INFRASTRUCTURE ONLY (like the rest of oracle/): imported by tests and the
benchmark's CPU leg, never by the product library; it shares no code with
the HIP path.

Source: "From GPU to NPU: Qwen3-Embedding model adaptation and performance
optimisation on Ascend":
  * 2.2 (normalisation layer): RMSNorm takes the variance of the fp32 values
    as the mean of their squares over the last dimension, multiplies by
    rsqrt(variance + eps), and the fused npu_rms_norm applies the weight;
  * 2.3 (linear layer): q_norm and k_norm act on the projections viewed as
    [T, num_heads, head_dim], i.e. per head over head_dim;
  * 2.4 (rotary embedding): npu_rotary_mul on q and k with per-token cos and
    sin of head_dim entries (reshaped to [1, T, 1, D]), so one (cos, sin)
    row serves every head of a token.
Readings where the page is silent (also listed in the design notes):
  * npu_rotary_mul's rotation is the rotate-half form:
    out = x * cos + rotate_half(x) * sin, rotate_half(x) = [-x[D/2:], x[:D/2]];
  * the whole prologue is computed in high precision and rounded once to the
    output dtype (the fused NPU operators' behaviour the page adopts), not
    rounded between the norm, the weight and the rotation.
"""
from __future__ import annotations

import numpy as np

__all__ = ["rms_norm", "rotate_half", "rotary", "qk_norm_rope"]


def rms_norm(x, weight, eps: float):
    """x / sqrt(mean(x^2 over the last axis) + eps) * weight, in fp64 (2.2)."""
    x = np.asarray(x, dtype=np.float64)
    var = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(var + eps) * np.asarray(weight, dtype=np.float64)


def rotate_half(x):
    """[-x[..., D/2:], x[..., :D/2]] along the last axis."""
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    return np.concatenate([-x[..., h:], x[..., :h]], axis=-1)


def rotary(x, cos, sin):
    """x [T, N, D] with per-token cos, sin [T, D]: x * cos + rotate_half(x) * sin (2.4)."""
    x = np.asarray(x, dtype=np.float64)
    c = np.asarray(cos, dtype=np.float64)[:, None, :]
    s = np.asarray(sin, dtype=np.float64)[:, None, :]
    return x * c + rotate_half(x) * s


def qk_norm_rope(q, k, q_weight, k_weight, cos, sin, eps: float):
    """q [T, Hq, D], k [T, Hkv, D] -> (rotary(rms_norm(q)), rotary(rms_norm(k))), fp64."""
    return (rotary(rms_norm(q, q_weight, eps), cos, sin), rotary(rms_norm(k, k_weight, eps), cos, sin))
