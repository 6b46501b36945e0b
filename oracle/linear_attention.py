"""fp64 CPU oracle for the varlen gated delta rule (linear attention) forward.

TEST INFRASTRUCTURE ONLY (like the rest of oracle/): imported by tests and the
benchmark's CPU leg, never by the product library; it shares no code with
the HIP path.

Source: "Twinkle NPU kernels" page, Qwen3.5 flash linear attention section:
the hybrid model's linear-attention layers call chunk_gated_delta_rule, a
chunked (WY-representation) forward that handles variable-length sequences
through cu_seqlens. The page names the operator and its varlen interface but
gives no formula; the reading taken (also listed in the design notes) is the
gated delta rule as its name defines it. Per sequence and value head, a state
S [Dk, Dv] (zero, or a given initial state) is advanced token by token:
    S   <- exp(g_t) * S                          (gated decay, g_t <= 0 usually)
    u_t  = beta_t * (v_t - S^T k_t)              (delta-rule correction)
    S   <- S + k_t u_t^T                         (rank-1 write)
    o_t  = scale * S^T q_t                       (read with the updated state)
States do not cross sequence boundaries (cu_seqlens), and each value head h
reads query/key head h // (Hv / Hqk). The chunked form is a reorganisation
of this recurrence; the oracle is the recurrence itself.
"""
from __future__ import annotations

import numpy as np

__all__ = ["gated_delta_rule"]


def gated_delta_rule(q, k, v, g, beta, cu_seqlens, scale: float, initial_state=None):
    """q, k [T, Hqk, Dk]; v [T, Hv, Dv]; g, beta [T, Hv]; cu_seqlens int [B+1].

    Returns o [T, Hv, Dv] and the final states [B, Hv, Dk, Dv], in fp64.
    initial_state: [B, Hv, Dk, Dv] or None (zeros).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    t_all, hqk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    if hv % hqk != 0:
        raise ValueError("the value head count must be a multiple of the query/key head count")
    rep = hv // hqk
    batch = len(cu) - 1
    out = np.zeros((t_all, hv, dv), dtype=np.float64)
    final = np.zeros((batch, hv, dk, dv), dtype=np.float64)
    for b in range(batch):
        for h in range(hv):
            s = (np.zeros((dk, dv)) if initial_state is None
                 else np.array(initial_state[b, h], dtype=np.float64))
            hk = h // rep
            for t in range(int(cu[b]), int(cu[b + 1])):
                s = np.exp(g[t, h]) * s
                u = beta[t, h] * (v[t, h] - s.T @ k[t, hk])
                s = s + np.outer(k[t, hk], u)
                out[t, h] = scale * (s.T @ q[t, hk])
            final[b, h] = s
    return out, final
