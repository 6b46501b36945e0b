"""fp64 CPU oracle for varlen attention, the AttentionUpdate merge and the last-token gather.

TEST INFRASTRUCTURE ONLY. Nothing in the product library imports, links or
calls this module; only tests, the smoke check and the benchmark's CPU
baseline do. It shares no code with the HIP path.

Everything here is the plain definition written out in float64 numpy: scores
are materialised, masked entries are computed and then discarded, softmax is
max-subtract / exp / sum / divide in one pass over all visible keys of a row
(no online softmax, no tiling, no exp2). The only library primitive used is
a matrix product for the dot products.

Sources (page title, section):
  [P1] "From GPU to NPU: Qwen3-Embedding model adaptation and performance
       optimisation on Ascend" -- core optimisation 1 (TND format, cu_seqlens,
       last-token indexing in embed()), 2.1 (npu_fusion_attention call with
       scale, causal triu(diagonal=1) mask, sparse_mode 3), core optimisation
       5 (FIA with num_heads / num_key_value_heads: native GQA that replaces
       repeat_interleave(G, dim=1) of K/V).
  [P2] "Qwen3-MoE low-latency inference on Atlas A3" -- flash attention fused
       operator section: one attention op serves full (prefill) and
       incremental (decode) computation.
  [P4] "attention_update operator optimisation practice" -- operator function
       description (the four-line lse_max / lse / lse_m / O formula) and the
       InferShape / op-plugin sections (lse [sp, bsh], go [sp, bsh, hd] ->
       out [bsh, hd], lse_out [bsh]; out takes go's dtype; lse_out only when
       update_type == 1). Its background section names PagedAttention as the
       operator whose per-chunk partials the merge combines.

Readings where the pages are silent (each also listed in the design notes):
  * cu_seqlens: int32, length B+1, cu[0] = 0, non-decreasing ([P1] core
    optimisation 1, which indexes the last token of sequence b as cu[b+1]-1).
  * GQA: query head h reads kv head h // G with G = Hq / Hkv, which is what
    repeat_interleave(G, dim=1) produces ([P1] core optimisation 5).
  * Causal mask when Lq != Lk: aligned bottom-right, query i sees key j iff
    j <= i + (Lk - Lq). With Lq == Lk this is exactly [P1] 2.1's
    triu(ones, diagonal=1) == masked. An explicit per-sequence offset may
    replace Lk - Lq: it is the position of the sequence's first query minus
    that of its first key, which is how a key chunk [a, c) of a sequence
    ([P4]'s sequence-parallel chunks) keeps the absolute mask: offset -a.
  * lse is the natural log of sum_j exp(scale * q.k_j) over visible keys
    ([P4]: "log-sum-exp, the normalisation factor of the attention weights").
  * A row with no visible key: lse = -inf and O = 0. The merge ignores
    chunks with lse = -inf; if every chunk is -inf, lse_m = -inf and out = 0.
  * Chunk c of sp covers keys [floor(c*Lk/sp), floor((c+1)*Lk/sp)); inside a
    chunk the causal mask uses absolute key positions.
  * Merge row order "bsh" is the [T, Hq] flattening r = token * Hq + head.
  * Paged K/V ([P4] names PagedAttention but gives no cache layout): a cache
    [num_pages, page_size, Hkv, D] per tensor, an int block table
    [B, max_pages] and the key count of each sequence; key j of sequence b is
    slot j % page_size of page block_table[b, j // page_size]. Queries stay
    in TND with cu_seqlens_q, and the mask is the one above with
    Lk = the sequence's key count.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "varlen_attention",
    "varlen_attention_rows",
    "attn_update",
    "last_token_gather",
    "chunked_partials",
    "paged_gather",
    "paged_attention_rows",
]


def _as64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _visible(i_pos: np.ndarray, lq: int, lk: int, causal: bool, key_lo: int, key_hi: int,
             offset=None) -> np.ndarray:
    """Boolean [n, key_hi-key_lo]: key j (absolute in the sequence) is visible to query i.

    [P1] 2.1: the causal mask is triu(ones, diagonal=1) with True = masked,
    i.e. key j is hidden from query i when j > i. Bottom-right alignment
    shifts that by Lk - Lq; an explicit offset (first query's position minus
    first key's position) replaces Lk - Lq.
    """
    j = np.arange(key_lo, key_hi, dtype=np.int64)[None, :]
    vis = np.ones((len(i_pos), key_hi - key_lo), dtype=bool)
    if causal:
        off = (lk - lq) if offset is None else int(offset)
        vis &= j <= (i_pos[:, None] + off)
    return vis


def _attend_rows(q_rows: np.ndarray, k_seq: np.ndarray, v_seq: np.ndarray, scale: float,
                 vis: np.ndarray):
    """Naive softmax attention for a block of query rows against one key set.

    q_rows [n, D], k_seq [m, D], v_seq [m, D], vis [n, m] -> O [n, D], lse [n].
    s_ij = scale * q_i . k_j; M_i = max over visible j; l_i = sum exp(s_ij - M_i);
    O_i = sum exp(s_ij - M_i) v_j / l_i; lse_i = M_i + ln l_i.
    """
    n, d = q_rows.shape
    out = np.zeros((n, v_seq.shape[1]), dtype=np.float64)
    lse = np.full(n, -np.inf, dtype=np.float64)
    if n == 0 or k_seq.shape[0] == 0:
        return out, lse
    s = scale * (q_rows @ k_seq.T)                 # every score, masked or not
    s = np.where(vis, s, -np.inf)
    has = vis.any(axis=1)
    if not has.any():
        return out, lse
    m = np.where(has, s.max(axis=1, initial=-np.inf), 0.0)
    e = np.where(vis, np.exp(s - m[:, None]), 0.0)
    l_sum = e.sum(axis=1)
    o = (e @ v_seq)
    out[has] = o[has] / l_sum[has, None]
    lse[has] = m[has] + np.log(l_sum[has])
    return out, lse


def varlen_attention_rows(q, k, v, cu_seqlens_q, cu_seqlens_k, num_heads_kv: int, scale: float,
                          causal: bool, tokens=None, key_range=None, row_block: int = 1024, causal_offset=None):
    """Attention for selected packed query tokens (all heads), TND layout.

    q [Tq, Hq, D], k / v [Tk, Hkv, D]; cu_seqlens_* int [B+1] ([P1] core
    optimisation 1). ``tokens`` is an iterable of packed query indices (None =
    all). ``key_range`` optionally restricts every sequence to keys
    [lo_b, hi_b) given as a callable b -> (lo, hi), with the mask still using
    absolute positions. ``causal_offset`` (int [B] or None) replaces Lk - Lq
    in the causal mask per sequence. Returns O [len(tokens), Hq, D] and
    lse [len(tokens), Hq].

    [P1] core optimisation 5: query head h shares kv head h // (Hq / Hkv).
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    cu_q = np.asarray(cu_seqlens_q, dtype=np.int64)
    cu_k = np.asarray(cu_seqlens_k, dtype=np.int64)
    tq, hq, d = q.shape
    hkv = int(num_heads_kv)
    if hq % hkv != 0:
        raise ValueError("num_heads_q must be a multiple of num_heads_kv")
    grp = hq // hkv
    batch = len(cu_q) - 1
    if tokens is None:
        tokens = np.arange(tq, dtype=np.int64)
    tokens = np.asarray(list(tokens) if not isinstance(tokens, np.ndarray) else tokens, dtype=np.int64)
    out = np.zeros((len(tokens), hq, v.shape[2]), dtype=np.float64)
    lse = np.full((len(tokens), hq), -np.inf, dtype=np.float64)
    if len(tokens) == 0:
        return out, lse
    # sequence of each selected token: cu_q[b] <= t < cu_q[b+1]
    seq_of = np.searchsorted(cu_q, tokens, side="right") - 1
    for b in range(batch):
        sel = np.nonzero(seq_of == b)[0]
        if len(sel) == 0:
            continue
        qs, lq = int(cu_q[b]), int(cu_q[b + 1] - cu_q[b])
        ks, lk = int(cu_k[b]), int(cu_k[b + 1] - cu_k[b])
        lo, hi = (0, lk) if key_range is None else key_range(b)
        for blk in range(0, len(sel), row_block):
            rows = sel[blk:blk + row_block]
            i_pos = tokens[rows] - qs                      # position inside the sequence
            vis = _visible(i_pos, lq, lk, causal, lo, hi,
                           None if causal_offset is None else causal_offset[b])
            for h in range(hq):
                g = h // grp
                o_h, lse_h = _attend_rows(q[tokens[rows], h, :], k[ks + lo:ks + hi, g, :],
                                          v[ks + lo:ks + hi, g, :], scale, vis)
                out[rows, h, :] = o_h
                lse[rows, h] = lse_h
    return out, lse


def varlen_attention(q, k, v, cu_seqlens_q, cu_seqlens_k, num_heads_kv: int, scale: float,
                     causal: bool, row_block: int = 1024, causal_offset=None):
    """Whole-batch varlen attention: O [Tq, Hq, D] and natural-log lse [Tq, Hq], fp64.

    The call [P1] 2.1 makes: TND layout, per-sequence lengths from cu_seqlens,
    head counts, softmax scale and an optional causal mask; [P2] uses the same
    op for prefill (Lq = Lk) and decode (Lq = 1).
    """
    return varlen_attention_rows(q, k, v, cu_seqlens_q, cu_seqlens_k, num_heads_kv, scale,
                                 causal, tokens=None, row_block=row_block, causal_offset=causal_offset)


def attn_update(lse, go, update_type: int = 1):
    """[P4] AttentionUpdate: merge sp partials computed over key chunks.

    lse [sp, bsh], go [sp, bsh, hd] -> (out [bsh, hd], lse_out [bsh] or None).
      lse_max = max_i lse_i
      lse     = sum_i exp(lse_i - lse_max)
      lse_m   = lse_max + log(lse)
      O       = sum_i O_i * exp(lse_i - lse_m)
    sp is read from dim 0 of lse. Rows whose every chunk has lse = -inf get
    lse_m = -inf and out = 0. lse_out is returned only when update_type == 1.
    """
    lse = _as64(lse)
    go = _as64(go)
    if lse.ndim != 2 or go.ndim != 3 or go.shape[:2] != lse.shape:
        raise ValueError("expected lse [sp, bsh] and go [sp, bsh, hd]")
    if update_type not in (0, 1):
        raise ValueError("update_type must be 0 or 1")
    sp, bsh = lse.shape
    lse_max = lse.max(axis=0)                                   # [bsh]
    live = np.isfinite(lse_max)
    safe_max = np.where(live, lse_max, 0.0)
    w_un = np.where(np.isfinite(lse), np.exp(lse - safe_max[None, :]), 0.0)   # [sp, bsh]
    ssum = w_un.sum(axis=0)
    lse_m = np.where(live, safe_max + np.log(np.where(live, ssum, 1.0)), -np.inf)
    w = np.where(np.isfinite(lse) & live[None, :],
                 np.exp(lse - np.where(live, lse_m, 0.0)[None, :]), 0.0)      # exp(lse_i - lse_m)
    out = np.einsum("sr,srd->rd", w, go)
    return out, (lse_m if update_type == 1 else None)


def last_token_gather(x, cu_seqlens_q):
    """[P1] core optimisation 1, embed(): the last token of every sequence, x[cu[1:] - 1].

    Works on any array whose first axis is the packed token axis ([T, ...]).
    A sequence of length 0 has no last token; that is an error here.
    """
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    idx = cu[1:] - 1
    if np.any(cu[1:] <= cu[:-1]):
        raise ValueError("every sequence needs at least one token to have a last token")
    return np.asarray(x)[idx]


def chunked_partials(q, k, v, cu_seqlens_q, cu_seqlens_k, num_heads_kv: int, scale: float,
                     causal: bool, sp: int, tokens=None):
    """Per-chunk partials (O_c, lse_c) over sp key chunks, in the merge's layout.

    Chunk c of sequence b covers keys [floor(c*Lk/sp), floor((c+1)*Lk/sp)); the
    causal mask keeps absolute key positions. Returns lse [sp, n*Hq] and
    go [sp, n*Hq, D] with rows r = token * Hq + head ([P4] [sp, bsh] layout).
    """
    cu_k = np.asarray(cu_seqlens_k, dtype=np.int64)
    q = _as64(q)
    hq = q.shape[1]
    n = q.shape[0] if tokens is None else len(list(tokens))
    lse_all = np.empty((sp, n * hq), dtype=np.float64)
    go_all = np.empty((sp, n * hq, v.shape[2]), dtype=np.float64)
    for c in range(sp):
        def rng_c(b, c=c):
            lk = int(cu_k[b + 1] - cu_k[b])
            return (c * lk) // sp, ((c + 1) * lk) // sp
        o_c, lse_c = varlen_attention_rows(q, k, v, cu_seqlens_q, cu_seqlens_k, num_heads_kv,
                                           scale, causal, tokens=tokens, key_range=rng_c)
        lse_all[c] = lse_c.reshape(-1)
        go_all[c] = o_c.reshape(n * hq, -1)
    return lse_all, go_all


def paged_gather(cache, block_table, seqused_k):
    """The key (or value) rows of every sequence, read through its block table.

    cache [num_pages, page_size, Hkv, D]; block_table [B, max_pages] ints;
    seqused_k [B] ints (keys of each sequence). Key j of sequence b is
    cache[block_table[b, j // page_size], j % page_size] (the paged-cache
    reading listed in the module docstring). Returns the rows packed in TND
    order, [sum_b seqused_k[b], Hkv, D], and their cu_seqlens [B + 1]. Pages
    and slots that no key of a sequence names are never read.
    """
    cache = np.asarray(cache)
    table = np.asarray(block_table, dtype=np.int64)
    used = np.asarray(seqused_k, dtype=np.int64)
    page_size = cache.shape[1]
    parts = []
    for b in range(len(used)):
        j = np.arange(int(used[b]), dtype=np.int64)
        parts.append(cache[table[b, j // page_size], j % page_size])
    packed = (np.concatenate(parts, axis=0) if parts else np.zeros((0,) + cache.shape[2:], cache.dtype))
    cu = np.concatenate([[0], np.cumsum(used)]).astype(np.int64)
    return packed, cu


def paged_attention_rows(q, k_cache, v_cache, block_table, seqused_k, cu_seqlens_q, num_heads_kv: int,
                         scale: float, causal: bool, tokens=None):
    """Varlen attention whose keys and values sit in a paged cache.

    Same definition as varlen_attention_rows (TND queries, GQA h -> h // G,
    bottom-right causal mask, natural-log lse, -inf / 0 for rows without a
    visible key), with sequence b's keys and values gathered by paged_gather.
    Returns O [len(tokens), Hq, D] and lse [len(tokens), Hq] in fp64.
    """
    k, cu_k = paged_gather(k_cache, block_table, seqused_k)
    v, _ = paged_gather(v_cache, block_table, seqused_k)
    return varlen_attention_rows(q, k, v, cu_seqlens_q, cu_k, num_heads_kv, scale, causal, tokens=tokens)
