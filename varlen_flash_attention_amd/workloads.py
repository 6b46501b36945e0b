"""Seeded synthetic inputs for varlen attention and the AttentionUpdate merge.

This module only draws numbers: sequence lengths, Q/K/V values and the
chunk boundaries a caller asks for. It holds none of the attention or merge
arithmetic, so the CPU oracle and the HIP path can both be fed from it
without sharing any of the method.

Shapes follow the workloads the pages describe:
  * "From GPU to NPU: Qwen3-Embedding on Ascend", core optimisation 1 (TND
    format): all tokens of a batch flattened to [total_tokens, heads, head_dim],
    sequence boundaries in an int32 cu_seqlens of length B+1.
  * same page, core optimisation 5 (FIA, native GQA): 16 query heads, 8 kv
    heads, head_dim 128 for the embedding model.
  * "Qwen3-MoE low-latency inference on Atlas A3", attention TP section: the
    same fused attention op serves prefill and decode.

Random draws use numpy's PCG64. Lengths come from default_rng(seed); Q, K
and V come from the three children of SeedSequence(seed), each tensor drawn
in blocks of 2^22 values with one spawned PCG64 stream per block (so the
values do not depend on the thread count). Values are i.i.d. N(0,1) drawn in
fp32; for bf16 workloads they are rounded to bf16 (round to nearest even) and
both sides receive the rounded values.
"""
from __future__ import annotations

import concurrent.futures as cf
import math
import os
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Workload",
    "make_growing_scores",
    "round_to_bf16",
    "bf16_bits",
    "make_workload",
    "make_custom",
    "chunk_bounds",
    "PagedCache",
    "make_paged",
    "PrologueInputs",
    "make_prologue",
    "GatedDeltaInputs",
    "make_gated_delta",
    "WORKLOAD_NAMES",
]


_BLOCK = 1 << 22          # values per independently seeded block
_THREADS = min(16, os.cpu_count() or 1)


def _round_slice(u: np.ndarray) -> None:
    lsb = (u >> 16) & 1
    u += np.uint32(0x7FFF)
    u += lsb
    u &= np.uint32(0xFFFF0000)


def round_to_bf16(x: np.ndarray, inplace: bool = False) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32 holding them.

    Finite inputs only. Works in slices with uint32 arithmetic, on a copy
    unless ``inplace`` (then x must be a C-contiguous fp32 array).
    """
    if inplace:
        if x.dtype != np.float32 or not x.flags.c_contiguous:
            raise ValueError("in-place rounding needs a C-contiguous float32 array")
        y = x
    else:
        y = np.array(x, dtype=np.float32, copy=True, order="C")
    u = y.reshape(-1).view(np.uint32)
    with cf.ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(lambda lo: _round_slice(u[lo:lo + _BLOCK]), range(0, u.size, _BLOCK)))
    return y


def _normal(seq: np.random.SeedSequence, shape) -> np.ndarray:
    """i.i.d. N(0,1) fp32 of the given shape.

    Block i of _BLOCK consecutive values (in C order) comes from its own PCG64
    stream seeded by the i-th child of ``seq``, so the values do not depend on
    how many threads draw them.
    """
    out = np.empty(int(np.prod(shape)), dtype=np.float32)
    n_blocks = (out.size + _BLOCK - 1) // _BLOCK
    children = seq.spawn(n_blocks)

    def fill(i):
        lo = i * _BLOCK
        np.random.Generator(np.random.PCG64(children[i])).standard_normal(
            out=out[lo:lo + _BLOCK], dtype=np.float32)

    with cf.ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(fill, range(n_blocks)))
    return out.reshape(shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The upper 16 bits of fp32 values that are already bf16-exact, as uint16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    halves = x.reshape(-1).view(np.uint16)          # little-endian: (low, high) pairs
    if halves[0::2].any():
        raise ValueError("values are not bf16-exact; round them first")
    return np.ascontiguousarray(halves[1::2]).reshape(x.shape)


@dataclass
class Workload:
    name: str
    lengths_q: np.ndarray          # int64 [B]
    lengths_k: np.ndarray          # int64 [B]
    num_heads_q: int
    num_heads_kv: int
    head_dim: int
    dtype: str                     # "fp32" or "bf16"
    causal: bool
    scale: float
    seed: int
    q: np.ndarray = field(repr=False, default=None)   # fp32 [Tq, Hq, D]
    k: np.ndarray = field(repr=False, default=None)   # fp32 [Tk, Hkv, D]
    v: np.ndarray = field(repr=False, default=None)   # fp32 [Tk, Hkv, D]

    @property
    def batch(self) -> int:
        return int(len(self.lengths_q))

    @property
    def cu_seqlens_q(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lengths_q)]).astype(np.int32)

    @property
    def cu_seqlens_k(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lengths_k)]).astype(np.int32)

    @property
    def total_q(self) -> int:
        return int(self.lengths_q.sum())

    @property
    def total_k(self) -> int:
        return int(self.lengths_k.sum())

    @property
    def max_seqlen_q(self) -> int:
        return int(self.lengths_q.max()) if self.batch else 0

    @property
    def max_seqlen_k(self) -> int:
        return int(self.lengths_k.max()) if self.batch else 0

    def with_causal(self, causal: bool) -> "Workload":
        w = Workload(**{**self.__dict__})
        w.causal = bool(causal)
        return w

    def visible_pairs(self) -> int:
        """Number of (query row, key) pairs the mask leaves visible, per query head.

        Causal masking is aligned bottom-right: query i of a sequence with Lq
        queries and Lk keys sees key j iff j <= i + Lk - Lq.
        """
        total = 0
        for lq, lk in zip(self.lengths_q.tolist(), self.lengths_k.tolist()):
            if not self.causal:
                total += lq * lk
                continue
            off = lk - lq
            for_i = np.clip(np.arange(lq, dtype=np.int64) + off + 1, 0, lk)
            total += int(for_i.sum())
        return total

    def useful_flops(self) -> float:
        """4 * head_dim per visible (query row, query head, key); masked pairs excluded."""
        return 4.0 * self.head_dim * self.num_heads_q * self.visible_pairs()

    def compulsory_bytes(self, out_bytes_per_elem: int | None = None) -> int:
        """Q, K, V read once; O and lse written once."""
        eb = 4 if self.dtype == "fp32" else 2
        ob = eb if out_bytes_per_elem is None else out_bytes_per_elem
        tq, tk = self.total_q, self.total_k
        hq, hkv, d = self.num_heads_q, self.num_heads_kv, self.head_dim
        return tq * hq * d * eb + 2 * tk * hkv * d * eb + tq * hq * d * ob + tq * hq * 4


def _draw_values(seed: int, lq: np.ndarray, lk: np.ndarray, hq: int, hkv: int, d: int, dtype: str):
    """Q, K, V from three child seeds of SeedSequence(seed), in that order."""
    tq, tk = int(lq.sum()), int(lk.sum())
    sq, sk, sv = np.random.SeedSequence(seed).spawn(3)
    q = _normal(sq, (tq, hq, d))
    k = _normal(sk, (tk, hkv, d))
    v = _normal(sv, (tk, hkv, d))
    if dtype == "bf16":
        q, k, v = (round_to_bf16(t, inplace=True) for t in (q, k, v))
    elif dtype != "fp32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return q, k, v


# name -> (description, default seed)
WORKLOAD_NAMES = {
    "tiny_fp32": "4 sequences {17,64,5,128}, Hq=4 Hkv=2 D=64, fp32, causal",
    "embed_prefill": "64 sequences uniform in [32,512], Hq=16 Hkv=8 D=128, bf16, causal",
    "long_prefill": "16 sequences log-normal (median 2048, clip [256,8192]), Hq=32 Hkv=8 D=128, bf16, causal",
    "long_prefill_full": "long_prefill shapes with full (non-causal) masking",
    "decode": "64 sequences, 1 query each, KV lengths uniform in [1024,32768], Hq=32 Hkv=4 D=128, bf16",
}


def _lengths(name: str, rng: np.random.Generator):
    if name == "tiny_fp32":
        lq = np.array([17, 64, 5, 128], dtype=np.int64)
        return lq, lq.copy()
    if name == "embed_prefill":
        lq = rng.integers(32, 513, 64).astype(np.int64)
        return lq, lq.copy()
    if name in ("long_prefill", "long_prefill_full"):
        raw = rng.lognormal(mean=math.log(2048.0), sigma=1.0, size=16)
        lq = np.clip(np.rint(raw), 256, 8192).astype(np.int64)
        return lq, lq.copy()
    if name == "decode":
        lk = rng.integers(1024, 32769, 64).astype(np.int64)
        return np.ones(64, dtype=np.int64), lk
    raise KeyError(name)


_SHAPES = {
    # name: (Hq, Hkv, D, dtype, causal, seed)
    "tiny_fp32": (4, 2, 64, "fp32", True, 1),
    "embed_prefill": (16, 8, 128, "bf16", True, 2),
    "long_prefill": (32, 8, 128, "bf16", True, 3),
    "long_prefill_full": (32, 8, 128, "bf16", False, 3),
    "decode": (32, 4, 128, "bf16", True, 4),
}


def make_workload(name: str, seed: int | None = None, values: bool = True) -> Workload:
    """Build one of the named workloads. ``values=False`` draws only the lengths."""
    hq, hkv, d, dtype, causal, default_seed = _SHAPES[name]
    seed = default_seed if seed is None else int(seed)
    rng = np.random.default_rng(seed)
    lq, lk = _lengths(name, rng)
    w = Workload(name=name, lengths_q=lq, lengths_k=lk, num_heads_q=hq, num_heads_kv=hkv,
                 head_dim=d, dtype=dtype, causal=causal, scale=1.0 / math.sqrt(d), seed=seed)
    if values:
        w.q, w.k, w.v = _draw_values(seed, lq, lk, hq, hkv, d, dtype)
    return w


def make_custom(lengths_q, lengths_k=None, num_heads_q=4, num_heads_kv=2, head_dim=64,
                dtype="fp32", causal=True, scale=None, seed=0, name="custom") -> Workload:
    """A workload with caller-chosen lengths (e.g. small parity cases and edge cases)."""
    lq = np.asarray(lengths_q, dtype=np.int64).reshape(-1)
    lk = lq.copy() if lengths_k is None else np.asarray(lengths_k, dtype=np.int64).reshape(-1)
    if lq.shape != lk.shape:
        raise ValueError("lengths_q and lengths_k must have the same number of sequences")
    q, k, v = _draw_values(seed, lq, lk, num_heads_q, num_heads_kv, head_dim, dtype)
    sc = 1.0 / math.sqrt(head_dim) if scale is None else float(scale)
    return Workload(name=name, lengths_q=lq, lengths_k=lk, num_heads_q=num_heads_q,
                    num_heads_kv=num_heads_kv, head_dim=head_dim, dtype=dtype,
                    causal=bool(causal), scale=sc, seed=seed, q=q, k=k, v=v)


def make_growing_scores(lengths, num_heads_q=8, num_heads_kv=2, head_dim=128, dtype="bf16", causal=True,
                        seed=0, top_score=1000.0, name="growing_scores") -> Workload:
    """Scores that climb along every sequence: Q entries near 1 and key row j of a sequence of length L
    scaled by (j + 1) / L, so q . k runs from about 0 to about ``top_score`` (raw, before the softmax scale)
    over each sequence, with noise of a tenth around the trend. With the default scale 1/sqrt(D) a row's
    later keys then outgrow its earlier ones by far more than 2^32 in probability units, which moves an
    online softmax's reference several times per row."""
    lq = np.asarray(lengths, dtype=np.int64).reshape(-1)
    sq, sk, sv = np.random.SeedSequence(seed).spawn(3)
    tq = int(lq.sum())
    q = 1.0 + 0.1 * _normal(sq, (tq, num_heads_q, head_dim))
    k = 1.0 + 0.1 * _normal(sk, (tq, num_heads_kv, head_dim))
    v = _normal(sv, (tq, num_heads_kv, head_dim))
    ramp = np.concatenate([(np.arange(n, dtype=np.float64) + 1.0) / max(int(n), 1) for n in lq]) if tq else \
        np.zeros(0)
    k = k * (top_score / head_dim * ramp)[:, None, None]
    q, k, v = (np.ascontiguousarray(t, dtype=np.float32) for t in (q, k, v))
    if dtype == "bf16":
        q, k, v = (round_to_bf16(t, inplace=True) for t in (q, k, v))
    elif dtype != "fp32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return Workload(name=name, lengths_q=lq, lengths_k=lq.copy(), num_heads_q=num_heads_q,
                    num_heads_kv=num_heads_kv, head_dim=head_dim, dtype=dtype, causal=bool(causal),
                    scale=1.0 / math.sqrt(head_dim), seed=seed, q=q, k=k, v=v)


def chunk_bounds(length: int, sp: int) -> list[tuple[int, int]]:
    """Key range [lo, hi) of each of ``sp`` chunks of a sequence of ``length`` keys.

    Chunk c covers [floor(c*L/sp), floor((c+1)*L/sp)): equal chunks when sp
    divides L, otherwise sizes differ by at most one.
    """
    return [((c * length) // sp, ((c + 1) * length) // sp) for c in range(sp)]


@dataclass
class PagedCache:
    """A workload's K/V laid out in fixed-size pages behind a per-sequence block table."""
    page_size: int
    k_cache: np.ndarray = field(repr=False)      # fp32 values [num_pages, page_size, Hkv, D]
    v_cache: np.ndarray = field(repr=False)
    block_table: np.ndarray = field(repr=False)  # int32 [B, max_pages]; -1 past a sequence's pages
    seqused_k: np.ndarray = field(repr=False)    # int32 [B], keys of each sequence

    @property
    def num_pages(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])


def make_paged(w: Workload, page_size: int, seed: int = 0, spare_pages: int = 3) -> PagedCache:
    """Write the workload's K and V into a paged cache.

    Layout (the reading taken for a PagedAttention cache, whose layout the
    pages do not give): key j of sequence b sits in slot j % page_size of
    page block_table[b, j // page_size]. Logical pages go to physical pages
    in a seeded random order, so consecutive pages of a sequence are
    scattered; slots past a sequence's last key and ``spare_pages`` unused
    pages hold other N(0,1) draws (bf16-rounded for bf16 workloads), so a
    read from a wrong page or slot changes the result.
    """
    if page_size < 1:
        raise ValueError("page_size must be positive")
    lk = w.lengths_k.astype(np.int64)
    need = (lk + page_size - 1) // page_size
    num_pages = int(need.sum()) + int(spare_pages)
    max_pages = max(int(need.max()) if len(need) else 0, 1)
    s_perm, s_k, s_v = np.random.SeedSequence([int(seed), int(page_size)]).spawn(3)
    perm = np.random.default_rng(s_perm).permutation(num_pages)
    shape = (num_pages, page_size, w.num_heads_kv, w.head_dim)
    k_cache = np.empty(shape, dtype=np.float32)
    v_cache = np.empty(shape, dtype=np.float32)
    filled = np.zeros((num_pages, page_size), dtype=bool)
    table = np.full((w.batch, max_pages), -1, dtype=np.int32)
    cu = w.cu_seqlens_k.astype(np.int64)
    nxt = 0
    for b in range(w.batch):
        phys = perm[nxt:nxt + need[b]]
        nxt += int(need[b])
        table[b, :need[b]] = phys
        n = int(lk[b])
        full, rem = n // page_size, n % page_size
        for cache, src in ((k_cache, w.k), (v_cache, w.v)):
            rows = src[cu[b]:cu[b + 1]]
            if full:            # whole pages: key j -> page phys[j // page_size], slot j % page_size
                cache[phys[:full]] = rows[:full * page_size].reshape(full, page_size, *rows.shape[1:])
            if rem:
                cache[phys[full], :rem] = rows[full * page_size:]
        filled[phys[:full]] = True
        if rem:
            filled[phys[full], :rem] = True
    n_free = int((~filled).sum())
    for cache, ss in ((k_cache, s_k), (v_cache, s_v)):
        junk = _normal(ss, (n_free, w.num_heads_kv, w.head_dim))
        cache[~filled] = round_to_bf16(junk, inplace=True) if w.dtype == "bf16" else junk
    return PagedCache(page_size=int(page_size), k_cache=k_cache, v_cache=v_cache, block_table=table,
                      seqused_k=lk.astype(np.int32))


@dataclass
class PrologueInputs:
    """Inputs of the attention prologue (per-head q/k RMSNorm, then the rotary embedding)."""
    lengths: np.ndarray                            # int64 [B]
    q: np.ndarray = field(repr=False)              # bf16 values in fp32 [T, Hq, D]
    k: np.ndarray = field(repr=False)              # bf16 values in fp32 [T, Hkv, D]
    q_weight: np.ndarray = field(repr=False)       # bf16 values in fp32 [D]
    k_weight: np.ndarray = field(repr=False)
    cos: np.ndarray = field(repr=False)            # fp32 [T, D]
    sin: np.ndarray = field(repr=False)
    eps: float = 1e-6

    @property
    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lengths)]).astype(np.int32)


def make_prologue(lengths, num_heads_q=32, num_heads_kv=8, head_dim=128, theta=1.0e6, eps=1e-6,
                  seed=0) -> PrologueInputs:
    """Seeded prologue inputs for packed sequences.

    q and k are N(0, 4) (projection outputs are not unit scale; the norm
    removes the scale), rounded to bf16; the weights are 1 + N(0, 0.01),
    rounded to bf16. cos / sin rows follow the usual rotary tables: token i of
    a sequence (positions restart at 0 in each sequence, as TND packs whole
    sequences) at frequency j < D/2 has angle i * theta^(-2j/D), used for
    both element j and element j + D/2; computed in fp64, stored fp32.
    theta = 1e6 is the Qwen3 family's base.
    """
    lens = np.asarray(lengths, dtype=np.int64).reshape(-1)
    t = int(lens.sum())
    sq, sk, sw = np.random.SeedSequence(seed).spawn(3)
    q = round_to_bf16(2.0 * _normal(sq, (t, num_heads_q, head_dim)), inplace=True)
    k = round_to_bf16(2.0 * _normal(sk, (t, num_heads_kv, head_dim)), inplace=True)
    w = round_to_bf16(1.0 + 0.1 * _normal(sw, (2, head_dim)), inplace=True)
    pos = np.concatenate([np.arange(int(n), dtype=np.float64) for n in lens]) if t else np.zeros(0)
    inv_freq = theta ** (-np.arange(0, head_dim, 2, dtype=np.float64) / head_dim)
    ang = pos[:, None] * inv_freq[None, :]
    ang = np.concatenate([ang, ang], axis=1)
    return PrologueInputs(lengths=lens, q=q, k=k, q_weight=np.ascontiguousarray(w[0]),
                          k_weight=np.ascontiguousarray(w[1]), cos=np.cos(ang).astype(np.float32),
                          sin=np.sin(ang).astype(np.float32), eps=float(eps))


@dataclass
class GatedDeltaInputs:
    """Inputs of the varlen gated delta rule (linear attention) forward."""
    lengths: np.ndarray                          # int64 [B]
    q: np.ndarray = field(repr=False)            # bf16 values in fp32 [T, Hqk, Dk]
    k: np.ndarray = field(repr=False)            # bf16 values in fp32 [T, Hqk, Dk]
    v: np.ndarray = field(repr=False)            # bf16 values in fp32 [T, Hv, Dv]
    g: np.ndarray = field(repr=False)            # fp32 [T, Hv], log decay <= 0
    beta: np.ndarray = field(repr=False)         # fp32 [T, Hv], in (0, 1)
    scale: float = 1.0

    @property
    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lengths)]).astype(np.int32)


def make_gated_delta(lengths, num_heads_qk=16, num_heads_v=32, head_dim_k=128, head_dim_v=128,
                     seed=0) -> GatedDeltaInputs:
    """Seeded inputs shaped like a hybrid model's linear-attention layers.

    q and k are N(0, 1) rows scaled to unit length per head (the layers
    normalise q and k before the operator), then rounded to bf16; v is
    N(0, 1) rounded to bf16; the decay exp(g) is uniform in [0.5, 1) and
    beta = sigmoid(N(0, 1)), both stored fp32. scale = 1/sqrt(Dk).
    """
    lens = np.asarray(lengths, dtype=np.int64).reshape(-1)
    t = int(lens.sum())
    sq, sk, sv, sgb = np.random.SeedSequence(seed).spawn(4)
    q = _normal(sq, (t, num_heads_qk, head_dim_k)).astype(np.float64)
    k = _normal(sk, (t, num_heads_qk, head_dim_k)).astype(np.float64)
    q /= np.maximum(np.linalg.norm(q, axis=-1, keepdims=True), 1e-30)
    k /= np.maximum(np.linalg.norm(k, axis=-1, keepdims=True), 1e-30)
    rng = np.random.default_rng(sgb)
    g = np.log(rng.uniform(0.5, 1.0, (t, num_heads_v))).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((t, num_heads_v))))).astype(np.float32)
    return GatedDeltaInputs(lengths=lens, q=round_to_bf16(q.astype(np.float32), inplace=True),
                            k=round_to_bf16(k.astype(np.float32), inplace=True),
                            v=round_to_bf16(_normal(sv, (t, num_heads_v, head_dim_v)), inplace=True),
                            g=g, beta=beta, scale=1.0 / math.sqrt(head_dim_k))
