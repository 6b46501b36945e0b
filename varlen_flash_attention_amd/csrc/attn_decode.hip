// Split-KV varlen attention for few queries against long key sets (decode), bf16 in.
//
// Same result as the prefill kernel (softmax(scale q K^T) V and the natural
// log-sum-exp per query row, TND queries, GQA head h -> h / G, bottom-right
// causal mask), for the shape where one fused attention op serves
// incremental decoding ("Qwen3-MoE low-latency inference on Atlas A3", flash
// attention fused operator section).
//
// Decode reads every K/V byte once and does little arithmetic per byte, so it
// is bound by HBM bandwidth. Sequence lengths vary widely, so each
// (sequence, kv head) is cut into fixed-size key chunks ("splits") and the
// splits become independent workgroups. Each split produces a partial
// (O_s, lse_s); the partials are merged with the AttentionUpdate rule
// ("attention_update operator optimisation practice", operator function
// description) using the same device helpers as the attn_update entry point.
//
// Two K/V layouts share one kernel template:
//   contiguous: K/V in TND with cu_seqlens_k. Partials go to a row-indexed
//               workspace and a combine kernel merges them.
//   paged:      K/V in fixed-size pages reached through a per-sequence block
//               table (the PagedAttention operator that page names as the
//               source of the partials it merges). Queries may exceed the 16
//               columns of one workgroup: the (token, head) columns of a kv
//               head are cut into groups of 16. With a single split the split
//               kernel writes the output itself.
// In both layouts the partials are merged by a second kernel rather than by
// the last split to finish: handing partials between workgroups inside one
// launch needs a device-scope release (an L2 writeback on every XCD) per
// workgroup, which measured 718 us against 453 us without it at the decode
// shape.
//
// Inside a workgroup (4 waves) every wave owns a strided subset of 32-key
// steps of the split and keeps its own online-softmax state; the four states
// are merged through LDS at the end. The G query heads of the kv head (times
// the query tokens) fill the 16 columns of v_mfma_f32_16x16x32_bf16:
//   S^T = K Q^T   : A = K rows parked in a wave-private LDS buffer and read
//                   back 16 B per lane, B = Q^T in registers.
//   O^T += V^T P^T: V rows go through the same buffer so that
//                   ds_read_b64_tr_b16 can deliver V^T; B = P^T from registers.
#include "common.h"
#include "launch.h"

namespace vfa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kCols = 16;      // query columns (heads x tokens) per workgroup
constexpr int kStep = 32;      // keys per wave step
// Paged K/V: the page ids of one split are staged in LDS. A split holds at
// most kMaxChunk keys and a page at least kMinPage keys (so a 32-key step
// touches at most two pages).
constexpr int kMaxChunk = 4096;
constexpr int kMinPage = 16;
constexpr int kPageSlots = kMaxChunk / kMinPage;

// Kernel arguments of the split kernel (contiguous or paged K/V).
struct SplitArgs {
  const bf16* q;                // [total_q, hq, D]
  const bf16* k;                // contiguous: [total_k, hkv, D]; paged: [num_pages, 2^lg_page, hkv, D]
  const bf16* v;
  const int32_t* cu_q;          // [batch + 1]
  const int32_t* cu_k;          // contiguous: [batch + 1]
  const int32_t* causal_off;    // contiguous: per-sequence causal offset, or NULL (bottom-right)
  const int32_t* seqused_k;     // paged: keys of each sequence [batch]
  const int32_t* block_table;   // paged: [batch, max_pages]
  int batch, hq, hkv, grp, chunk, n_splits;
  int max_pages, num_pages, lg_page, max_seqlen_k, n_cg;
  long long rows_total;         // total_q * hq (row-indexed partials)
  float scale, scale_log2;
  float* ws_o;                  // partial O [n_splits][rows_total][D]
  float* ws_lse;                // partial lse [n_splits][rows_total]
  void* out;                    // paged with one split: final [total_q, hq, D]
  float* lse;                   // paged with one split: final [total_q, hq]
};

template <int D>
struct DSmem {
  static constexpr int VSTR = D * 2 + 64;                 // bytes per V row (conflict-free tr reads)
  static constexpr int KSTR = D * 2 + 16;                 // bytes per K row (conflict-free b128 reads)
  static constexpr int WAVE_BYTES = kStep * (VSTR + KSTR); // one step of K and V per wave (see below)
  static constexpr int VBYTES = kWaves * WAVE_BYTES;
  static constexpr int MERGE_BYTES = kWaves * kCols * (D + 2) * 4;
  static constexpr int TOTAL = VBYTES > MERGE_BYTES ? VBYTES : MERGE_BYTES;
  static constexpr int KREGS = kStep * D / 8 / 64;         // 16-byte K loads per lane per step
  static constexpr int VREGS = kStep * D / 8 / 64;         // 16-byte V loads per lane per step
};

__device__ __forceinline__ bf16x8 tr_pair(const char VFA_LDS* p0, const char VFA_LDS* p1) {
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 VFA_LDS*)p0);
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 VFA_LDS*)p1);
  typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8;
  i16x8 r = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, r);
}

// Writes one column slice of a final output row: O (D / 16 values from md on)
// and, from the column's first thread, its lse.
template <int D, typename OutT>
__device__ __forceinline__ void store_row(void* out, float* lse, long long row, int md, bool lead,
                                          const f32x4 (&o)[D / 64], float lse_v) {
  OutT* dst = (OutT*)out + row * D + md;
#pragma unroll
  for (int x = 0; x < D / 64; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) dst[x * 4 + y] = from_f32<OutT>(o[x][y]);
  if (lead) lse[row] = lse_v;
}

// Grid, contiguous: n_splits * batch * hkv workgroups. Grid, paged:
// n_splits * batch * hkv * n_cg workgroups (column group fastest). Partials
// go to ws_o[split][row][D] and ws_lse[split][row], row = token * hq + head;
// paged with n_splits == 1 writes out and lse instead.
template <int D, bool CAUSAL, bool PAGED, typename OutT>
__global__ __launch_bounds__(kThreads, 2) void attn_decode_split_kernel(const SplitArgs p) {
  using S = DSmem<D>;
  __shared__ __attribute__((aligned(16))) char smem[S::TOTAL];
  __shared__ int pages[PAGED ? kPageSlots : 1];
  char VFA_LDS* lds = (char VFA_LDS*)smem;

  // Longest splits first: split index descends with the block id.
  const int per_s = p.batch * p.hkv;
  int split, b, g, cg = 0;
  if constexpr (PAGED) {
    cg = (int)(blockIdx.x % p.n_cg);
    const int r = (int)(blockIdx.x / p.n_cg);
    split = p.n_splits - 1 - r / per_s;
    b = (r % per_s) / p.hkv;
    g = r % p.hkv;
  } else {
    split = p.n_splits - 1 - (int)(blockIdx.x / per_s);
    const int bg = blockIdx.x % per_s;
    b = bg / p.hkv;
    g = bg % p.hkv;
  }
  const int grp = p.grp;
  const float scale_log2 = p.scale_log2;

  const int q0 = p.cu_q[b];
  const int lq = p.cu_q[b + 1] - q0;
  int k0 = 0, lk;
  if constexpr (PAGED) {
    // Keys past the host bound are ignored, so the block table is never read
    // past max_seqlen_k / page_size entries.
    lk = min(max(p.seqused_k[b], 0), p.max_seqlen_k);
  } else {
    k0 = p.cu_k[b];
    lk = p.cu_k[b + 1] - k0;
  }
  const int key_lo = split * p.chunk;
  if constexpr (PAGED) {
    if (lq * grp <= cg * kCols) return;                  // no (token, head) column in this group
    // A sequence without keys still owes its rows out = 0, lse = -inf; split 0 writes them.
    if (key_lo >= lk && !(lk == 0 && split == 0)) return;
  } else {
    if (lq <= 0 || key_lo >= lk) return;                 // this split holds no key of the sequence
  }
  const int key_hi = min(lk, key_lo + p.chunk);
  const int diag = causal_diag(PAGED ? nullptr : p.causal_off, b, lq, lk);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int c16 = lane & 15;
  const int grp4 = lane >> 4;

  // Column -> (token, head): tokens outer, the G heads of this kv head inner.
  int tq, head;
  bool qvalid;
  if constexpr (PAGED) {
    const int col = cg * kCols + c16;
    tq = col / grp;
    head = g * grp + col % grp;
    qvalid = tq < lq;
  } else {
    const int tpc = kCols / grp;                         // tokens per workgroup (>= 1)
    const bool colvalid = c16 < tpc * grp;
    tq = colvalid ? c16 / grp : 0;
    head = g * grp + (colvalid ? c16 % grp : 0);
    qvalid = colvalid && tq < lq;
  }

  // Q^T (B operand): column c16, k-slot grp4*8 + e <-> d = ks*32 + grp4*8 + e.
  bf16x8 qreg[D / 32];
  {
    const bf16* qrow = p.q + ((size_t)(q0 + (qvalid ? tq : 0)) * p.hq + head) * D + grp4 * 8;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      bf16x8 t = *(const bf16x8*)(qrow + ks * 32);
      if (!qvalid) t = bf16x8{};
      qreg[ks] = t;
    }
  }

  // Paged: the split's page ids, clamped to the cache so that a bad table
  // entry cannot send a load outside it.
  int lg = 0, pbase = 0;
  if constexpr (PAGED) {
    lg = p.lg_page;
    pbase = key_lo >> lg;
    const int npg = key_hi > key_lo ? ((key_hi - 1) >> lg) - pbase + 1 : 0;   // <= kPageSlots
    const int32_t* trow = p.block_table + (long long)b * p.max_pages + pbase;
    for (int i = tid; i < npg; i += kThreads) pages[i] = (int)min((unsigned)trow[i], (unsigned)(p.num_pages - 1));
    __syncthreads();
  }

  f32x4 acc[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) acc[i] = f32x4{};
  float m_run = neg_inf();
  float l_run = 0.f;

  const int n_steps = (key_hi - key_lo + kStep - 1) / kStep;

  // Registers for one step: K as MFMA A operands, V rows on their way to LDS.
  // Keys past the split end are clamped to its last key (unconditional loads:
  // a per-lane zero-fill would force a wait on every outstanding load); the
  // mask gives them probability 0. Two register sets keep two steps of loads
  // in flight per wave while a third is computed.
  typedef u32x4 KRegs[S::KREGS];
  typedef u32x4 VRegs[S::VREGS];
  KRegs kA, kB;
  VRegs vA, vB;
  const size_t kv_stride = (size_t)p.hkv * D;
  const bf16* kg = p.k + ((size_t)k0 * p.hkv + g) * D;
  const bf16* vg = p.v + ((size_t)k0 * p.hkv + g) * D;
  // K and V rows are loaded whole (each instruction covers 64 / (D/8) rows of
  // contiguous bytes) and parked in the wave's LDS buffers.
  auto gload = [&](KRegs& kr, VRegs& vr, int st) {
    const int base = key_lo + st * kStep;
    if constexpr (PAGED) {
      // Steps start at multiples of 32 and pages hold a power of two >= 16
      // keys, so keys 0-15 of a step lie in the page of `base` and keys 16-31
      // (clamped to the last key) in the page of min(base + 16, last key).
      const size_t page_elems = kv_stride << lg;
      const size_t lo_off = (size_t)pages[(base >> lg) - pbase] * page_elems;
      const size_t hi_off = (size_t)pages[(min(base + 16, key_hi - 1) >> lg) - pbase] * page_elems;
      const int in_page = (1 << lg) - 1;
#pragma unroll
      for (int i = 0; i < S::VREGS; ++i) {
        const int f = i * 64 + lane;
        const int key = min(base + f / (D / 8), key_hi - 1);
        // In-page offset: fits 32 bits (page_size * hkv * D < 2^31, checked on the host).
        const uint32_t off = (uint32_t)(key & in_page) * (uint32_t)kv_stride + (f % (D / 8)) * 8;
        const size_t pg = (i * (64 / (D / 8)) < 16) ? lo_off : hi_off;
        kr[i] = __builtin_nontemporal_load((const u32x4*)(kg + pg + off));
        vr[i] = __builtin_nontemporal_load((const u32x4*)(vg + pg + off));
      }
    } else {
#pragma unroll
      for (int i = 0; i < S::VREGS; ++i) {
        const int f = i * 64 + lane;
        const int key = min(base + f / (D / 8), key_hi - 1);
        const size_t off = (size_t)key * kv_stride + (f % (D / 8)) * 8;
        // Streaming loads: every K/V byte is read once (measured 9% faster on
        // MI355X at the decode shape than plain loads).
        kr[i] = __builtin_nontemporal_load((const u32x4*)(kg + off));
        vr[i] = __builtin_nontemporal_load((const u32x4*)(vg + off));
      }
    }
  };
  const int tr_i = lane & 15;
  const int tr_key = grp4 * 4 + (tr_i >> 2);
  const int tr_d = 4 * (tr_i & 3);
  // A wave's LDS operations execute in issue order, so one V buffer per wave is
  // enough: the next step's writes cannot overtake this step's reads.
  char VFA_LDS* vb = lds + wave * S::WAVE_BYTES;
  char VFA_LDS* kbw = vb + kStep * S::VSTR;

  auto step = [&](const KRegs& kr, const VRegs& vr, int st) {
#pragma unroll
    for (int i = 0; i < S::VREGS; ++i) {
      const int f = i * 64 + lane;
      *(u32x4 VFA_LDS*)(vb + (f / (D / 8)) * S::VSTR + (f % (D / 8)) * 16) = vr[i];
      *(u32x4 VFA_LDS*)(kbw + (f / (D / 8)) * S::KSTR + (f % (D / 8)) * 16) = kr[i];
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    // S^T for two 16-key blocks: lane holds keys sb*16 + grp4*4 + r of column c16.
    // A operand: row = key sb*16 + c16, k-slot grp4*8 + e <-> d = ks*32 + grp4*8 + e.
    f32x4 s[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      s[sb] = f32x4{};
      const char VFA_LDS* krow = kbw + (sb * 16 + c16) * S::KSTR + grp4 * 16;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
        s[sb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8 VFA_LDS*)(krow + ks * 64), qreg[ks], s[sb],
                                                        0, 0, 0);
    }

    const int base = key_lo + st * kStep;
    const bool need_mask = (base + kStep > key_hi) || (CAUSAL && base + kStep - 1 > diag);
    if (need_mask) {
      const int lim = CAUSAL ? min(key_hi - 1, tq + diag) : key_hi - 1;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (base + sb * 16 + grp4 * 4 + r > lim) s[sb][r] = neg_inf();
    }

    float mx = neg_inf();
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[sb][r]);
    mx = fmaxf(mx, xor_shuffle(mx, 16));
    mx = fmaxf(mx, xor_shuffle(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == neg_inf()) ? 0.f : m_new;
    const float alpha = fast_exp2((m_run - m_use) * scale_log2);
    const float ms = m_use * scale_log2;
    m_run = m_new;

    float e[8];
    float psum = 0.f;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      e[x] = fast_exp2(__builtin_fmaf(s[x >> 2][x & 3], scale_log2, -ms));
      psum += e[x];
    }
    l_run = l_run * alpha + psum;
    // P^T (B operand): k-slot grp4*8 + x <-> key (x / 4) * 16 + grp4 * 4 + x % 4.
    bf16x2 p01 = f32x2_to_bf16x2(e[0], e[1]);
    bf16x2 p23 = f32x2_to_bf16x2(e[2], e[3]);
    bf16x2 p45 = f32x2_to_bf16x2(e[4], e[5]);
    bf16x2 p67 = f32x2_to_bf16x2(e[6], e[7]);
    const bf16x8 p = bf16x8{p01[0], p01[1], p23[0], p23[1], p45[0], p45[1], p67[0], p67[1]};

#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[db][r] *= alpha;

    // The V rows written above must be visible to the transposed reads of the
    // same wave; LDS executes one wave's operations in order, so a compiler
    // barrier is enough.
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    const char VFA_LDS* vrow = vb + tr_key * S::VSTR + tr_d * 2;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      bf16x8 a = tr_pair(vrow + db * 32, vrow + 16 * S::VSTR + db * 32);
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, p, acc[db], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  };

  // This wave's steps are wave, wave + 4, ...; sets A and B alternate.
  int st = wave;
  if (st < n_steps) gload(kA, vA, st);
  if (st + kWaves < n_steps) gload(kB, vB, st + kWaves);
  for (; st < n_steps; st += 2 * kWaves) {
    step(kA, vA, st);
    if (st + 2 * kWaves < n_steps) gload(kA, vA, st + 2 * kWaves);
    if (st + kWaves < n_steps) {
      step(kB, vB, st + kWaves);
      if (st + 3 * kWaves < n_steps) gload(kB, vB, st + 3 * kWaves);
    }
  }

  // Per-wave totals: the four lanes of a column hold disjoint keys.
  float l_tot = l_run + xor_shuffle(l_run, 16);
  l_tot += xor_shuffle(l_tot, 32);

  __syncthreads();   // all waves are done with their V buffers; reuse LDS for the merge
  float VFA_LDS* m_lse = (float VFA_LDS*)lds;                       // [kWaves][kCols]
  float VFA_LDS* m_o = m_lse + kWaves * kCols;                      // [kWaves][kCols][D]
  if (grp4 == 0)
    m_lse[wave * kCols + c16] = l_tot > 0.f ? m_run * p.scale + fast_log2(l_tot) * kLn2 : neg_inf();
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) m_o[(wave * kCols + c16) * D + db * 16 + grp4 * 4 + r] = acc[db][r] * inv;
  __syncthreads();

  // 256 threads = 16 columns x 16 threads; each thread merges D/16 values of one column.
  const int mc = tid >> 4;
  const int md = (tid & 15) * (D / 16);
  int colm;
  bool mvalid;
  if constexpr (PAGED) {
    colm = cg * kCols + mc;
    mvalid = colm < lq * grp;
  } else {
    colm = mc;
    mvalid = mc < (kCols / grp) * grp && (mc / grp) < lq;
  }
  if (!mvalid) return;
  float lw[kWaves], w[kWaves];
#pragma unroll
  for (int i = 0; i < kWaves; ++i) lw[i] = m_lse[i * kCols + mc];
  const float lse_m = merge_weights<kWaves>(lw, kWaves, w);
  f32x4 o[D / 64];
#pragma unroll
  for (int x = 0; x < D / 64; ++x) {
    o[x] = f32x4{};
#pragma unroll
    for (int i = 0; i < kWaves; ++i)
#pragma unroll
      for (int y = 0; y < 4; ++y) o[x][y] += w[i] * m_o[(i * kCols + mc) * D + md + x * 4 + y];
  }
  const long long row = (long long)(q0 + colm / grp) * p.hq + g * grp + colm % grp;
  if (PAGED && p.n_splits == 1) {                                  // the only split: final result
    store_row<D, OutT>(p.out, p.lse, row, md, (tid & 15) == 0, o, lse_m);
    return;
  }
  float* dst = p.ws_o + ((long long)split * p.rows_total + row) * D + md;
#pragma unroll
  for (int x = 0; x < D / 64; ++x) *(f32x4*)(dst + x * 4) = o[x];
  if ((tid & 15) == 0) p.ws_lse[(long long)split * p.rows_total + row] = lse_m;
}

// Merge the splits of every row with the AttentionUpdate rule. Grid: (row
// chunk, sequence); one row per TPR lanes with 16-byte loads. NS is a
// compile-time bound on the split count so that every lse and partial load of
// a row is issued before the first one is consumed (NS = 0: streaming loop
// for very long key sets).
template <int D, int NS, typename OutT>
__global__ __launch_bounds__(256) void attn_decode_combine_kernel(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, const int32_t* __restrict__ seqused_k,
    int max_seqlen_k, int hq, int chunk, int n_splits, long long rows_total, const float* __restrict__ ws_o,
    const float* __restrict__ ws_lse, OutT* __restrict__ out, float* __restrict__ lse) {
  constexpr int TPR = D / 4;
  constexpr int RPB = 256 / TPR;
  const int b = blockIdx.y;
  const int q0 = cu_q[b];
  const int rows_b = (cu_q[b + 1] - q0) * hq;
  const int r_in = blockIdx.x * RPB + threadIdx.x / TPR;
  if (r_in >= rows_b) return;
  const long long row = (long long)q0 * hq + r_in;
  const int c4 = (threadIdx.x % TPR) * 4;
  // Keys of the sequence: from cu_seqlens_k, or (paged) from seqused_k clamped
  // as the split kernel clamps it.
  const int lk = seqused_k ? min(max(seqused_k[b], 0), max_seqlen_k) : cu_k[b + 1] - cu_k[b];
  // Splits written for this sequence (keys past a too-small max_seqlen_k bound
  // were never split: the count is capped at the workspace's split count).
  const int n = lk > 0 ? min((lk + chunk - 1) / chunk, n_splits) : 0;
  f32x4 o = f32x4{};
  float lse_m;
  if constexpr (NS > 0) {
    float l[NS], w[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) l[i] = i < n ? ws_lse[(long long)i * rows_total + row] : neg_inf();
    lse_m = merge_weights<NS>(l, n, w);
#pragma unroll
    for (int i0 = 0; i0 < NS; i0 += 8) {
      f32x4 x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        x[i] = i0 + i < n ? *(const f32x4*)(ws_o + ((long long)(i0 + i) * rows_total + row) * D + c4) : f32x4{};
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int y = 0; y < 4; ++y) o[y] += w[i0 + i] * x[i][y];
    }
  } else {
    const MergeStats st = merge_stats(ws_lse + row, rows_total, n);
    for (int s = 0; s < n; ++s) {
      const float w = merge_weight(ws_lse[(long long)s * rows_total + row], st);
      const f32x4 x = *(const f32x4*)(ws_o + ((long long)s * rows_total + row) * D + c4);
#pragma unroll
      for (int y = 0; y < 4; ++y) o[y] += w * x[y];
    }
    lse_m = st.lse_m;
  }
  OutT* dst = out + row * D + c4;
#pragma unroll
  for (int y = 0; y < 4; ++y) dst[y] = from_f32<OutT>(o[y]);
  if (c4 == 0) lse[row] = lse_m;
}

// Combine launch shared by both layouts (seqused_k == NULL: contiguous).
template <int D, typename OutT>
void launch_combine(const int32_t* cu_q, const int32_t* cu_k, const int32_t* seqused_k, int max_seqlen_k,
                    int batch, int max_seqlen_q, int hq, const DecodePlan& p, long long rows, const float* ws_o,
                    const float* ws_lse, void* out, float* lse, void* stream) {
  constexpr int RPB = 256 / (D / 4);
  const long long max_rows = (long long)max_seqlen_q * hq;
  const dim3 grid((unsigned)((max_rows + RPB - 1) / RPB), (unsigned)batch);
  hipStream_t st = (hipStream_t)stream;
#define VFA_COMBINE(NS)                                                                                    \
  hipLaunchKernelGGL((attn_decode_combine_kernel<D, NS, OutT>), grid, dim3(256), 0, st, cu_q, cu_k, seqused_k, \
                     max_seqlen_k, hq, p.chunk, p.n_splits, rows, ws_o, ws_lse, (OutT*)out, lse)
  if (p.n_splits <= 8) VFA_COMBINE(8);
  else if (p.n_splits <= 16) VFA_COMBINE(16);
  else if (p.n_splits <= 32) VFA_COMBINE(32);
  else if (p.n_splits <= 64) VFA_COMBINE(64);
  else VFA_COMBINE(0);
#undef VFA_COMBINE
}

template <int D, bool CAUSAL, typename OutT>
int launch_t(const AttnArgs& a, const DecodePlan& p) {
  const long long rows = (long long)a.total_q * a.hq;
  float* ws_o = (float*)a.workspace;
  float* ws_lse = ws_o + (size_t)p.n_splits * rows * D;
  const long long blocks = (long long)p.n_splits * a.batch * a.hkv;
  if (blocks > 0x7fffffffLL) return -1;
  SplitArgs s{};
  s.q = (const bf16*)a.q; s.k = (const bf16*)a.k; s.v = (const bf16*)a.v;
  s.cu_q = a.cu_q; s.cu_k = a.cu_k; s.causal_off = a.causal_off;
  s.batch = a.batch; s.hq = a.hq; s.hkv = a.hkv; s.grp = a.grp; s.chunk = p.chunk; s.n_splits = p.n_splits;
  s.n_cg = 1; s.rows_total = rows;
  s.scale = a.scale; s.scale_log2 = a.scale * kLog2e;
  s.ws_o = ws_o; s.ws_lse = ws_lse;
  hipLaunchKernelGGL((attn_decode_split_kernel<D, CAUSAL, false, float>), dim3((unsigned)blocks), dim3(kThreads),
                     0, (hipStream_t)a.stream, s);
  if (hipGetLastError() != hipSuccess) return -1;
  launch_combine<D, OutT>(a.cu_q, a.cu_k, nullptr, a.max_seqlen_k, a.batch, a.max_seqlen_q, a.hq, p, rows, ws_o,
                          ws_lse, a.out, a.lse, a.stream);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int D, bool CAUSAL, typename OutT>
int launch_paged_t(const PagedArgs& a, const PagedPlan& p) {
  if (p.chunk > kMaxChunk || a.page_size < kMinPage) return -1;
  const long long blocks = (long long)p.n_splits * a.batch * a.hkv * p.n_cg;
  if (blocks > 0x7fffffffLL) return -1;
  const long long rows = (long long)a.total_q * a.hq;
  SplitArgs s{};
  s.q = (const bf16*)a.q; s.k = (const bf16*)a.k_cache; s.v = (const bf16*)a.v_cache;
  s.cu_q = a.cu_q; s.seqused_k = a.seqused_k; s.block_table = a.block_table;
  s.batch = a.batch; s.hq = a.hq; s.hkv = a.hkv; s.grp = a.grp; s.chunk = p.chunk; s.n_splits = p.n_splits;
  s.max_pages = a.max_pages; s.num_pages = a.num_pages; s.max_seqlen_k = a.max_seqlen_k; s.n_cg = p.n_cg;
  s.lg_page = 0;
  while ((1 << s.lg_page) < a.page_size) ++s.lg_page;
  s.rows_total = rows;
  s.scale = a.scale; s.scale_log2 = a.scale * kLog2e;
  s.out = a.out; s.lse = a.lse;
  if (p.n_splits > 1) {
    s.ws_o = (float*)a.workspace;
    s.ws_lse = s.ws_o + (size_t)p.n_splits * rows * D;
  }
  hipLaunchKernelGGL((attn_decode_split_kernel<D, CAUSAL, true, OutT>), dim3((unsigned)blocks), dim3(kThreads),
                     0, (hipStream_t)a.stream, s);
  if (hipGetLastError() != hipSuccess) return -1;
  if (p.n_splits > 1) {
    const DecodePlan dp{true, p.chunk, p.n_splits, p.ws_bytes};
    launch_combine<D, OutT>(a.cu_q, nullptr, a.seqused_k, a.max_seqlen_k, a.batch, a.max_seqlen_q, a.hq, dp, rows,
                            s.ws_o, s.ws_lse, a.out, a.lse, a.stream);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_attn_decode_bf16(const AttnArgs& a, const DecodePlan& p) {
  const bool f32out = a.out_dtype == 0;
  if (a.head_dim == 128) {
    if (a.causal) return f32out ? launch_t<128, true, float>(a, p) : launch_t<128, true, bf16>(a, p);
    return f32out ? launch_t<128, false, float>(a, p) : launch_t<128, false, bf16>(a, p);
  }
  if (a.causal) return f32out ? launch_t<64, true, float>(a, p) : launch_t<64, true, bf16>(a, p);
  return f32out ? launch_t<64, false, float>(a, p) : launch_t<64, false, bf16>(a, p);
}

int launch_paged_decode_bf16(const PagedArgs& a, const PagedPlan& p) {
  const bool f32out = a.out_dtype == 0;
  if (a.head_dim == 128) {
    if (a.causal) return f32out ? launch_paged_t<128, true, float>(a, p) : launch_paged_t<128, true, bf16>(a, p);
    return f32out ? launch_paged_t<128, false, float>(a, p) : launch_paged_t<128, false, bf16>(a, p);
  }
  if (a.causal) return f32out ? launch_paged_t<64, true, float>(a, p) : launch_paged_t<64, true, bf16>(a, p);
  return f32out ? launch_paged_t<64, false, float>(a, p) : launch_paged_t<64, false, bf16>(a, p);
}

}  // namespace vfa
