// Varlen attention forward, bf16 inputs, on gfx950 bf16 MFMA with fp32 accumulation.
//
// What is computed: for every packed sequence, query head h and query i,
// softmax(scale * q_i K^T) V over the visible keys, plus the natural-log
// log-sum-exp of the scaled scores. Layout TND with int32 cu_seqlens ("From
// GPU to NPU: Qwen3-Embedding on Ascend", core optimisation 1 and section
// 2.1); query head h reads kv head h / G ("native GQA", core optimisation 5 of
// the same page); causal mask aligned bottom-right (with Lq == Lk it is the
// page's triu(diagonal=1)-is-masked mask).
//
// This file holds the kernel for short sequences and the prefill dispatch:
// batches whose sequences average at least eight 256-column query tiles go to
// attn_fwd_overlap.hip (eight waves, the softmax overlapped with the matrix
// products, a persistent grid); shorter ones run here.
//
// Work decomposition. One workgroup = one (sequence b, kv head g, query tile
// m). Its 128 "columns" are the G query heads of kv head g times 128 / G
// consecutive tokens, so every K/V sub-block brought into LDS serves all G
// heads (no repeat_interleave of K/V is ever materialised). Workgroups are
// dispatched round-robin over the 8 XCDs, each with its own L2: XCD x takes
// the (sequence, kv head) pairs x, x + 8, ... one after another and each
// pair's query tiles back to back, last tile first (causal rows grow with
// the tile index), so the workgroups resident on an XCD at one time mostly
// share one pair's K/V in L2. Key sub-blocks that the causal mask hides from
// every row of the workgroup are never visited; only sub-blocks that
// straddle the diagonal or the sequence end are masked.
//
// A workgroup here lives for a few 32-key sub-blocks (the embedding
// workload's sequences hold 32-512 tokens), so its own load and store
// latency is what sets the time, and other workgroups on the same CU are
// what hides it. The kernel is therefore sized for three resident
// workgroups per CU (149 VGPRs, 37.9 KB of LDS): four waves of 32 query
// columns, one 32-key sub-block per step, K and V double-buffered in LDS and
// filled straight from global memory (buffer_load ... lds, one dword per
// lane and one padded 256-byte line per load), so no registers stage them.
//
// Per wave, per 32-key sub-block:
//   S^T = K Q^T   : v_mfma_f32_32x32x16_bf16, A = K rows from LDS (16 B
//                   reads), B = Q^T held in registers.
//   online softmax: each lane owns one column (query row) in the S^T
//                   accumulator, so the running statistics stay lane-local
//                   apart from one exchange with lane ^ 32 for the max.
//   O^T += V^T P^T: A = V^T read with ds_read_b64_tr_b16 (gfx950 LDS
//                   transpose read) straight from the row-major V tile,
//                   B = P^T converted to bf16 in registers.
// The first sub-block has no history, so its exact max becomes the softmax
// reference at once and its PV products start O. bf16 output leaves through
// LDS as whole rows (16 lanes to a 256-byte row) instead of 32-byte pieces
// of 32 rows per store.
//
// Batches whose key sets pass 4 GiB per sequence also come here: the
// persistent kernel addresses a sequence through one 32-bit buffer range,
// and this one makes a buffer per sub-block.
#include <type_traits>

#include "common.h"
#include "launch.h"

// Kernel-body lambdas are forced inline: one left out of line takes the
// register arrays it touches by reference, which moves them to scratch.
#define VFA_INLINE __attribute__((always_inline))

namespace vfa {
namespace {

constexpr int kXcds = 8;             // MI355X: 8 XCDs, blocks dispatched round-robin

__device__ __forceinline__ bf16x8 lds_read_b128(const char VFA_LDS* p) { return *(const bf16x8 VFA_LDS*)p; }

__device__ __forceinline__ bf16x8 lds_read_tr_pair(const char VFA_LDS* p0, const char VFA_LDS* p1) {
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 VFA_LDS*)p0);
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 VFA_LDS*)p1);
  typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8;
  i16x8 r = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, r);
}

// LDS layout. The global-to-LDS loads write 256 contiguous bytes each (64
// lanes x 4 bytes): a "line" of RPD = 256 / (2 D) key rows (one at D = 128,
// two at D = 64). Lines are padded as measured conflict-free on gfx950: +16
// bytes for the per-lane-row ds_read_b128 of K, +64 bytes for the transposed
// reads of V.
template <int D>
struct ShortSmem {
  static constexpr int RPD = 256 / (D * 2);      // rows per 256-byte load line
  static constexpr int LINES = 32 / RPD;          // lines per sub-block
  static constexpr int KLSTR = RPD * D * 2 + 16;  // line stride in the K buffer
  static constexpr int VLSTR = RPD * D * 2 + 64;  // line stride in the V buffer
  static constexpr int KBUF = LINES * KLSTR;
  static constexpr int VBUF = LINES * VLSTR;
  static constexpr int TOTAL = 2 * (KBUF + VBUF);  // K and V, two sub-blocks each
  static constexpr int PW = LINES / 4;            // lines per wave per tensor
  // Byte offset of key row r inside a sub-block buffer.
  static __device__ __forceinline__ int krow(int r) { return (r / RPD) * KLSTR + (r % RPD) * (D * 2); }
  static __device__ __forceinline__ int vrow(int r) { return (r / RPD) * VLSTR + (r % RPD) * (D * 2); }
};

template <int D, bool CAUSAL, typename OutT>
__global__ __attribute__((amdgpu_flat_work_group_size(1, 256), amdgpu_waves_per_eu(3, 3))) void
attn_fwd_short_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
                     const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
                     const int32_t* __restrict__ coff, int batch, int hq, int hkv, int grp, int tokw, int n_mtiles,
                     float scale, float scale_log2, OutT* __restrict__ out, float* __restrict__ lse) {
  using S = ShortSmem<D>;
  __shared__ __attribute__((aligned(16))) char smem[S::TOTAL];
  char VFA_LDS* kbuf = (char VFA_LDS*)smem;
  char VFA_LDS* vbuf = kbuf + 2 * S::KBUF;

  const int per_m = batch * hkv;
  const int id = blockIdx.x;
  const int xcd = id % kXcds;
  const int slot = id / kXcds;
  const int bg = (slot / n_mtiles) * kXcds + xcd;
  if (bg >= per_m) return;
  const int m = n_mtiles - 1 - slot % n_mtiles;
  const int b = bg / hkv;
  const int g = bg % hkv;
  const int q0 = cu_q[b];
  const int lq = cu_q[b + 1] - q0;
  const int tok_lo = m * tokw;
  if (tok_lo >= lq) return;
  const int k0 = cu_k[b];
  const int lk = cu_k[b + 1] - k0;
  const int tok_hi = min(lq, tok_lo + tokw);
  const int diag = causal_diag(coff, b, lq, lk);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int col = wave * 32 + l32;
  const bool colvalid = col < tokw * grp;
  const int hg = colvalid ? col / tokw : 0;
  const int tq = tok_lo + (colvalid ? col - hg * tokw : 0);
  const int head = g * grp + hg;
  const bool qvalid = colvalid && tq < lq;

  const int n_end = CAUSAL ? min(lk, tok_hi + diag) : lk;
  const int n_sub = n_end > 0 ? (n_end + 31) / 32 : 0;
  // Sub-blocks [0, j_full) hold only keys that every row of the workgroup sees: no mask.
  int j_full = lk / 32;
  if (CAUSAL) j_full = min(j_full, max(0, (tok_lo + diag + 1) / 32));

  // Global-to-LDS loads. Each call makes one buffer per tensor over the 32
  // key rows of kv head g in the sub-block, its size ending at the sequence's
  // last key, so rows past the end read as zero (those keys are masked).
  // Rebasing per sub-block keeps every byte offset below 32 rows whatever the
  // sequence length. Wave w moves lines w * PW .. w * PW + PW - 1 of K and of
  // V; lane L brings 4 bytes of key row L / (64 / RPD) of the line, the row
  // offset of each line going to the scalar offset and its LDS address to M0.
  const uint32_t row_bytes = (uint32_t)hkv * D * sizeof(bf16);
  const size_t sub_elems = (size_t)32 * hkv * D;
  const bf16* kseq = k + ((size_t)k0 * hkv + g) * D;
  const bf16* vseq = v + ((size_t)k0 * hkv + g) * D;
  const uint32_t l_voff = (uint32_t)(lane / (64 / S::RPD)) * row_bytes + (uint32_t)(lane % (64 / S::RPD)) * 4u;
  const uint32_t w_soff = (uint32_t)wave * S::PW * S::RPD * row_bytes;
  auto dma = [&](int sub, int bsel) VFA_INLINE {
    // readfirstlane keeps the (uniform) size in an SGPR: a size the compiler
    // leaves in a VGPR would make it loop over lanes for every load.
    const uint32_t nrec =
        (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)min(max(lk - sub * 32, 0), 32) * row_bytes));
    const __amdgpu_buffer_rsrc_t krsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(kseq + sub * sub_elems), (short)0, (int)nrec, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(vseq + sub * sub_elems), (short)0, (int)nrec, 0x00020000);
    char VFA_LDS* kd = kbuf + bsel * S::KBUF + wave * S::PW * S::KLSTR;
    char VFA_LDS* vd = vbuf + bsel * S::VBUF + wave * S::PW * S::VLSTR;
#pragma unroll
    for (int i = 0; i < S::PW; ++i) {
      const uint32_t so = w_soff + (uint32_t)(i * S::RPD) * row_bytes;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krsrc, (VFA_LDS void*)(kd + i * S::KLSTR), 4, l_voff, so, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrsrc, (VFA_LDS void*)(vd + i * S::VLSTR), 4, l_voff, so, 0, 0);
    }
  };

  // Q^T as the B operand: column = query, k-slot (half*8 + e) <-> d = ks*16 + half*8 + e.
  // A column without a query reads the sequence's first query: its results are never stored.
  bf16x8 qreg[D / 16];
  {
    const bf16* qrow = q + ((size_t)(q0 + (qvalid ? tq : 0)) * hq + head) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qreg[ks] = *(const bf16x8*)(qrow + ks * 16);
  }
  // The Q loads go out first; sub-block 0's loads follow (they run even for a
  // workgroup without keys, whose rows then read as zero and are never used).
  __builtin_amdgcn_sched_barrier(0);
  dma(0, 0);

  const int tr_grp = lane >> 4;
  const int tr_i = lane & 15;
  const int tr_key = (tr_grp >> 1) * 4 + (tr_i >> 2);
  const int tr_d = (tr_grp & 1) * 16 + 4 * (tr_i & 3);
  // Transposed V reads (ds_read_b64_tr_b16): in each 16-lane group, lane i
  // receives d = dbase + i for 4 consecutive keys.
  const int k_lane = S::krow(l32) + half * 16;
  const int v_lane = S::vrow(tr_key) + tr_d * 2;

  f32x16 acc[D / 32];
  // Per column: reference max m_run (raw score units; -inf until the column
  // has seen a visible key), the same pre-scaled to log2 units, and the
  // running sum of probabilities against it. The reference only has to keep
  // probabilities finite (bf16 P and the fp32 sums share fp32's exponent
  // range): the fast path exponentiates against the current reference and
  // only a sum above 2^32, or a column without a reference, moves it to the
  // exact running max (rescaling O and the sum) and recomputes.
  float m_run = neg_inf(), mref = 0.f, l_run = 0.f;
  constexpr float kSumLimit = 4294967296.f;

  // One 32-key sub-block. The first has no history: its exact max becomes
  // the reference directly (O and the sum are zero, so nothing is rescaled)
  // and its PV products start O.
  auto sub_block = [&](int j, auto first_c) VFA_INLINE {
    constexpr bool FIRST = decltype(first_c)::value;
    const int bsel = j & 1;
    // The other buffer held sub-block j - 1, which every wave finished before
    // the barrier that ended iteration j - 1.
    if (j + 1 < n_sub) dma(j + 1, bsel ^ 1);
    f32x16 s = f32x16{};
    const char VFA_LDS* krow = kbuf + bsel * S::KBUF + k_lane;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read_b128(krow + ks * 32), qreg[ks], s, 0, 0, 0);
    if (j >= j_full) {
      // Keys past the row's last visible one, as offsets from this lane's first key.
      const int rel = (CAUSAL ? min(lk - 1, tq + diag) : lk - 1) - (j * 32 + half * 4);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if ((r >> 2) * 8 + (r & 3) > rel) s[r] = neg_inf();
    }
    // Probabilities against the current reference and their fp32 sum (of the
    // unrounded values, so lse stays fp32-accurate), summed as a tree.
    float e[16], ts;
    auto exps = [&]() VFA_INLINE {
#pragma unroll
      for (int r = 0; r < 16; ++r) e[r] = fast_exp2(__builtin_fmaf(s[r], scale_log2, -mref));
      float t8[8], t4[4];
#pragma unroll
      for (int r = 0; r < 8; ++r) t8[r] = e[r] + e[r + 8];
#pragma unroll
      for (int r = 0; r < 4; ++r) t4[r] = t8[r] + t8[r + 4];
      ts = (t4[0] + t4[2]) + (t4[1] + t4[3]);
    };
    // The sub-block's exact max per column; the other lane half holds the
    // other keys of the same column.
    auto block_max = [&]() VFA_INLINE {
      float x = neg_inf();
#pragma unroll
      for (int r = 0; r < 16; ++r) x = fmaxf(x, s[r]);
      auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
      return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    };
    if constexpr (FIRST) {
      m_run = block_max();
      mref = m_run == neg_inf() ? 0.f : m_run * scale_log2;
      exps();
      l_run = ts;
    } else {
      exps();
      if (__builtin_amdgcn_ballot_w64(!(ts <= kSumLimit) || m_run == neg_inf())) {
        const float m_new = fmaxf(m_run, block_max());
        // Unchanged references scale by exactly 1 (m_run may be -inf); one moving
        // up from -inf scales the (zero) history by 0.
        const float alpha = m_new == m_run ? 1.f : fast_exp2((m_run - m_new) * scale_log2);
        m_run = m_new;
        mref = m_new == neg_inf() ? 0.f : m_new * scale_log2;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
        exps();
      }
      l_run += ts;
    }
    // P^T (B operand) for the sub-block's two 16-key steps.
    bf16x8 pp[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      bf16x2 pr[4];
#pragma unroll
      for (int y = 0; y < 4; ++y) pr[y] = f32x2_to_bf16x2(e[hh * 8 + 2 * y], e[hh * 8 + 2 * y + 1]);
      pp[hh] = bf16x8{pr[0][0], pr[0][1], pr[1][0], pr[1][1], pr[2][0], pr[2][1], pr[3][0], pr[3][1]};
    }
    const char VFA_LDS* vb = vbuf + bsel * S::VBUF + v_lane;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const char VFA_LDS* vrow = vb + S::vrow(hh * 16);
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read_tr_pair(vrow + db * 64, vrow + S::vrow(8) + db * 64),
                                                          pp[hh], (FIRST && hh == 0) ? f32x16{} : acc[db], 0, 0, 0);
    }
    // Sub-block j + 1 has landed (this wave's share), and nobody reads buffer j any more.
    asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };

  // Sub-block 0 (and Q) landed in every wave, then the workgroup barrier.
  asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (n_sub > 0) {
    sub_block(0, std::true_type{});
    for (int j = 1; j < n_sub; ++j) sub_block(j, std::false_type{});
  } else {
#pragma unroll
    for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};
  }

  // Epilogue: combine the two lane halves' partial sums, normalise, store.
  // A lane holds, per 32-dim block and group g4, the 4 dims g4*8 + half*4 ..
  const float l_tot = l_run + xor_shuffle(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const size_t row = (size_t)(q0 + tq) * hq + head;
  if constexpr (sizeof(OutT) == 2) {
    // bf16: lanes i and i + 32 (the same query) trade one group of each pair,
    // so that each holds 8 contiguous dims (16 B); the wave lays its 32 rows
    // out in LDS (the K/V buffers, which every wave has finished with at the
    // last barrier) and then stores whole rows, D * 2 / 16 lanes to a row,
    // instead of 32-byte pieces of 32 rows per store. Each row's 16-byte pad
    // carries its output row index (-1: not stored).
    constexpr int RS = D * 2 + 16;
    static_assert(4 * 32 * RS <= S::TOTAL, "the four waves' rows fit in the K/V buffers");
    char VFA_LDS* ot = (char VFA_LDS*)smem + wave * 32 * RS;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const f32x16& a = acc[db];
      auto pk = [&](int r) VFA_INLINE {
        return __builtin_bit_cast(uint32_t, f32x2_to_bf16x2(a[r] * inv, a[r + 1] * inv));
      };
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        const int ga = 2 * gp, gb = 2 * gp + 1;   // the groups the lower and upper half keep
        const uint32_t a0 = pk(ga * 4), a1 = pk(ga * 4 + 2), b0 = pk(gb * 4), b1 = pk(gb * 4 + 2);
        // The swap trades lanes 32-63 of its first operand with lanes 0-31 of
        // its second, which leaves both halves holding their 8 dims in order:
        // a lower lane group ga (its own 4, then its partner's), an upper lane
        // group gb (its partner's 4, then its own).
        const auto s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
        *(u32x4 VFA_LDS*)(ot + l32 * RS + (db * 32 + (2 * gp + half) * 8) * 2) = u32x4{s0[0], s1[0], s0[1], s1[1]};
      }
    }
    if (half == 0) *(long long VFA_LDS*)(ot + l32 * RS + D * 2) = qvalid ? (long long)row : -1LL;
    constexpr int LPR = D * 2 / 16;   // lanes per row
    constexpr int RPI = 64 / LPR;     // rows per store
    const int rsub = lane / LPR, chunk = lane % LPR;
    // All reads first (the accumulators are dead by now), then the stores.
    long long orow_i[32 / RPI];
    u32x4 ov[32 / RPI];
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const char VFA_LDS* rp = ot + (i * RPI + rsub) * RS;
      orow_i[i] = *(const long long VFA_LDS*)(rp + D * 2);
      ov[i] = *(const u32x4 VFA_LDS*)(rp + chunk * 16);
    }
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i)
      if (orow_i[i] >= 0) *(u32x4*)((char*)out + orow_i[i] * (D * 2) + chunk * 16) = ov[i];
  } else {
    OutT* orow = out + row * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const f32x16& a = acc[db];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 val{a[g4 * 4 + 0] * inv, a[g4 * 4 + 1] * inv, a[g4 * 4 + 2] * inv, a[g4 * 4 + 3] * inv};
        f32x4* dst = (f32x4*)(orow + db * 32 + g4 * 8 + half * 4);
        if (qvalid) *dst = val;
      }
    }
  }
  if (qvalid && half == 0) lse[row] = l_tot > 0.f ? m_run * scale + fast_log2(l_tot) * kLn2 : neg_inf();
}

template <int D, bool CAUSAL, typename OutT>
int launch_short(const AttnArgs& a) {
  const int tokw = 128 / a.grp;
  const int n_mtiles = (a.max_seqlen_q + tokw - 1) / tokw;
  const long long pairs_per_xcd = ((long long)a.batch * a.hkv + kXcds - 1) / kXcds;
  const long long blocks = (long long)n_mtiles * pairs_per_xcd * kXcds;
  if (blocks <= 0) return 0;
  if (blocks > 0x7fffffffLL) return -1;
  hipLaunchKernelGGL((attn_fwd_short_kernel<D, CAUSAL, OutT>), dim3((unsigned)blocks), dim3(256), 0,
                     (hipStream_t)a.stream, (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, a.cu_q, a.cu_k,
                     a.causal_off, a.batch, a.hq, a.hkv, a.grp, tokw, n_mtiles, a.scale, a.scale * kLog2e,
                     (OutT*)a.out, a.lse);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_attn_fwd_bf16(const AttnArgs& a) {
  if (wide_prefill(a.batch, a.total_q, a.max_seqlen_k, a.hq, a.hkv, a.head_dim)) return launch_attn_fwd_overlap(a);
  const bool f32out = a.out_dtype == 0;
  if (a.head_dim == 128) {
    if (a.causal) return f32out ? launch_short<128, true, float>(a) : launch_short<128, true, bf16>(a);
    return f32out ? launch_short<128, false, float>(a) : launch_short<128, false, bf16>(a);
  }
  if (a.causal) return f32out ? launch_short<64, true, float>(a) : launch_short<64, true, bf16>(a);
  return f32out ? launch_short<64, false, float>(a) : launch_short<64, false, bf16>(a);
}

}  // namespace vfa
