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
// Work decomposition. One workgroup = one (sequence b, kv head g, query tile
// m). Its 128 "columns" are the G query heads of kv head g times 128/G
// consecutive tokens, so every K/V tile brought into LDS serves all G heads
// (no repeat_interleave of K/V is ever materialised). Tiles are walked in
// descending m so the longest causal rows start first. Key tiles that the
// causal mask hides from every row of the workgroup are never visited; only
// tiles that straddle the diagonal or the sequence end are masked.
//
// Per wave (4 waves, 32 columns each), per 64-key tile:
//   S^T = K Q^T   : v_mfma_f32_32x32x16_bf16, A = K rows from LDS (16 B
//                   reads), B = Q^T held in registers for the whole loop.
//   online softmax: each lane owns one column (query row) in the S^T
//                   accumulator, so running max / sum stay lane-local apart
//                   from one exchange with lane ^ 32 for the max.
//   O^T += V^T P^T: A = V^T read with ds_read_b64_tr_b16 (gfx950 LDS
//                   transpose read) straight from the row-major V tile,
//                   B = P^T converted to bf16 in registers.
// K/V tiles are double-buffered in LDS; the next tile's global loads are in
// flight while the current tile is computed.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace vfa {
namespace {

constexpr int kBN = 64;              // keys per tile
constexpr int kXcds = 8;             // MI355X: 8 XCDs, blocks dispatched round-robin

// Workgroup shapes: WAVES waves of 32 query columns each. Four waves (two
// workgroups per CU) suit short sequences; eight waves (one workgroup per CU)
// halve the K/V tile traffic per query column for long ones.
template <int WAVES>
struct Shape {
  static constexpr int THREADS = WAVES * 64;
  static constexpr int COLS = WAVES * 32;
  static constexpr int MIN_BLOCKS = WAVES == 4 ? 2 : 1;
};

// LDS row strides, chosen from measured bank behaviour on gfx950: a 16-byte pad
// makes the per-lane-row ds_read_b128 of K conflict-free; a 64-byte pad makes
// the ds_read_b64_tr_b16 of V conflict-free (a 32-byte pad costs 2x).
template <int D, int THREADS>
struct Smem {
  static constexpr int KSTR = D * 2 + 16;
  static constexpr int VSTR = D * 2 + 64;
  static constexpr int KBYTES = kBN * KSTR;
  static constexpr int VBYTES = kBN * VSTR;
  static constexpr int TOTAL = 2 * (KBYTES + VBYTES);
  static constexpr int CHUNKS = kBN * D / 8;          // 16-byte chunks per tile (per tensor)
  static constexpr int PER_THREAD = CHUNKS / THREADS;
  static_assert(CHUNKS % THREADS == 0, "tile must split evenly over the workgroup");
};

__device__ __forceinline__ bf16x8 lds_read_b128(const char VFA_LDS* p) {
  return *(const bf16x8 VFA_LDS*)p;
}

__device__ __forceinline__ bf16x8 lds_read_tr_pair(const char VFA_LDS* p0, const char VFA_LDS* p1) {
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 VFA_LDS*)p0);
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 VFA_LDS*)p1);
  typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8;
  i16x8 r = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, r);
}

template <int WAVES, int D, bool CAUSAL, typename OutT>
__global__ __launch_bounds__(Shape<WAVES>::THREADS, Shape<WAVES>::MIN_BLOCKS) void attn_fwd_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int batch, int hq, int hkv,
    int grp, int tokw, int n_mtiles, float scale, float scale_log2, OutT* __restrict__ out,
    float* __restrict__ lse) {
  constexpr int kThreads = Shape<WAVES>::THREADS;
  using S = Smem<D, kThreads>;
  __shared__ __attribute__((aligned(16))) char smem[S::TOTAL];
  char VFA_LDS* lds = (char VFA_LDS*)smem;
  char VFA_LDS* kbufs = lds;                      // two K tiles
  char VFA_LDS* vbufs = lds + 2 * S::KBYTES;      // two V tiles

  // Block -> work. Consecutive block ids go round-robin to the 8 XCDs, each
  // with its own L2. XCD x takes the (sequence, kv head) pairs x, x + 8, ...
  // one after another, and for each pair all of its query tiles back to back
  // (last tile first: causal rows grow with the tile index), so the blocks
  // resident on an XCD at one time mostly share one pair's K/V in L2.
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
  const int diag = lk - lq;  // query i sees key j iff j <= i + diag (causal)

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // This lane's query column. Columns past tokw * grp (when grp does not
  // divide the column count) carry no query.
  const int col = wave * 32 + l32;
  const bool colvalid = col < tokw * grp;
  const int hg = colvalid ? col / tokw : 0;
  const int tq = tok_lo + (colvalid ? col - hg * tokw : 0);
  const int head = g * grp + hg;
  const bool qvalid = colvalid && tq < lq;

  // Q^T as the B operand: column = query, k-slot (half*8 + e) <-> d = ks*16 + half*8 + e.
  bf16x8 qreg[D / 16];
  {
    const bf16* qrow = q + ((size_t)(q0 + (qvalid ? tq : 0)) * hq + head) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      bf16x8 t = *(const bf16x8*)(qrow + ks * 16);
      if (!qvalid) t = bf16x8{};
      qreg[ks] = t;
    }
  }

  const int n_end = CAUSAL ? min(lk, tok_hi + diag) : lk;
  const int n_tiles = n_end > 0 ? (n_end + kBN - 1) / kBN : 0;
  // Tiles [0, j_full) hold only keys that every row of the workgroup sees: no mask.
  int j_full = lk / kBN;
  if (CAUSAL) j_full = min(j_full, max(0, (tok_lo + diag + 1) / kBN));
  j_full = min(j_full, n_tiles);

  // Global -> register staging; K runs one tile ahead of V.
  u32x4 kst[S::PER_THREAD], vst[S::PER_THREAD];
  const int st_key = tid / (D / 8);              // key of chunk i is st_key + i * (kThreads / (D / 8))
  const int st_c8 = (tid % (D / 8)) * 8;
  constexpr int KEYS_PER_PASS = kThreads / (D / 8);
  const bf16* kbase = k + ((size_t)k0 * hkv + g) * D + st_c8;
  const bf16* vbase = v + ((size_t)k0 * hkv + g) * D + st_c8;
  const size_t kv_stride = (size_t)hkv * D;
  // Rows past the sequence end are clamped to its last key instead of being
  // skipped: the loads stay unconditional (a per-lane branch that zero-fills
  // the destination forces a wait on every outstanding load), and those keys
  // are masked to probability 0 anyway.
  auto gload = [&](u32x4 (&dst)[S::PER_THREAD], const bf16* base, int tile) {
#pragma unroll
    for (int i = 0; i < S::PER_THREAD; ++i) {
      const int kk = min(tile * kBN + st_key + i * KEYS_PER_PASS, lk - 1);
      dst[i] = *(const u32x4*)(base + (size_t)kk * kv_stride);
    }
  };
  auto sstore = [&](const u32x4 (&src)[S::PER_THREAD], char VFA_LDS* buf, int stride) {
#pragma unroll
    for (int i = 0; i < S::PER_THREAD; ++i)
      *(u32x4 VFA_LDS*)(buf + (st_key + i * KEYS_PER_PASS) * stride + st_c8 * 2) = src[i];
  };

  // S^T for one 64-key tile: two 32-key sub-blocks, rows = keys, column = this lane's query.
  auto qk = [&](const char VFA_LDS* kb, f32x16 (&s)[2]) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      s[sb] = f32x16{};
      const char VFA_LDS* krow = kb + (sb * 32 + l32) * S::KSTR + half * 16;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
        s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read_b128(krow + ks * 32), qreg[ks], s[sb], 0, 0, 0);
    }
  };

  // Transposed V reads (ds_read_b64_tr_b16): in each 16-lane group, lane i
  // receives d = dbase + i for 4 consecutive keys.
  const int tr_grp = lane >> 4;
  const int tr_i = lane & 15;
  const int tr_key = (tr_grp >> 1) * 4 + (tr_i >> 2);
  const int tr_d = (tr_grp & 1) * 16 + 4 * (tr_i & 3);

  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};
  // Running reference max (raw score units) and running sum. The reference is
  // only moved when some column's tile max exceeds it by more than 2^8 in
  // probability terms, so most tiles skip the rescale of O.
  float m_run = neg_inf();
  float l_run = 0.f;
  const float tau = 8.f / scale_log2;

  auto softmax_pv = [&](auto masked, f32x16 (&s)[2], int j) {
    if constexpr (decltype(masked)::value) {
      const int lim = CAUSAL ? min(lk - 1, tq + diag) : lk - 1;
      const int kb0 = j * kBN + half * 4;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb0 + sb * 32 + (r >> 2) * 8 + (r & 3) > lim) s[sb][r] = neg_inf();
    }
    float lm = neg_inf();
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) lm = fmaxf(lm, s[sb][r]);
    // The other lane half holds the other keys of the same column.
    {
      auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lm), __float_as_uint(lm), false, false);
      lm = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    // Probabilities against the current reference (speculative: redone below if it moves).
    bf16x8 p[4];
    float ts = 0.f;
    auto make_p = [&](float mref) {
      ts = 0.f;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int sb = x >> 1, hh = x & 1;
        bf16x2 pr[4];
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          const float e0 = fast_exp2(__builtin_fmaf(s[sb][hh * 8 + 2 * y], scale_log2, -mref));
          const float e1 = fast_exp2(__builtin_fmaf(s[sb][hh * 8 + 2 * y + 1], scale_log2, -mref));
          pr[y] = f32x2_to_bf16x2(e0, e1);
          ts += e0 + e1;   // fp32 sum of the unrounded probabilities: lse stays fp32-accurate
        }
        p[x] = bf16x8{pr[0][0], pr[0][1], pr[1][0], pr[1][1], pr[2][0], pr[2][1], pr[3][0], pr[3][1]};
      }
    };
    make_p(m_run == neg_inf() ? 0.f : m_run * scale_log2);
    const bool need = lm > m_run + tau;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float m_new = need ? lm : m_run;
      // Lanes that keep their reference scale by exactly 1 (their m_run may be -inf);
      // a reference moving up from -inf scales the (zero) history by 0.
      const float alpha = need ? fast_exp2((m_run - m_new) * scale_log2) : 1.f;
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
      make_p(m_run == neg_inf() ? 0.f : m_run * scale_log2);
    }
    l_run += ts;

    // O^T += V^T P^T over four 16-key steps.
    const char VFA_LDS* vb = vbufs + (j & 1) * S::VBYTES;
#pragma unroll
    for (int kstep = 0; kstep < 4; ++kstep) {
      const char VFA_LDS* vrow = vb + (kstep * 16 + tr_key) * S::VSTR + tr_d * 2;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        bf16x8 a = lds_read_tr_pair(vrow + db * 64, vrow + 8 * S::VSTR + db * 64);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p[kstep], acc[db], 0, 0, 0);
      }
    }
  };

  // Prologue: K(0), V(0), K(1) in LDS; K(2), V(1) in registers; S = QK(0).
  if (n_tiles > 0) {
    gload(kst, kbase, 0);
    gload(vst, vbase, 0);
    sstore(kst, kbufs, S::KSTR);
    sstore(vst, vbufs, S::VSTR);
    if (n_tiles > 1) {
      gload(kst, kbase, 1);
      sstore(kst, kbufs + S::KBYTES, S::KSTR);
    }
  }
  __syncthreads();
  if (n_tiles > 2) gload(kst, kbase, 2);
  if (n_tiles > 1) gload(vst, vbase, 1);
  f32x16 s_cur[2];
  qk(kbufs, s_cur);

  auto tile_step = [&](auto masked, int j) {
    // Everyone is done with QK(j) and PV(j-1): K buffer j%2 and V buffer (j+1)%2
    // are free, and K(j+1), V(j) (stored last iteration) are visible.
    __syncthreads();
    if (j + 2 < n_tiles) sstore(kst, kbufs + (j & 1) * S::KBYTES, S::KSTR);
    if (j + 1 < n_tiles) sstore(vst, vbufs + ((j + 1) & 1) * S::VBYTES, S::VSTR);
    if (j + 3 < n_tiles) gload(kst, kbase, j + 3);
    if (j + 2 < n_tiles) gload(vst, vbase, j + 2);
    // QK of the next tile (harmless garbage after the last tile) overlaps this tile's softmax.
    f32x16 s_next[2];
    qk(kbufs + ((j + 1) & 1) * S::KBYTES, s_next);
    softmax_pv(masked, s_cur, j);
    s_cur[0] = s_next[0];
    s_cur[1] = s_next[1];
  };
  int j = 0;
  for (; j < j_full; ++j) tile_step(std::integral_constant<bool, false>{}, j);
  for (; j < n_tiles; ++j) tile_step(std::integral_constant<bool, true>{}, j);

  // Epilogue: combine the two lane halves' partial sums, normalise, store.
  const float l_tot = l_run + xor_shuffle(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qvalid) {
    const size_t row = (size_t)(q0 + tq) * hq + head;
    OutT* orow = out + row * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = db * 32 + g4 * 8 + half * 4;
        if constexpr (sizeof(OutT) == 2) {
          bf16x2 a = f32x2_to_bf16x2(acc[db][g4 * 4 + 0] * inv, acc[db][g4 * 4 + 1] * inv);
          bf16x2 c = f32x2_to_bf16x2(acc[db][g4 * 4 + 2] * inv, acc[db][g4 * 4 + 3] * inv);
          *(bf16x4*)(orow + d0) = bf16x4{a[0], a[1], c[0], c[1]};
        } else {
          *(f32x4*)(orow + d0) = f32x4{acc[db][g4 * 4 + 0] * inv, acc[db][g4 * 4 + 1] * inv,
                                       acc[db][g4 * 4 + 2] * inv, acc[db][g4 * 4 + 3] * inv};
        }
      }
    if (half == 0)
      lse[row] = l_tot > 0.f ? m_run * scale + fast_log2(l_tot) * kLn2 : neg_inf();
  }
}

template <int WAVES, int D, bool CAUSAL, typename OutT>
int launch_t(const AttnArgs& a) {
  const int tokw = Shape<WAVES>::COLS / a.grp;
  const int n_mtiles = (a.max_seqlen_q + tokw - 1) / tokw;
  const long long pairs_per_xcd = ((long long)a.batch * a.hkv + kXcds - 1) / kXcds;
  const long long blocks = (long long)n_mtiles * pairs_per_xcd * kXcds;
  if (blocks <= 0) return 0;
  if (blocks > 0x7fffffffLL) return -1;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<WAVES, D, CAUSAL, OutT>), dim3((unsigned)blocks),
                     dim3(Shape<WAVES>::THREADS), 0, (hipStream_t)a.stream, (const bf16*)a.q, (const bf16*)a.k,
                     (const bf16*)a.v, a.cu_q, a.cu_k, a.batch, a.hq, a.hkv, a.grp, tokw, n_mtiles, a.scale,
                     a.scale * kLog2e, (OutT*)a.out, a.lse);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int WAVES>
int launch_w(const AttnArgs& a) {
  const bool f32out = a.out_dtype == 0;
  if (a.head_dim == 128) {
    if (a.causal) return f32out ? launch_t<WAVES, 128, true, float>(a) : launch_t<WAVES, 128, true, bf16>(a);
    return f32out ? launch_t<WAVES, 128, false, float>(a) : launch_t<WAVES, 128, false, bf16>(a);
  }
  if (a.causal) return f32out ? launch_t<WAVES, 64, true, float>(a) : launch_t<WAVES, 64, true, bf16>(a);
  return f32out ? launch_t<WAVES, 64, false, float>(a) : launch_t<WAVES, 64, false, bf16>(a);
}

}  // namespace

// Eight-wave workgroups once sequences average at least eight of their
// query tiles (256 / G tokens); shorter ones waste less with four waves.
int launch_attn_fwd_bf16(const AttnArgs& a) {
  const long long mean_q = a.batch > 0 ? (long long)a.total_q / a.batch : 0;
  if (mean_q >= 8LL * (Shape<8>::COLS / a.grp)) return launch_w<8>(a);
  return launch_w<4>(a);
}

}  // namespace vfa
