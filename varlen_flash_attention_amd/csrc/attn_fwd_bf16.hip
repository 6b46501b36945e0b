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
// m). Its "columns" are the G query heads of kv head g times tokw consecutive
// tokens, so every K/V tile brought into LDS serves all G heads (no
// repeat_interleave of K/V is ever materialised). Key tiles that the causal
// mask hides from every row of the workgroup are never visited; only tiles
// that straddle the diagonal or the sequence end are masked.
//
// Per wave (NQ blocks of 32 query columns), per 32-key sub-block:
//   S^T = K Q^T   : v_mfma_f32_32x32x16_bf16, A = K rows from LDS (16 B
//                   reads, each feeding NQ MFMAs), B = Q^T held in registers.
//   online softmax: each lane owns one column (query row) per block in the S^T
//                   accumulator, so running max / sum stay lane-local apart
//                   from one exchange with lane ^ 32 for the max.
//   O^T += V^T P^T: A = V^T read with ds_read_b64_tr_b16 (gfx950 LDS
//                   transpose read) straight from the row-major V tile (each
//                   read feeding NQ MFMAs), B = P^T converted to bf16 in
//                   registers.
// The QK of the next sub-block is issued before the softmax of the current
// one. K and V stream through LDS in tiles of BN keys with one barrier per
// tile (see the pipeline comment in the kernel): 64 keys for the 4-wave
// shape, whose two workgroups per CU share the LDS.
//
// This kernel serves batches of short sequences (four waves, 128 columns).
// Batches whose sequences average at least eight 256-column query tiles go to
// attn_fwd_overlap.hip, eight waves with the softmax overlapped with the
// matrix products.
#include <type_traits>

#include "common.h"
#include "launch.h"

// Kernel-body lambdas are forced inline: one left out of line takes the
// register arrays it touches by reference, which moves them to scratch.
#define VFA_INLINE __attribute__((always_inline))

namespace vfa {
namespace {

constexpr int kXcds = 8;             // MI355X: 8 XCDs, blocks dispatched round-robin

// Workgroup shapes: WAVES waves of NQ x 32 query columns each.
//   <4, 1>: 128 columns, two workgroups per CU (short sequences).
//   <8, 1>: 256 columns, one workgroup per CU, two waves per SIMD.
//   <4, 2>: 256 columns, one workgroup per CU, one wave per SIMD with every
//           K/V operand read from LDS feeding two MFMAs (half the LDS read
//           traffic per FLOP of the 32-column waves).
template <int WAVES, int NQ>
struct Shape {
  static constexpr int THREADS = WAVES * 64;
  static constexpr int COLS = WAVES * 32 * NQ;
  // Waves per SIMD the register budget is sized for: 2 (256 VGPR+AGPR per
  // wave) for the 32-column shapes, 1 (512) for the 64-column shape.
  static constexpr int WAVES_PER_EU = NQ == 1 ? 2 : 1;
};

// LDS row strides, chosen from measured bank behaviour on gfx950: a 16-byte pad
// makes the per-lane-row ds_read_b128 of K conflict-free; a 64-byte pad makes
// the ds_read_b64_tr_b16 of V conflict-free (a 32-byte pad costs 2x).
template <int D, int THREADS, int BN>
struct Smem {
  static constexpr int KSTR = D * 2 + 16;
  static constexpr int VSTR = D * 2 + 64;
  static constexpr int KBYTES = BN * KSTR;
  static constexpr int VBYTES = BN * VSTR;
  static constexpr int TOTAL = 2 * (KBYTES + VBYTES);
  static constexpr int CHUNKS = BN * D / 8;           // 16-byte chunks per tile (per tensor)
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

template <int WAVES, int NQ, int D, bool CAUSAL, typename OutT, int BN>
__global__ __attribute__((amdgpu_flat_work_group_size(1, Shape<WAVES, NQ>::THREADS),
                          amdgpu_waves_per_eu(Shape<WAVES, NQ>::WAVES_PER_EU, Shape<WAVES, NQ>::WAVES_PER_EU))) void
attn_fwd_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, const int32_t* __restrict__ coff,
    int batch, int hq, int hkv, int grp, int tokw, int n_mtiles, float scale, float scale_log2,
    OutT* __restrict__ out, float* __restrict__ lse) {
  constexpr int kThreads = Shape<WAVES, NQ>::THREADS;
  using S = Smem<D, kThreads, BN>;
  constexpr int kBN = BN;
  constexpr int SUBS = BN / 32;                   // 32-key sub-blocks per tile
  __shared__ __attribute__((aligned(16))) char smem[S::TOTAL];
  char VFA_LDS* lds = (char VFA_LDS*)smem;
  char VFA_LDS* kbufs = lds;                      // 2 * SUBS 32-key K slots
  char VFA_LDS* vbufs = lds + 2 * S::KBYTES;      // two BN-key V tiles

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
  const int diag = causal_diag(coff, b, lq, lk);  // query i sees key j iff j <= i + diag (causal)

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // This lane's query column in each of its NQ blocks. Columns past tokw * grp
  // (when grp does not divide the column count) carry no query.
  int tq[NQ], head[NQ];
  bool qvalid[NQ];
  // Q^T as the B operand: column = query, k-slot (half*8 + e) <-> d = ks*16 + half*8 + e.
  bf16x8 qreg[NQ][D / 16];
#pragma unroll
  for (int qb = 0; qb < NQ; ++qb) {
    const int col = (wave * NQ + qb) * 32 + l32;
    const bool colvalid = col < tokw * grp;
    const int hg = colvalid ? col / tokw : 0;
    tq[qb] = tok_lo + (colvalid ? col - hg * tokw : 0);
    head[qb] = g * grp + hg;
    qvalid[qb] = colvalid && tq[qb] < lq;
    const bf16* qrow = q + ((size_t)(q0 + (qvalid[qb] ? tq[qb] : 0)) * hq + head[qb]) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      bf16x8 t = *(const bf16x8*)(qrow + ks * 16);
      if (!qvalid[qb]) t = bf16x8{};
      qreg[qb][ks] = t;
    }
  }

  const int n_end = CAUSAL ? min(lk, tok_hi + diag) : lk;
  const int n_tiles = n_end > 0 ? (n_end + kBN - 1) / kBN : 0;
  // Tiles [0, j_full) hold only keys that every row of the workgroup sees: no mask.
  int j_full = lk / kBN;
  if (CAUSAL) j_full = min(j_full, max(0, (tok_lo + diag + 1) / kBN));
  j_full = min(j_full, n_tiles);

  // Global -> register staging. Rows past the sequence end are clamped to its
  // last key instead of being skipped: the loads stay unconditional (a
  // per-lane branch that zero-fills the destination forces a wait on every
  // outstanding load), and those keys are masked to probability 0 anyway.
  u32x4 kst[S::PER_THREAD], vst[S::PER_THREAD];
  const int st_key = tid / (D / 8);
  const int st_c8 = (tid % (D / 8)) * 8;
  constexpr int KEYS_PER_PASS = kThreads / (D / 8);
  // Sequence bases are wave-uniform; each lane adds fixed 32-bit byte offsets
  // (BN rows of hkv * D bf16 stay far below 4 GiB), so a tile that lies wholly
  // inside the sequence needs no per-lane address arithmetic. Only the tail
  // tile clamps rows one by one.
  const char* kbase = (const char*)(k + ((size_t)k0 * hkv + g) * D);
  const char* vbase = (const char*)(v + ((size_t)k0 * hkv + g) * D);
  const size_t row_bytes = (size_t)hkv * D * sizeof(bf16);
  uint32_t st_off[S::PER_THREAD];
#pragma unroll
  for (int i = 0; i < S::PER_THREAD; ++i)
    st_off[i] = (uint32_t)((st_key + i * KEYS_PER_PASS) * row_bytes + st_c8 * sizeof(bf16));
  // BN consecutive keys starting at key0.
  auto gload = [&](u32x4 (&dst)[S::PER_THREAD], const char* base, int key0) {
    if (key0 + kBN <= lk) {
      const char* tile = base + (size_t)key0 * row_bytes;
#pragma unroll
      for (int i = 0; i < S::PER_THREAD; ++i) dst[i] = *(const u32x4*)(tile + st_off[i]);
    } else {
#pragma unroll
      for (int i = 0; i < S::PER_THREAD; ++i) {
        const int kk = min(key0 + st_key + i * KEYS_PER_PASS, lk - 1);
        dst[i] = *(const u32x4*)(base + (size_t)kk * row_bytes + st_c8 * sizeof(bf16));
      }
    }
  };
  // V: one BN-key tile per buffer.
  auto sstore_v = [&](const u32x4 (&src)[S::PER_THREAD], char VFA_LDS* buf) {
#pragma unroll
    for (int i = 0; i < S::PER_THREAD; ++i)
      *(u32x4 VFA_LDS*)(buf + (st_key + i * KEYS_PER_PASS) * S::VSTR + st_c8 * 2) = src[i];
  };
  // K: a ring of 2 * SUBS 32-key slots; sub-block n lives in slot
  // n % (2 * SUBS). Stores BN keys = sub-blocks sub0 .. sub0 + SUBS-1.
  auto k_slot = [&](int sub) { return kbufs + (sub & (2 * SUBS - 1)) * (32 * S::KSTR); };
  auto sstore_k = [&](const u32x4 (&src)[S::PER_THREAD], int sub0) {
#pragma unroll
    for (int i = 0; i < S::PER_THREAD; ++i) {
      const int r = st_key + i * KEYS_PER_PASS;
      *(u32x4 VFA_LDS*)(k_slot(sub0 + (r >> 5)) + (r & 31) * S::KSTR + st_c8 * 2) = src[i];
    }
  };

  // S^T for one 32-key sub-block (rows = keys, column = this lane's query),
  // for all NQ column blocks; each K operand read feeds NQ MFMAs.
  auto qk = [&](int sub, f32x16 (&s)[NQ]) {
#pragma unroll
    for (int qb = 0; qb < NQ; ++qb) s[qb] = f32x16{};
    const char VFA_LDS* krow = k_slot(sub) + l32 * S::KSTR + half * 16;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const bf16x8 a = lds_read_b128(krow + ks * 32);
#pragma unroll
      for (int qb = 0; qb < NQ; ++qb)
        s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[qb][ks], s[qb], 0, 0, 0);
    }
  };

  // Transposed V reads (ds_read_b64_tr_b16): in each 16-lane group, lane i
  // receives d = dbase + i for 4 consecutive keys.
  const int tr_grp = lane >> 4;
  const int tr_i = lane & 15;
  const int tr_key = (tr_grp >> 1) * 4 + (tr_i >> 2);
  const int tr_d = (tr_grp & 1) * 16 + 4 * (tr_i & 3);

  f32x16 acc[NQ][D / 32];
#pragma unroll
  for (int qb = 0; qb < NQ; ++qb)
#pragma unroll
    for (int i = 0; i < D / 32; ++i) acc[qb][i] = f32x16{};
  // Per column: reference max m_run (raw score units; -inf until the column
  // has seen a visible key), the same reference pre-scaled to log2 units, and
  // the running sum of probabilities against it.
  float m_run[NQ], mref[NQ], l_run[NQ];
#pragma unroll
  for (int qb = 0; qb < NQ; ++qb) {
    m_run[qb] = neg_inf();
    mref[qb] = 0.f;
    l_run[qb] = 0.f;
  }
  // The reference only has to keep probabilities finite (bf16 P and the fp32
  // sums share fp32's exponent range), not at or below 1. So the fast path
  // takes exponentials against the current reference and checks their sum:
  // only a sum above 2^32 (a score more than 32 log2 units above the
  // reference) or a column without a reference yet takes the slow path, which
  // moves the reference to the exact running max, rescales O and the sum, and
  // recomputes. This drops the per-block max from the common path.
  constexpr float kSumLimit = 4294967296.f;

  // Softmax and PV for sub-block sb of tile j (keys j*BN + sb*32 ...).
  auto softmax_pv = [&](auto masked, f32x16 (&s)[NQ], int j, int sb) {
    if constexpr (decltype(masked)::value) {
#pragma unroll
      for (int qb = 0; qb < NQ; ++qb) {
        const int lim = CAUSAL ? min(lk - 1, tq[qb] + diag) : lk - 1;
        const int kb0 = j * kBN + sb * 32 + half * 4;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb0 + (r >> 2) * 8 + (r & 3) > lim) s[qb][r] = neg_inf();
      }
    }
    float e[NQ][16], ts[NQ];
    auto exps = [&]() {
#pragma unroll
      for (int qb = 0; qb < NQ; ++qb) {
        ts[qb] = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          e[qb][r] = fast_exp2(__builtin_fmaf(s[qb][r], scale_log2, -mref[qb]));
          ts[qb] += e[qb][r];   // fp32 sum of the unrounded probabilities: lse stays fp32-accurate
        }
      }
    };
    exps();
    bool slow = false;
#pragma unroll
    for (int qb = 0; qb < NQ; ++qb) slow |= !(ts[qb] <= kSumLimit) || m_run[qb] == neg_inf();
    if (__builtin_amdgcn_ballot_w64(slow)) {
#pragma unroll
      for (int qb = 0; qb < NQ; ++qb) {
        float x = neg_inf();
#pragma unroll
        for (int r = 0; r < 16; ++r) x = fmaxf(x, s[qb][r]);
        // The other lane half holds the other keys of the same column.
        auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        const float m_new = fmaxf(m_run[qb], fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])));
        // Unchanged references scale by exactly 1 (m_run may be -inf); one moving
        // up from -inf scales the (zero) history by 0.
        const float alpha = m_new == m_run[qb] ? 1.f : fast_exp2((m_run[qb] - m_new) * scale_log2);
        m_run[qb] = m_new;
        mref[qb] = m_new == neg_inf() ? 0.f : m_new * scale_log2;
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[qb][db][r] *= alpha;
      }
      exps();
    }
    // P^T (B operand) for the two 16-key steps.
    bf16x8 p[NQ][2];
#pragma unroll
    for (int qb = 0; qb < NQ; ++qb) {
      l_run[qb] += ts[qb];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        bf16x2 pr[4];
#pragma unroll
        for (int y = 0; y < 4; ++y) pr[y] = f32x2_to_bf16x2(e[qb][hh * 8 + 2 * y], e[qb][hh * 8 + 2 * y + 1]);
        p[qb][hh] = bf16x8{pr[0][0], pr[0][1], pr[1][0], pr[1][1], pr[2][0], pr[2][1], pr[3][0], pr[3][1]};
      }
    }

    // O^T += V^T P^T over the sub-block's two 16-key steps; each V^T read feeds NQ MFMAs.
    const char VFA_LDS* vb = vbufs + (j & 1) * S::VBYTES + sb * 32 * S::VSTR;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const char VFA_LDS* vrow = vb + (hh * 16 + tr_key) * S::VSTR + tr_d * 2;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const bf16x8 a = lds_read_tr_pair(vrow + db * 64, vrow + 8 * S::VSTR + db * 64);
#pragma unroll
        for (int qb = 0; qb < NQ; ++qb)
          acc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p[qb][hh], acc[qb][db], 0, 0, 0);
      }
    }
  };

  // Pipeline (SUBS = BN / 32 sub-blocks per tile). Iteration j does softmax +
  // PV for sub-blocks SUBS*j .. SUBS*j + SUBS-1 (V tile j) and the QK of
  // sub-blocks SUBS*j + 1 .. SUBS*j + SUBS, each QK issued before the previous
  // sub-block's softmax. It refills the SUBS K slots freed by the previous
  // iteration (whose QKs it ran) with sub-blocks SUBS*j + SUBS+1 ..
  // SUBS*j + 2*SUBS, and V buffer (j+1)%2 with V tile j+1 (both loaded into
  // registers one iteration earlier), so one barrier per iteration separates
  // every LDS write from the reads of the same slot.
  const int n_sub = SUBS * n_tiles;
  const int n_sub_vis = (n_end + 31) / 32;         // sub-blocks holding a visible key
  if (n_tiles > 0) {
    // All three first loads in flight together (one memory round trip).
    u32x4 kst2[S::PER_THREAD];
    gload(kst, kbase, 0);
    gload(vst, vbase, 0);
    gload(kst2, kbase, kBN);
    sstore_k(kst, 0);
    sstore_v(vst, vbufs);
    sstore_k(kst2, SUBS);
  }
  __syncthreads();
  if (n_sub > SUBS + 1) gload(kst, kbase, (SUBS + 1) * 32);
  if (n_tiles > 1) gload(vst, vbase, kBN);
  f32x16 s_cur[NQ], s_next[NQ];
  qk(0, s_cur);

  auto tile_step = [&](auto masked, int j) {
    __syncthreads();
    if (SUBS * j + SUBS + 1 < n_sub) sstore_k(kst, SUBS * j + SUBS + 1);
    if (j + 1 < n_tiles) sstore_v(vst, vbufs + ((j + 1) & 1) * S::VBYTES);
    if (SUBS * j + 2 * SUBS + 1 < n_sub) gload(kst, kbase, (SUBS * j + 2 * SUBS + 1) * 32);
    if (j + 2 < n_tiles) gload(vst, vbase, (j + 2) * kBN);
#pragma unroll
    for (int sb = 0; sb < SUBS; ++sb) {
      // Masked tiles: sub-blocks wholly past the block's last visible key hold
      // nothing for any row (n_sub_vis is uniform over the workgroup).
      if (decltype(masked)::value && SUBS * j + sb >= n_sub_vis) break;
      // The QK after the block's last visible sub-block would never be used
      // (masked tiles only: in full tiles it is the next sub-block's).
      if (!decltype(masked)::value || SUBS * j + sb + 1 < n_sub_vis) qk(SUBS * j + sb + 1, s_next);
      softmax_pv(masked, s_cur, j, sb);
#pragma unroll
      for (int qb = 0; qb < NQ; ++qb) s_cur[qb] = s_next[qb];
    }
  };
  int j = 0;
  for (; j < j_full; ++j) tile_step(std::integral_constant<bool, false>{}, j);
  for (; j < n_tiles; ++j) tile_step(std::integral_constant<bool, true>{}, j);

  // Epilogue: combine the two lane halves' partial sums, normalise, store.
  // A lane holds, per 32-dim block and group g4, the 4 dims g4*8 + half*4 ..;
  // for bf16 output the two halves trade one group of each pair (lane i and
  // i + 32 own the same query), so each lane stores 8 contiguous dims (16 B)
  // instead of 4.
#pragma unroll
  for (int qb = 0; qb < NQ; ++qb) {
    const float l_tot = l_run[qb] + xor_shuffle(l_run[qb], 32);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const size_t row = (size_t)(q0 + tq[qb]) * hq + head[qb];
    OutT* orow = out + row * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const f32x16& a = acc[qb][db];
      if constexpr (sizeof(OutT) == 2) {
        auto pk = [&](int r) VFA_INLINE {
          return __builtin_bit_cast(uint32_t, f32x2_to_bf16x2(a[r] * inv, a[r + 1] * inv));
        };
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {
          const int ga = 2 * gp, gb = 2 * gp + 1;   // half 0 stores group ga, half 1 group gb
          const uint32_t a0 = pk(ga * 4), a1 = pk(ga * 4 + 2), b0 = pk(gb * 4), b1 = pk(gb * 4 + 2);
          // Lanes 0-31 receive the upper half's group ga, lanes 32-63 the lower half's group gb.
          const auto s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
          const u32x4 val = half == 0 ? u32x4{a0, a1, s0[1], s1[1]} : u32x4{s0[0], s1[0], b0, b1};
          u32x4* dst = (u32x4*)(orow + db * 32 + (half == 0 ? ga : gb) * 8);
          if (qvalid[qb]) *dst = val;
        }
      } else {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 val{a[g4 * 4 + 0] * inv, a[g4 * 4 + 1] * inv, a[g4 * 4 + 2] * inv, a[g4 * 4 + 3] * inv};
          f32x4* dst = (f32x4*)(orow + db * 32 + g4 * 8 + half * 4);
          if (qvalid[qb]) *dst = val;
        }
      }
    }
    if (qvalid[qb] && half == 0)
      lse[row] = l_tot > 0.f ? m_run[qb] * scale + fast_log2(l_tot) * kLn2 : neg_inf();
  }
}

template <int WAVES, int NQ, int D, bool CAUSAL, typename OutT>
int launch_t(const AttnArgs& a) {
  constexpr int BN = WAVES == 8 ? 128 : 64;
  const int tokw = Shape<WAVES, NQ>::COLS / a.grp;
  const int n_mtiles = (a.max_seqlen_q + tokw - 1) / tokw;
  const long long pairs_per_xcd = ((long long)a.batch * a.hkv + kXcds - 1) / kXcds;
  const long long blocks = (long long)n_mtiles * pairs_per_xcd * kXcds;
  if (blocks <= 0) return 0;
  if (blocks > 0x7fffffffLL) return -1;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<WAVES, NQ, D, CAUSAL, OutT, BN>), dim3((unsigned)blocks),
                     dim3(Shape<WAVES, NQ>::THREADS), 0, (hipStream_t)a.stream, (const bf16*)a.q,
                     (const bf16*)a.k, (const bf16*)a.v, a.cu_q, a.cu_k, a.causal_off, a.batch, a.hq, a.hkv,
                     a.grp, tokw, n_mtiles, a.scale, a.scale * kLog2e, (OutT*)a.out, a.lse);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int WAVES, int NQ>
int launch_w(const AttnArgs& a) {
  const bool f32out = a.out_dtype == 0;
  if (a.head_dim == 128) {
    if (a.causal)
      return f32out ? launch_t<WAVES, NQ, 128, true, float>(a) : launch_t<WAVES, NQ, 128, true, bf16>(a);
    return f32out ? launch_t<WAVES, NQ, 128, false, float>(a) : launch_t<WAVES, NQ, 128, false, bf16>(a);
  }
  if (a.causal) return f32out ? launch_t<WAVES, NQ, 64, true, float>(a) : launch_t<WAVES, NQ, 64, true, bf16>(a);
  return f32out ? launch_t<WAVES, NQ, 64, false, float>(a) : launch_t<WAVES, NQ, 64, false, bf16>(a);
}

}  // namespace

// 256-column workgroups (attn_fwd_overlap.hip) once sequences average at
// least eight of their query tiles (256 / G tokens); shorter ones waste less
// with 128 columns.
int launch_attn_fwd_bf16(const AttnArgs& a) {
  if (wide_prefill(a.batch, a.total_q, a.hq, a.hkv)) return launch_attn_fwd_overlap(a);
  return launch_w<4, 1>(a);
}

}  // namespace vfa
