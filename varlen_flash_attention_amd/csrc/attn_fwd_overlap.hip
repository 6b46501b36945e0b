// Varlen attention forward for long sequences: bf16 inputs on gfx950 bf16
// MFMA with fp32 accumulation, with each wave's softmax overlapped with its
// own matrix products.
//
// What is computed is the same as in attn_fwd_bf16.hip: for every packed
// sequence, query head h and query i, softmax(scale * q_i K^T) V over the
// visible keys plus the natural-log log-sum-exp of the scaled scores, in the
// TND layout with int32 cu_seqlens ("From GPU to NPU: Qwen3-Embedding on
// Ascend", core optimisation 1 and section 2.1), query head h reading kv head
// h / G (core optimisation 5 of the same page), causal mask aligned
// bottom-right.
//
// Work decomposition: a work item is one (sequence, kv head, query tile) with
// 256 query columns (G heads x 256/G tokens). Key sub-blocks that the causal
// mask hides from the whole tile are never visited. The grid is persistent:
// one workgroup of 8 waves per CU, each taking items one after another from a
// ticket counter of its XCD (workgroups are dispatched round-robin over the 8
// XCDs, so workgroup i serves XCD i % 8). XCD x's tickets run over the
// (sequence, kv head) pairs x, x + 8, ... and, within a pair, its query tiles
// last first (causal tiles grow with the index), so the items an XCD works on
// at one time mostly share one pair's K/V in its L2, the longest items start
// first and a CU that finishes early takes the next item instead of idling.
// Tickets are slots of a (pair, max_seqlen_q / tokens-per-tile) grid; the
// first workgroup that draws an empty slot of a pair (a tile past a shorter
// sequence's end) moves the counter past all of them. The counters sit in the
// caller's workspace and a one-wave kernel zeroes them before each call.
//
// Software pipeline. Per 32-key sub-block a wave runs S_j^T = K_j Q^T (8
// MFMAs), the online softmax of S_j (exponentials, sums and bf16 conversions
// on the vector ALU) and O^T += V_j^T P_j^T (8 MFMAs). PV_j
// needs the softmax of S_j, and the softmax needs QK_j, so a wave that runs
// them in that order leaves the matrix unit idle during its softmax. Here
// iteration j issues QK_{j+1} and PV_{j-1}, which need nothing from iteration
// j, and the softmax of S_j between those 16 MFMAs, in a pinned instruction
// order, so the vector ALU works under the MFMAs of the same wave. The two
// waves of each SIMD run this freely and fill each other's remaining gaps.
//
// K and V stream through LDS rings of 4 sub-block slots with one barrier per
// tile of 2 sub-blocks. Waves 0-3 move K and waves 4-7 move V, one sub-block
// per iteration: iteration j stores K_{j+3} and V_{j+1} (loaded into registers
// one iteration earlier) and loads K_{j+4} and V_{j+2}. Iteration j reads K_{j+1}
// and V_{j-1}; a sub-block stored in iteration j is first read in iteration
// j+2, the next tile, and it replaces one last read in iteration j-2, the
// previous tile (K_0, read by QK_0 before the first iteration, has a barrier
// of its own), so the tile barriers order every LDS write after the reads of
// the slot it replaces and before the first read of its data.
#include <type_traits>

#include "common.h"
#include "launch.h"

#define VFA_INLINE __attribute__((always_inline))

namespace vfa {
namespace {

constexpr int kXcds = 8;        // MI355X: 8 XCDs, blocks dispatched round-robin
constexpr int kThreads = 512;   // 8 waves, two per SIMD
constexpr int kCols = 256;      // 8 waves x 32 query columns
constexpr int kSub = 32;        // keys per sub-block
constexpr int kRing = 4;        // sub-block slots per LDS ring (two tiles of two)
constexpr int kTicketStride = 32;   // ints between two XCDs' counters (one 128-byte line each)

// LDS row strides as in the short-sequence kernel: a 16-byte pad keeps the
// per-lane-row ds_read_b128 of K conflict-free, a 64-byte pad the transposed
// reads of V.
template <int D>
struct OverlapSmem {
  static constexpr int KSTR = D * 2 + 16;
  static constexpr int VSTR = D * 2 + 64;
  static constexpr int KSLOT = kSub * KSTR;
  static constexpr int VSLOT = kSub * VSTR;
  static constexpr int TOTAL = kRing * (KSLOT + VSLOT);
  // Four waves (256 threads) move one sub-block of one tensor: 32 rows of D
  // bf16 = 32 * D / 8 16-byte pieces.
  static constexpr int PER_THREAD = kSub * D / 8 / 256;
  static constexpr int KEYS_PER_PASS = 256 / (D / 8);
  static_assert(kSub * D / 8 % 256 == 0, "a sub-block must split evenly over four waves");
};

__device__ __forceinline__ bf16x8 ov_read_b128(const char VFA_LDS* p) { return *(const bf16x8 VFA_LDS*)p; }

__device__ __forceinline__ bf16x8 ov_read_tr_pair(const char VFA_LDS* p0, const char VFA_LDS* p1) {
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 VFA_LDS*)p0);
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 VFA_LDS*)p1);
  typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8;
  i16x8 r = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, r);
}

// Tile boundary: this wave's LDS writes complete, then a workgroup barrier
// that no instruction crosses in either direction.
__device__ __forceinline__ void tile_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Zeroes the 8 ticket counters (one wave; kernel stores, so a captured graph
// holds no memset node).
__global__ void zero_tickets_kernel(int* __restrict__ tickets) {
  if (threadIdx.x < kXcds) tickets[threadIdx.x * kTicketStride] = 0;
}

// Next non-empty slot of XCD xcd's ticket range [0, n_slots), or -1 when
// there is none (run by one thread). A slot whose tile lies past its
// sequence's end moves the counter to the pair's first non-empty slot. The
// value drawn grows strictly on every pass, so the loop ends.
__device__ __forceinline__ int next_slot(int* ctr, int n_slots, int n_mtiles, int xcd, int hkv, int tokw,
                                      const int32_t* __restrict__ cu_q) {
  int t = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  while (t < n_slots) {
    const int pl = t / n_mtiles;
    const int kk = t - pl * n_mtiles;
    const int b = (pl * kXcds + xcd) / hkv;
    const int lq = cu_q[b + 1] - cu_q[b];
    const int k0 = n_mtiles - min(n_mtiles, max(0, (lq + tokw - 1) / tokw));
    if (kk >= k0) return t;
    __hip_atomic_fetch_max(ctr, pl * n_mtiles + k0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    t = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return -1;
}

template <int D, bool CAUSAL, typename OutT>
__global__ __attribute__((amdgpu_flat_work_group_size(1, kThreads), amdgpu_waves_per_eu(2, 2))) void
attn_fwd_overlap_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
                        const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
                        const int32_t* __restrict__ coff, int batch, int hq, int hkv, int grp, int tokw,
                        int n_mtiles, float scale, float scale_log2, OutT* __restrict__ out,
                        float* __restrict__ lse, int* __restrict__ tickets) {
  using S = OverlapSmem<D>;
  constexpr int PT = S::PER_THREAD;
  __shared__ __attribute__((aligned(16))) char smem[S::TOTAL];
  __shared__ int s_slot;
  char VFA_LDS* kring = (char VFA_LDS*)smem;
  char VFA_LDS* vring = kring + kRing * S::KSLOT;

  // XCD x serves the (sequence, kv head) pairs x, x + 8, ..., n_mtiles slots each.
  const int per_m = batch * hkv;
  const int xcd = blockIdx.x % kXcds;
  const int n_slots = per_m > xcd ? ((per_m - xcd + kXcds - 1) / kXcds) * n_mtiles : 0;
  int* ctr = tickets + xcd * kTicketStride;

  for (;;) {
  // The thread index goes through an opaque copy in every item: the per-lane
  // offsets derived from it are then recomputed per item (a few instructions)
  // instead of being hoisted out of this loop and held in registers through
  // the item's own loop.
  int tid;
  asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"((int)threadIdx.x));
  // The barrier after the draw also ends every wave's previous item, so the
  // new item's stores into the rings follow all reads of the old one.
  if (tid == 0) s_slot = next_slot(ctr, n_slots, n_mtiles, xcd, hkv, tokw, cu_q);
  __syncthreads();
  const int slot = s_slot;
  if (slot < 0) break;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave (scalar registers)
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int group = wave >> 2;                    // 0: waves moving K, 1: waves moving V
  const int bg = (slot / n_mtiles) * kXcds + xcd;
  const int m = n_mtiles - 1 - slot % n_mtiles;
  const int b = bg / hkv;
  const int g = bg % hkv;

  const int q0 = cu_q[b];
  const int lq = cu_q[b + 1] - q0;
  const int tok_lo = m * tokw;
  const int k0 = cu_k[b];
  const int lk = cu_k[b + 1] - k0;
  const int tok_hi = min(lq, tok_lo + tokw);
  const int diag = causal_diag(coff, b, lq, lk);  // query i sees key j iff j <= i + diag (causal)

  // This lane's query column: (query head of kv head g, token).
  const int col = wave * 32 + l32;
  const bool colvalid = col < tokw * grp;
  const int hg = colvalid ? col / tokw : 0;
  const int tq = tok_lo + (colvalid ? col - hg * tokw : 0);
  const int head = g * grp + hg;
  const bool qvalid = colvalid && tq < lq;
  // Q^T as the B operand: column = query, k-slot (half*8 + e) <-> d = ks*16 + half*8 + e.
  // A column without a query reads the sequence's first query instead: its
  // results are never stored.
  bf16x8 qreg[D / 16];
  {
    const bf16* qrow = q + ((size_t)(q0 + (qvalid ? tq : 0)) * hq + head) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qreg[ks] = *(const bf16x8*)(qrow + ks * 16);
  }

  const int n_end = CAUSAL ? min(lk, tok_hi + diag) : lk;
  const int n_sub = n_end > 0 ? (n_end + kSub - 1) / kSub : 0;
  // Loads run the same on every path: sub-block indices past the last one are
  // clamped to it (stores past it fill slots that nothing reads), so the
  // number of loads in flight is the same at every point and each store waits
  // only for its own set's loads.
  const int last = n_sub - 1;
  // Sub-blocks [0, j_full) hold only keys that every row of the tile sees.
  int j_full = lk / kSub;
  if (CAUSAL) j_full = min(j_full, max(0, (tok_lo + diag + 1) / kSub));

  // Global -> register -> LDS staging through buffer loads: the sequence's
  // rows of kv head g form one buffer whose size ends at its last key, so rows
  // past the end read as zero (those keys are masked to probability 0). A
  // sub-block's offset is wave-uniform (an SGPR); each lane adds a fixed
  // offset of its own.
  const int gt = tid & 255;
  const int st_key = gt / (D / 8);
  const int st_c8 = (gt % (D / 8)) * 8;
  const uint32_t row_bytes = (uint32_t)hkv * D * sizeof(bf16);
  const __amdgpu_buffer_rsrc_t srsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((group == 0 ? k : v) + ((size_t)k0 * hkv + g) * D), (short)0, (int)((uint32_t)lk * row_bytes),
      0x00020000);
  char VFA_LDS* ring = group == 0 ? kring : vring;
  const int sstr = group == 0 ? S::KSTR : S::VSTR;
  const int sslot = group == 0 ? S::KSLOT : S::VSLOT;
  // Iteration j stores sub-block j + ahead of the group's tensor: K_{j+3}, V_{j+1}.
  const int ahead = group == 0 ? 3 : 1;
  uint32_t g_off[PT], l_off[PT];
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    g_off[i] = (st_key + i * S::KEYS_PER_PASS) * row_bytes + st_c8 * (uint32_t)sizeof(bf16);
    l_off[i] = (uint32_t)((st_key + i * S::KEYS_PER_PASS) * sstr + st_c8 * 2);
  }
  auto gload = [&](u32x4 (&dst)[PT], int sub) VFA_INLINE {
    const uint32_t soff = (uint32_t)sub * kSub * row_bytes;
#pragma unroll
    for (int i = 0; i < PT; ++i) dst[i] = __builtin_amdgcn_raw_buffer_load_b128(srsrc, g_off[i], soff, 0);
  };
  auto sstore = [&](const u32x4 (&src)[PT], int sub) VFA_INLINE {
    char VFA_LDS* dst = ring + (sub & (kRing - 1)) * sslot;
#pragma unroll
    for (int i = 0; i < PT; ++i) *(u32x4 VFA_LDS*)(dst + l_off[i]) = src[i];
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
  // Running reference max (raw score units; -inf until the column has seen a
  // visible key), the same pre-scaled to log2 units, and the running sum.
  float m_run = neg_inf(), mref = 0.f, l_run = 0.f;
  // The reference only has to keep probabilities finite, not at or below 1:
  // the common path exponentiates against the current reference and only a
  // sum above 2^32, or a column without a reference yet, moves it to the
  // exact running max (rescaling O and the sum) and recomputes.
  constexpr float kSumLimit = 4294967296.f;

  // S_j^T = K_j Q^T: K operands from LDS (A), Q^T in registers (B).
  auto qk = [&](int j, f32x16& sd) VFA_INLINE {
    bf16x8 ka[D / 16];
    const char VFA_LDS* krow = kring + (j & (kRing - 1)) * S::KSLOT + l32 * S::KSTR + half * 16;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) ka[ks] = ov_read_b128(krow + ks * 32);
    sd = f32x16{};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) sd = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qreg[ks], sd, 0, 0, 0);
  };
  // O^T += V_j^T P_j^T: V^T operands through the transposed LDS read (A), P^T in registers (B).
  auto pv = [&](int j, const bf16x8 (&pp)[2]) VFA_INLINE {
    bf16x8 va[2][D / 32];
    const char VFA_LDS* vb = vring + (j & (kRing - 1)) * S::VSLOT;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const char VFA_LDS* vrow = vb + (hh * 16 + tr_key) * S::VSTR + tr_d * 2;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) va[hh][db] = ov_read_tr_pair(vrow + db * 64, vrow + 8 * S::VSTR + db * 64);
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[hh][db], pp[hh], acc[db], 0, 0, 0);
  };
  // Probabilities against the current reference and their fp32 sum (of the
  // unrounded values, so lse stays fp32-accurate), summed as a tree.
  auto exps = [&](const f32x16& sc, float (&e)[16], float& ts) VFA_INLINE {
#pragma unroll
    for (int r = 0; r < 16; ++r) e[r] = fast_exp2(__builtin_fmaf(sc[r], scale_log2, -mref));
    float t8[8], t4[4];
#pragma unroll
    for (int r = 0; r < 8; ++r) t8[r] = e[r] + e[r + 8];
#pragma unroll
    for (int r = 0; r < 4; ++r) t4[r] = t8[r] + t8[r + 4];
    ts = (t4[0] + t4[2]) + (t4[1] + t4[3]);
  };

  // P^T (B operand) for a sub-block's two 16-key steps.
  auto to_p = [&](const float (&e)[16], bf16x8 (&pp)[2]) VFA_INLINE {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      bf16x2 pr[4];
#pragma unroll
      for (int y = 0; y < 4; ++y) pr[y] = f32x2_to_bf16x2(e[hh * 8 + 2 * y], e[hh * 8 + 2 * y + 1]);
      pp[hh] = bf16x8{pr[0][0], pr[0][1], pr[1][0], pr[1][1], pr[2][0], pr[2][1], pr[3][0], pr[3][1]};
    }
  };

  // One iteration: the softmax of sub-block j (scores in s_cur, P_j into
  // p_cur) between the MFMAs of QK_{j+1} (into s_next) and PV_{j-1} (with
  // p_prev), plus the group's staging. A reference move (the slow path)
  // recomputes P_j. `st` is the staging set that holds sub-block j + ahead.
  auto step = [&](auto do_qk, auto do_pv, int j, f32x16& s_cur, f32x16& s_next, bf16x8 (&p_cur)[2],
                  const bf16x8 (&p_prev)[2], u32x4 (&st)[PT]) VFA_INLINE {
    constexpr bool QK = decltype(do_qk)::value, PV = decltype(do_pv)::value;
    if (j >= j_full) {   // a tile-edge sub-block: mask keys past the row's last visible one
      const int lim = CAUSAL ? min(lk - 1, tq + diag) : lk - 1;
      const int kb0 = j * kSub + half * 4;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kb0 + (r >> 2) * 8 + (r & 3) > lim) s_cur[r] = neg_inf();
    }
    __builtin_amdgcn_sched_barrier(0);
    float e[16], ts;
    if constexpr (QK && PV) {
      // Sixteen MFMA slots, the order fixed by scheduling barriers between
      // them. Slot i < 8: the probability of score i, QK MFMA i, and the two
      // transposed reads of PV operand i. Slot 8 + i: the probability of
      // score 8 + i, its share of the running sum, and PV MFMA i, whose
      // operand was read 8 slots earlier. Each pair of probabilities becomes
      // bf16 P as soon as both exist, so few fp32 values stay live. The K
      // operands are read up front.
      bf16x8 ka[D / 16], va[2][D / 32];
      const char VFA_LDS* krow = kring + ((j + 1) & (kRing - 1)) * S::KSLOT + l32 * S::KSTR + half * 16;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) ka[ks] = ov_read_b128(krow + ks * 32);
      const char VFA_LDS* vb = vring + ((j - 1) & (kRing - 1)) * S::VSLOT + tr_key * S::VSTR + tr_d * 2;
      s_next = f32x16{};
      constexpr int NQK = D / 16, NPV = 2 * (D / 32);   // 8 and 8 at D = 128, 4 and 4 at D = 64
      constexpr int SPS = 8 / NQK;                       // scores per slot
      static_assert(NQK == NPV && SPS * NQK == 8, "the 16 scores spread evenly over the slots");
      bf16x2 pr[8];
      float sum_a, sum_b;   // each starts at its first pair's sum (no add of zero)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NQK; ++i) {
#pragma unroll
        for (int u = 0; u < SPS; ++u) {
          const int r = i * SPS + u;
          e[r] = fast_exp2(__builtin_fmaf(s_cur[r], scale_log2, -mref));
          if (r & 1) {
            pr[r >> 1] = f32x2_to_bf16x2(e[r - 1], e[r]);
            sum_a = r == 1 ? e[0] + e[1] : sum_a + (e[r - 1] + e[r]);
          }
        }
        s_next = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[i], qreg[i], s_next, 0, 0, 0);
        const int hh = i / (D / 32), db = i % (D / 32);
        const char VFA_LDS* vrow = vb + hh * 16 * S::VSTR;
        va[hh][db] = ov_read_tr_pair(vrow + db * 64, vrow + 8 * S::VSTR + db * 64);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
#pragma unroll
        for (int u = 0; u < SPS; ++u) {
          const int r = 8 + i * SPS + u;
          e[r] = fast_exp2(__builtin_fmaf(s_cur[r], scale_log2, -mref));
          if (r & 1) {
            pr[r >> 1] = f32x2_to_bf16x2(e[r - 1], e[r]);
            sum_b = r == 9 ? e[8] + e[9] : sum_b + (e[r - 1] + e[r]);
          }
        }
        const int hh = i / (D / 32), db = i % (D / 32);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[hh][db], p_prev[hh], acc[db], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      ts = sum_a + sum_b;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        p_cur[hh] = bf16x8{pr[4 * hh][0], pr[4 * hh][1], pr[4 * hh + 1][0], pr[4 * hh + 1][1],
                           pr[4 * hh + 2][0], pr[4 * hh + 2][1], pr[4 * hh + 3][0], pr[4 * hh + 3][1]};
    } else {
      if constexpr (QK) qk(j + 1, s_next);
      if constexpr (PV) pv(j - 1, p_prev);
      exps(s_cur, e, ts);
      to_p(e, p_cur);
    }
    sstore(st, j + ahead);
    gload(st, min(j + ahead + 1, last));
    __builtin_amdgcn_sched_barrier(0);
    const bool slow = !(ts <= kSumLimit) || m_run == neg_inf();
    if (__builtin_amdgcn_ballot_w64(slow)) {
      float x = neg_inf();
#pragma unroll
      for (int r = 0; r < 16; ++r) x = fmaxf(x, s_cur[r]);
      // The other lane half holds the other keys of the same column.
      auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
      const float m_new = fmaxf(m_run, fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])));
      // Unchanged references scale by exactly 1 (m_run may be -inf); one moving
      // up from -inf scales the (zero) history by 0. O here already holds PV_{j-1}.
      const float alpha = m_new == m_run ? 1.f : fast_exp2((m_run - m_new) * scale_log2);
      m_run = m_new;
      mref = m_new == neg_inf() ? 0.f : m_new * scale_log2;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
      exps(s_cur, e, ts);
      to_p(e, p_cur);
    }
    l_run += ts;
  };

  // Prologue: sub-blocks 0-2 of the group's tensor into the ring (the V waves
  // store V_1 and V_2 here and again in iterations 0 and 1, with the same
  // data, so that both groups run the same loads), then the first staged
  // sub-block in flight.
  u32x4 st[PT];
  if (n_sub > 0) {
    u32x4 t1[PT], t2[PT];
    gload(st, 0);
    gload(t1, min(1, last));
    gload(t2, min(2, last));
    sstore(st, 0);
    sstore(t1, 1);
    sstore(t2, 2);
    gload(st, min(ahead, last));
  }
  tile_barrier();

  using yes = std::integral_constant<bool, true>;
  using no = std::integral_constant<bool, false>;
  f32x16 sa, sb;
  bf16x8 pa[2], pb[2];
  // Iteration j uses scores / probabilities a or b by the parity of j. A tile
  // barrier precedes every even iteration after the first, and the final PV
  // when it falls on an even position.
  if (n_sub > 0) {
    // QK_0 reads K_0, whose slot iteration 1 refills with K_4: every wave's
    // reads of it complete before any wave goes on.
    qk(0, sa);
    tile_barrier();
    if (n_sub == 1) {
      step(no{}, no{}, 0, sa, sb, pa, pb, st);
      pv(0, pa);
    } else {
      step(yes{}, no{}, 0, sa, sb, pa, pb, st);
      int j = 1;
      for (; j + 2 < n_sub; j += 2) {
        step(yes{}, yes{}, j, sb, sa, pb, pa, st);
        tile_barrier();
        step(yes{}, yes{}, j + 1, sa, sb, pa, pb, st);
      }
      if (j == n_sub - 1) {          // last sub-block odd
        step(no{}, yes{}, j, sb, sa, pb, pa, st);
        tile_barrier();
        pv(j, pb);
      } else {                       // j == n_sub - 2: last sub-block even
        step(yes{}, yes{}, j, sb, sa, pb, pa, st);
        tile_barrier();
        step(no{}, yes{}, j + 1, sa, sb, pa, pb, st);
        pv(j + 1, pa);
      }
    }
  }

  // Epilogue: combine the two lane halves' partial sums, normalise, store.
  const float l_tot = l_run + xor_shuffle(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const size_t row = (size_t)(q0 + tq) * hq + head;
  OutT* orow = out + row * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const f32x16& a = acc[db];
    if constexpr (sizeof(OutT) == 2) {
      // A lane holds, per 32-dim block and group g4, the 4 dims g4*8 + half*4 ..;
      // the two halves trade one group of each pair (lanes i and i + 32 own the
      // same query) so that each lane stores 8 contiguous dims (16 B).
      auto pk = [&](int r) VFA_INLINE {
        return __builtin_bit_cast(uint32_t, f32x2_to_bf16x2(a[r] * inv, a[r + 1] * inv));
      };
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        const int ga = 2 * gp, gb = 2 * gp + 1;   // half 0 stores group ga, half 1 group gb
        const uint32_t a0 = pk(ga * 4), a1 = pk(ga * 4 + 2), b0 = pk(gb * 4), b1 = pk(gb * 4 + 2);
        const auto s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
        const u32x4 val = half == 0 ? u32x4{a0, a1, s0[1], s1[1]} : u32x4{s0[0], s1[0], b0, b1};
        u32x4* dst = (u32x4*)(orow + db * 32 + (half == 0 ? ga : gb) * 8);
        if (qvalid) *dst = val;
      }
    } else {
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
}

// Persistent grid: one workgroup per CU of the stream's device (a multiple of
// the 8 XCDs), looked up once per device.
int persistent_grid(hipStream_t stream) {
  static int cus[64] = {};
  hipDevice_t dev = 0;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return -1;
    cus[dev] = n;
  }
  return cus[dev] < kXcds ? kXcds : cus[dev] / kXcds * kXcds;
}

template <int D, bool CAUSAL, typename OutT>
int launch_t(const AttnArgs& a) {
  const int tokw = kCols / a.grp;
  const int n_mtiles = (a.max_seqlen_q + tokw - 1) / tokw;
  const long long pairs_per_xcd = ((long long)a.batch * a.hkv + kXcds - 1) / kXcds;
  const long long slots = (long long)n_mtiles * pairs_per_xcd;
  if (slots <= 0) return 0;
  if (slots > 0x7fffff00LL) return -1;   // the counters run past the last slot by one draw per workgroup
  hipStream_t st = (hipStream_t)a.stream;
  const int grid = persistent_grid(st);
  if (grid <= 0) return -1;
  int* tickets = (int*)a.workspace;
  hipLaunchKernelGGL(zero_tickets_kernel, dim3(1), dim3(64), 0, st, tickets);
  hipLaunchKernelGGL((attn_fwd_overlap_kernel<D, CAUSAL, OutT>), dim3((unsigned)grid), dim3(kThreads), 0, st,
                     (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, a.cu_q, a.cu_k, a.causal_off, a.batch,
                     a.hq, a.hkv, a.grp, tokw, n_mtiles, a.scale, a.scale * kLog2e, (OutT*)a.out, a.lse, tickets);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_attn_fwd_overlap(const AttnArgs& a) {
  const bool f32out = a.out_dtype == 0;
  if (a.head_dim == 128) {
    if (a.causal) return f32out ? launch_t<128, true, float>(a) : launch_t<128, true, bf16>(a);
    return f32out ? launch_t<128, false, float>(a) : launch_t<128, false, bf16>(a);
  }
  if (a.causal) return f32out ? launch_t<64, true, float>(a) : launch_t<64, true, bf16>(a);
  return f32out ? launch_t<64, false, float>(a) : launch_t<64, false, bf16>(a);
}

}  // namespace vfa
