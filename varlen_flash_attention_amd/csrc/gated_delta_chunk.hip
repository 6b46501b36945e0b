// Varlen gated delta rule forward in the chunked (WY) form, on bf16 MFMA with
// fp32 state.
//
// "Twinkle NPU kernels" (Qwen3.5 flash linear attention section) runs
// chunk_gated_delta_rule: the recurrence, per (sequence, value head),
//   S <- exp(g_t) S ;  u_t = beta_t (v_t - S^T k_t) ;  S <- S + k_t u_t^T ;
//   o_t = scale * S^T q_t
// reorganised over chunks of C = 64 tokens. Inside a chunk starting from state
// S, with gamma_i the cumulative log decay of its first i + 1 tokens:
//   (I + A) U = beta (V - e^gamma (K S)),  A_ij = beta_i e^(gamma_i - gamma_j) k_i.k_j (j < i)
//   O = scale (e^gamma (Q S) + M U),       M_ij = e^(gamma_i - gamma_j) q_i.k_j     (j <= i)
//   S' = e^gamma_end S + K^T (e^(gamma_end - gamma) U)
//
// Two kernels:
//   gdn_prep_kernel  one wave per (sequence, chunk, value head), all in
//                    parallel: gamma (fp64 scan), K K^T and K Q^T on MFMA,
//                    T = (I + A)^-1 by forward substitution in fp32, then T and
//                    M as bf16 hi / lo pairs and the two decay factors per token
//                    into the workspace. Its first workgroups also rank the
//                    sequences by length (longest first) for the second kernel.
//   gdn_chunk_kernel one workgroup per (sequence, value head, 64 state
//                    columns), one wave per 16 columns, chunks in order: y = K S and Q S, then
//                    U = T r with r = beta (V - e^gamma y), then M U for the
//                    output and K^T U~ for the state. Workgroups take the
//                    sequences longest first: each one's chunks form a serial
//                    chain, and a long chain started late ends after the rest
//                    of the grid has drained.
//
// Precision: the state stays fp32 in MFMA accumulators. Products with an fp32
// operand split it into bf16 hi + lo and take hi.hi + hi.lo + lo.hi (K and Q
// are bf16 already, so their products take hi and lo of the other side); the
// dropped lo.lo term is below 2^-16 relative. (Taking S's hi part alone in
// y = K S leaves the output within its bound, but a nonzero initial state then
// drifts past the state's bound, so the lo pass stays.)
//
// Operand layout: accumulators feed the next product as B operands directly
// when the memory-side A operand reads its k values in the accumulator's row
// order; K^T and V come from the staged chunk through the LDS transpose read,
// which delivers that order.
#include "common.h"
#include "launch.h"

namespace vfa {
namespace {

constexpr int kC = kGdnChunk;          // tokens per chunk

typedef __attribute__((__vector_size__(2 * sizeof(double)))) double f64x2;

__device__ __forceinline__ bf16x8 join(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x8 lds_read_tr(const char VFA_LDS* p0, const char VFA_LDS* p1) {
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 VFA_LDS*)p0);
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 VFA_LDS*)p1);
  return join(__builtin_bit_cast(bf16x4, lo), __builtin_bit_cast(bf16x4, hi));
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Workgroup id -> (item, inner) with the `inner` workgroups of one item on one
// XCD (workgroups are dispatched round-robin over the 8 XCDs), 8 ids apart, so
// they share that XCD's L2: the value heads of one query / key head read the
// same K and Q rows, the column groups of one head the same staged chunks.
// Bijective on [0, items * inner); the last items % 8 items keep plain order.
__device__ __forceinline__ void xcd_decode(int idx, int items, int inner, int& item, int& in) {
  const int full = (items / 8) * 8 * inner;
  if (idx < full) {
    const int slot = idx / 8;
    item = (slot / inner) * 8 + idx % 8;
    in = slot % inner;
  } else {
    const int r = idx - full;
    item = (items / 8) * 8 + r / inner;
    in = r % inner;
  }
}

// e^x for a log decay held in fp64: x rounded to fp32, then the hardware exp2.
__device__ __forceinline__ float decay_factor(double x) { return fast_exp2((float)x * kLog2e); }

// Workspace rows, one per (token, value head): T (hi then lo, kC each) and M
// (the same), bf16; then two fp32 decay factors per (token, value head); then
// the chunk kernel's sequence order (a fixed slot of kOrderMax int32).
__device__ __forceinline__ size_t ws_row(size_t t, int hv, int h) { return (t * hv + h) * (2 * kC); }

// ---------------------------------------------------------------------------
// Phase 1: per (sequence, chunk, value head), independent of the state.
template <int DK>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2))) void gdn_prep_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const float* __restrict__ g,
    const float* __restrict__ beta, const int32_t* __restrict__ cu, int batch, int hqk, int hv, int n_chunks,
    bf16* __restrict__ wt, bf16* __restrict__ wm, float* __restrict__ we, int32_t* __restrict__ order) {
  // Sequence order for the chunk kernel: order[r] = the sequence of rank r by
  // length, longest first, ties by index (a permutation). One sequence per
  // lane of the first ceil(batch / 64) workgroups, ranked against all others.
  if (order && (int)blockIdx.x * 64 < batch) {
    const int sq = (int)blockIdx.x * 64 + (int)threadIdx.x;
    if (sq < batch) {
      const int ls = cu[sq + 1] - cu[sq];
      int rank = 0;
      for (int b2 = 0; b2 < batch; ++b2) {
        const int l2 = cu[b2 + 1] - cu[b2];
        rank += (l2 > ls) || (l2 == ls && b2 < sq);
      }
      order[rank] = sq;
    }
  }
  __shared__ __attribute__((aligned(16))) double sgam[kC];
  __shared__ float sbeta[kC];
  __shared__ __attribute__((aligned(16))) float sat[kC][kC + 4];   // A transposed: sat[j][i] = A_ij

  const int rep_v = hv / hqk;           // value heads per query / key head
  int item, vi;
  xcd_decode(blockIdx.x, gridDim.x / rep_v, rep_v, item, vi);
  const int hk0 = item % hqk;
  const int c = (item / hqk) % n_chunks;
  const int b = item / (hqk * n_chunks);
  const int h = hk0 * rep_v + vi;
  const int len = cu[b + 1] - cu[b];
  if (c * kC >= len) return;
  const int t0 = cu[b] + c * kC;
  const int n = min(kC, len - c * kC);
  const int hk = hk0;
  const int lane = threadIdx.x;
  const int l32 = lane & 31, half = lane >> 5;

  // g and beta first (rows past n repeat the last token, then are zeroed),
  // then the K and Q operands of the products below (rows m = key token j,
  // columns n = token i, same clamp): the scan waits only for the first two,
  // and the operands arrive while it runs.
  const size_t gb_row = (size_t)(t0 + min(lane, n - 1)) * hv + h;
  const float g_raw = g[gb_row];
  const float b_raw = beta[gb_row];
  bf16x8 ka[2][DK / 16], qa[2][DK / 16];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const size_t row = ((size_t)(t0 + min(32 * t + l32, n - 1)) * hqk + hk) * DK + 8 * half;
#pragma unroll
    for (int ks = 0; ks < DK / 16; ++ks) {
      ka[t][ks] = *(const bf16x8*)(k + row + 16 * ks);
      qa[t][ks] = *(const bf16x8*)(q + row + 16 * ks);
    }
  }

  // gamma: inclusive prefix sum of g over the chunk, in fp64 so that the
  // differences gamma_i - gamma_j keep fp32 accuracy however long the decay
  // runs; each difference is then rounded to fp32 and exponentiated there.
  double gl = lane < n ? (double)g_raw : 0.0;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double o = __shfl_up(gl, off, 64);
    if (lane >= off) gl += o;
  }
  sgam[lane] = gl;                              // lanes past n repeat gamma_{n-1}
  sbeta[lane] = lane < n ? b_raw : 0.f;
  __syncthreads();
  if (lane < n) {
    const size_t o = (size_t)(t0 + lane) * hv + h;
    we[2 * o] = decay_factor(gl);                     // e^gamma_i
    we[2 * o + 1] = decay_factor(sgam[n - 1] - gl);   // e^(gamma_end - gamma_i)
  }

  // Products with rows m = key token j and columns n = token i, so that a
  // lane (column i) holds four consecutive j of row i of A and M: K K^T (for
  // A) and K Q^T (for M). Tiles (mt, nt) = (0,0), (0,1), (1,1); tile (1, 0)
  // has j > i only, where both are zero.
  // Every operand is consumed here, so all loads are in flight together and
  // the products below wait on memory once (left alone, the compiler keeps
  // only a few loads ahead of the products and pays several round trips).
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int ks = 0; ks < DK / 16; ++ks) __asm__ volatile("" ::"v"(ka[t][ks]), "v"(qa[t][ks]));
  constexpr int kMt[3] = {0, 0, 1}, kNt[3] = {0, 1, 1};
  f32x16 kk[3] = {}, kq[3] = {};
#pragma unroll
  for (int ks = 0; ks < DK / 16; ++ks)
#pragma unroll
    for (int tile = 0; tile < 3; ++tile) {
      kk[tile] = mfma(ka[kMt[tile]][ks], ka[kNt[tile]][ks], kk[tile]);
      kq[tile] = mfma(ka[kMt[tile]][ks], qa[kNt[tile]][ks], kq[tile]);
    }

  // The workspace rows of T and M (256 bytes each, 8 KB apart from token to
  // token) leave through LDS: each matrix is first laid out there by rows
  // (272-byte stride), then written as whole rows, 16 bytes per lane. Stored
  // straight from registers they take 2- or 8-byte pieces of many rows per
  // instruction. The staging reuses the array that holds A.
  constexpr int SROW = 2 * kC * 2 + 16;
  static_assert(kC * SROW <= (int)sizeof(sat), "staging must fit the A array");
  char VFA_LDS* stg = (char VFA_LDS*)&sat[0][0];
  // Lane l moves 16-byte piece l % 16 of rows l / 16 + 4 it. All pieces are
  // read before the first store, and full chunks store without a row test
  // (a per-row branch makes the compiler pair each read with its store).
  auto store_rows = [&](bf16* base) __attribute__((always_inline)) {
    constexpr int NP = kC * 16 / 64;
    const int r0 = lane >> 4, c16 = lane & 15;
    u32x4 val[NP];
#pragma unroll
    for (int it = 0; it < NP; ++it) val[it] = *(const u32x4 VFA_LDS*)(stg + (r0 + 4 * it) * SROW + 16 * c16);
    bf16* dst = base + ws_row(t0 + r0, hv, h) + 8 * c16;
    const size_t step = (size_t)4 * hv * (2 * kC);      // 4 rows further
    if (n == kC) {
#pragma unroll
      for (int it = 0; it < NP; ++it) *(u32x4*)(dst + it * step) = val[it];
    } else {
#pragma unroll
      for (int it = 0; it < NP; ++it)
        if (r0 + 4 * it < n) *(u32x4*)(dst + it * step) = val[it];
    }
  };

  // A_ij = beta_i e^(gamma_i - gamma_j) k_i.k_j (j < i), kept in registers
  // until M has left; M_ij = e^(gamma_i - gamma_j) q_i.k_j (j <= i), hi / lo,
  // four consecutive columns per 8-byte write into the staging rows.
  float av[3][16];
#pragma unroll
  for (int tile = 0; tile < 3; ++tile) {
    const int i = 32 * kNt[tile] + l32;
    const double gi = sgam[i];
    const float bi = sbeta[i];
    const bool live = i < n;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int jb = 32 * kMt[tile] + 8 * g4 + 4 * half;
      double gj[4];
      *(f64x2*)&gj[0] = *(const f64x2*)&sgam[jb];
      *(f64x2*)&gj[2] = *(const f64x2*)&sgam[jb + 2];
      float mv[4];
#pragma unroll
      for (int z = 0; z < 4; ++z) {
        const int r = 4 * g4 + z;
        const int j = jb + z;
        // Computed for every j and selected after (for j > i it may be inf,
        // which the select drops): no branch around the fp64 difference.
        const float e = decay_factor(gi - gj[z]);
        const float d = (j <= i) ? e : 0.f;
        av[tile][r] = (live && j < i) ? bi * d * kk[tile][r] : 0.f;
        mv[z] = d * kq[tile][r];
      }
      const bf16x2 h01 = f32x2_to_bf16x2(mv[0], mv[1]), h23 = f32x2_to_bf16x2(mv[2], mv[3]);
      const bf16x2 l01 = f32x2_to_bf16x2(mv[0] - (float)h01[0], mv[1] - (float)h01[1]);
      const bf16x2 l23 = f32x2_to_bf16x2(mv[2] - (float)h23[0], mv[3] - (float)h23[1]);
      char VFA_LDS* mrow = stg + i * SROW + 2 * jb;
      *(bf16x4 VFA_LDS*)mrow = bf16x4{h01[0], h01[1], h23[0], h23[1]};
      *(bf16x4 VFA_LDS*)(mrow + 2 * kC) = bf16x4{l01[0], l01[1], l23[0], l23[1]};
    }
  }
  // Tile (1, 0): j >= 32 > i, zero in A and M.
#pragma unroll
  for (int g4 = 0; g4 < 4; ++g4) {
    char VFA_LDS* mrow = stg + l32 * SROW + 2 * (32 + 8 * g4 + 4 * half);
    *(bf16x4 VFA_LDS*)mrow = bf16x4{};
    *(bf16x4 VFA_LDS*)(mrow + 2 * kC) = bf16x4{};
  }
  __syncthreads();
  store_rows(wm);
  __syncthreads();
  // A into the same array, transposed: sat[j][i] = A_ij.
#pragma unroll
  for (int tile = 0; tile < 3; ++tile) {
    const int i = 32 * kNt[tile] + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) sat[32 * kMt[tile] + 8 * (r / 4) + 4 * half + r % 4][i] = av[tile][r];
  }
#pragma unroll
  for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
    for (int z = 0; z < 4; ++z) sat[32 + 8 * g4 + 4 * half + z][l32] = 0.f;
  __syncthreads();

  // T = (I + A)^-1 by forward substitution, lane = column c of T, in the
  // right-looking order: x starts as e_c; once x_j is final, every later row
  // takes its term, x_i -= A_ij x_j (i > j). The updates of one step are
  // independent, and column j of A is one broadcast read per four rows.
  // Column j + 1 of A is read while step j's updates run (read just before
  // its use, each broadcast read waits out a full LDS round trip).
  float x[kC];
#pragma unroll
  for (int i = 0; i < kC; ++i) x[i] = (i == lane) ? 1.f : 0.f;
  f32x4 acol[2][kC / 4];
#pragma unroll
  for (int q4 = 0; q4 < kC / 4; ++q4) acol[0][q4] = *(const f32x4*)&sat[0][4 * q4];
#pragma unroll
  for (int j = 0; j < kC - 1; ++j) {
    const int cur = j & 1;
    if (j + 1 < kC - 1) {
#pragma unroll
      for (int q4 = (j + 2) >> 2; q4 < kC / 4; ++q4) acol[cur ^ 1][q4] = *(const f32x4*)&sat[j + 1][4 * q4];
    }
    __builtin_amdgcn_sched_barrier(0);
    const float xj = x[j];
#pragma unroll
    for (int q4 = (j + 1) >> 2; q4 < kC / 4; ++q4) {
#pragma unroll
      for (int z = 0; z < 4; ++z)
        if (4 * q4 + z > j) x[4 * q4 + z] -= acol[cur][q4][z] * xj;
    }
    // Materialise this step's updates here. Left free, the compiler defers
    // each row's chain of updates to its end, keeping every loaded A value
    // live at once (far more than the register file).
#pragma unroll
    for (int i = j + 1; i < kC; ++i) __asm__ volatile("" : "+v"(x[i]));
  }
  __syncthreads();
  // T rows (hi then lo) through the staging rows: lane c holds column c.
#pragma unroll
  for (int i = 0; i < kC; ++i) {
    const bf16 th = (bf16)x[i];
    *(bf16 VFA_LDS*)(stg + i * SROW + 2 * lane) = th;
    *(bf16 VFA_LDS*)(stg + i * SROW + 2 * kC + 2 * lane) = (bf16)(x[i] - (float)th);
  }
  __syncthreads();
  store_rows(wt);
}

// ---------------------------------------------------------------------------
// Phase 2: per (sequence, value head, 64-column group), chunks in order. The
// four "chain" waves own 16 state columns each and run the dependent chain
// y = K S -> r -> U = T r -> S' = e^gamma_end S + K^T U~; four "output" waves,
// one per chain wave, compute O = scale (e^gamma Q S + M U) for the same
// columns from S and U that the chain waves leave in LDS already split into
// bf16 hi / lo B operands. Each role stages what it reads: during chunk c the
// chain waves load chunk c+1's K, T and V rows into registers and store them
// after their state update (K into the second of two buffers, since the
// update still reads this chunk's K); the output waves do the same for Q, M
// and the per-token beta and decay factors after their stores, having taken
// their M operands into registers before the mid-chunk barrier. Per chunk:
// barrier A (chunk staged, S published), chain y, r, U / output Q S, barrier
// B (U published), chain state update and staging / output M U, stores and
// staging.
//
// Products use v_mfma_f32_16x16x32_bf16 (lane (c16, g) holds k-slots 8 g + 0..7
// of its row or column, and accumulator rows 4 g + 0..3). Two 16-row
// accumulator tiles form one 32-deep B operand, k-slot 8 g + x holding row
// {4 g + x, 16 + 4 g + x - 4}; memory-side A operands read their k values in
// that order (two 8-byte runs 32 bytes apart), and the transposed LDS read
// pair 16 rows apart delivers it too.
constexpr int kChainWaves = 4;
constexpr int kChunkWaves = 2 * kChainWaves;       // chain + output waves
constexpr int kGroupCols = kChainWaves * 16;       // state columns per workgroup

template <int DK>
struct ChunkSmem {
  static constexpr int STAGERS = kChainWaves * 64;  // threads of one role (each role stages its tensors)
  static constexpr int DV = kGroupCols;         // staged V columns
  // Row strides of 2 D + 16 bytes (D = 64 or 128): both the A-operand row
  // reads (lane (c16, g) at row c16, dword 2 g) and the transposed reads (rows
  // 4 g + 0..3, dwords 2 (i & 3)) then touch each of the 64 banks exactly
  // twice per wave, the minimum for 8-byte accesses (a 64-byte pad folds
  // them four ways).
  static constexpr int KSTR = DK * 2 + 16;     // K rows (row and transposed reads)
  static constexpr int QSTR = DK * 2 + 16;     // Q rows
  static constexpr int TSTR = 2 * kC * 2 + 16; // T and M rows (hi | lo)
  static constexpr int VSTR = DV * 2 + 16;     // V rows of this group's columns (transposed reads)
  static constexpr int K_OFF = 0;              // two K buffers (chunk parity)
  static constexpr int KBUF = kC * KSTR;
  static constexpr int Q_OFF = K_OFF + 2 * KBUF;
  static constexpr int T_OFF = Q_OFF + kC * QSTR;
  static constexpr int M_OFF = T_OFF + kC * TSTR;
  static constexpr int V_OFF = M_OFF + kC * TSTR;
  // Hand-over buffers, one 16-byte B operand per lane: S (DK / 32 k steps, hi
  // and lo) and U (2 k steps, hi and lo) per chain wave.
  static constexpr int SB_OFF = V_OFF + kC * VSTR;
  static constexpr int SB_WAVE = (DK / 32) * 2 * 64 * 16;
  static constexpr int UB_OFF = SB_OFF + kChainWaves * SB_WAVE;
  static constexpr int UB_WAVE = 2 * 2 * 64 * 16;
  static constexpr int BYTES = UB_OFF + kChainWaves * UB_WAVE;
  // 16-byte pieces per staging thread for each staged tensor.
  static constexpr int PK = kC * DK / 8 / STAGERS;
  static constexpr int PT = kC * (2 * kC) / 8 / STAGERS;
  static constexpr int PV = kC * DV / 8 / STAGERS;
  static_assert(PK * STAGERS * 8 == kC * DK && PT * STAGERS * 8 == kC * 2 * kC && PV * STAGERS * 8 == kC * DV,
                "pieces must split evenly over the staging threads");
};

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// A operand read for the 16x16x32 k order: runs at p and p + 32 bytes.
__device__ __forceinline__ bf16x8 lds_perm16(const char VFA_LDS* p) {
  return join(*(const bf16x4 VFA_LDS*)p, *(const bf16x4 VFA_LDS*)(p + 32));
}

// bf16 hi / lo of two 16-row accumulator tiles as one 32-deep B operand.
__device__ __forceinline__ void split_pair(const f32x4& t0, const f32x4& t1, bf16x8& hi, bf16x8& lo) {
  const float x[8] = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
#pragma unroll
  for (int y = 0; y < 8; y += 2) {
    const bf16x2 h = f32x2_to_bf16x2(x[y], x[y + 1]);
    const bf16x2 l = f32x2_to_bf16x2(x[y] - (float)h[0], x[y + 1] - (float)h[1]);
    hi[y] = h[0]; hi[y + 1] = h[1];
    lo[y] = l[0]; lo[y + 1] = l[1];
  }
}

template <int DK, int DV>
__global__ __launch_bounds__(kChunkWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void gdn_chunk_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ beta, const int32_t* __restrict__ cu, int hqk, int hv, float scale,
    const float* __restrict__ s_init, bf16* __restrict__ out, float* __restrict__ s_final,
    const bf16* __restrict__ wt, const bf16* __restrict__ wm, const float* __restrict__ we,
    const int32_t* __restrict__ order) {
  using S = ChunkSmem<DK>;
  constexpr int NCG = DV / kGroupCols;  // column groups per head
  constexpr int NDT = DK / 16;          // 16-row tiles of the state
  constexpr int NKS = DK / 32;          // 32-deep k steps over the state rows
  __shared__ __attribute__((aligned(16))) char smem[S::BYTES];
  __shared__ __attribute__((aligned(16))) float se1[kC], se2[kC], sbt[kC];
  char VFA_LDS* lds = (char VFA_LDS*)smem;
  char VFA_LDS* sq = lds + S::Q_OFF;
  char VFA_LDS* stt = lds + S::T_OFF;
  char VFA_LDS* smm = lds + S::M_OFF;
  char VFA_LDS* sv = lds + S::V_OFF;

  int item, cg;
  xcd_decode(blockIdx.x, gridDim.x / NCG, NCG, item, cg);
  const int h = item % hv;
  const int b = order ? order[item / hv] : item / hv;   // longest sequences first
  const int hk = h / (hv / hqk);
  const int ts = cu[b];
  const int len = cu[b + 1] - ts;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const bool chain = wave < kChainWaves;           // wave-uniform role
  // Chain wave w and output wave w + 4 share a SIMD, both at the default issue
  // priority (raising the chain's measured 1% slower).
  const int pw = wave % kChainWaves;               // column slot shared by a chain / output pair
  const int stid = tid % (kChainWaves * 64);       // staging thread index within the role
  const int lane = tid & 63, c16 = lane & 15, g = lane >> 4;
  const int lcol0 = pw * 16;                       // first column of the pair within the group
  const int col = cg * kGroupCols + lcol0 + c16;
  // This pair's hand-over slots, indexed [k step][hi, lo][lane] of 16 bytes.
  char VFA_LDS* sbuf = lds + S::SB_OFF + pw * S::SB_WAVE + lane * 16;
  char VFA_LDS* ubuf = lds + S::UB_OFF + pw * S::UB_WAVE + lane * 16;

  // Transposed reads: lane (c16, g) receives column c16 of a 16-wide block for
  // rows {4 g + 0..3} (first read) and {16 + 4 g + 0..3} (second, 16 rows on).
  const int tr_i = lane & 15;
  const int tr_key = g * 4 + (tr_i >> 2);
  const int tr_d = 4 * (tr_i & 3);

  // Chain waves: state rows d = 16 dt + 4 g + r, column col; and its bf16
  // hi / lo B operands, published to the output wave through sbuf.
  f32x4 st[NDT];
  bf16x8 sh[NKS], sl[NKS];
  const size_t sbase = ((size_t)b * hv + h) * DK * DV + col;
  if (chain) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        st[dt][r] = s_init ? s_init[sbase + (size_t)(16 * dt + 4 * g + r) * DV] : 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      split_pair(st[2 * ks], st[2 * ks + 1], sh[ks], sl[ks]);
      *(bf16x8 VFA_LDS*)(sbuf + (2 * ks) * 64 * 16) = sh[ks];
      *(bf16x8 VFA_LDS*)(sbuf + (2 * ks + 1) * 64 * 16) = sl[ks];
    }
  }

  // Staging. Rows past a chunk's end repeat its last row (finite values):
  // their beta and decay factors are zero, so they add nothing. Chain waves:
  // K, T, V; output waves: Q, M and the factors.
  u32x4 pk[S::PK], pt[S::PT], pv[S::PV];      // chain
  u32x4 pq[S::PK], pm[S::PT];                  // output
  float pe1 = 0.f, pe2 = 0.f, pbt = 0.f;      // output
  // Piece e = stid + i STAGERS of a staged tensor is row e / PR, 16-byte
  // column e % PR. In a full chunk its address is the chunk's first row (a
  // wave-uniform pointer) plus a 32-bit lane offset that stays the same for
  // every chunk (the entry point keeps 64 rows of each tensor under 4 GiB);
  // only a sequence's last, partial chunk clamps rows to its end.
  auto gather = [&](auto& dst, int pr, const char* base, uint32_t row_bytes, int n) __attribute__((always_inline)) {
    constexpr int CNT = sizeof(dst) / sizeof(dst[0]);
    if (n == kC) {
#pragma unroll
      for (int i = 0; i < CNT; ++i) {
        const int e = stid + i * S::STAGERS;
        dst[i] = *(const u32x4*)(base + ((uint32_t)(e / pr) * row_bytes + 16u * (uint32_t)(e % pr)));
      }
    } else {
#pragma unroll
      for (int i = 0; i < CNT; ++i) {
        const int e = stid + i * S::STAGERS;
        dst[i] = *(const u32x4*)(base + (size_t)min(e / pr, n - 1) * row_bytes + 16 * (e % pr));
      }
    }
  };
  const uint32_t k_row = (uint32_t)hqk * DK * sizeof(bf16);          // K and Q
  const uint32_t w_row = (uint32_t)hv * 2 * kC * sizeof(bf16);       // T and M
  const uint32_t v_row = (uint32_t)hv * DV * sizeof(bf16);
  auto load_chain = [&](int c0) __attribute__((always_inline)) {
    const int n = min(kC, len - c0);
    const int t0 = ts + c0;
    gather(pk, DK / 8, (const char*)(k + ((size_t)t0 * hqk + hk) * DK), k_row, n);
    gather(pt, 2 * kC / 8, (const char*)(wt + ws_row(t0, hv, h)), w_row, n);
    gather(pv, S::DV / 8, (const char*)(v + ((size_t)t0 * hv + h) * DV + cg * kGroupCols), v_row, n);
  };
  auto store_chain = [&](int parity) __attribute__((always_inline)) {
    char VFA_LDS* skw = lds + S::K_OFF + parity * S::KBUF;
#pragma unroll
    for (int i = 0; i < S::PK; ++i) {
      const int e = stid + i * S::STAGERS;
      *(u32x4 VFA_LDS*)(skw + (e / (DK / 8)) * S::KSTR + 16 * (e % (DK / 8))) = pk[i];
    }
#pragma unroll
    for (int i = 0; i < S::PT; ++i) {
      const int e = stid + i * S::STAGERS;
      *(u32x4 VFA_LDS*)(stt + (e / (2 * kC / 8)) * S::TSTR + 16 * (e % (2 * kC / 8))) = pt[i];
    }
#pragma unroll
    for (int i = 0; i < S::PV; ++i) {
      const int e = stid + i * S::STAGERS;
      *(u32x4 VFA_LDS*)(sv + (e / (S::DV / 8)) * S::VSTR + 16 * (e % (S::DV / 8))) = pv[i];
    }
  };
  auto load_out = [&](int c0) __attribute__((always_inline)) {
    const int n = min(kC, len - c0);
    const int t0 = ts + c0;
    gather(pq, DK / 8, (const char*)(q + ((size_t)t0 * hqk + hk) * DK), k_row, n);
    gather(pm, 2 * kC / 8, (const char*)(wm + ws_row(t0, hv, h)), w_row, n);
    if (stid < kC) {
      const bool ok = stid < n;
      const size_t o = (size_t)(t0 + (ok ? stid : 0)) * hv + h;
      pe1 = ok ? we[2 * o] : 0.f;
      pe2 = ok ? we[2 * o + 1] : 0.f;
      pbt = ok ? beta[o] : 0.f;
    }
  };
  auto store_out = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < S::PK; ++i) {
      const int e = stid + i * S::STAGERS;
      *(u32x4 VFA_LDS*)(sq + (e / (DK / 8)) * S::QSTR + 16 * (e % (DK / 8))) = pq[i];
    }
#pragma unroll
    for (int i = 0; i < S::PT; ++i) {
      const int e = stid + i * S::STAGERS;
      *(u32x4 VFA_LDS*)(smm + (e / (2 * kC / 8)) * S::TSTR + 16 * (e % (2 * kC / 8))) = pm[i];
    }
    if (stid < kC) {
      se1[stid] = pe1;
      se2[stid] = pe2;
      sbt[stid] = pbt;
    }
  };

  // The two roles run separate loops (so that neither holds the other's
  // registers), each with the same two barriers per chunk.
  if (chain) {
    if (len > 0) {
      load_chain(0);
      store_chain(0);
    }
    for (int c0 = 0; c0 < len; c0 += kC) {
      const int n = min(kC, len - c0);
      const char VFA_LDS* sk = lds + S::K_OFF + ((c0 / kC) & 1) * S::KBUF;   // this chunk's K
      __syncthreads();                  // A: chunk staged, S of this chunk start in sbuf

      // y = K S (hi and lo); rows: chunk tokens 16 mt + 4 g + r. All products
      // below run k step outer, row tile inner: each step's operands are read
      // together and the tiles' independent accumulators alternate, instead of
      // one tile's dependent chain at a time behind one read per step (each
      // accumulator still sums in the same order).
      f32x4 y[4] = {};
      const char VFA_LDS* kr = sk + c16 * S::KSTR + 8 * g;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        bf16x8 ak[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) ak[mt] = lds_perm16(kr + 16 * mt * S::KSTR + 64 * ks);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) y[mt] = mfma16(ak[mt], sh[ks], y[mt]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) y[mt] = mfma16(ak[mt], sl[ks], y[mt]);
      }
      // The next chunk's K, T and V go in flight after y, so that y starts right
      // at the barrier; they are needed only at the end of this chunk.
      if (c0 + kC < len) load_chain(c0 + kC);
      // r = beta (v - e^gamma y) in place; V comes through the transposed read,
      // already in accumulator row order.
#pragma unroll
      for (int s32 = 0; s32 < 2; ++s32) {
        const char VFA_LDS* p = sv + (32 * s32 + tr_key) * S::VSTR + tr_d * 2 + 2 * lcol0;
        const bf16x8 vv = lds_read_tr(p, p + 16 * S::VSTR);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int mt = 2 * s32 + hh;
          const int i0 = 16 * mt + 4 * g;
          const f32x4 e1 = *(const f32x4*)&se1[i0];
          const f32x4 bt = *(const f32x4*)&sbt[i0];
#pragma unroll
          for (int z = 0; z < 4; ++z) y[mt][z] = bt[z] * ((float)vv[4 * hh + z] - e1[z] * y[mt][z]);
        }
      }
      bf16x8 rh[2], rl[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) split_pair(y[2 * kk], y[2 * kk + 1], rh[kk], rl[kk]);

      // U = T r, published (hi / lo) for the output wave's M U.
      f32x4 u[4] = {};
      const char VFA_LDS* tr = stt + c16 * S::TSTR + 8 * g;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8 th[4], tl[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          th[mt] = lds_perm16(tr + 16 * mt * S::TSTR + 64 * kk);
          tl[mt] = lds_perm16(tr + 16 * mt * S::TSTR + 2 * kC + 64 * kk);
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) u[mt] = mfma16(th[mt], rh[kk], u[mt]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) u[mt] = mfma16(th[mt], rl[kk], u[mt]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) u[mt] = mfma16(tl[mt], rh[kk], u[mt]);
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8 uh, ul;
        split_pair(u[2 * kk], u[2 * kk + 1], uh, ul);
        *(bf16x8 VFA_LDS*)(ubuf + (2 * kk) * 64 * 16) = uh;
        *(bf16x8 VFA_LDS*)(ubuf + (2 * kk + 1) * 64 * 16) = ul;
      }
      // U~ = e^(gamma_end - gamma) U as B operands for the state update; the
      // decay is read now, before the staging after barrier B overwrites it.
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const f32x4 e2 = *(const f32x4*)&se2[16 * mt + 4 * g];
#pragma unroll
        for (int z = 0; z < 4; ++z) u[mt][z] *= e2[z];
      }
      bf16x8 wh[2], wl[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) split_pair(u[2 * kk], u[2 * kk + 1], wh[kk], wl[kk]);
      const float decay = se1[n - 1];

      __syncthreads();                  // B: U published; the output waves are done with sbuf

      // S <- e^gamma_end S + K^T U~ (this chunk's K buffer, which the staging
      // of the next chunk does not touch), then its split for the next chunk.
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) st[dt][r] *= decay;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int d0 = 0; d0 < NDT; d0 += 4) {       // four row tiles per batch of reads
          bf16x8 a[4];
#pragma unroll
          for (int dd = 0; dd < 4; ++dd) {
            const char VFA_LDS* p = sk + (32 * kk + tr_key) * S::KSTR + tr_d * 2 + 32 * (d0 + dd);
            a[dd] = lds_read_tr(p, p + 16 * S::KSTR);
          }
#pragma unroll
          for (int dd = 0; dd < 4; ++dd) st[d0 + dd] = mfma16(a[dd], wh[kk], st[d0 + dd]);
#pragma unroll
          for (int dd = 0; dd < 4; ++dd) st[d0 + dd] = mfma16(a[dd], wl[kk], st[d0 + dd]);
        }
      }
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        split_pair(st[2 * ks], st[2 * ks + 1], sh[ks], sl[ks]);
        *(bf16x8 VFA_LDS*)(sbuf + (2 * ks) * 64 * 16) = sh[ks];
        *(bf16x8 VFA_LDS*)(sbuf + (2 * ks + 1) * 64 * 16) = sl[ks];
      }
      // Stage the next chunk's K (other buffer), T and V: this wave's reads of
      // this chunk's T and V ended before barrier B.
      if (c0 + kC < len) store_chain(((c0 / kC) + 1) & 1);
    }
  } else {
    if (len > 0) {
      load_out(0);
      store_out();
    }
    for (int c0 = 0; c0 < len; c0 += kC) {
      const int n = min(kC, len - c0);
      const int t0 = ts + c0;
      __syncthreads();                  // A: chunk staged, S of this chunk start in sbuf

      // Q S from the chain wave's published S (hi and lo), scaled by e^gamma.
      f32x4 qs[4] = {};
      const char VFA_LDS* qr = sq + c16 * S::QSTR + 8 * g;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8 bh = *(const bf16x8 VFA_LDS*)(sbuf + (2 * ks) * 64 * 16);
        const bf16x8 bl = *(const bf16x8 VFA_LDS*)(sbuf + (2 * ks + 1) * 64 * 16);
        bf16x8 aq[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) aq[mt] = lds_perm16(qr + 16 * mt * S::QSTR + 64 * ks);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) qs[mt] = mfma16(aq[mt], bh, qs[mt]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) qs[mt] = mfma16(aq[mt], bl, qs[mt]);
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const f32x4 e1 = *(const f32x4*)&se1[16 * mt + 4 * g];
#pragma unroll
        for (int z = 0; z < 4; ++z) qs[mt][z] *= e1[z];
      }
      // The next chunk's Q, M and factors go in flight only now: right after
      // barrier A the address unit is left to the chain waves' loads, which
      // the chain waits behind.
      if (c0 + kC < len) load_out(c0 + kC);
      // M operands into registers now: the staging after barrier B overwrites M.
      bf16x8 mh[4][2], ml[4][2];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const char VFA_LDS* mr = smm + (16 * mt + c16) * S::TSTR + 8 * g;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          mh[mt][kk] = lds_perm16(mr + 64 * kk);
          ml[mt][kk] = lds_perm16(mr + 2 * kC + 64 * kk);
        }
      }

      __syncthreads();                  // B: U published by the chain wave

      // O = scale (e^gamma Q S + M U), rows below n stored (without a per-row
      // test on full chunks, so the stores do not split the code into blocks).
      bf16x8 uh[2], ul[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        uh[kk] = *(const bf16x8 VFA_LDS*)(ubuf + (2 * kk) * 64 * 16);
        ul[kk] = *(const bf16x8 VFA_LDS*)(ubuf + (2 * kk + 1) * 64 * 16);
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) qs[mt] = mfma16(mh[mt][kk], uh[kk], qs[mt]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) qs[mt] = mfma16(mh[mt][kk], ul[kk], qs[mt]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) qs[mt] = mfma16(ml[mt][kk], uh[kk], qs[mt]);
      }
      bf16* orow = out + ((size_t)(t0 + 4 * g) * hv + h) * DV + col;   // row 4 g of the chunk
      const size_t ostride = (size_t)hv * DV;                           // elements per token
      if (n == kC) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) orow[(16 * mt + r) * ostride] = (bf16)(scale * qs[mt][r]);
      } else {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (16 * mt + 4 * g + r < n) orow[(16 * mt + r) * ostride] = (bf16)(scale * qs[mt][r]);
      }
      // Stage the next chunk's Q, M and factors: every read of them for this
      // chunk (the chain's included) happened before barrier B.
      if (c0 + kC < len) store_out();
    }
  }

  if (chain && s_final) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) s_final[sbase + (size_t)(16 * dt + 4 * g + r) * DV] = st[dt][r];
  }
}

template <int DK, int DV>
int launch_t(const GatedDeltaArgs& a, int n_chunks, bf16* wt, bf16* wm, float* we, int32_t* order) {
  const long long prep = (long long)a.batch * a.hv * n_chunks;
  const long long main_blocks = (long long)a.batch * a.hv * (DV / kGroupCols);
  if (prep > 0x7fffffffLL || main_blocks > 0x7fffffffLL) return -1;
  hipStream_t s = (hipStream_t)a.stream;
  hipLaunchKernelGGL((gdn_prep_kernel<DK>), dim3((unsigned)prep), dim3(64), 0, s, (const bf16*)a.q,
                     (const bf16*)a.k, a.g, a.beta, a.cu, a.batch, a.hqk, a.hv, n_chunks, wt, wm, we, order);
  if (hipGetLastError() != hipSuccess) return -1;
  hipLaunchKernelGGL((gdn_chunk_kernel<DK, DV>), dim3((unsigned)main_blocks), dim3(kChunkWaves * 64), 0, s,
                     (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, a.beta, a.cu, a.hqk, a.hv, a.scale,
                     a.s_init, (bf16*)a.out, a.s_final, (const bf16*)wt, (const bf16*)wm, (const float*)we,
                     (const int32_t*)order);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

// Up to this many sequences are ranked by length for the chunk kernel; larger
// batches keep their own order. The ranking costs O(batch) per sequence.
constexpr int kOrderMax = kGdnOrderMax;
static_assert(sizeof(bf16) == 2, "the workspace size in launch.h counts bf16 as 2 bytes");

int launch_gated_delta_chunked(const GatedDeltaArgs& a, int max_seqlen, void* workspace) {
  if (a.batch <= 0 || max_seqlen <= 0 || a.tokens <= 0) return 0;
  const int n_chunks = (max_seqlen + kC - 1) / kC;
  char* ws = (char*)workspace;
  const size_t rows = (size_t)a.tokens * a.hv * 2 * kC;
  bf16* wt = (bf16*)ws;
  bf16* wm = wt + rows;
  float* we = (float*)(wm + rows);
  int32_t* order = a.batch <= kOrderMax ? (int32_t*)(we + 2 * (size_t)a.tokens * a.hv) : nullptr;
  if (a.dk == 128)
    return a.dv == 128 ? launch_t<128, 128>(a, n_chunks, wt, wm, we, order)
                       : launch_t<128, 64>(a, n_chunks, wt, wm, we, order);
  return a.dv == 128 ? launch_t<64, 128>(a, n_chunks, wt, wm, we, order)
                     : launch_t<64, 64>(a, n_chunks, wt, wm, we, order);
}

}  // namespace vfa
