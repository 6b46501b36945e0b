// Split-KV varlen attention for few queries against long key sets (decode), bf16 in.
//
// Same result as the prefill kernel (softmax(scale q K^T) V and the natural
// log-sum-exp per query row, TND layout, cu_seqlens, GQA head h -> h / G,
// bottom-right causal mask), for the shape where one fused attention op
// serves incremental decoding ("Qwen3-MoE low-latency inference on Atlas A3",
// flash attention fused operator section).
//
// Decode reads every K/V byte once and does little arithmetic per byte, so it
// is bound by HBM bandwidth. Sequence lengths vary widely, so each
// (sequence, kv head) is cut into fixed-size key chunks ("splits") and the
// splits become independent workgroups. Each split produces a partial
// (O_s, lse_s) in the workspace; a combine kernel then merges the splits with
// the AttentionUpdate rule ("attention_update operator optimisation
// practice", operator function description) using the same device helpers as
// the attn_update entry point.
//
// Inside a workgroup (4 waves) every wave owns a strided subset of 32-key
// steps of the split and keeps its own online-softmax state; the four states
// are merged through LDS at the end. The G query heads of the kv head (times
// up to 16 / G query tokens) fill the 16 columns of v_mfma_f32_16x16x32_bf16:
//   S^T = K Q^T   : A = K rows loaded straight from global memory (16 B per
//                   lane), B = Q^T in registers.
//   O^T += V^T P^T: V rows go through a wave-private LDS buffer so that
//                   ds_read_b64_tr_b16 can deliver V^T; B = P^T from registers.
#include "common.h"
#include "launch.h"

namespace vfa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kCols = 16;      // query columns (heads x tokens) per workgroup
constexpr int kStep = 32;      // keys per wave step

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

// Grid: n_splits * batch * hkv workgroups. Partials go to
// ws_o[split][row][D] and ws_lse[split][row], row = token * hq + head.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void attn_decode_split_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int batch, int hq, int hkv,
    int grp, int chunk, int n_splits, long long rows_total, float scale, float scale_log2,
    float* __restrict__ ws_o, float* __restrict__ ws_lse) {
  using S = DSmem<D>;
  __shared__ __attribute__((aligned(16))) char smem[S::TOTAL];
  char VFA_LDS* lds = (char VFA_LDS*)smem;

  // Longest splits first: split index descends with the block id.
  const int per_s = batch * hkv;
  const int split = n_splits - 1 - (int)(blockIdx.x / per_s);
  const int bg = blockIdx.x % per_s;
  const int b = bg / hkv;
  const int g = bg % hkv;

  const int q0 = cu_q[b];
  const int lq = cu_q[b + 1] - q0;
  const int k0 = cu_k[b];
  const int lk = cu_k[b + 1] - k0;
  const int key_lo = split * chunk;
  if (lq <= 0 || key_lo >= lk) return;     // this split holds no key of the sequence
  const int key_hi = min(lk, key_lo + chunk);
  const int diag = lk - lq;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int c16 = lane & 15;
  const int grp4 = lane >> 4;

  // Column -> (token, head): tokens outer, the G heads of this kv head inner.
  const int tpc = kCols / grp;                 // tokens per workgroup (>= 1)
  const bool colvalid = c16 < tpc * grp;
  const int tq = colvalid ? c16 / grp : 0;
  const int head = g * grp + (colvalid ? c16 % grp : 0);
  const bool qvalid = colvalid && tq < lq;

  // Q^T (B operand): column c16, k-slot grp4*8 + e <-> d = ks*32 + grp4*8 + e.
  bf16x8 qreg[D / 32];
  {
    const bf16* qrow = q + ((size_t)(q0 + (qvalid ? tq : 0)) * hq + head) * D + grp4 * 8;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      bf16x8 t = *(const bf16x8*)(qrow + ks * 32);
      if (!qvalid) t = bf16x8{};
      qreg[ks] = t;
    }
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
  const bf16* kg = k + ((size_t)k0 * hkv + g) * D;
  const bf16* vg = v + ((size_t)k0 * hkv + g) * D;
  const size_t kv_stride = (size_t)hkv * D;
  // K and V rows are loaded whole (each instruction covers 64 / (D/8) rows of
  // contiguous bytes) and parked in the wave's LDS buffers.
  auto gload = [&](KRegs& kr, VRegs& vr, int st) {
    const int base = key_lo + st * kStep;
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
    m_lse[wave * kCols + c16] = l_tot > 0.f ? m_run * scale + fast_log2(l_tot) * kLn2 : neg_inf();
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) m_o[(wave * kCols + c16) * D + db * 16 + grp4 * 4 + r] = acc[db][r] * inv;
  __syncthreads();

  // 256 threads = 16 columns x 16 threads; each thread merges D/16 values of one column.
  const int mc = tid >> 4;
  const int md = (tid & 15) * (D / 16);
  const bool mvalid = mc < tpc * grp && (mc / grp) < lq;
  if (!mvalid) return;
  float lw[kWaves], w[kWaves];
#pragma unroll
  for (int i = 0; i < kWaves; ++i) lw[i] = m_lse[i * kCols + mc];
  const float lse_m = merge_weights<kWaves>(lw, kWaves, w);
  const long long row = (long long)(q0 + mc / grp) * hq + g * grp + (mc % grp);
  float* dst = ws_o + ((long long)split * rows_total + row) * D + md;
#pragma unroll
  for (int x = 0; x < D / 16; x += 4) {
    f32x4 o = f32x4{};
#pragma unroll
    for (int i = 0; i < kWaves; ++i)
#pragma unroll
      for (int y = 0; y < 4; ++y) o[y] += w[i] * m_o[(i * kCols + mc) * D + md + x + y];
    *(f32x4*)(dst + x) = o;
  }
  if ((tid & 15) == 0) ws_lse[(long long)split * rows_total + row] = lse_m;
}

// Merge the splits of every row with the AttentionUpdate rule. Grid: (row
// chunk, sequence); one row per TPR lanes with 16-byte loads. NS is a
// compile-time bound on the split count so that every lse and partial load of
// a row is issued before the first one is consumed (NS = 0: streaming loop
// for very long key sets).
template <int D, int NS, typename OutT>
__global__ __launch_bounds__(256) void attn_decode_combine_kernel(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int hq, int chunk, int n_splits,
    long long rows_total, const float* __restrict__ ws_o, const float* __restrict__ ws_lse,
    OutT* __restrict__ out, float* __restrict__ lse) {
  constexpr int TPR = D / 4;
  constexpr int RPB = 256 / TPR;
  const int b = blockIdx.y;
  const int q0 = cu_q[b];
  const int rows_b = (cu_q[b + 1] - q0) * hq;
  const int r_in = blockIdx.x * RPB + threadIdx.x / TPR;
  if (r_in >= rows_b) return;
  const long long row = (long long)q0 * hq + r_in;
  const int c4 = (threadIdx.x % TPR) * 4;
  const int lk = cu_k[b + 1] - cu_k[b];
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

template <int D, typename OutT>
void launch_combine(const AttnArgs& a, const DecodePlan& p, long long rows, const float* ws_o,
                    const float* ws_lse) {
  constexpr int RPB = 256 / (D / 4);
  const long long max_rows = (long long)a.max_seqlen_q * a.hq;
  const dim3 grid((unsigned)((max_rows + RPB - 1) / RPB), (unsigned)a.batch);
  hipStream_t st = (hipStream_t)a.stream;
#define VFA_COMBINE(NS)                                                                                    \
  hipLaunchKernelGGL((attn_decode_combine_kernel<D, NS, OutT>), grid, dim3(256), 0, st, a.cu_q, a.cu_k, a.hq, \
                     p.chunk, p.n_splits, rows, ws_o, ws_lse, (OutT*)a.out, a.lse)
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
  hipLaunchKernelGGL((attn_decode_split_kernel<D, CAUSAL>), dim3((unsigned)blocks), dim3(kThreads), 0,
                     (hipStream_t)a.stream, (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, a.cu_q,
                     a.cu_k, a.batch, a.hq, a.hkv, a.grp, p.chunk, p.n_splits, rows, a.scale,
                     a.scale * kLog2e, ws_o, ws_lse);
  if (hipGetLastError() != hipSuccess) return -1;
  launch_combine<D, OutT>(a, p, rows, ws_o, ws_lse);
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

}  // namespace vfa
