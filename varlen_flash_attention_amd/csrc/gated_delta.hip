// Varlen gated delta rule forward (linear attention), bf16 q/k/v, fp32 state.
//
// The linear-attention layers of the hybrid model on "Twinkle NPU kernels"
// (Qwen3.5 flash linear attention section) call chunk_gated_delta_rule over
// packed sequences delimited by cu_seqlens. Per sequence and value head h a
// state S [Dk, Dv] (zero or a given initial state) advances token by token:
//   S <- exp(g_t) S ;  u = beta_t (v_t - S^T k_t) ;  S <- S + k_t u^T ;
//   o_t = scale * S^T q_t
// with query / key head h / (Hv / Hqk). States never cross sequences.
//
// This kernel runs the recurrence itself in fp32, token by token; it serves
// calls whose sequences are at most 16 tokens long (decode steps, speculative
// tokens), where it needs no workspace and one launch. Longer sequences take
// the chunked form (gated_delta_chunk.hip). The tokens of a sequence are
// sequential, so the parallelism is across (sequence, head, state column). A
// column j of S belongs to 8 consecutive lanes, each holding Dk / 8 of its
// rows in registers, so a token's dependency chain (S^T k, then the write) is
// Dk / 8 deep per lane; the two dot products per token (S^T k and S^T q)
// finish with three DPP exchanges inside the 8 lanes. A workgroup takes 32
// columns of one (sequence, value head); q, k (converted to fp32), v, g and
// beta of kTC tokens at a time are staged in LDS and read back as broadcasts.
#include "common.h"
#include "launch.h"

namespace vfa {
namespace {

constexpr int kThreads = 256;
constexpr int kLanesPerCol = 8;         // lanes sharing one state column
constexpr int kColsPerBlock = kThreads / kLanesPerCol;   // 32 state columns per workgroup
constexpr int kTC = 16;                 // tokens staged per pass (the calls this kernel serves fit one)

// Sum over 8 consecutive lanes with DPP: within each quad (lane ^ 1, then
// lane ^ 2), then across the two quads of the 8 (row_half_mirror pairs lane i
// with lane 7 - i). VALU operations, so the per-token dependency chain does not
// wait on an LDS round trip.
__device__ __forceinline__ float lane8_sum(float x) {
  constexpr int kXor1 = 1 | (0 << 2) | (3 << 4) | (2 << 6);   // quad_perm [1, 0, 3, 2]
  constexpr int kXor2 = 2 | (3 << 2) | (0 << 4) | (1 << 6);   // quad_perm [2, 3, 0, 1]
  constexpr int kHalfMirror = 0x141;                          // row_half_mirror
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kXor1, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kXor2, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kHalfMirror, 0xf, 0xf, false));
  return x;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

template <int DK>
__global__ __launch_bounds__(kThreads) void gated_delta_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const int32_t* __restrict__ cu, int hqk, int hv,
    int dv, float scale, const float* __restrict__ s_init, bf16* __restrict__ out, float* __restrict__ s_final) {
  constexpr int RP = DK / kLanesPerCol;  // state rows per lane
  constexpr int KSTR = DK + 4;           // fp32 words per staged q / k row
  // Staged k rows then q rows, one array so that the state slice fits it too.
  __shared__ __attribute__((aligned(16))) float skq[2][kTC][KSTR];
  float (*sk)[KSTR] = skq[0];
  float (*sq)[KSTR] = skq[1];
  __shared__ float sv[kTC][kColsPerBlock];
  __shared__ float sg[kTC], sb[kTC];

  const int ncb = dv / kColsPerBlock;
  const int cb = blockIdx.x % ncb;
  const int h = (blockIdx.x / ncb) % hv;
  const int b = blockIdx.x / (ncb * hv);
  const int hk = h / (hv / hqk);
  const int t0 = cu[b];
  const int len = cu[b + 1] - t0;

  const int tid = threadIdx.x;
  const int part = tid % kLanesPerCol;   // which eighth of the column's rows
  const int col = tid / kLanesPerCol;    // 0 .. kColsPerBlock - 1
  const int j = cb * kColsPerBlock + col;
  const int r0 = part * RP;

  // The state moves between HBM and registers through LDS (the q / k staging
  // array, free before and after the token loop): in memory, each of the
  // slice's DK rows holds this workgroup's 32 columns contiguously (128 B),
  // moved as 16-byte pieces; a lane's registers hold one column. A decode
  // step is almost only this traffic (non-temporal accesses measured 15%
  // slower here). Row stride 33 floats: the lanes of a
  // wave then read 32 or 64 distinct banks.
  float st[RP];
  float* ss = &skq[0][0][0];
  constexpr int SSTR = kColsPerBlock + 1;
  static_assert(DK * SSTR <= 2 * kTC * KSTR, "state slice must fit the staging array");
  const size_t sslice = (((size_t)b * hv + h) * DK) * dv + cb * kColsPerBlock;   // state [b][h][i][j]
  if (s_init) {
    for (int e = tid; e < DK * (kColsPerBlock / 4); e += kThreads) {
      const int row = e / (kColsPerBlock / 4), c4 = (e % (kColsPerBlock / 4)) * 4;
      const f32x4 x = *(const f32x4*)(s_init + sslice + (size_t)row * dv + c4);
#pragma unroll
      for (int z = 0; z < 4; ++z) ss[row * SSTR + c4 + z] = x[z];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < RP; ++i) st[i] = ss[(r0 + i) * SSTR + col];
  } else {
#pragma unroll
    for (int i = 0; i < RP; ++i) st[i] = 0.f;
  }

  for (int c0 = 0; c0 < len; c0 += kTC) {
    const int n = min(kTC, len - c0);
    __syncthreads();                     // the previous staging pass is no longer read
    // Stage q and k rows (bf16 -> fp32), this block's v columns, g and beta.
    for (int e = tid; e < kTC * (DK / 2); e += kThreads) {
      const int t = e / (DK / 2), d2 = (e % (DK / 2)) * 2;
      if (t < n) {
        const size_t row = ((size_t)(t0 + c0 + t) * hqk + hk) * DK + d2;
        const uint32_t kk = *(const uint32_t*)(k + row), qq = *(const uint32_t*)(q + row);
        sk[t][d2] = bf16_bits_to_f32(kk & 0xffffu);
        sk[t][d2 + 1] = bf16_bits_to_f32(kk >> 16);
        sq[t][d2] = bf16_bits_to_f32(qq & 0xffffu);
        sq[t][d2 + 1] = bf16_bits_to_f32(qq >> 16);
      }
    }
    for (int e = tid; e < kTC * kColsPerBlock; e += kThreads) {
      const int t = e / kColsPerBlock, cc = e % kColsPerBlock;
      if (t < n) sv[t][cc] = (float)v[((size_t)(t0 + c0 + t) * hv + h) * dv + cb * kColsPerBlock + cc];
    }
    if (tid < kTC && tid < n) {
      sg[tid] = g[(size_t)(t0 + c0 + tid) * hv + h];
      sb[tid] = beta[(size_t)(t0 + c0 + tid) * hv + h];
    }
    __syncthreads();

    for (int t = 0; t < n; ++t) {
      const float a = fast_exp2(sg[t] * kLog2e);                  // gated decay exp(g_t)
      const float* kr = &sk[t][r0];
      float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
#pragma unroll
      for (int i = 0; i < RP; i += 4) {
        const f32x4 kk = *(const f32x4*)(kr + i);
        d0 = __builtin_fmaf(st[i], kk[0], d0);
        d1 = __builtin_fmaf(st[i + 1], kk[1], d1);
        d2 = __builtin_fmaf(st[i + 2], kk[2], d2);
        d3 = __builtin_fmaf(st[i + 3], kk[3], d3);
      }
      const float dot = lane8_sum((d0 + d1) + (d2 + d3));          // (S^T k) before the decay
      const float u = sb[t] * (sv[t][col] - a * dot);
      const float* qr = &sq[t][r0];
      float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
#pragma unroll
      for (int i = 0; i < RP; i += 4) {
        const f32x4 kk = *(const f32x4*)(kr + i);
        const f32x4 qq = *(const f32x4*)(qr + i);
        st[i] = __builtin_fmaf(kk[0], u, a * st[i]);
        st[i + 1] = __builtin_fmaf(kk[1], u, a * st[i + 1]);
        st[i + 2] = __builtin_fmaf(kk[2], u, a * st[i + 2]);
        st[i + 3] = __builtin_fmaf(kk[3], u, a * st[i + 3]);
        o0 = __builtin_fmaf(st[i], qq[0], o0);
        o1 = __builtin_fmaf(st[i + 1], qq[1], o1);
        o2 = __builtin_fmaf(st[i + 2], qq[2], o2);
        o3 = __builtin_fmaf(st[i + 3], qq[3], o3);
      }
      const float o = lane8_sum((o0 + o1) + (o2 + o3));
      if (part == 0) out[((size_t)(t0 + c0 + t) * hv + h) * dv + j] = (bf16)(scale * o);
    }
  }
  if (s_final) {
    __syncthreads();                     // the token loop's reads of the staging array are done
#pragma unroll
    for (int i = 0; i < RP; ++i) ss[(r0 + i) * SSTR + col] = st[i];
    __syncthreads();
    for (int e = tid; e < DK * (kColsPerBlock / 4); e += kThreads) {
      const int row = e / (kColsPerBlock / 4), c4 = (e % (kColsPerBlock / 4)) * 4;
      f32x4 x;
#pragma unroll
      for (int z = 0; z < 4; ++z) x[z] = ss[row * SSTR + c4 + z];
      *(f32x4*)(s_final + sslice + (size_t)row * dv + c4) = x;
    }
  }
}

template <int DK>
int launch_t(const GatedDeltaArgs& a) {
  const long long blocks = (long long)a.batch * a.hv * (a.dv / kColsPerBlock);
  if (blocks <= 0) return 0;
  if (blocks > 0x7fffffffLL) return -1;
  hipLaunchKernelGGL((gated_delta_kernel<DK>), dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)a.stream,
                     (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, a.g, a.beta, a.cu, a.hqk, a.hv, a.dv,
                     a.scale, a.s_init, (bf16*)a.out, a.s_final);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_gated_delta(const GatedDeltaArgs& a) {
  return a.dk == 128 ? launch_t<128>(a) : launch_t<64>(a);
}

}  // namespace vfa
