// The attention prologue on TND tensors: per-head RMSNorm of q and k, then the
// rotary embedding, written back in the [T, heads, head_dim] layout the
// attention kernels read ("From GPU to NPU: Qwen3-Embedding on Ascend", 2.2:
// variance as the fp32 mean of squares, x * rsqrt(variance + eps), then the
// weight; 2.3: q_norm / k_norm per head over head_dim; 2.4: npu_rotary_mul
// with one (cos, sin) row per token for every head, taken in its rotate-half
// form out = y * cos + rotate_half(y) * sin).
//
// Everything is computed in fp32 and rounded to bf16 once. The op is bound by
// HBM bandwidth: each (token, head) row is read once and written once, and the
// cos / sin rows and weights are shared by all heads of a token: a group of
// D / 8 consecutive lanes (16 bytes of a row each) takes a chunk of a token's
// heads. The sum of squares is reduced across the group with lane
// shuffles, and the rotate-half partner of a lane's 8 values sits in the lane
// D / 16 away, so the raw 16 bytes are exchanged in registers. Each row is read
// by its group before the group writes it, and no group touches another
// group's rows, so the output may alias the input.
#include "common.h"
#include "launch.h"

namespace vfa {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t lane_swap(uint32_t v, int mask) {
  const int src = (__lane_id() ^ mask) << 2;
  return (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)v);
}

__device__ __forceinline__ void unpack8(const u32x4& r, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(r[i] << 16);
    x[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
  }
}

// The rotated, normalised 8 values of one row held by this lane.
template <int D>
__device__ __forceinline__ u32x4 norm_rope_row(const u32x4& raw, float eps, const float (&w)[8], const float (&wp)[8],
                                              const float (&c)[8], const float (&s)[8], float sign) {
  constexpr int LPR = D / 8;
  u32x4 praw;
#pragma unroll
  for (int i = 0; i < 4; ++i) praw[i] = lane_swap(raw[i], LPR / 2);
  float x[8], xp[8];
  unpack8(raw, x);
  unpack8(praw, xp);
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(x[e], x[e], ss);
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) ss += xor_shuffle(ss, m);
  const float inv = 1.f / sqrtf(ss * (1.f / D) + eps);
  u32x4 packed;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float o[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = 2 * i + j;
      const float y = x[e] * inv * w[e];
      const float yp = xp[e] * inv * wp[e];
      o[j] = __builtin_fmaf(y, c[e], sign * yp * s[e]);
    }
    packed[i] = __builtin_bit_cast(uint32_t, f32x2_to_bf16x2(o[0], o[1]));
  }
  return packed;
}

// Grid: one group of D / 8 lanes per (token, chunk of kU heads), q chunks
// first: short work items keep the last round of workgroups small. Each lane
// loads the token's cos / sin values and the chunk's weights, then all kU
// rows of the chunk before computing the first. q and k are read and written
// once: streaming (non-temporal) accesses.
constexpr int kU = 8;   // heads per chunk

template <int D>
__global__ __launch_bounds__(kThreads) void qk_norm_rope_kernel(
    const bf16* q_in, const bf16* k_in, const bf16* __restrict__ wq, const bf16* __restrict__ wk,
    const float* __restrict__ cos_t, const float* __restrict__ sin_t, long long items, int hq, int hkv, float eps,
    bf16* q_out, bf16* k_out) {
  constexpr int LPR = D / 8;               // lanes per row
  constexpr int IPB = kThreads / LPR;      // (token, chunk) items per workgroup
  const int li = threadIdx.x % LPR;
  const long long item = (long long)blockIdx.x * IPB + threadIdx.x / LPR;
  if (item >= items) return;               // an item's lanes leave together; shuffles stay inside them
  const int cq = (hq + kU - 1) / kU, ck = (hkv + kU - 1) / kU;
  const long long t = item / (cq + ck);
  const int chunk = (int)(item - t * (cq + ck));
  const bool is_q = chunk < cq;
  const int nh = is_q ? hq : hkv;
  const int h0 = (is_q ? chunk : chunk - cq) * kU;
  const int d0 = li * 8;
  const int dp = d0 ^ (D / 2);             // the rotate-half partner's first element
  const float sign = d0 < D / 2 ? -1.f : 1.f;   // rotate_half: first half takes -partner

  const size_t base = ((size_t)t * nh + h0) * D + d0;
  const bf16* src = (is_q ? q_in : k_in) + base;
  u32x4 raw[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u)
    raw[u] = __builtin_nontemporal_load((const u32x4*)(src + (size_t)min(u, nh - 1 - h0) * D));

  float c[8], s[8];
  {
    const float* crow = cos_t + t * D + d0;
    const float* srow = sin_t + t * D + d0;
    const f32x4 c0 = *(const f32x4*)crow, c1 = *(const f32x4*)(crow + 4);
    const f32x4 s0 = *(const f32x4*)srow, s1 = *(const f32x4*)(srow + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { c[e] = c0[e]; c[e + 4] = c1[e]; s[e] = s0[e]; s[e + 4] = s1[e]; }
  }
  const bf16* w = is_q ? wq : wk;
  float wo[8], wp[8];
  unpack8(*(const u32x4*)(w + d0), wo);
  unpack8(*(const u32x4*)(w + dp), wp);

  bf16* dst = (is_q ? q_out : k_out) + base;
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    if (h0 + u >= nh) break;
    __builtin_nontemporal_store(norm_rope_row<D>(raw[u], eps, wo, wp, c, s, sign), (u32x4*)(dst + (size_t)u * D));
  }
}

template <int D>
int launch_t(const QkNormRopeArgs& a) {
  constexpr int IPB = kThreads / (D / 8);
  const long long items = (long long)a.tokens * ((a.hq + kU - 1) / kU + (a.hkv + kU - 1) / kU);
  const long long blocks = (items + IPB - 1) / IPB;
  if (blocks > 0x7fffffffLL) return -1;
  hipLaunchKernelGGL((qk_norm_rope_kernel<D>), dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)a.stream,
                     (const bf16*)a.q_in, (const bf16*)a.k_in, (const bf16*)a.q_weight, (const bf16*)a.k_weight,
                     a.cos, a.sin, items, a.hq, a.hkv, a.eps, (bf16*)a.q_out, (bf16*)a.k_out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_qk_norm_rope(const QkNormRopeArgs& a) {
  return a.head_dim == 128 ? launch_t<128>(a) : launch_t<64>(a);
}

}  // namespace vfa
