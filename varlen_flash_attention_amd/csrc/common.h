// Device-side building blocks shared by the libvfa kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vfa {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

#define VFA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 2^x by the hardware instruction (v_exp_f32). -inf -> 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) by the hardware instruction (v_log_f32), x > 0.
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// Value exchange with the lane `mask` away (XOR) inside the wave, via ds_bpermute.
__device__ __forceinline__ float xor_shuffle(float v, int mask) {
  int lane = __lane_id();
  int src = (lane ^ mask) << 2;
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(v)));
}

__device__ __forceinline__ float bf16_to_f32(bf16 x) { return (float)x; }

// Round-to-nearest-even fp32 -> bf16 (the hardware conversion on gfx950).
__device__ __forceinline__ bf16x2 f32x2_to_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_convertvector(v, bf16x2);
}

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

template <typename T>
__device__ __forceinline__ float to_f32(T x) { return (float)x; }

// Causal diagonal of sequence b: query i sees key j iff j <= i + diag. The
// caller's offset (the position of the sequence's first query minus that of
// its first key), or Lk - Lq when there is none (bottom-right alignment), is
// clamped to [-lq, lk]: that keeps every visible set (no offset can show more
// than all keys or hide more than every row) and keeps i + diag from
// overflowing.
__device__ __forceinline__ int causal_diag(const int32_t* off, int b, int lq, int lk) {
  const int d = off ? off[b] : lk - lq;
  return d < -lq ? -lq : (d > lk ? lk : d);
}

// ---------------------------------------------------------------------------
// AttentionUpdate merge statistics for one row over n partials ("attention_update
// operator optimisation practice", operator function description):
//   lse_max = max_i lse_i ; lse_m = lse_max + ln sum_i exp(lse_i - lse_max)
//   weight_i = exp(lse_i - lse_m) = exp(lse_i - lse_max) / sum
// Partials with lse_i = -inf get weight 0; if all are -inf, lse_m = -inf and
// every weight is 0. Base 2 inside: exp(x) = 2^(x * log2 e).
struct MergeStats {
  float mx;       // lse_max (or 0 when every partial is -inf)
  float inv_sum;  // 1 / sum_i exp(lse_i - lse_max) (0 when every partial is -inf)
  float lse_m;    // merged log-sum-exp
};

__device__ __forceinline__ MergeStats merge_stats(const float* lse, long long stride, int n) {
  float mx = neg_inf();
  for (int i = 0; i < n; ++i) mx = fmaxf(mx, lse[i * stride]);
  if (mx == neg_inf()) return MergeStats{0.f, 0.f, neg_inf()};
  float sum = 0.f;
  for (int i = 0; i < n; ++i) sum += fast_exp2((lse[i * stride] - mx) * kLog2e);
  return MergeStats{mx, 1.f / sum, mx + fast_log2(sum) * kLn2};
}

__device__ __forceinline__ float merge_weight(float lse_i, const MergeStats& st) {
  // -inf partials: exp2(-inf) = 0. All--inf rows: inv_sum = 0.
  return fast_exp2((lse_i - st.mx) * kLog2e) * st.inv_sum;
}

// ---------------------------------------------------------------------------
// The same merge for a compile-time bound N of partials held in registers:
// `lse` holds n <= N values; weights exp(lse_i - lse_m) are written to `w`
// and lse_m is returned.
template <int N>
__device__ __forceinline__ float merge_weights(const float (&lse)[N], int n, float (&w)[N]) {
  float mx = neg_inf();
#pragma unroll
  for (int i = 0; i < N; ++i)
    if (i < n) mx = fmaxf(mx, lse[i]);
  if (mx == neg_inf()) {
#pragma unroll
    for (int i = 0; i < N; ++i) w[i] = 0.f;
    return neg_inf();
  }
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    w[i] = (i < n) ? fast_exp2((lse[i] - mx) * kLog2e) : 0.f;
    sum += w[i];
  }
  float inv = 1.f / sum;
#pragma unroll
  for (int i = 0; i < N; ++i) w[i] *= inv;
  return mx + fast_log2(sum) * kLn2;
}

}  // namespace vfa
