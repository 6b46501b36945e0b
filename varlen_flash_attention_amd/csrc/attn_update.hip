// AttentionUpdate merge and last-token gather kernels.
//
// attn_update ("attention_update operator optimisation practice", operator
// function description): partial results (O_i, lse_i) of sp key chunks are
// merged per row r as
//   lse_m = max_i lse_i + ln sum_i exp(lse_i - max_i lse_i),
//   out[r] = sum_i O_i[r] * exp(lse_i - lse_m).
// Inputs are whole tensors lse [sp, bsh] and go [sp, bsh, hd] (the page's
// plain-tensor form: chunk i of row r sits at i * bsh + r). The kernel is
// bound by HBM bandwidth: each row is owned by hd / VEC lanes that each issue
// all sp 16-byte loads of their slice up front (coalesced across the row), the
// weights come from the row's sp lse values, and the row is written once.
//
// Last-token gather ("From GPU to NPU: Qwen3-Embedding on Ascend", core
// optimisation 1, embed()): out[b] = x[cu_seqlens[b + 1] - 1].
#include "common.h"
#include "launch.h"

namespace vfa {
namespace {

template <typename T>
struct Vec16;
template <>
struct Vec16<float> { typedef f32x4 type; static constexpr int N = 4; };
template <>
struct Vec16<bf16> { typedef bf16x8 type; static constexpr int N = 8; };

// SPMAX: compile-time bound on sp (partials held in registers); sp <= SPMAX.
// The TPR lanes of a row read its sp lse values with one load each (lane t
// takes chunk t, t + TPR, ...) and exchange them with lane shuffles, so the
// load instructions per row are the sp data loads plus one or two. Partials
// are read and the merged row written with streaming (non-temporal) accesses:
// neither is touched again by this kernel. NR rows per thread (all their loads
// in flight together): 2 for large merges, measured 4% faster cold at 608 MB
// on MI355X; 1 when there are few rows, so that more workgroups share them.
template <typename T, int HD, int SPMAX, int NR>
__global__ __launch_bounds__(256) void attn_update_kernel(const float* __restrict__ lse,
                                                          const T* __restrict__ go, int sp, long long bsh,
                                                          T* __restrict__ out, float* __restrict__ lse_out,
                                                          int write_lse) {
  typedef typename Vec16<T>::type VT;
  constexpr int VEC = Vec16<T>::N;
  constexpr int TPR = HD / VEC;     // lanes per row
  constexpr int RPB = 256 / TPR;    // rows per block per pass
  constexpr int NL = (SPMAX + TPR - 1) / TPR;
  static_assert(64 % TPR == 0, "a row's lanes must sit in one wavefront");
  const int t = threadIdx.x % TPR;
  const int c = t * VEC;
  const int row_lane0 = (threadIdx.x & 63) - t;   // first lane of this row within the wave
  {
    const long long grp = blockIdx.x;
    long long row[NR], rr[NR];
    VT x[NR][SPMAX];
    float lv[NR][NL];
#pragma unroll
    for (int qq = 0; qq < NR; ++qq) {
      row[qq] = (grp * NR + qq) * RPB + threadIdx.x / TPR;
      rr[qq] = row[qq] < bsh ? row[qq] : bsh - 1;   // rows past the end load a valid row and store nothing
#pragma unroll
      for (int i = 0; i < SPMAX; ++i)
        if (i < sp) x[qq][i] = __builtin_nontemporal_load((const VT*)(go + ((long long)i * bsh + rr[qq]) * HD + c));
#pragma unroll
      for (int u = 0; u < NL; ++u) {
        const int i = u * TPR + t;
        lv[qq][u] = i < sp ? lse[(long long)i * bsh + rr[qq]] : neg_inf();
      }
    }
#pragma unroll
    for (int qq = 0; qq < NR; ++qq) {
      float l[SPMAX];
#pragma unroll
      for (int i = 0; i < SPMAX; ++i) l[i] = __shfl(lv[qq][i / TPR], row_lane0 + i % TPR, 64);
      float w[SPMAX];
      const float lse_m = merge_weights<SPMAX>(l, sp, w);
      float acc[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
#pragma unroll
      for (int i = 0; i < SPMAX; ++i)
        if (i < sp)
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[e] += w[i] * to_f32(x[qq][i][e]);
      if (row[qq] < bsh) {
        VT r;
#pragma unroll
        for (int e = 0; e < VEC; ++e) r[e] = from_f32<T>(acc[e]);
        __builtin_nontemporal_store(r, (VT*)(out + row[qq] * HD + c));
        if (write_lse && t == 0) lse_out[row[qq]] = lse_m;
      }
    }
  }
}

// sp above the register bound: two passes over lse, then a streaming
// accumulation over the chunks (same arithmetic, loads not all in flight).
template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_update_long_kernel(const float* __restrict__ lse,
                                                               const T* __restrict__ go, int sp,
                                                               long long bsh, T* __restrict__ out,
                                                               float* __restrict__ lse_out, int write_lse) {
  typedef typename Vec16<T>::type VT;
  constexpr int VEC = Vec16<T>::N;
  constexpr int TPR = HD / VEC;
  constexpr int RPB = 256 / TPR;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  if (row >= bsh) return;
  const int c = (threadIdx.x % TPR) * VEC;
  const MergeStats st = merge_stats(lse + row, bsh, sp);
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
  for (int i = 0; i < sp; ++i) {
    const float w = merge_weight(lse[(long long)i * bsh + row], st);
    const VT x = *(const VT*)(go + ((long long)i * bsh + row) * HD + c);
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] += w * to_f32(x[e]);
  }
  VT r;
#pragma unroll
  for (int e = 0; e < VEC; ++e) r[e] = from_f32<T>(acc[e]);
  *(VT*)(out + row * HD + c) = r;
  if (write_lse && c == 0) lse_out[row] = st.lse_m;
}

template <typename T, int HD>
int launch_update_t(const float* lse, const void* go, int sp, long long bsh, void* out, float* lse_out,
                    int write_lse, hipStream_t stream) {
  constexpr int TPR = HD / Vec16<T>::N;
  constexpr int RPB = 256 / TPR;
  const long long blocks = (bsh + RPB - 1) / RPB;
  if (blocks > 0x7fffffffLL) return -1;
  const bool two = blocks >= 4096;                   // two rows per thread for large merges
  const dim3 grid((unsigned)blocks), block(256), grid2((unsigned)((bsh + 2 * RPB - 1) / (2 * RPB)));
  const T* g = (const T*)go;
  T* o = (T*)out;
#define VFA_UPD(N)                                                                                            \
  do {                                                                                                        \
    if (two)                                                                                                  \
      hipLaunchKernelGGL((attn_update_kernel<T, HD, N, 2>), grid2, block, 0, stream, lse, g, sp, bsh, o,      \
                         lse_out, write_lse);                                                                 \
    else                                                                                                      \
      hipLaunchKernelGGL((attn_update_kernel<T, HD, N, 1>), grid, block, 0, stream, lse, g, sp, bsh, o,       \
                         lse_out, write_lse);                                                                 \
  } while (0)
  if (sp <= 1) VFA_UPD(1);
  else if (sp <= 2) VFA_UPD(2);
  else if (sp <= 4) VFA_UPD(4);
  else if (sp <= 8) VFA_UPD(8);
  else if (sp <= 16) VFA_UPD(16);
  else hipLaunchKernelGGL((attn_update_long_kernel<T, HD>), grid, block, 0, stream, lse, g, sp, bsh, o, lse_out,
                          write_lse);
#undef VFA_UPD
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// One workgroup per sequence; 16-byte copies when the row allows, else element copies.
template <typename E>
__global__ __launch_bounds__(256) void gather_kernel(const E* __restrict__ x, const int32_t* __restrict__ cu,
                                                     long long row_units, E* __restrict__ out) {
  const int b = blockIdx.x;
  const int lo = cu[b], hi = cu[b + 1];
  E* dst = out + (long long)b * row_units;
  if (hi <= lo) {
    for (long long e = threadIdx.x; e < row_units; e += blockDim.x) dst[e] = E{};
    return;
  }
  const E* src = x + (long long)(hi - 1) * row_units;
  for (long long e = threadIdx.x; e < row_units; e += blockDim.x) dst[e] = src[e];
}

}  // namespace

int launch_attn_update(const float* lse, const void* go, int go_dtype, int sp, int64_t bsh, int hd,
                       int update_type, void* out, float* lse_out, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const int wl = update_type == 1;
  if (go_dtype == 0)
    return hd == 128 ? launch_update_t<float, 128>(lse, go, sp, bsh, out, lse_out, wl, s)
                     : launch_update_t<float, 64>(lse, go, sp, bsh, out, lse_out, wl, s);
  return hd == 128 ? launch_update_t<bf16, 128>(lse, go, sp, bsh, out, lse_out, wl, s)
                   : launch_update_t<bf16, 64>(lse, go, sp, bsh, out, lse_out, wl, s);
}

int launch_last_token_gather(const void* x, int esize, const int32_t* cu, int batch, int64_t row_elems,
                             void* out, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const long long bytes = row_elems * esize;
  const bool wide = bytes % 16 == 0 && ((uintptr_t)x % 16 == 0) && ((uintptr_t)out % 16 == 0);
  if (wide)
    hipLaunchKernelGGL((gather_kernel<u32x4>), dim3(batch), dim3(256), 0, s, (const u32x4*)x, cu, bytes / 16,
                       (u32x4*)out);
  else if (esize == 4)
    hipLaunchKernelGGL((gather_kernel<uint32_t>), dim3(batch), dim3(256), 0, s, (const uint32_t*)x, cu,
                       (long long)row_elems, (uint32_t*)out);
  else
    hipLaunchKernelGGL((gather_kernel<uint16_t>), dim3(batch), dim3(256), 0, s, (const uint16_t*)x, cu,
                       (long long)row_elems, (uint16_t*)out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace vfa
