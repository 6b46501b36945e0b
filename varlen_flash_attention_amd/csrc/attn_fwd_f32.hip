// Varlen attention forward for fp32 inputs and outputs.
//
// Same definition as the bf16 kernels (TND layout with cu_seqlens, GQA head
// h -> kv head h / G, optional bottom-right causal mask, natural-log lse; "From
// GPU to NPU: Qwen3-Embedding on Ascend", core optimisation 1, section 2.1 and
// core optimisation 5), computed entirely in fp32 FMA arithmetic so that the
// result keeps fp32 accuracy. One thread owns one (token, query head) row,
// keeps q and the output accumulator in registers and walks the visible keys
// of its sequence with a running max / running sum (the max only moves up, so
// earlier terms are rescaled when it does). This path serves small fp32
// problems; bf16 is the throughput path.
#include "common.h"
#include "launch.h"

namespace vfa {
namespace {

template <int D>
__global__ __launch_bounds__(64) void attn_fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, const int32_t* __restrict__ coff,
    int batch, int hq, int hkv, int grp, long long rows_total, float scale, int causal, float* __restrict__ out,
    float* __restrict__ lse) {
  const long long row = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= rows_total) return;
  const int tok = (int)(row / hq);
  const int head = (int)(row % hq);
  const int g = head / grp;
  int lo = 0, hi = batch;   // sequence of this token: largest b with cu_q[b] <= tok
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu_q[mid] <= tok) lo = mid; else hi = mid;
  }
  const int i = tok - cu_q[lo];
  const int lq = cu_q[lo + 1] - cu_q[lo];
  const int k0 = cu_k[lo];
  const int lk = cu_k[lo + 1] - k0;
  int n_end = lk;
  if (causal) n_end = max(0, min(lk, i + causal_diag(coff, lo, lq, lk) + 1));

  float qr[D], o[D];
  const float* qp = q + row * D;
#pragma unroll
  for (int d = 0; d < D; ++d) { qr[d] = qp[d]; o[d] = 0.f; }
  float m = neg_inf(), l = 0.f;
  for (int j = 0; j < n_end; ++j) {
    const float* kp = k + ((long long)(k0 + j) * hkv + g) * D;
    const float* vp = v + ((long long)(k0 + j) * hkv + g) * D;
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) s = __builtin_fmaf(qr[d], kp[d], s);
    s *= scale;
    if (s > m) {
      const float corr = expf(m - s);   // 0 when m = -inf
      l *= corr;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] *= corr;
      m = s;
    }
    const float p = expf(s - m);
    l += p;
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] = __builtin_fmaf(p, vp[d], o[d]);
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* op = out + row * D;
#pragma unroll
  for (int d = 0; d < D; ++d) op[d] = o[d] * inv;
  lse[row] = l > 0.f ? m + logf(l) : neg_inf();
}

template <int D>
int launch_t(const AttnArgs& a) {
  const long long rows = (long long)a.total_q * a.hq;
  const long long blocks = (rows + 63) / 64;
  if (blocks > 0x7fffffffLL) return -1;
  hipLaunchKernelGGL((attn_fwd_f32_kernel<D>), dim3((unsigned)blocks), dim3(64), 0, (hipStream_t)a.stream,
                     (const float*)a.q, (const float*)a.k, (const float*)a.v, a.cu_q, a.cu_k, a.causal_off,
                     a.batch, a.hq, a.hkv, a.grp, rows, a.scale, a.causal, (float*)a.out, a.lse);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_attn_fwd_f32(const AttnArgs& a) {
  return a.head_dim == 128 ? launch_t<128>(a) : launch_t<64>(a);
}

}  // namespace vfa
