// Device check of the cu_seqlens caller contract, run only when the VFA_DEBUG
// environment variable is set (see include/vfa.h).
//
// The contract follows the TND layout of "From GPU to NPU: Qwen3-Embedding on
// Ascend", core optimisation 1: cu_seqlens holds the running token count,
// starting at 0, non-decreasing, ending at the total; every sequence fits the
// host's max_seqlen bound.
#include "common.h"
#include "launch.h"

namespace vfa {
namespace {

// Violation bits of the last checked call on this device (one word per device).
__device__ int g_contract_bits;

// One workgroup: thread t checks entries t, t + 256, ... of cu[0 .. batch].
// total < 0 skips the end check; every index stays within cu[0 .. batch].
__global__ __launch_bounds__(256) void check_cu_kernel(const int32_t* __restrict__ cu, int batch, int total,
                                                       int max_len, int* __restrict__ bits) {
  for (int b = threadIdx.x; b <= batch; b += blockDim.x) {
    const int c = cu[b];
    int f = 0;
    if (b == 0 && c != 0) f |= 1;
    if (b == batch && total >= 0 && c != total) f |= 2;
    if (b < batch) {
      const int n = cu[b + 1];
      if (n < c) f |= 4;
      else if (n - c > max_len) f |= 8;
    }
    if (f) atomicOr(bits, f);
  }
}

}  // namespace

int check_cu_seqlens(const int32_t* cu_a, int total_a, int max_a, const int32_t* cu_b, int total_b, int max_b,
                     int batch, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  int* bits = nullptr;
  if (hipGetSymbolAddress((void**)&bits, HIP_SYMBOL(g_contract_bits)) != hipSuccess) return -1;
  if (hipMemsetAsync(bits, 0, sizeof(int), st) != hipSuccess) return -1;
  hipLaunchKernelGGL(check_cu_kernel, dim3(1), dim3(256), 0, st, cu_a, batch, total_a, max_a, bits);
  if (cu_b) hipLaunchKernelGGL(check_cu_kernel, dim3(1), dim3(256), 0, st, cu_b, batch, total_b, max_b, bits);
  if (hipGetLastError() != hipSuccess) return -1;
  int host = 0;
  if (hipMemcpyAsync(&host, bits, sizeof(int), hipMemcpyDeviceToHost, st) != hipSuccess) return -1;
  if (hipStreamSynchronize(st) != hipSuccess) return -1;
  return host != 0 ? 1 : 0;
}

}  // namespace vfa
