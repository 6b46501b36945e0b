// Device checks of the caller contracts (cu_seqlens; paged key counts and
// block tables), run only when the VFA_DEBUG environment variable is set (see
// include/vfa.h).
//
// The contract follows the TND layout of "From GPU to NPU: Qwen3-Embedding on
// Ascend", core optimisation 1: cu_seqlens holds the running token count,
// starting at 0, non-decreasing, ending at the total; every sequence fits the
// host's max_seqlen bound.
#include <mutex>

#include "common.h"
#include "launch.h"

namespace vfa {
namespace {

// Violation bits of the checked call in progress on this device (one word per
// device). Checked calls are serialised by g_check_mutex, so two of them on
// different streams never share the word at the same time.
__device__ int g_contract_bits;
std::mutex g_check_mutex;

// The check synchronises its stream, which a stream under graph capture does
// not allow: report that instead of breaking the capture. Returns 0 when the
// stream is not capturing, -2 when it is, -1 on a HIP error.
int capture_state(hipStream_t st) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess) return -1;
  return cs == hipStreamCaptureStatusNone ? 0 : -2;
}

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

// One workgroup per sequence: its key count must lie in [0, max_len], and
// every block-table entry naming one of its (clamped) keys' pages must lie in
// [0, num_pages). max_len <= max_pages * page_size (checked on the host), so
// the table row is read within its max_pages entries.
__global__ __launch_bounds__(256) void check_paged_kernel(const int32_t* __restrict__ used,
                                                          const int32_t* __restrict__ table, int max_pages,
                                                          int page_size, int num_pages, int max_len,
                                                          int* __restrict__ bits) {
  const int b = blockIdx.x;
  const int n = used[b];
  if (threadIdx.x == 0 && (n < 0 || n > max_len)) atomicOr(bits, 16);
  const int keys = min(max(n, 0), max_len);
  const int np = (keys + page_size - 1) / page_size;
  for (int i = threadIdx.x; i < np; i += blockDim.x) {
    const int e = table[(long long)b * max_pages + i];
    if (e < 0 || e >= num_pages) atomicOr(bits, 32);
  }
}

int* contract_word(hipStream_t st) {
  int* bits = nullptr;
  if (hipGetSymbolAddress((void**)&bits, HIP_SYMBOL(g_contract_bits)) != hipSuccess) return nullptr;
  if (hipMemsetAsync(bits, 0, sizeof(int), st) != hipSuccess) return nullptr;
  return bits;
}

int read_contract_word(const int* bits, hipStream_t st) {
  if (hipGetLastError() != hipSuccess) return -1;
  int host = 0;
  if (hipMemcpyAsync(&host, bits, sizeof(int), hipMemcpyDeviceToHost, st) != hipSuccess) return -1;
  if (hipStreamSynchronize(st) != hipSuccess) return -1;
  return host != 0 ? 1 : 0;
}

}  // namespace

int check_cu_seqlens(const int32_t* cu_a, int total_a, int max_a, const int32_t* cu_b, int total_b, int max_b,
                     int batch, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (const int c = capture_state(st)) return c;
  std::lock_guard<std::mutex> hold(g_check_mutex);
  int* bits = contract_word(st);
  if (!bits) return -1;
  hipLaunchKernelGGL(check_cu_kernel, dim3(1), dim3(256), 0, st, cu_a, batch, total_a, max_a, bits);
  if (cu_b) hipLaunchKernelGGL(check_cu_kernel, dim3(1), dim3(256), 0, st, cu_b, batch, total_b, max_b, bits);
  return read_contract_word(bits, st);
}

int check_paged(const int32_t* seqused_k, const int32_t* block_table, int batch, int max_pages, int page_size,
                int num_pages, int max_seqlen_k, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (const int c = capture_state(st)) return c;
  std::lock_guard<std::mutex> hold(g_check_mutex);
  int* bits = contract_word(st);
  if (!bits) return -1;
  hipLaunchKernelGGL(check_paged_kernel, dim3((unsigned)batch), dim3(256), 0, st, seqused_k, block_table, max_pages,
                     page_size, num_pages, max_seqlen_k, bits);
  return read_contract_word(bits, st);
}

}  // namespace vfa
