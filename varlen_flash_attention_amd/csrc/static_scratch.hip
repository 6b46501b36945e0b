// A fixed device buffer for callers that cannot allocate (code under graph
// capture, serving loops, harnesses that forbid hipMalloc): the split-KV
// partials of varlen_attn_fwd_noalloc live here instead of in a caller's
// workspace.
//
// Every device the library runs on holds its own copy of the array from the
// moment the code object is loaded there until the process ends. In host code
// the name `scratch` is only a host-side stand-in, so the device address of
// each copy is looked up once per device with hipGetSymbolAddress (with that
// device current) and kept; only that address is ever handed to kernels.
#include <mutex>

#include "common.h"
#include "launch.h"

namespace vfa {
namespace {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

int static_scratch(void* stream, void** ptr) {
  *ptr = nullptr;
  hipDevice_t dev = 0;
  if (hipStreamGetDevice((hipStream_t)stream, &dev) != hipSuccess) return -1;
  if (dev < 0 || dev >= kMaxDevices) return -1;
  std::lock_guard<std::mutex> hold(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return -1;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return -1;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return -1;
    if (e != hipSuccess || !p) return -1;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return 0;
}

}  // namespace vfa
