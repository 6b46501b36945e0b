// Host-only stand-ins for the HIP side of libvfa, so that the C-ABI layer
// (api.cpp, plain C++) can be built with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer and driven from Python without a GPU.
//
// Every launcher, device check and device-memory lookup that api.cpp can reach
// is replaced by a function that only counts the call. The count is exported
// as vfa_stub_launch_count(): the argument-validation tests assert that it
// stays unchanged, i.e. that every rejected (or empty) call returns before it
// reaches the GPU side. The plans and sizes that validation depends on
// (plan_decode, plan_paged, gated_delta_chunk_workspace, wide_prefill) are the
// real ones: api.cpp and launch.h define them.
#include "launch.h"

static int g_calls = 0;

extern "C" __attribute__((visibility("default"))) int vfa_stub_launch_count() { return g_calls; }

namespace vfa {

int static_scratch(void*, void** ptr) {
  ++g_calls;
  *ptr = nullptr;
  return -1;
}
int launch_attn_fwd_bf16(const AttnArgs&) { return ++g_calls, -1; }
int launch_attn_fwd_overlap(const AttnArgs&) { return ++g_calls, -1; }
int launch_attn_decode_bf16(const AttnArgs&, const DecodePlan&) { return ++g_calls, -1; }
int launch_attn_fwd_f32(const AttnArgs&) { return ++g_calls, -1; }
int launch_paged_decode_bf16(const PagedArgs&, const PagedPlan&) { return ++g_calls, -1; }
int launch_attn_update(const float*, const void*, int, int, int64_t, int, int, void*, float*, void*) {
  return ++g_calls, -1;
}
int launch_qk_norm_rope(const QkNormRopeArgs&) { return ++g_calls, -1; }
int launch_gated_delta(const GatedDeltaArgs&) { return ++g_calls, -1; }
int launch_gated_delta_chunked(const GatedDeltaArgs&, int, void*) { return ++g_calls, -1; }
int launch_last_token_gather(const void*, int, const int32_t*, int, int64_t, void*, void*) {
  return ++g_calls, -1;
}
int check_cu_seqlens(const int32_t*, int, int, const int32_t*, int, int, int, void*) { return ++g_calls, -1; }
int check_paged(const int32_t*, const int32_t*, int, int, int, int, int, void*) { return ++g_calls, -1; }

}  // namespace vfa
