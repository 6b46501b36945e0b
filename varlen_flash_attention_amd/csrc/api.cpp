// libvfa C ABI: argument validation, launch planning and dispatch.
//
// Plain C++ with no HIP headers: every check here runs on host values only
// and returns before anything is launched, so the error paths can be tested
// without a GPU. Kernels are reached through launch.h.
//
// The boundary follows the operator conventions of "attention_update operator
// optimisation practice" (ACLNN and op-plugin sections): plain tensors, sizes
// taken from the caller, outputs allocated by the caller, a status code, and
// validation before execution. The attention arguments follow the fused
// attention call of "From GPU to NPU: Qwen3-Embedding on Ascend" (section 2.1
// and core optimisation 5: head counts, TND layout, per-sequence lengths,
// scale, causal flag).
#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <cstdint>

#include "../../include/vfa.h"
#include "launch.h"

#define VFA_API extern "C" __attribute__((visibility("default")))

namespace vfa {

// Split-KV (decode) path: only when the queries of one sequence fit the
// 16-column tile together with the G heads that share a kv head, and the key
// sets are long enough for splitting to pay. Keys per split start at 4096
// and halve (down to 256) until there are enough workgroups to fill the chip.
DecodePlan plan_decode(int batch, int total_q, int max_seqlen_q, int max_seqlen_k, int hq, int hkv,
                       int head_dim) {
  DecodePlan p{false, 0, 0, 0};
  if (batch <= 0 || total_q <= 0 || hq <= 0 || hkv <= 0 || hq % hkv != 0) return p;
  const int grp = hq / hkv;
  if (grp > 16 || (long long)max_seqlen_q * grp > 16 || max_seqlen_q < 1) return p;
  if (max_seqlen_k < 512) return p;
  // Longer splits amortise each workgroup's start (first loads in flight, Q,
  // the final merge): measured on MI355X at the decode shape, 4096-key splits
  // beat 1024 by 4-5% and match 8192. Halve while fewer than 2048 (sequence,
  // kv head, split) work units would leave CUs idle.
  int chunk = 4096;
  while (chunk > 256 && (long long)batch * hkv * ((max_seqlen_k + chunk - 1) / chunk) < 2048) chunk /= 2;
  p.use = true;
  p.chunk = chunk;
  p.n_splits = (max_seqlen_k + chunk - 1) / chunk;
  p.ws_bytes = (size_t)p.n_splits * (size_t)total_q * (size_t)hq * (size_t)(head_dim + 1) * sizeof(float);
  return p;
}

// Paged path: the (token, head) columns of a kv head are cut into groups of
// 16 (one workgroup's MFMA columns); splits follow the same rule as above
// over (sequence, kv head, column group) units.
PagedPlan plan_paged(int batch, int total_q, int max_seqlen_q, int max_seqlen_k, int hq, int hkv, int head_dim) {
  PagedPlan p{256, 1, 1, 0};
  if (batch <= 0 || total_q <= 0 || max_seqlen_q <= 0 || hq <= 0 || hkv <= 0 || hq % hkv != 0) return p;
  const long long grp = hq / hkv;
  p.n_cg = (int)(((long long)max_seqlen_q * grp + 15) / 16);
  const long long units = (long long)batch * hkv * p.n_cg;
  int chunk = 4096;
  while (chunk > 256 && units * ((max_seqlen_k + chunk - 1) / chunk) < 2048) chunk /= 2;
  p.chunk = chunk;
  p.n_splits = max_seqlen_k > chunk ? (max_seqlen_k + chunk - 1) / chunk : 1;
  if (p.n_splits > 1)
    p.ws_bytes = (size_t)p.n_splits * (size_t)total_q * (size_t)hq * (size_t)(head_dim + 1) * sizeof(float);
  return p;
}

}  // namespace vfa

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// VFA_DEBUG set to anything but "" or "0": check cu_seqlens on the device
// before launching (read on every call, so a process can switch it).
bool debug_checks() {
  const char* e = std::getenv("VFA_DEBUG");
  return e && *e && std::strcmp(e, "0") != 0;
}

// Status of a VFA_DEBUG contract check: violated -> VFA_ERR_SHAPE; asked for
// on a stream that is capturing a graph (the check must synchronise) ->
// VFA_ERR_UNSUPPORTED; a HIP error -> VFA_ERR_LAUNCH.
int32_t debug_status(int r) {
  if (r == 0) return VFA_OK;
  if (r == 1) return VFA_ERR_SHAPE;
  if (r == -2) return VFA_ERR_UNSUPPORTED;
  return VFA_ERR_LAUNCH;
}

}  // namespace

VFA_API int32_t vfa_abi_version(void) { return VFA_ABI_VERSION; }

VFA_API const char* vfa_status_string(int32_t status) {
  switch (status) {
    case VFA_OK: return "VFA_OK: success";
    case VFA_ERR_NULL: return "VFA_ERR_NULL: a required pointer is NULL";
    case VFA_ERR_SHAPE: return "VFA_ERR_SHAPE: a size or count is out of range or inconsistent";
    case VFA_ERR_UNSUPPORTED: return "VFA_ERR_UNSUPPORTED: request not supported by this library";
    case VFA_ERR_WORKSPACE: return "VFA_ERR_WORKSPACE: workspace missing or too small";
    case VFA_ERR_LAUNCH: return "VFA_ERR_LAUNCH: the HIP runtime reported a launch error";
    default: return "unknown vfa status";
  }
}

VFA_API size_t varlen_attn_fwd_workspace_size(int32_t batch, int32_t total_q, int32_t max_seqlen_q,
                                              int32_t max_seqlen_k, int32_t num_heads_q,
                                              int32_t num_heads_kv, int32_t head_dim) {
  const vfa::DecodePlan p =
      vfa::plan_decode(batch, total_q, max_seqlen_q, max_seqlen_k, num_heads_q, num_heads_kv, head_dim);
  if (p.use) return p.ws_bytes;
  const bool wide = vfa::wide_prefill(batch, total_q, max_seqlen_k, num_heads_q, num_heads_kv, head_dim);
  return wide ? vfa::kWidePrefillWorkspace : 0;
}

namespace {

int32_t attn_fwd_impl(const void* q, const void* k, const void* v, int32_t in_dtype, const int32_t* cu_seqlens_q,
                      const int32_t* cu_seqlens_k, const int32_t* causal_offset, int32_t batch, int32_t total_q,
                      int32_t total_k, int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t num_heads_q,
                      int32_t num_heads_kv, int32_t head_dim, float softmax_scale, int32_t causal, void* out,
                      int32_t out_dtype, float* lse, void* workspace, size_t workspace_bytes, void* stream,
                      bool static_ws = false) {
  if (batch < 0 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 || max_seqlen_k < 0) return VFA_ERR_SHAPE;
  if (batch == 0 || total_q == 0) return VFA_OK;
  if (!q || !k || !v || !cu_seqlens_q || !cu_seqlens_k || !out || !lse) return VFA_ERR_NULL;
  if (num_heads_q <= 0 || num_heads_kv <= 0 || num_heads_q % num_heads_kv != 0) return VFA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return VFA_ERR_SHAPE;
  if (max_seqlen_q > total_q || max_seqlen_k > total_k) return VFA_ERR_SHAPE;
  if ((long long)max_seqlen_q * batch < total_q || (long long)max_seqlen_k * batch < total_k)
    return VFA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return VFA_ERR_UNSUPPORTED;
  if (num_heads_q / num_heads_kv > 32) return VFA_ERR_UNSUPPORTED;
  if (in_dtype == VFA_F32) {
    if (out_dtype != VFA_F32) return VFA_ERR_UNSUPPORTED;
  } else if (in_dtype == VFA_BF16) {
    if (out_dtype != VFA_F32 && out_dtype != VFA_BF16) return VFA_ERR_UNSUPPORTED;
  } else {
    return VFA_ERR_UNSUPPORTED;
  }
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return VFA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return VFA_ERR_UNSUPPORTED;

  // bf16 calls take the split-KV (decode) path with its partials workspace,
  // or, for long sequences, the persistent prefill kernel with its ticket
  // counters; the fp32 kernel needs no workspace.
  const vfa::DecodePlan plan =
      in_dtype == VFA_BF16
          ? vfa::plan_decode(batch, total_q, max_seqlen_q, max_seqlen_k, num_heads_q, num_heads_kv, head_dim)
          : vfa::DecodePlan{false, 0, 0, 0};
  const bool wide = in_dtype == VFA_BF16 && !plan.use &&
                    vfa::wide_prefill(batch, total_q, max_seqlen_k, num_heads_q, num_heads_kv, head_dim);
  const size_t ws_need = plan.use ? plan.ws_bytes : (wide ? vfa::kWidePrefillWorkspace : 0);
  if (ws_need > 0) {
    if (static_ws) {
      if (ws_need > vfa::kStaticScratchBytes) return VFA_ERR_WORKSPACE;
    } else if (!workspace || workspace_bytes < ws_need || !aligned16(workspace)) {
      return VFA_ERR_WORKSPACE;
    }
  }

  if (debug_checks()) {
    const int r = vfa::check_cu_seqlens(cu_seqlens_q, total_q, max_seqlen_q, cu_seqlens_k, total_k, max_seqlen_k,
                                        batch, stream);
    if (r != 0) return debug_status(r);
  }
  if (ws_need > 0 && static_ws) {
    if (vfa::static_scratch(stream, &workspace) != 0) return VFA_ERR_LAUNCH;
    workspace_bytes = vfa::kStaticScratchBytes;
  }

  vfa::AttnArgs a{};
  a.q = q; a.k = k; a.v = v;
  a.cu_q = cu_seqlens_q; a.cu_k = cu_seqlens_k; a.causal_off = causal_offset;
  a.batch = batch; a.total_q = total_q; a.total_k = total_k;
  a.max_seqlen_q = max_seqlen_q; a.max_seqlen_k = max_seqlen_k;
  a.hq = num_heads_q; a.hkv = num_heads_kv; a.grp = num_heads_q / num_heads_kv; a.head_dim = head_dim;
  a.scale = softmax_scale; a.causal = causal;
  a.out = out; a.out_dtype = out_dtype == VFA_BF16 ? 1 : 0; a.lse = lse;
  a.workspace = workspace; a.workspace_bytes = workspace_bytes; a.stream = stream;

  if (in_dtype == VFA_F32) return vfa::launch_attn_fwd_f32(a) == 0 ? VFA_OK : VFA_ERR_LAUNCH;
  if (plan.use) return vfa::launch_attn_decode_bf16(a, plan) == 0 ? VFA_OK : VFA_ERR_LAUNCH;
  return vfa::launch_attn_fwd_bf16(a) == 0 ? VFA_OK : VFA_ERR_LAUNCH;
}

}  // namespace

VFA_API int32_t varlen_attn_fwd(const void* q, const void* k, const void* v, int32_t in_dtype,
                                const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t batch,
                                int32_t total_q, int32_t total_k, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                float softmax_scale, int32_t causal, void* out, int32_t out_dtype, float* lse,
                                void* workspace, size_t workspace_bytes, void* stream) {
  return attn_fwd_impl(q, k, v, in_dtype, cu_seqlens_q, cu_seqlens_k, nullptr, batch, total_q, total_k,
                       max_seqlen_q, max_seqlen_k, num_heads_q, num_heads_kv, head_dim, softmax_scale, causal, out,
                       out_dtype, lse, workspace, workspace_bytes, stream);
}

VFA_API int32_t varlen_attn_fwd_offset(const void* q, const void* k, const void* v, int32_t in_dtype,
                                       const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                       const int32_t* causal_offset, int32_t batch, int32_t total_q,
                                       int32_t total_k, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                       int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                       float softmax_scale, int32_t causal, void* out, int32_t out_dtype,
                                       float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  if (batch > 0 && total_q > 0 && causal != 0 && !causal_offset) return VFA_ERR_NULL;
  return attn_fwd_impl(q, k, v, in_dtype, cu_seqlens_q, cu_seqlens_k, causal != 0 ? causal_offset : nullptr,
                       batch, total_q, total_k, max_seqlen_q, max_seqlen_k, num_heads_q, num_heads_kv, head_dim,
                       softmax_scale, causal, out, out_dtype, lse, workspace, workspace_bytes, stream);
}

static_assert(vfa::kStaticScratchBytes == VFA_STATIC_SCRATCH_BYTES, "static scratch size differs from the header");

VFA_API int32_t varlen_attn_fwd_noalloc(const void* q, const void* k, const void* v, int32_t in_dtype,
                                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t batch,
                                        int32_t total_q, int32_t total_k, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                        int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                        float softmax_scale, int32_t causal, void* out, int32_t out_dtype,
                                        float* lse, void* stream) {
  return attn_fwd_impl(q, k, v, in_dtype, cu_seqlens_q, cu_seqlens_k, nullptr, batch, total_q, total_k,
                       max_seqlen_q, max_seqlen_k, num_heads_q, num_heads_kv, head_dim, softmax_scale, causal, out,
                       out_dtype, lse, nullptr, 0, stream, true);
}

VFA_API int32_t attn_update(const float* lse, const void* go, int32_t go_dtype, int32_t sp, int64_t bsh,
                            int32_t hd, int32_t update_type, void* out, float* lse_out, void* stream) {
  if (sp < 1 || bsh < 0) return VFA_ERR_SHAPE;
  if (update_type != 0 && update_type != 1) return VFA_ERR_SHAPE;
  if (bsh == 0) return VFA_OK;
  if (!lse || !go || !out) return VFA_ERR_NULL;
  if (update_type == 1 && !lse_out) return VFA_ERR_NULL;
  if (hd != 64 && hd != 128) return VFA_ERR_UNSUPPORTED;
  if (go_dtype != VFA_F32 && go_dtype != VFA_BF16) return VFA_ERR_UNSUPPORTED;
  if (!aligned16(go) || !aligned16(out)) return VFA_ERR_UNSUPPORTED;
  return vfa::launch_attn_update(lse, go, go_dtype == VFA_BF16 ? 1 : 0, sp, bsh, hd, update_type, out, lse_out,
                                 stream) == 0
             ? VFA_OK
             : VFA_ERR_LAUNCH;
}

VFA_API int32_t varlen_last_token_gather(const void* x, int32_t dtype, const int32_t* cu_seqlens, int32_t batch,
                                         int64_t row_elems, void* out, void* stream) {
  if (batch < 0 || row_elems < 0) return VFA_ERR_SHAPE;
  if (batch == 0 || row_elems == 0) return VFA_OK;
  if (!x || !cu_seqlens || !out) return VFA_ERR_NULL;
  if (dtype != VFA_F32 && dtype != VFA_BF16) return VFA_ERR_UNSUPPORTED;
  if (debug_checks()) {
    const int r = vfa::check_cu_seqlens(cu_seqlens, -1, 0x7fffffff, nullptr, 0, 0, batch, stream);
    if (r != 0) return debug_status(r);
  }
  return vfa::launch_last_token_gather(x, dtype == VFA_F32 ? 4 : 2, cu_seqlens, batch, row_elems, out, stream) == 0
             ? VFA_OK
             : VFA_ERR_LAUNCH;
}

VFA_API size_t paged_attn_decode_workspace_size(int32_t batch, int32_t total_q, int32_t max_seqlen_q,
                                                int32_t max_seqlen_k, int32_t num_heads_q, int32_t num_heads_kv,
                                                int32_t head_dim) {
  return vfa::plan_paged(batch, total_q, max_seqlen_q, max_seqlen_k, num_heads_q, num_heads_kv, head_dim).ws_bytes;
}

VFA_API int32_t paged_attn_decode(const void* q, int32_t in_dtype, const void* k_cache, const void* v_cache,
                                  const int32_t* block_table, int32_t max_pages_per_seq, int32_t num_pages,
                                  int32_t page_size, const int32_t* cu_seqlens_q, const int32_t* seqused_k,
                                  int32_t batch, int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                  int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim, float softmax_scale,
                                  int32_t causal, void* out, int32_t out_dtype, float* lse, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (batch < 0 || total_q < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || max_pages_per_seq < 0 || num_pages < 0 ||
      page_size <= 0)
    return VFA_ERR_SHAPE;
  if (batch == 0 || total_q == 0) return VFA_OK;
  if (!q || !k_cache || !v_cache || !block_table || !cu_seqlens_q || !seqused_k || !out || !lse) return VFA_ERR_NULL;
  if (num_heads_q <= 0 || num_heads_kv <= 0 || num_heads_q % num_heads_kv != 0) return VFA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return VFA_ERR_SHAPE;
  if (max_seqlen_q > total_q || (long long)max_seqlen_q * batch < total_q) return VFA_ERR_SHAPE;
  if ((long long)max_seqlen_k > (long long)max_pages_per_seq * page_size) return VFA_ERR_SHAPE;
  if (max_seqlen_k > 0 && num_pages == 0) return VFA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return VFA_ERR_UNSUPPORTED;
  if (in_dtype != VFA_BF16) return VFA_ERR_UNSUPPORTED;
  if (out_dtype != VFA_F32 && out_dtype != VFA_BF16) return VFA_ERR_UNSUPPORTED;
  // Page sizes: powers of two from 16 keys (a 32-key step then spans at most two pages) to 4096.
  if (page_size < 16 || page_size > 4096 || (page_size & (page_size - 1)) != 0) return VFA_ERR_UNSUPPORTED;
  if ((long long)page_size * num_heads_kv * head_dim >= (1LL << 31)) return VFA_ERR_UNSUPPORTED;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return VFA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)) return VFA_ERR_UNSUPPORTED;

  const vfa::PagedPlan plan =
      vfa::plan_paged(batch, total_q, max_seqlen_q, max_seqlen_k, num_heads_q, num_heads_kv, head_dim);
  if (plan.ws_bytes > 0 && (!workspace || workspace_bytes < plan.ws_bytes || !aligned16(workspace)))
    return VFA_ERR_WORKSPACE;

  if (debug_checks()) {
    int r = vfa::check_cu_seqlens(cu_seqlens_q, total_q, max_seqlen_q, nullptr, 0, 0, batch, stream);
    if (r == 0)
      r = vfa::check_paged(seqused_k, block_table, batch, max_pages_per_seq, page_size, num_pages, max_seqlen_k,
                           stream);
    if (r != 0) return debug_status(r);
  }

  vfa::PagedArgs a{};
  a.q = q; a.k_cache = k_cache; a.v_cache = v_cache;
  a.block_table = block_table; a.max_pages = max_pages_per_seq; a.num_pages = num_pages; a.page_size = page_size;
  a.cu_q = cu_seqlens_q; a.seqused_k = seqused_k;
  a.batch = batch; a.total_q = total_q; a.max_seqlen_q = max_seqlen_q; a.max_seqlen_k = max_seqlen_k;
  a.hq = num_heads_q; a.hkv = num_heads_kv; a.grp = num_heads_q / num_heads_kv; a.head_dim = head_dim;
  a.scale = softmax_scale; a.causal = causal;
  a.out = out; a.out_dtype = out_dtype == VFA_BF16 ? 1 : 0; a.lse = lse;
  a.workspace = workspace; a.workspace_bytes = workspace_bytes; a.stream = stream;
  return vfa::launch_paged_decode_bf16(a, plan) == 0 ? VFA_OK : VFA_ERR_LAUNCH;
}

VFA_API int32_t qk_norm_rope(const void* q_in, const void* k_in, int32_t dtype, const void* q_weight,
                             const void* k_weight, const float* cos, const float* sin, int32_t total_tokens,
                             int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim, float eps, void* q_out,
                             void* k_out, void* stream) {
  if (total_tokens < 0 || num_heads_q < 0 || num_heads_kv < 0) return VFA_ERR_SHAPE;
  if (total_tokens == 0 || num_heads_q + num_heads_kv == 0) return VFA_OK;
  if (!cos || !sin) return VFA_ERR_NULL;
  if (num_heads_q > 0 && (!q_in || !q_weight || !q_out)) return VFA_ERR_NULL;
  if (num_heads_kv > 0 && (!k_in || !k_weight || !k_out)) return VFA_ERR_NULL;
  if (head_dim != 64 && head_dim != 128) return VFA_ERR_UNSUPPORTED;
  if (dtype != VFA_BF16) return VFA_ERR_UNSUPPORTED;
  if (!std::isfinite(eps) || eps < 0.f) return VFA_ERR_UNSUPPORTED;
  const void* ptrs[] = {q_in, k_in, q_weight, k_weight, q_out, k_out};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return VFA_ERR_UNSUPPORTED;
  if (!aligned16(cos) || !aligned16(sin)) return VFA_ERR_UNSUPPORTED;
  vfa::QkNormRopeArgs a{};
  a.q_in = q_in; a.k_in = k_in; a.q_weight = q_weight; a.k_weight = k_weight; a.cos = cos; a.sin = sin;
  a.tokens = total_tokens; a.hq = num_heads_q; a.hkv = num_heads_kv; a.head_dim = head_dim; a.eps = eps;
  a.q_out = q_out; a.k_out = k_out; a.stream = stream;
  return vfa::launch_qk_norm_rope(a) == 0 ? VFA_OK : VFA_ERR_LAUNCH;
}

// Sequences up to this length take the token-by-token recurrence (one
// kernel, no workspace); longer ones the chunked form.
constexpr int kGdnRecurrentMaxLen = 16;

VFA_API int64_t gated_delta_rule_fwd_workspace_size(int32_t total_tokens, int32_t num_heads_v, int32_t max_seqlen) {
  if (total_tokens <= 0 || num_heads_v <= 0 || max_seqlen <= kGdnRecurrentMaxLen) return 0;
  return (int64_t)vfa::gated_delta_chunk_workspace(total_tokens, num_heads_v);
}

VFA_API int32_t gated_delta_rule_fwd(const void* q, const void* k, const void* v, int32_t dtype, const float* g,
                                     const float* beta, const int32_t* cu_seqlens, int32_t batch,
                                     int32_t total_tokens, int32_t max_seqlen, int32_t num_heads_qk,
                                     int32_t num_heads_v, int32_t head_dim_k, int32_t head_dim_v, float scale,
                                     const float* initial_state, void* out, float* final_state, void* workspace,
                                     int64_t workspace_bytes, void* stream) {
  if (batch < 0 || total_tokens < 0 || max_seqlen < 0 || num_heads_qk <= 0 || num_heads_v <= 0)
    return VFA_ERR_SHAPE;
  if (num_heads_v % num_heads_qk != 0) return VFA_ERR_SHAPE;
  if (batch == 0) return VFA_OK;
  // With no tokens the token tensors may be NULL; the final state is still written.
  if (!cu_seqlens || (total_tokens > 0 && (!q || !k || !v || !g || !beta || !out))) return VFA_ERR_NULL;
  if (dtype != VFA_BF16) return VFA_ERR_UNSUPPORTED;
  if (head_dim_k != 64 && head_dim_k != 128) return VFA_ERR_UNSUPPORTED;
  if (head_dim_v != 64 && head_dim_v != 128) return VFA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return VFA_ERR_UNSUPPORTED;
  // Token rows, states and the workspace move in 16-byte pieces.
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return VFA_ERR_UNSUPPORTED;
  if (!aligned16(initial_state) || !aligned16(final_state)) return VFA_ERR_UNSUPPORTED;
  const int64_t need = gated_delta_rule_fwd_workspace_size(total_tokens, num_heads_v, max_seqlen);
  // The chunked path addresses a 64-token chunk of each tensor with 32-bit offsets.
  constexpr int64_t kChunkSpan = 64LL * 2;   // 64 tokens, bf16
  if (need > 0 && (kChunkSpan * num_heads_qk * head_dim_k >= (1LL << 32) ||
                   kChunkSpan * num_heads_v * std::max(head_dim_v, 128) >= (1LL << 32)))
    return VFA_ERR_UNSUPPORTED;
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace))) return VFA_ERR_WORKSPACE;
  if (debug_checks()) {
    const int r = vfa::check_cu_seqlens(cu_seqlens, total_tokens, max_seqlen, nullptr, 0, 0, batch, stream);
    if (r != 0) return debug_status(r);
  }
  vfa::GatedDeltaArgs a{};
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.cu = cu_seqlens;
  a.batch = batch; a.tokens = total_tokens; a.hqk = num_heads_qk; a.hv = num_heads_v;
  a.dk = head_dim_k; a.dv = head_dim_v; a.scale = scale;
  a.s_init = initial_state; a.out = out; a.s_final = final_state; a.stream = stream;
  const int rc = need > 0 ? vfa::launch_gated_delta_chunked(a, max_seqlen, workspace) : vfa::launch_gated_delta(a);
  return rc == 0 ? VFA_OK : VFA_ERR_LAUNCH;
}
