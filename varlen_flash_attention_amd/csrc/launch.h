// Host-side launch interface between the C-ABI layer (api.cpp, plain C++)
// and the HIP kernels. Plain data only: no HIP types cross this header.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace vfa {

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* causal_off;  // per-sequence causal offset, or NULL for Lk - Lq (bottom-right)
  int batch, total_q, total_k, max_seqlen_q, max_seqlen_k;
  int hq, hkv, grp, head_dim;
  float scale;
  int causal;
  void* out;
  int out_dtype;  // 0 = fp32, 1 = bf16
  float* lse;
  void* workspace;
  size_t workspace_bytes;
  void* stream;
};

// Long-sequence prefill: batches whose sequences average at least eight
// 256-column query tiles (8 * 256 / G tokens, G = hq / hkv) run on the
// persistent 256-column kernel (attn_fwd_overlap.hip), which takes its work
// items from ticket counters in a small workspace; shorter ones on the
// 128-column kernel, which needs none. The persistent kernel addresses all
// keys of a sequence and kv head through one buffer with 32-bit byte offsets,
// so a sequence whose keys span 4 GiB or more (with a 256-row margin for the
// last sub-block) goes to the 128-column kernel, which rebases per sub-block.
constexpr size_t kWidePrefillWorkspace = 1024;   // 8 XCD counters, one 128-byte line each
inline bool wide_prefill(int batch, int total_q, int max_seqlen_k, int hq, int hkv, int head_dim) {
  if (batch <= 0 || hq <= 0 || hkv <= 0 || hq % hkv != 0 || max_seqlen_k < 0 || head_dim <= 0) return false;
  if (((long long)max_seqlen_k + 256) * hkv * head_dim * 2 >= (1LL << 32)) return false;
  return (long long)total_q / batch >= 8LL * (256 / (hq / hkv));
}

// Split-KV plan for short query sets against long key sets (decode).
struct DecodePlan {
  bool use;          // take the split-KV path
  int chunk;         // keys per split
  int n_splits;      // splits per sequence at max_seqlen_k
  size_t ws_bytes;   // partial O (fp32) + partial lse (fp32)
};
DecodePlan plan_decode(int batch, int total_q, int max_seqlen_q, int max_seqlen_k, int hq, int hkv,
                       int head_dim);

// Paged K/V (decode-shaped): caches [num_pages, page_size, hkv, D], block
// table [batch, max_pages], keys per sequence in seqused_k.
struct PagedArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  int max_pages, num_pages, page_size;
  const int32_t* cu_q;
  const int32_t* seqused_k;
  int batch, total_q, max_seqlen_q, max_seqlen_k;
  int hq, hkv, grp, head_dim;
  float scale;
  int causal;
  void* out;
  int out_dtype;  // 0 = fp32, 1 = bf16
  float* lse;
  void* workspace;
  size_t workspace_bytes;
  void* stream;
};

// Split plan of the paged path: (token, head) columns of a kv head in n_cg
// groups of 16, keys per split, splits at max_seqlen_k.
struct PagedPlan {
  int chunk;
  int n_splits;
  int n_cg;
  size_t ws_bytes;   // partial O + partial lse (fp32) per split and row; 0 with one split
};
PagedPlan plan_paged(int batch, int total_q, int max_seqlen_q, int max_seqlen_k, int hq, int hkv, int head_dim);

// Attention prologue: per-head RMSNorm of q [tokens, hq, D] and k [tokens, hkv, D]
// (bf16, weights bf16 [D]) then the rotary embedding with fp32 cos / sin [tokens, D].
struct QkNormRopeArgs {
  const void* q_in;
  const void* k_in;
  const void* q_weight;
  const void* k_weight;
  const float* cos;
  const float* sin;
  int tokens, hq, hkv, head_dim;
  float eps;
  void* q_out;
  void* k_out;
  void* stream;
};

// Varlen gated delta rule forward: q, k [tokens, hqk, dk], v [tokens, hv, dv] bf16;
// g, beta [tokens, hv] fp32; states [batch, hv, dk, dv] fp32 (optional); out
// [tokens, hv, dv] bf16.
struct GatedDeltaArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const int32_t* cu;
  int batch, tokens, hqk, hv, dk, dv;
  float scale;
  const float* s_init;
  void* out;
  float* s_final;
  void* stream;
};

// Size of the library's static per-device scratch array (static_scratch.hip),
// which holds the split-KV partials of varlen_attn_fwd_noalloc. Equal to
// VFA_STATIC_SCRATCH_BYTES in include/vfa.h.
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;

// Device address of that array on the device of `stream`, looked up once per
// device (hipGetSymbolAddress with the device current) and cached. Returns 0,
// or -1 on a HIP error.
int static_scratch(void* stream, void** ptr);

// Each returns 0 on success, -1 if the HIP runtime reported a launch error.
int launch_attn_fwd_bf16(const AttnArgs& a);
// The 256-column kernel for long sequences (attn_fwd_overlap.hip).
int launch_attn_fwd_overlap(const AttnArgs& a);
int launch_attn_decode_bf16(const AttnArgs& a, const DecodePlan& plan);
int launch_attn_fwd_f32(const AttnArgs& a);
int launch_paged_decode_bf16(const PagedArgs& a, const PagedPlan& plan);
int launch_attn_update(const float* lse, const void* go, int go_dtype, int sp, int64_t bsh, int hd,
                       int update_type, void* out, float* lse_out, void* stream);
int launch_qk_norm_rope(const QkNormRopeArgs& a);
int launch_gated_delta(const GatedDeltaArgs& a);
// Chunked form (gated_delta_chunk.hip): tokens per chunk; sequences ranked by
// length for the chunk kernel's order (larger batches keep their own order);
// bytes of workspace for `tokens` packed tokens and hv value heads (per token
// and value head, T and M as bf16 hi/lo rows of kGdnChunk, 2 bytes each, and
// two fp32 decay factors; then a fixed slot of kGdnOrderMax int32 for the
// order); and the two-kernel launch using it.
constexpr int kGdnChunk = 64;
constexpr int kGdnOrderMax = 4096;
inline size_t gated_delta_chunk_workspace(long long tokens, int hv) {
  return (size_t)tokens * hv * (2 * 2 * kGdnChunk * 2 + 2 * sizeof(float)) + kGdnOrderMax * sizeof(int32_t);
}
int launch_gated_delta_chunked(const GatedDeltaArgs& a, int max_seqlen, void* workspace);
int launch_last_token_gather(const void* x, int esize, const int32_t* cu, int batch, int64_t row_elems,
                             void* out, void* stream);

// Caller-contract check of one or two cu_seqlens arrays of batch + 1 entries
// (cu_b may be NULL; a negative total skips the end check). Synchronises the
// stream; checked calls are serialised process-wide. Returns 0 if the
// contract holds, 1 if it is violated, -1 on a HIP error, -2 (nothing
// launched) if the stream is capturing a graph.
int check_cu_seqlens(const int32_t* cu_a, int total_a, int max_a, const int32_t* cu_b, int total_b, int max_b,
                     int batch, void* stream);

// Caller-contract check of the paged inputs: 0 <= seqused_k[b] <= max_seqlen_k
// and every block-table entry that names one of those keys' pages lies in
// [0, num_pages). Synchronises the stream; same serialisation and return values.
int check_paged(const int32_t* seqused_k, const int32_t* block_table, int batch, int max_pages, int page_size,
                int num_pages, int max_seqlen_k, void* stream);

}  // namespace vfa
