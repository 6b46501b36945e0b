/*
 * vfa.h -- C ABI of libvfa: attention over packed variable-length sequences
 * and the AttentionUpdate merge, on AMD MI355X (gfx950).
 *
 * Conventions shared by every entry point
 *   - Tensor arguments are DEVICE pointers to contiguous row-major buffers
 *     that the caller allocates, owns and frees. The library never allocates,
 *     frees, synchronises or copies device memory to the host, and keeps no
 *     state between calls (it is reentrant). The one exception is
 *     varlen_attn_fwd_noalloc, whose split-KV partials and long-prefill work
 *     counters live in a static per-device array (see there).
 *   - `stream` is a hipStream_t (NULL = the null stream). Work is enqueued
 *     on it asynchronously; results are ready when the stream reaches them.
 *   - Sizes and flags are HOST values. Every condition that can be checked
 *     from them is checked before anything is launched; a failed check
 *     returns its status code and launches nothing. After a launch, a HIP
 *     launch error is reported as VFA_ERR_LAUNCH.
 *   - Return values are vfa_status codes (0 = success).
 *   - Debug check: with the environment variable VFA_DEBUG set to anything but
 *     "" or "0" (read on every call), varlen_attn_fwd, paged_attn_decode and
 *     varlen_last_token_gather first check the cu_seqlens contract on the
 *     device:
 *       - cu[0] == 0;
 *       - entries non-decreasing;
 *       - cu[batch] equals the total (attention only);
 *       - no length above the max_seqlen bound;
 *       - paged_attn_decode also: 0 <= seqused_k[b] <= max_seqlen_k, and
 *         every block-table entry naming a page of those keys lies in
 *         [0, num_pages).
 *     A violation returns VFA_ERR_SHAPE and launches nothing. The check
 *     synchronises the stream, copies one word to the host and clears a
 *     library word in device memory with hipMemsetAsync. Checked calls are
 *     serialised process-wide by a host lock (calls on several streams or
 *     threads each see only their own violations). A checked call on a
 *     stream that is capturing a graph returns VFA_ERR_UNSUPPORTED and
 *     launches nothing, leaving the capture intact.
 *
 * The argument conventions follow the problem as the source pages state it:
 *   [P1] "From GPU to NPU: Qwen3-Embedding model adaptation and performance
 *        optimisation on Ascend", core optimisation 1 (TND layout and
 *        cu_seqlens), section 2.1 (the fused attention call: head count,
 *        TND layout, softmax scale, per-sequence lengths, causal mask) and
 *        core optimisation 5 (native GQA through num_heads and
 *        num_key_value_heads).
 *   [P2] "Qwen3-MoE low-latency inference on Atlas A3", flash attention
 *        fused operator section (one op for prefill and decode).
 *   [P4] "attention_update operator optimisation practice", operator
 *        function description (the merge formula) and the InferShape,
 *        ACLNN and op-plugin sections (plain-tensor inputs, sp read from
 *        dim 0, output shapes and dtypes, update_type).
 */
#ifndef VFA_H
#define VFA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VFA_ABI_VERSION 8

typedef enum vfa_status {
  VFA_OK = 0,
  VFA_ERR_NULL = 1,         /* a required pointer is NULL                          */
  VFA_ERR_SHAPE = 2,        /* a size or count is out of range or inconsistent     */
  VFA_ERR_UNSUPPORTED = 3,  /* valid request this library does not support         */
  VFA_ERR_WORKSPACE = 4,    /* workspace missing or smaller than the size query    */
  VFA_ERR_LAUNCH = 5        /* the HIP runtime reported an error at launch         */
} vfa_status;

typedef enum vfa_dtype {
  VFA_F32 = 0,
  VFA_BF16 = 1
} vfa_dtype;

/* Version of this ABI compiled into the loaded library; a caller compares it
 * with VFA_ABI_VERSION to detect a stale library picked up from another path
 * (the failure mode [P4]'s troubleshooting section describes for a
 * same-named older operator). */
int32_t vfa_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* vfa_status_string(int32_t status);

/* Bytes of device workspace varlen_attn_fwd needs for these host sizes.
 * 0 means no workspace is needed. Same arguments as varlen_attn_fwd. */
size_t varlen_attn_fwd_workspace_size(int32_t batch, int32_t total_q,
                                      int32_t max_seqlen_q, int32_t max_seqlen_k,
                                      int32_t num_heads_q, int32_t num_heads_kv,
                                      int32_t head_dim);

/* Varlen attention forward ([P1] section 2.1 and core optimisation 5; [P2]).
 *
 * For every sequence b (queries cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1,
 * keys cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1), query head h and query i:
 *   s_j   = softmax_scale * <q[i, h, :], k[j, h / G, :]>,  G = Hq / Hkv
 *   vis   = all keys, or with causal != 0 the keys j <= i + Lk_b - Lq_b
 *           (bottom-right alignment; with Lq_b == Lk_b this is the
 *           triu(ones, diagonal=1)-is-masked mask of [P1] 2.1)
 *   out[i, h, :] = sum_vis exp(s_j - M) v[j, h / G, :] / sum_vis exp(s_j - M)
 *   lse[i, h]    = ln sum_vis exp(s_j)                     (natural log)
 * A row with no visible key gets out = 0 and lse = -inf.
 *
 * q       [total_q, num_heads_q, head_dim]    in_dtype
 * k, v    [total_k, num_heads_kv, head_dim]   in_dtype
 * cu_seqlens_q, cu_seqlens_k: device int32 [batch + 1], cu[0] = 0,
 *         non-decreasing, cu_q[batch] = total_q, cu_k[batch] = total_k.
 *         Not read on the host and not checked (caller contract), except
 *         on the device under VFA_DEBUG (see above).
 * max_seqlen_q / max_seqlen_k: host upper bounds of the per-sequence
 *         lengths; they size the launch so that no device-to-host copy of
 *         cu_seqlens is needed ([P1] core optimisation 1 keeps cu_seqlens
 *         on the host for the same reason). A bound below a real length
 *         is a caller error: that sequence's excess query rows are left
 *         unwritten and, on the split-KV (decode) path, its keys past the
 *         bound are ignored; nothing is read or written out of bounds.
 * out     [total_q, num_heads_q, head_dim]    out_dtype
 * lse     [total_q, num_heads_q]              fp32
 * workspace / workspace_bytes: device scratch of at least
 *         varlen_attn_fwd_workspace_size(...) bytes (may be NULL when that
 *         size is 0). Its contents on entry do not matter. Decode-shaped
 *         calls keep split-KV partials there; long-sequence prefill (bf16,
 *         sequences averaging at least 8 * 256 / G query tokens, and
 *         (max_seqlen_k + 256) * num_heads_kv * head_dim * 2 < 2^32, i.e. one
 *         sequence's keys short of 4 GiB) keeps the 1 KB of work counters its
 *         persistent kernel hands items out with, zeroed on the stream before
 *         the kernel starts. Longer key sets run on the kernel that needs no
 *         workspace. Calls that run at the same time need workspaces of their
 *         own.
 * Supported: head_dim 64 or 128; in bf16 -> out bf16 or fp32; in fp32 ->
 *         out fp32. num_heads_q % num_heads_kv == 0 and
 *         num_heads_q / num_heads_kv <= 32.
 * batch == 0 or total_q == 0 returns VFA_OK and launches nothing.
 */
int32_t varlen_attn_fwd(const void* q, const void* k, const void* v, int32_t in_dtype,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                        int32_t batch, int32_t total_q, int32_t total_k,
                        int32_t max_seqlen_q, int32_t max_seqlen_k,
                        int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                        float softmax_scale, int32_t causal,
                        void* out, int32_t out_dtype, float* lse,
                        void* workspace, size_t workspace_bytes, void* stream);

/* varlen_attn_fwd with an explicit causal alignment per sequence.
 *
 * Identical to varlen_attn_fwd except that, when causal != 0, query i of
 * sequence b sees key j iff
 *   j <= i + causal_offset[b]
 * instead of j <= i + Lk_b - Lq_b. causal_offset[b] is the position of the
 * sequence's first query minus the position of its first key, so:
 *   - Lk_b - Lq_b reproduces varlen_attn_fwd (queries are the last Lq_b
 *     positions of the key sequence);
 *   - 0 aligns the first query with the first key (top-left);
 *   - -a computes the partial of a key chunk [a, c) of a sequence against
 *     all of its queries with the sequence's absolute causal mask: the
 *     per-chunk partials of [P4]'s sequence-parallel setting, which
 *     attn_update then merges. With the query shard starting at position s,
 *     the offset is s - a.
 * Rows that see no key get out = 0 and lse = -inf. Any int32 value is
 * accepted (values beyond -Lq_b or Lk_b act as those bounds).
 *
 * causal_offset: device int32 [batch]; required (non-NULL) when causal != 0,
 *         ignored when causal == 0. Every other argument, the supported set
 *         and the workspace are those of varlen_attn_fwd (same
 *         varlen_attn_fwd_workspace_size).
 */
int32_t varlen_attn_fwd_offset(const void* q, const void* k, const void* v, int32_t in_dtype,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                               const int32_t* causal_offset,
                               int32_t batch, int32_t total_q, int32_t total_k,
                               int32_t max_seqlen_q, int32_t max_seqlen_k,
                               int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                               float softmax_scale, int32_t causal,
                               void* out, int32_t out_dtype, float* lse,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the library's static scratch array on each device: the most
 * split-KV partial storage varlen_attn_fwd_noalloc can use. */
#define VFA_STATIC_SCRATCH_BYTES (16u << 20)

/* varlen_attn_fwd for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. It takes no workspace: the split-KV partials, and the 1 KB of
 * work counters of long-sequence prefill (cleared by a kernel on every
 * call), go to a static device array of VFA_STATIC_SCRATCH_BYTES (16 MiB)
 * that every device the library runs on holds from the moment the library's
 * code is loaded there until the process ends. The call itself allocates and frees nothing and
 * calls no allocating library routine; the first call on a device looks up
 * that device's copy of the array (hipGetSymbolAddress) and caches it.
 *
 * Arguments, results, the supported set and the error codes are those of
 * varlen_attn_fwd without workspace / workspace_bytes, plus:
 *   - VFA_ERR_WORKSPACE if the call needs more split-KV storage than the
 *     static array holds, i.e. varlen_attn_fwd_workspace_size(...) >
 *     VFA_STATIC_SCRATCH_BYTES (the decode shape of 64 sequences x 32 heads
 *     with keys up to 32768 needs 8.5 MB). Nothing is launched.
 *   - VFA_ERR_LAUNCH if the array's address cannot be looked up.
 * Every call on one device shares that device's array, and each call's
 * kernels write every byte of it they read, so no state carries over
 * between calls. Calls that overlap on one device (several streams or
 * threads at once) race on the array: serialise them, or use
 * varlen_attn_fwd with a workspace per stream.
 */
int32_t varlen_attn_fwd_noalloc(const void* q, const void* k, const void* v, int32_t in_dtype,
                                const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                int32_t batch, int32_t total_q, int32_t total_k,
                                int32_t max_seqlen_q, int32_t max_seqlen_k,
                                int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                float softmax_scale, int32_t causal,
                                void* out, int32_t out_dtype, float* lse, void* stream);

/* AttentionUpdate merge ([P4], operator function description):
 *   lse_max = max_i lse[i, r]
 *   lse_m   = lse_max + ln sum_i exp(lse[i, r] - lse_max)
 *   out[r, :] = sum_i go[i, r, :] * exp(lse[i, r] - lse_m)
 * for r in [0, bsh). Chunks with lse = -inf contribute nothing; a row whose
 * every chunk is -inf gets lse_m = -inf and out = 0.
 *
 * lse     [sp, bsh]        fp32 (sp is dim 0, as in [P4]'s plain-tensor form)
 * go      [sp, bsh, hd]    go_dtype (fp32 or bf16)
 * out     [bsh, hd]        same dtype as go ([P4] op-plugin section)
 * lse_out [bsh]            fp32; written only when update_type == 1, and
 *                          then it must not be NULL; ignored when 0.
 * Row order is free to the caller; varlen_attn_fwd's partials use
 * r = token * num_heads_q + head, so its out/lse feed this call directly.
 * Supported: hd in {64, 128}, any sp >= 1 (sp <= 16 keeps every partial's
 * load in flight at once; larger sp streams). go and out 16-byte aligned.
 * bsh == 0 returns VFA_OK.
 */
int32_t attn_update(const float* lse, const void* go, int32_t go_dtype,
                    int32_t sp, int64_t bsh, int32_t hd, int32_t update_type,
                    void* out, float* lse_out, void* stream);

/* Bytes of device workspace paged_attn_decode needs for these host sizes
 * (0 when no sequence can need more than one key split). Same arguments as
 * varlen_attn_fwd_workspace_size. */
size_t paged_attn_decode_workspace_size(int32_t batch, int32_t total_q,
                                        int32_t max_seqlen_q, int32_t max_seqlen_k,
                                        int32_t num_heads_q, int32_t num_heads_kv,
                                        int32_t head_dim);

/* Attention of packed queries against a paged K/V cache ([P4] background:
 * the per-chunk partials its merge combines come from PagedAttention).
 *
 * Computes exactly what varlen_attn_fwd computes (same formula, GQA mapping,
 * bottom-right causal mask, natural-log lse, out = 0 / lse = -inf for a row
 * with no visible key), with the keys and values of sequence b read from
 * pages: key j (0 <= j < seqused_k[b]) is slot j % page_size of page
 * block_table[b, j / page_size] of k_cache and v_cache. The pages give no
 * cache layout; this is the layout taken.
 *
 * q            [total_q, num_heads_q, head_dim]                 bf16
 * k_cache,
 * v_cache      [num_pages, page_size, num_heads_kv, head_dim]   bf16
 * block_table  device int32 [batch, max_pages_per_seq]; only the entries of
 *              pages holding keys < min(seqused_k[b], max_seqlen_k) are
 *              read. Entries outside [0, num_pages) are a caller error; they
 *              are clamped into that range (wrong values, no out-of-range
 *              read).
 * cu_seqlens_q device int32 [batch + 1], as in varlen_attn_fwd.
 * seqused_k    device int32 [batch], keys of each sequence. Keys past the
 *              host bound max_seqlen_k are ignored (caller error).
 * max_seqlen_q / max_seqlen_k: host upper bounds, as in varlen_attn_fwd;
 *              max_seqlen_k <= max_pages_per_seq * page_size is required.
 * out          [total_q, num_heads_q, head_dim]   out_dtype (bf16 or fp32)
 * lse          [total_q, num_heads_q]             fp32
 * workspace / workspace_bytes: device scratch of at least
 *              paged_attn_decode_workspace_size(...) bytes, 16-byte
 *              aligned (may be NULL when that size is 0). Its contents on
 *              entry do not matter. Calls that overlap in time must not
 *              share a workspace.
 * Supported: in_dtype bf16; head_dim 64 or 128; page_size a power of two in
 *              [16, 4096] with page_size * num_heads_kv * head_dim < 2^31;
 *              any num_heads_q / num_heads_kv. Built for few queries per
 *              sequence (decode, a few speculative tokens): each group of 16
 *              (token, head) columns of a kv head reads that sequence's
 *              keys again, so long query sets belong on varlen_attn_fwd.
 * batch == 0 or total_q == 0 returns VFA_OK and launches nothing.
 */
int32_t paged_attn_decode(const void* q, int32_t in_dtype,
                          const void* k_cache, const void* v_cache,
                          const int32_t* block_table, int32_t max_pages_per_seq,
                          int32_t num_pages, int32_t page_size,
                          const int32_t* cu_seqlens_q, const int32_t* seqused_k,
                          int32_t batch, int32_t total_q,
                          int32_t max_seqlen_q, int32_t max_seqlen_k,
                          int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                          float softmax_scale, int32_t causal,
                          void* out, int32_t out_dtype, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Attention prologue on TND tensors: per-head RMSNorm of q and k, then the
 * rotary embedding ([P1] 2.2 normalisation layer, 2.3 q_norm / k_norm on the
 * [T, heads, head_dim] view, 2.4 rotary embedding with per-token cos / sin).
 *
 * For every token t and head h of q (weight q_weight) and of k (k_weight):
 *   r   = x / sqrt(mean_d x[d]^2 + eps)            x = in[t, h, :]
 *   y   = r * weight
 *   out[t, h, d] = y[d] * cos[t, d] + rot[d] * sin[t, d],
 *   rot = [-y[D/2:], y[:D/2]]                      (rotate-half form)
 * computed in fp32 and rounded once to bf16. The page gives npu_rotary_mul
 * without its formula; the rotate-half form is the reading taken.
 *
 * q_in / q_out  [total_tokens, num_heads_q, head_dim]   bf16
 * k_in / k_out  [total_tokens, num_heads_kv, head_dim]  bf16
 *               (out may be the same buffer as in: each row is read before
 *               it is written; the two must not overlap otherwise)
 * q_weight, k_weight  [head_dim] bf16
 * cos, sin      [total_tokens, head_dim] fp32, one row per token for all of
 *               its heads (positions are the caller's: in TND each sequence
 *               usually restarts at 0)
 * dtype         VFA_BF16 (the only supported value)
 * eps           finite, >= 0
 * Supported: head_dim 64 or 128. Pointers 16-byte aligned. num_heads_q or
 * num_heads_kv may be 0 (that side's pointers may then be NULL).
 * total_tokens == 0 returns VFA_OK.
 */
int32_t qk_norm_rope(const void* q_in, const void* k_in, int32_t dtype,
                     const void* q_weight, const void* k_weight,
                     const float* cos, const float* sin,
                     int32_t total_tokens, int32_t num_heads_q, int32_t num_heads_kv,
                     int32_t head_dim, float eps,
                     void* q_out, void* k_out, void* stream);

/* Varlen gated delta rule forward: the linear-attention operator of the
 * hybrid model on "Twinkle NPU kernels" (Qwen3.5 flash linear attention
 * section: chunk_gated_delta_rule over packed sequences with cu_seqlens).
 * The page names the operator only; the recurrence below is the reading
 * taken. For every sequence b and value head h, with S [Dk, Dv] starting at
 * initial_state[b, h] (or zero):
 *   S   <- exp(g[t, h]) * S
 *   u    = beta[t, h] * (v[t, h, :] - S^T k[t, h / R, :])        R = Hv / Hqk
 *   S   <- S + k[t, h / R, :] u^T
 *   out[t, h, :] = scale * S^T q[t, h / R, :]
 * over the sequence's tokens in order; final_state[b, h] = S.
 *
 * q, k          [total_tokens, num_heads_qk, head_dim_k]   bf16
 * v             [total_tokens, num_heads_v, head_dim_v]    bf16
 * g, beta       [total_tokens, num_heads_v]                fp32
 * cu_seqlens    device int32 [batch + 1], as for varlen_attn_fwd (caller
 *               contract; checked on the device under VFA_DEBUG)
 * max_seqlen    host upper bound of every sequence's length (caller
 *               contract, checked under VFA_DEBUG). It selects the path:
 *               up to 16, a token-by-token fp32 recurrence that needs no
 *               workspace; above, the chunked form (64-token chunks, two
 *               kernels) whose per-chunk matrices go to the workspace.
 * initial_state [batch, num_heads_v, head_dim_k, head_dim_v] fp32, or NULL;
 *               16-byte aligned (else VFA_ERR_UNSUPPORTED)
 * out           [total_tokens, num_heads_v, head_dim_v]    bf16
 * final_state   [batch, num_heads_v, head_dim_k, head_dim_v] fp32, or NULL;
 *               16-byte aligned (else VFA_ERR_UNSUPPORTED)
 * workspace     device memory of at least
 *               gated_delta_rule_fwd_workspace_size(total_tokens,
 *               num_heads_v, max_seqlen) bytes, 16-byte aligned, owned by
 *               the caller; its contents need no initialisation and are
 *               overwritten. NULL with 0 bytes when the size query returns 0.
 * Both paths keep the state in fp32 and round out once to bf16.
 * Supported: dtype VFA_BF16; head_dim_k and head_dim_v in {64, 128};
 * num_heads_v a multiple of num_heads_qk; scale finite; on the chunked
 * path, num_heads_v * max(head_dim_v, 128) < 2^25 and num_heads_qk *
 * head_dim_k < 2^25 (else VFA_ERR_UNSUPPORTED).
 * q, k, v and out must be 16-byte aligned (else VFA_ERR_UNSUPPORTED).
 * q, k, v, g, beta and out may be NULL when total_tokens == 0; the final
 * state (the initial state, or zeros) is still written.
 * Errors: VFA_ERR_WORKSPACE if the workspace is NULL, smaller than the
 * query or not 16-byte aligned (nothing is launched). batch == 0 returns
 * VFA_OK.
 */
int64_t gated_delta_rule_fwd_workspace_size(int32_t total_tokens, int32_t num_heads_v, int32_t max_seqlen);

int32_t gated_delta_rule_fwd(const void* q, const void* k, const void* v, int32_t dtype,
                             const float* g, const float* beta, const int32_t* cu_seqlens,
                             int32_t batch, int32_t total_tokens, int32_t max_seqlen,
                             int32_t num_heads_qk, int32_t num_heads_v,
                             int32_t head_dim_k, int32_t head_dim_v, float scale,
                             const float* initial_state, void* out, float* final_state,
                             void* workspace, int64_t workspace_bytes, void* stream);

/* Last-token gather ([P1] core optimisation 1, embed(): x[cu_seqlens[1:] - 1]).
 *
 * x       [total, row_elems]   dtype (any packed-token tensor, e.g. the
 *                              attention output viewed as [total_q, Hq * D])
 * out     [batch, row_elems]   dtype; row b = x[cu_seqlens[b + 1] - 1]
 * cu_seqlens: device int32 [batch + 1]. A sequence of length 0 has no last
 *         token; its output row is written as zeros.
 * batch == 0 returns VFA_OK.
 */
int32_t varlen_last_token_gather(const void* x, int32_t dtype, const int32_t* cu_seqlens,
                                 int32_t batch, int64_t row_elems, void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VFA_H */
