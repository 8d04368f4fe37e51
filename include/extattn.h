/*
 * extattn: chunked-prefill "extend" attention for AMD Instinct MI355X (gfx950).
 *
 * What the library computes (zdszero "Chunked Prefill" notes, section "prefill
 * as several resumable extends", equation for o_i): a request whose first
 * P tokens already sit in the KV cache runs E new query tokens at global
 * positions P .. P+E-1. Query token i attends keys 0 .. P+i inclusive: the
 * whole prefix with no mask (stage 1, the rectangle) and its own chunk
 * causally (stage 2, the triangle). The two parts are combined with the
 * online-softmax merge of the same section, so chunked output equals one-shot
 * causal prefill up to floating-point order. A decode row is the case E = 1.
 * Several requests with different (P, E) run in one call (a mixed token-budget
 * step: the token-budget blog, sections 3 to 5; the zdszero notes, section
 * "mixed chunk").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All functions return EXTATTN_OK (0) or a negative status. On failure
 *    nothing has been enqueued, and extattn_last_error() returns a message
 *    (thread-local, valid until the next call on the same thread).
 *  - Pointers marked "device" must be device memory on the current HIP device;
 *    "host" pointers are read during the call only and may be reused after it
 *    returns. The library never allocates or frees device memory; the caller
 *    owns every buffer. Device work is enqueued on `stream` (a hipStream_t;
 *    NULL means the default stream) and the call returns without waiting;
 *    outputs are valid once the stream has reached that point. The library
 *    keeps pinned host staging buffers of its own for the small metadata it
 *    copies to the workspace (allocated on first use, reused afterwards).
 *  - Element types: EXTATTN_BF16 (bfloat16) or EXTATTN_F32 (float). q, the
 *    caches and out share one element type; lse is always float.
 *  - Heads: num_q_heads must be a multiple of num_kv_heads; query head h reads
 *    KV head h / (num_q_heads / num_kv_heads) (contiguous groups).
 *  - head_dim is 64 or 128; block_size is 16.
 *  - Paged cache layout, per physical block b and KV head g:
 *        k_cache[b][g][slot][d]   shape [num_blocks, Hkv, block_size, D]
 *        v_cache[b][g][d][slot]   shape [num_blocks, Hkv, D, block_size]
 *    Token at logical position p of request r lives in physical block
 *    block_table[r * max_blocks + p / block_size], slot p % block_size.
 *    V is stored slot-minor so that one block's values for one feature are
 *    contiguous over tokens, the order in which the P.V contraction reads them.
 *  - Request r's query rows are rows [q_off_r, q_off_r + E_r) of q and out,
 *    where q_off_r is the sum of extend_lens[0 .. r-1] (request order).
 */
#ifndef EXTATTN_H
#define EXTATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  EXTATTN_OK = 0,
  EXTATTN_EINVAL = -1,       /* invalid argument */
  EXTATTN_ENOSPC = -2,       /* workspace or output capacity too small */
  EXTATTN_EUNSUPPORTED = -3, /* valid but not implemented (head_dim, block_size, dtype) */
  EXTATTN_EHIP = -4          /* a HIP runtime call or launch failed */
};

enum { EXTATTN_BF16 = 0, EXTATTN_F32 = 1 };

/*
 * Chunk plan of one prompt (host only, pure, thread-safe).
 *
 * Sources: msmodeling chunked-prefill RFC, section 2.2 (cached prefix =
 * floor(n_tokens * hit_rate), chunking applies to the remaining effective
 * length) and section 3.1.3 (chunk plan); zdszero notes, section "prefill as
 * several resumable extends" (ceil(N/C) rounds, P_t = min(tC, N),
 * E_t = min(C, N - P_t)).
 *
 * The product n_tokens * hit_rate is one IEEE double multiply, then floor.
 * Prefixes are kernel-space: prefix_lens[t] = cached + min(t*C, effective),
 * extend_lens[t] = min(C, effective - min(t*C, effective)).
 *
 * Outputs: *cached, *effective, *n_chunks (always written on EXTATTN_OK and on
 * EXTATTN_ENOSPC), prefix_lens[0..n_chunks) and extend_lens[0..n_chunks)
 * (host arrays of `capacity` entries; may be NULL when capacity is 0).
 * Errors: EXTATTN_EINVAL if n_tokens < 1, chunk_size < 1, hit_rate is NaN or
 * outside [0, 1], or the effective length is below 1; EXTATTN_ENOSPC if
 * capacity < n_chunks (call with capacity 0 to size the arrays).
 */
int extattn_chunk_plan(int64_t n_tokens, int64_t chunk_size, double hit_rate,
                       int64_t* cached, int64_t* effective, int64_t* n_chunks,
                       int64_t* prefix_lens, int64_t* extend_lens, int64_t capacity);

/*
 * Workspace bytes that extattn_extend_attention needs for these requests
 * (host only). Arguments as for extattn_extend_attention. The result depends
 * only on the lengths, head counts, head_dim and dtype. Errors as for
 * extattn_extend_attention's argument checks.
 */
int extattn_workspace_bytes(int32_t num_seqs, const int32_t* prefix_lens, const int32_t* extend_lens,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t dtype, size_t* bytes);

/* Workspace bytes that extattn_kv_append needs for num_seqs requests (host only). */
size_t extattn_kv_append_workspace_bytes(int32_t num_seqs);

/*
 * Append each request's new tokens' K and V to the paged cache.
 *
 * The chunk's own keys and values are the "computed this round" part of the
 * extend equation (zdszero notes, section "prefill as several resumable
 * extends"); they go into the request's cache row, which persists across
 * chunks (same page, section on where the half-finished request's KV lives).
 *
 * k_new, v_new:  device [sum(E), Hkv, D], request order; token q_off_r + t of
 *                request r goes to logical position prefix_lens[r] + t.
 * k_cache, v_cache, block_table, max_blocks, num_blocks: the paged cache (see
 *                the layout above). Physical ids outside [0, num_blocks) are
 *                skipped (nothing written) and counted in the workspace's
 *                error word.
 * prefix_lens, extend_lens: host [num_seqs], prefix >= 0, extend >= 0.
 * workspace:     device, at least extattn_kv_append_workspace_bytes(num_seqs).
 * Errors: EXTATTN_EINVAL for null pointers, num_seqs < 1, negative lengths,
 * ceil((P_r + E_r) / block_size) > max_blocks, num_kv_heads < 1;
 * EXTATTN_EUNSUPPORTED for head_dim, block_size or dtype; EXTATTN_ENOSPC for a
 * small workspace; EXTATTN_EHIP on launch failure.
 */
int extattn_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                      const int32_t* block_table, int32_t max_blocks, int64_t num_blocks,
                      const int32_t* prefix_lens, const int32_t* extend_lens, int32_t num_seqs,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Extend attention for a batch of requests (chunk rows and decode rows mixed).
 *
 * For request r with prefix P = prefix_lens[r] and E = extend_lens[r], query
 * row q_off_r + i (global position P + i) and query head h:
 *   s_j   = scale * q . k_j        for keys j = 0 .. P+i of KV head h/(Hq/Hkv)
 *   out   = sum_j exp(s_j - m) v_j / sum_j exp(s_j - m),  m = max_j s_j
 *   lse   = m + ln sum_j exp(s_j - m)           (natural log, one per row and head)
 * (zdszero notes, section "prefill as several resumable extends": the o_i
 * equation, the stage 1 / stage 2 split and the log-sum-exp merge).
 * The K/V of all P+E positions must already be in the cache (the chunk's own
 * tokens appended with extattn_kv_append before this call).
 *
 * q:            device [sum(E), Hq, D]
 * k_cache, v_cache, block_table, max_blocks, num_blocks: the paged cache.
 *               Block ids outside [0, num_blocks) read as zeros and are counted
 *               in the workspace's error word.
 * prefix_lens, extend_lens: host [num_seqs]; prefix >= 0, extend >= 1.
 * scale:        finite and > 0 (the pages use 1/sqrt(D)).
 * out:          device [sum(E), Hq, D], element type of q.
 * lse:          device [sum(E), Hq] float, or NULL to skip.
 * workspace:    device, at least the extattn_workspace_bytes() result, 256-byte
 *               aligned; its first 4 bytes hold the error word after the call.
 * Accumulation is fp32 for both element types; bf16 scores' softmax weights
 * are rounded to bf16 before the P.V product.
 * Errors: EXTATTN_EINVAL for null required pointers, num_seqs < 1, any
 * extend < 1 or prefix < 0, Hq % Hkv != 0, a request needing more than
 * max_blocks blocks, a non-finite or non-positive scale, sum(E) above 2^31-1;
 * EXTATTN_EUNSUPPORTED for head_dim, block_size or dtype; EXTATTN_ENOSPC for a
 * small workspace; EXTATTN_EHIP on a HIP failure.
 */
int extattn_extend_attention(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_table, int32_t max_blocks, int64_t num_blocks,
                             const int32_t* prefix_lens, const int32_t* extend_lens, int32_t num_seqs,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, float scale, int32_t dtype,
                             void* out, float* lse, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Message for the last failing call on this thread ("" if none). */
const char* extattn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* EXTATTN_H */
