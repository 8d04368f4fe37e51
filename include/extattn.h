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
 *    keeps a pool of pinned host staging buffers per device (coherent and
 *    mapped into the device) for the small metadata that a copy kernel on
 *    `stream` moves into the workspace (a buffer is reused once the copy
 *    that last read it has completed; the pool grows instead of waiting, up to
 *    512 buffers in flight per device, beyond which a call waits on the host
 *    for the oldest copy to finish), and a bounded host table of launch plans
 *    keyed by the launch's shape (see extattn_plan_cache_configure).
 *  - Status words. Invalid input that only the GPU can see (a block id outside
 *    [0, num_blocks) in a row the launch reads) and a fused-append wait that
 *    gave up are not silent: each call that takes a workspace clears the first
 *    12 bytes of it (before its kernels run, in stream order) and its kernels
 *    record such events there; extattn_read_status returns them. Results of a
 *    call whose flags are not zero are not valid.
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

/* Status flags (see extattn_read_status). */
enum {
  EXTATTN_STATUS_BAD_BLOCK = 1,   /* a block id outside [0, num_blocks) was read */
  EXTATTN_STATUS_WAIT_TIMEOUT = 2 /* a fused-append wait gave up; results are not valid */
};

/* Entry kinds of extattn_mixed_chunk_step. */
enum { EXTATTN_ENTRY_DECODE = 0, EXTATTN_ENTRY_CHUNKED = 1, EXTATTN_ENTRY_WAITING = 2 };

/*
 * One mixed step under a token budget (host only, pure, thread-safe).
 *
 * Source: token-budget blog ("2.4 Chunked Prefill and the unified token
 * budget"), section 4 (a step is one map {request: tokens} whose sum is bounded
 * by the budget) and section 5 (the budget cuts chunks): running requests are
 * served first, in order, each with min(tokens still needed, budget left); then
 * waiting requests in queue order the same way, starting after their prefix-cache
 * hits, until the budget is used up. KV-cache allocation and preemption are not
 * modelled (every allocation succeeds).
 *
 * Running request i still needs running_total[i] - running_computed[i] >= 1
 * tokens (1 for a decode row); waiting request i needs waiting_total[i] -
 * waiting_cached[i] >= 1. Outputs (host arrays of `capacity` entries, scheduling
 * order): out_index (i for running i, n_running + i for waiting i), out_prefix
 * (tokens already in the cache: the launch's prefix_lens), out_extend (tokens this
 * step: the launch's extend_lens); *n_out entries and *budget_left are written on
 * EXTATTN_OK and EXTATTN_ENOSPC.
 * Errors: EXTATTN_EINVAL for budget < 1, negative queue sizes, null arrays, a
 * request with nothing left to compute; EXTATTN_ENOSPC if capacity < *n_out.
 */
int extattn_token_budget_step(int32_t n_running, const int64_t* running_total, const int64_t* running_computed,
                              int32_t n_waiting, const int64_t* waiting_total, const int64_t* waiting_cached,
                              int64_t budget, int32_t* out_index, int64_t* out_prefix, int64_t* out_extend,
                              int32_t capacity, int32_t* n_out, int64_t* budget_left);

/*
 * One round of the mixed-chunk scheduler (host only, pure, thread-safe).
 *
 * Source: zdszero notes, sections "only one half-finished request", "four things
 * per round", "mixed chunk" and "page alignment only at the first cut". With
 * `mixed` set, every decode row takes one token (prefix decode_prefix[i],
 * extend 1) and the running batch is taken out of the chunk budget first, so a
 * slice is chunk_size - n_decode. The half-finished request (chunked_total > 0,
 * chunked_done tokens done) continues first, without page alignment; waiting
 * requests then fill what is left in queue order, and the first one that does not
 * fit is cut with its end aligned down to a multiple of page_size and becomes the
 * next half-finished request (if alignment leaves nothing it waits).
 *
 * Outputs (host arrays of `capacity` entries): out_kind (EXTATTN_ENTRY_*),
 * out_index (decode row, 0 for the half-finished request, waiting index),
 * out_prefix, out_extend; *n_out, *chunk_left (budget not used) and the next
 * half-finished request (*next_kind = -1 if none, else its kind, *next_index and
 * *next_done = tokens done after this round) are written on EXTATTN_OK and
 * EXTATTN_ENOSPC.
 * Errors: EXTATTN_EINVAL for chunk_size or page_size < 1, negative sizes, null
 * arrays, 0 <= chunked_done < chunked_total violated, a waiting request with
 * nothing left; EXTATTN_ENOSPC if capacity < *n_out.
 */
int extattn_mixed_chunk_step(int32_t n_decode, const int64_t* decode_prefix, int64_t chunked_total,
                             int64_t chunked_done, int32_t n_waiting, const int64_t* waiting_total,
                             const int64_t* waiting_cached, int64_t chunk_size, int64_t page_size, int32_t mixed,
                             int32_t* out_kind, int32_t* out_index, int64_t* out_prefix, int64_t* out_extend,
                             int32_t capacity, int32_t* n_out, int64_t* chunk_left, int32_t* next_kind,
                             int32_t* next_index, int64_t* next_done);

/*
 * Default mixed-step scheduler of the msmodeling chunked-prefill RFC, section
 * 3.1.4 (host only, pure): d_step = min(ready_decode, max_batched_tokens),
 * limit = floor(max_batched_tokens * 1.15) as one IEEE double multiply (so a
 * budget of 100 gives 114), p_step = max(0, min(pending_prefill,
 * floor((limit - d_step) / chunk_query_len))).
 * Errors: EXTATTN_EINVAL for negative counts, chunk_query_len < 1,
 * max_batched_tokens < 1 or null outputs.
 */
int extattn_decode_first_with_slack(int64_t ready_decode, int64_t pending_prefill, int64_t chunk_query_len,
                                    int64_t max_batched_tokens, int64_t* p_step, int64_t* d_step, int64_t* limit);

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
 * extattn_extend_attention's argument checks, and EXTATTN_ENOSPC when the
 * launch's partial results would exceed 2^31 - 1 floats.
 */
int extattn_workspace_bytes(int32_t num_seqs, const int32_t* prefix_lens, const int32_t* extend_lens,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t dtype, size_t* bytes);

/*
 * Launch-plan cache (host only, thread-safe).
 *
 * The latency-table RFC (sections 3.1.3 and 3.1.4) keys the cost of one
 * forward by its dynamic shape and fills a table once per distinct shape. The
 * same idea here keys a launch's configuration: the work list, the combine
 * tasks, the workspace layout and the metadata image uploaded to the workspace
 * depend only on (dtype, num_q_heads, num_kv_heads, head_dim, and each
 * request's (prefix_len, extend_len) in order). extattn_workspace_bytes,
 * extattn_extend_attention, extattn_extend_attention_append and
 * extattn_extend_attention_timed look the shape up and build the plan only on
 * a miss; one record serves the plain and the fused-append call of a shape, so
 * sizing the workspace and then launching plans once. Results never depend on
 * whether a plan came from the table.
 *
 * extattn_plan_cache_configure: keep at most max_entries records using at most
 *   max_bytes of host memory, least recently used first out (defaults 256
 *   records, 64 MiB); max_entries = 0 turns the table off (every call plans).
 *   Shrinking evicts at once. Errors: EXTATTN_EINVAL for negative bounds.
 * extattn_plan_cache_stats: lookups that hit / missed since the last clear,
 *   records held and their host bytes. Errors: EXTATTN_EINVAL for a null
 *   output pointer.
 * extattn_plan_cache_clear: drop every record and zero the counters (the
 *   bounds stay). Records in use by a concurrent call stay valid for it.
 */
int extattn_plan_cache_configure(int32_t max_entries, int64_t max_bytes);
int extattn_plan_cache_stats(int64_t* hits, int64_t* misses, int32_t* entries, int64_t* bytes);
int extattn_plan_cache_clear(void);

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
 *                skipped (nothing written) and reported in the workspace's
 *                status words (EXTATTN_STATUS_BAD_BLOCK).
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
 *               Block ids outside [0, num_blocks) read as zeros and are
 *               reported in the workspace's status words
 *               (EXTATTN_STATUS_BAD_BLOCK; the results are then not valid).
 * prefix_lens, extend_lens: host [num_seqs]; prefix >= 0, extend >= 1.
 * scale:        finite and > 0 (the pages use 1/sqrt(D)).
 * out:          device [sum(E), Hq, D], element type of q.
 * lse:          device [sum(E), Hq] float, or NULL to skip.
 * workspace:    device, at least the extattn_workspace_bytes() result, 256-byte
 *               aligned; its first 8 bytes hold the status words after the call
 *               (extattn_read_status).
 * Accumulation is fp32 for both element types. The scores are the fp32 dot
 * products of the given q and k; the scale is applied to them in fp32 inside the
 * exponent. For bf16 the softmax weights are rounded to bf16 for the P.V product
 * only; lse and the normaliser sum the fp32 weights.
 * Errors: EXTATTN_EINVAL for null required pointers, num_seqs < 1, any
 * extend < 1 or prefix < 0, Hq % Hkv != 0, a request needing more than
 * max_blocks blocks, a non-finite or non-positive scale, sum(E) above 2^31-1;
 * EXTATTN_EUNSUPPORTED for head_dim, block_size or dtype; EXTATTN_ENOSPC for a
 * small workspace or a launch whose partial results exceed 2^31 - 1 floats;
 * EXTATTN_EHIP on a HIP failure.
 */
int extattn_extend_attention(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_table, int32_t max_blocks, int64_t num_blocks,
                             const int32_t* prefix_lens, const int32_t* extend_lens, int32_t num_seqs,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, float scale, int32_t dtype,
                             void* out, float* lse, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * KV append fused into the extend launch: the same result as
 * extattn_kv_append(k_new, v_new, ...) followed by extattn_extend_attention(...)
 * on the same requests, in one attention launch. The chunk's own keys and
 * values are the part of the extend equation computed in this round (zdszero
 * notes, section "prefill as several resumable extends"); here the launch's
 * first workgroups write them into the paged cache and the attention
 * workgroups that reach a request's new keys wait until those writes are done
 * (a device-scope counter in the workspace, release / acquire; the wait is
 * bounded: if it gives up, EXTATTN_STATUS_WAIT_TIMEOUT is set in the status
 * words and the results are not valid). Prefix keys need no wait.
 *
 * k_new, v_new: device [sum(E), Hkv, D], element type of q, request order;
 *               token q_off_r + t of request r goes to position prefix_lens[r] + t.
 * k_cache, v_cache: written (the new tokens' slots) and read.
 * Other arguments, ownership and errors as for extattn_extend_attention; the
 * workspace size is the same extattn_workspace_bytes() result. Block ids
 * outside [0, num_blocks) are skipped for writing, read as zeros and reported
 * (EXTATTN_STATUS_BAD_BLOCK). fp32 runs the append as its own launch first on
 * the same stream.
 */
int extattn_extend_attention_append(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                    void* v_cache, const int32_t* block_table, int32_t max_blocks,
                                    int64_t num_blocks, const int32_t* prefix_lens, const int32_t* extend_lens,
                                    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, float scale, int32_t dtype, void* out, float* lse,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Measurement variant of extattn_extend_attention: the same work and the same
 * results, and each workgroup of the bf16 attention kernel (one work item: a
 * chunk tile, a piece of one, or a piece of a decode / verify request's key
 * range) also records when it started and ended. This gives the span of the
 * decode rows inside a mixed launch (the mixed chunk-and-decode step of the
 * token-budget blog, section 5) next to the chunk rows' span.
 *
 * Arguments as for extattn_extend_attention, plus:
 * stamps:   device int64 [capacity][6]; item i writes {start, end, kind,
 *           request, clk_start, clk_end}: start / end in ticks of the device's
 *           constant-rate wall clock, kind 0 for chunk rows and 1 for decode /
 *           verify rows, request the index into prefix_lens, clk_start / clk_end
 *           the shader-clock cycle counter of the workgroup's CU at the same two
 *           points (so that cycles / ticks * tick_hz is the clock the kernel ran
 *           at). Items are in launch order. The combine kernel that follows split
 *           items is not recorded.
 * capacity: number of 6-entry records stamps can hold; 0 (stamps NULL) asks
 *           only for n_items and returns EXTATTN_ENOSPC without enqueuing work.
 * n_items:  host out: the launch's number of work items.
 * tick_hz:  host out: wall-clock ticks per second of the current device.
 * Errors: those of extattn_extend_attention; EXTATTN_ENOSPC when capacity <
 * n_items; EXTATTN_EUNSUPPORTED for fp32 (its kernel records nothing).
 */
int extattn_extend_attention_timed(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* block_table, int32_t max_blocks, int64_t num_blocks,
                                   const int32_t* prefix_lens, const int32_t* extend_lens, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, float scale, int32_t dtype,
                                   void* out, float* lse, void* workspace, size_t workspace_bytes,
                                   void* stream, int64_t* stamps, int32_t capacity, int32_t* n_items,
                                   double* tick_hz);

/*
 * Extend attention that allocates nothing, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation). The same computation, kernels and results as
 * extattn_extend_attention; the workspace is a static device scratch of 64 MiB
 * inside the library (each GPU the library runs on holds one until the process
 * ends), and the call's metadata reaches it through kernel arguments, so no
 * pinned staging is used either.
 *
 * Arguments, ownership and errors as for extattn_extend_attention, without
 * workspace / workspace_bytes; EXTATTN_ENOSPC when the launch needs more than the
 * 64 MiB scratch (extattn_workspace_bytes gives the need; partial results of
 * key-range pieces are the bulk of it).
 * All calls on one GPU share its scratch, which keeps the last call's contents:
 * calls that overlap on one GPU (several streams or threads) race and must be
 * serialised by the caller. The status words of the last call on the current
 * device are read with extattn_read_status(NULL, ...).
 */
int extattn_extend_attention_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* block_table, int32_t max_blocks, int64_t num_blocks,
                                     const int32_t* prefix_lens, const int32_t* extend_lens, int32_t num_seqs,
                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t block_size, float scale, int32_t dtype, void* out, float* lse,
                                     void* stream);

/*
 * Status of the last call that used `workspace` (any call taking a workspace:
 * extattn_kv_append, extattn_extend_attention and its _append / _timed
 * variants). The msmodeling chunked-prefill RFC, section 2.4 (reliability:
 * invalid input is reported at the entry with a clear error, never swallowed),
 * asks for this for the checks that only the GPU can make.
 *
 * workspace NULL reads the scratch of extattn_extend_attention_noalloc on the
 * current device.
 * Enqueues a copy of the workspace's status words on `stream`, then waits
 * on the host until the stream has completed it (hipStreamSynchronize): call
 * it where a host wait is acceptable (tests, a periodic health check, after a
 * fused-append call whose results matter).
 * flags:            host out, EXTATTN_STATUS_* bits (0: nothing to report).
 * bad_block_reads:  host out, number of invalid block-id reads recorded (each
 *                   workgroup that meets one counts it; wraps past 2^31 - 1).
 * exact_waves:      host out, number of waves of chunk rows that redid their
 *                   rows on the exact two-pass path because a tile's weights grew
 *                   past 2^64 against the first tile's row max (scores rising by
 *                   more than 64 in log2 units along the keys). Informational:
 *                   the results are valid; the count shows where time went.
 * Errors: EXTATTN_EINVAL for null output pointers or a workspace not 256-byte
 * aligned; EXTATTN_EHIP if the copy or the wait fails.
 */
int extattn_read_status(const void* workspace, uint32_t* flags, int32_t* bad_block_reads, int32_t* exact_waves,
                        void* stream);

/* Message for the last failing call on this thread ("" if none). */
const char* extattn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* EXTATTN_H */
