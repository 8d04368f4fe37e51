// Host-side mixed-step planning: which requests a forward serves and how many
// tokens each, returned as the (prefix, extend) pairs of one launch.
#include <cmath>
#include <cstdint>

#include "../../include/extattn.h"
#include "internal.hpp"

namespace extattn {

// Token-budget step (token-budget blog, sections 4 and 5): the running queue is
// served first, then the waiting queue, each request with min(still needed, budget
// left), until the budget is used up; a prompt longer than what is left is cut, and
// the cut is its chunk. Waiting requests start after their prefix-cache hits.
int token_budget_step_impl(int32_t n_running, const int64_t* running_total, const int64_t* running_computed,
                           int32_t n_waiting, const int64_t* waiting_total, const int64_t* waiting_cached,
                           int64_t budget, int32_t* out_index, int64_t* out_prefix, int64_t* out_extend,
                           int32_t capacity, int32_t* n_out, int64_t* budget_left, const char** why) {
  if (!n_out || !budget_left) { *why = "null output pointer"; return EXTATTN_EINVAL; }
  if (n_running < 0 || n_waiting < 0) { *why = "queue sizes must be >= 0"; return EXTATTN_EINVAL; }
  if (budget < 1) { *why = "token budget must be >= 1"; return EXTATTN_EINVAL; }
  if ((n_running > 0 && (!running_total || !running_computed)) ||
      (n_waiting > 0 && (!waiting_total || !waiting_cached))) {
    *why = "null queue array"; return EXTATTN_EINVAL;
  }
  for (int32_t i = 0; i < n_running; ++i)
    if (running_computed[i] < 0 || running_total[i] <= running_computed[i]) {
      *why = "a running request needs computed >= 0 and at least one token left"; return EXTATTN_EINVAL;
    }
  for (int32_t i = 0; i < n_waiting; ++i)
    if (waiting_cached[i] < 0 || waiting_total[i] <= waiting_cached[i]) {
      *why = "a waiting request needs cached >= 0 and at least one token left"; return EXTATTN_EINVAL;
    }
  // entries this step: walk the queues once to count, then fill
  int64_t left = budget;
  int32_t count = 0;
  for (int32_t k = 0; k < n_running + n_waiting && left > 0; ++k) {
    const bool run = k < n_running;
    const int64_t need = run ? running_total[k] - running_computed[k]
                             : waiting_total[k - n_running] - waiting_cached[k - n_running];
    left -= need < left ? need : left;
    ++count;
  }
  *n_out = count;
  *budget_left = left;
  if (capacity < count) { *why = "capacity is smaller than the number of scheduled requests"; return EXTATTN_ENOSPC; }
  if (count > 0 && (!out_index || !out_prefix || !out_extend)) { *why = "null output array"; return EXTATTN_EINVAL; }
  left = budget;
  for (int32_t k = 0; k < count; ++k) {
    const bool run = k < n_running;
    const int64_t base = run ? running_computed[k] : waiting_cached[k - n_running];
    const int64_t need = (run ? running_total[k] : waiting_total[k - n_running]) - base;
    const int64_t take = need < left ? need : left;
    out_index[k] = k;
    out_prefix[k] = base;
    out_extend[k] = take;
    left -= take;
  }
  return EXTATTN_OK;
}

// Mixed-chunk step (zdszero notes: "only one half-finished request", "four things
// per round", "mixed chunk", "page alignment only at the first cut"). With mixed
// chunks every decode row takes one token and the running batch is taken out of the
// chunk budget first; the half-finished request continues before anything new (its
// continuation is not page-aligned); waiting requests then fill what is left in
// queue order, and the first one that does not fit is cut with its end aligned down
// to a whole page and becomes the next half-finished request (a cut that would be
// empty after alignment admits nothing this round).
int mixed_chunk_step_impl(int32_t n_decode, const int64_t* decode_prefix, int64_t chunked_total,
                          int64_t chunked_done, int32_t n_waiting, const int64_t* waiting_total,
                          const int64_t* waiting_cached, int64_t chunk_size, int64_t page_size, int32_t mixed,
                          int32_t* out_kind, int32_t* out_index, int64_t* out_prefix, int64_t* out_extend,
                          int32_t capacity, int32_t* n_out, int64_t* chunk_left, int32_t* next_kind,
                          int32_t* next_index, int64_t* next_done, const char** why) {
  if (!n_out || !chunk_left || !next_kind || !next_index || !next_done) {
    *why = "null output pointer"; return EXTATTN_EINVAL;
  }
  if (n_decode < 0 || n_waiting < 0) { *why = "queue sizes must be >= 0"; return EXTATTN_EINVAL; }
  if (chunk_size < 1 || page_size < 1) { *why = "chunk size and page size must be >= 1"; return EXTATTN_EINVAL; }
  if ((mixed && n_decode > 0 && !decode_prefix) || (n_waiting > 0 && (!waiting_total || !waiting_cached))) {
    *why = "null queue array"; return EXTATTN_EINVAL;
  }
  const bool has_chunked = chunked_total > 0;
  if (has_chunked && (chunked_done < 0 || chunked_done >= chunked_total)) {
    *why = "the half-finished request needs 0 <= done < total"; return EXTATTN_EINVAL;
  }
  if (mixed)
    for (int32_t i = 0; i < n_decode; ++i)
      if (decode_prefix[i] < 0) { *why = "decode prefixes must be >= 0"; return EXTATTN_EINVAL; }
  for (int32_t i = 0; i < n_waiting; ++i)
    if (waiting_cached[i] < 0 || waiting_total[i] <= waiting_cached[i]) {
      *why = "a waiting request needs cached >= 0 and at least one token left"; return EXTATTN_EINVAL;
    }
  // Two passes: the first only counts (and finds the next half-finished request),
  // the second writes the entries.
  for (int pass = 0; pass < 2; ++pass) {
    const bool write = pass == 1;
    int32_t k = 0;
    int64_t left = chunk_size;
    int32_t nk = -1, ni = 0;
    int64_t nd = 0;
    auto put = [&](int32_t kind, int32_t idx, int64_t prefix, int64_t extend) {
      if (write) {
        out_kind[k] = kind;
        out_index[k] = idx;
        out_prefix[k] = prefix;
        out_extend[k] = extend;
      }
      ++k;
    };
    if (mixed) {
      for (int32_t i = 0; i < n_decode; ++i) put(EXTATTN_ENTRY_DECODE, i, decode_prefix[i], 1);
      left = chunk_size > n_decode ? chunk_size - n_decode : 0;
    }
    bool stop = false;
    if (has_chunked) {
      const int64_t rem = chunked_total - chunked_done;
      const int64_t take = rem < left ? rem : left;
      if (take > 0) {
        put(EXTATTN_ENTRY_CHUNKED, 0, chunked_done, take);
        left -= take;
      }
      if (chunked_done + take < chunked_total) {
        nk = EXTATTN_ENTRY_CHUNKED;
        ni = 0;
        nd = chunked_done + take;
        stop = true;
      }
    }
    for (int32_t i = 0; i < n_waiting && !stop && left > 0; ++i) {
      const int64_t need = waiting_total[i] - waiting_cached[i];
      if (need <= left) {
        put(EXTATTN_ENTRY_WAITING, i, waiting_cached[i], need);
        left -= need;
        continue;
      }
      const int64_t end = (waiting_cached[i] + left) / page_size * page_size;
      const int64_t take = end - waiting_cached[i];
      if (take > 0) {
        put(EXTATTN_ENTRY_WAITING, i, waiting_cached[i], take);
        left -= take;
        nk = EXTATTN_ENTRY_WAITING;
        ni = i;
        nd = waiting_cached[i] + take;
      }
      stop = true;
    }
    if (!write) {
      *n_out = k;
      *chunk_left = left;
      *next_kind = nk;
      *next_index = ni;
      *next_done = nd;
      if (capacity < k) { *why = "capacity is smaller than the number of entries"; return EXTATTN_ENOSPC; }
      if (k > 0 && (!out_kind || !out_index || !out_prefix || !out_extend)) {
        *why = "null output array"; return EXTATTN_EINVAL;
      }
    }
  }
  return EXTATTN_OK;
}

// Default mixed-step scheduler of the msmodeling chunked-prefill RFC (section 3.1.4):
// all ready decode rows up to the budget, then as many whole prefill chunks as fit
// under floor(budget * 1.15) -- one IEEE double multiply, then floor.
int decode_first_with_slack_impl(int64_t ready_decode, int64_t pending_prefill, int64_t chunk_query_len,
                                 int64_t max_batched_tokens, int64_t* p_step, int64_t* d_step, int64_t* limit,
                                 const char** why) {
  if (!p_step || !d_step || !limit) { *why = "null output pointer"; return EXTATTN_EINVAL; }
  if (ready_decode < 0 || pending_prefill < 0) { *why = "queue sizes must be >= 0"; return EXTATTN_EINVAL; }
  if (chunk_query_len < 1) { *why = "chunk_query_len must be >= 1"; return EXTATTN_EINVAL; }
  if (max_batched_tokens < 1) { *why = "max_batched_tokens must be >= 1"; return EXTATTN_EINVAL; }
  volatile double product = static_cast<double>(max_batched_tokens) * 1.15;  // one multiply, no fusion
  const int64_t lim = static_cast<int64_t>(std::floor(product));
  const int64_t d = ready_decode < max_batched_tokens ? ready_decode : max_batched_tokens;
  const int64_t room = lim - d;
  int64_t p = room > 0 ? room / chunk_query_len : 0;
  if (p > pending_prefill) p = pending_prefill;
  *p_step = p;
  *d_step = d;
  *limit = lim;
  return EXTATTN_OK;
}

}  // namespace extattn
