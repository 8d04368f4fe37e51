// The C ABI: argument checks, metadata upload, kernel launches.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <deque>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/extattn.h"
#include "internal.hpp"

namespace extattn {
int chunk_plan_impl(int64_t n_tokens, int64_t chunk_size, double hit_rate, int64_t* cached,
                    int64_t* effective, int64_t* n_chunks, int64_t* prefix_lens, int64_t* extend_lens,
                    int64_t capacity, const char** why);
}

using namespace extattn;

namespace {

thread_local std::string g_error;

int fail(int code, const std::string& msg) {
  g_error = msg;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  char buf[256];
  std::snprintf(buf, sizeof(buf), "%s: %s", what, hipGetErrorString(e));
  g_error = buf;
  return EXTATTN_EHIP;
}

// Pinned host staging for the metadata copied into the caller's workspace.
// Each device has a pool of pinned, coherent, device-mapped buffers; a copy kernel
// on the caller's stream reads a buffer over the host link (a DMA-engine copy would
// make the next kernel wait for a cross-engine signal). A buffer is reused only
// after the copy that last read it has completed (an event per buffer). A call
// takes a free buffer, or adds one to the pool, so it does not wait for the GPU;
// only when kMaxStaging buffers are in flight on the device does it wait (on the
// host, outside the pool's lock) for the oldest of them.
struct StagingSlot {
  void* host = nullptr;
  void* dev = nullptr;  // the same buffer's device address
  size_t cap = 0;
  hipEvent_t done = nullptr;
};

constexpr int kMaxStaging = 512;
constexpr size_t kStagingMinBytes = size_t(32) << 10;
constexpr int kMaxDevices = 64;

struct DeviceStaging {
  std::mutex mu;
  std::vector<StagingSlot*> free_slots;
  std::deque<StagingSlot*> in_flight;  // oldest first
  int total = 0;
};

DeviceStaging g_staging[kMaxDevices];

int upload(const void* src, size_t bytes, void* dst, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(EXTATTN_EHIP, "device index out of range");
  DeviceStaging& ds = g_staging[dev];
  StagingSlot* s = nullptr;
  bool must_wait = false;
  {
    std::lock_guard<std::mutex> lock(ds.mu);
    // buffers whose copies have completed go back to the free list
    for (auto it = ds.in_flight.begin(); it != ds.in_flight.end();) {
      if (hipEventQuery((*it)->done) == hipSuccess) {
        ds.free_slots.push_back(*it);
        it = ds.in_flight.erase(it);
      } else {
        ++it;
      }
    }
    if (!ds.free_slots.empty()) {
      s = ds.free_slots.back();
      ds.free_slots.pop_back();
    } else if (ds.total < kMaxStaging) {
      s = new StagingSlot();
      ++ds.total;
    } else {
      s = ds.in_flight.front();
      ds.in_flight.pop_front();
      must_wait = true;
    }
  }
  // from here on the buffer belongs to this call alone; on failure it goes back
  auto give_back = [&](int rc) {
    std::lock_guard<std::mutex> lock(ds.mu);
    ds.free_slots.push_back(s);
    return rc;
  };
  if (must_wait) {
    e = hipEventSynchronize(s->done);
    if (e != hipSuccess) return give_back(hip_fail(e, "hipEventSynchronize (staging)"));
  }
  if (!s->done) {
    e = hipEventCreateWithFlags(&s->done, hipEventDisableTiming);
    if (e != hipSuccess) {
      s->done = nullptr;
      return give_back(hip_fail(e, "hipEventCreate (staging)"));
    }
  }
  if (s->cap < bytes) {
    if (s->host) (void)hipHostFree(s->host);
    s->host = nullptr;
    s->dev = nullptr;
    s->cap = 0;
    size_t cap = kStagingMinBytes;
    while (cap < bytes) cap *= 2;
    e = hipHostMalloc(&s->host, cap, hipHostMallocMapped | hipHostMallocCoherent);
    if (e != hipSuccess) {
      s->host = nullptr;
      return give_back(hip_fail(e, "hipHostMalloc (staging)"));
    }
    e = hipHostGetDevicePointer(&s->dev, s->host, 0);
    if (e != hipSuccess || !s->dev) {
      (void)hipHostFree(s->host);
      s->host = nullptr;
      s->dev = nullptr;
      return give_back(hip_fail(e != hipSuccess ? e : hipErrorInvalidValue, "hipHostGetDevicePointer (staging)"));
    }
    s->cap = cap;
  }
  std::memcpy(s->host, src, bytes);
  e = launch_meta_copy(s->dev, dst, bytes, stream);
  if (e != hipSuccess) return give_back(hip_fail(e, "metadata copy launch"));
  e = hipEventRecord(s->done, stream);
  if (e != hipSuccess) {
    // the copy may still read the buffer: keep it out of the pool
    return hip_fail(e, "hipEventRecord (staging)");
  }
  std::lock_guard<std::mutex> lock(ds.mu);
  ds.in_flight.push_back(s);
  return EXTATTN_OK;
}

int check_common(int32_t num_seqs, const int32_t* prefix, const int32_t* extend, int32_t hq, int32_t hkv,
                 int32_t head_dim, int32_t dtype, bool extend_min_one) {
  if (num_seqs < 1) return fail(EXTATTN_EINVAL, "num_seqs must be >= 1");
  if (!prefix || !extend) return fail(EXTATTN_EINVAL, "prefix_lens and extend_lens must be host arrays");
  if (hkv < 1 || hq < 1) return fail(EXTATTN_EINVAL, "head counts must be >= 1");
  if (hq % hkv != 0) return fail(EXTATTN_EINVAL, "num_q_heads must be a multiple of num_kv_heads");
  if (head_dim != 64 && head_dim != 128) return fail(EXTATTN_EUNSUPPORTED, "head_dim must be 64 or 128");
  if (dtype != EXTATTN_BF16 && dtype != EXTATTN_F32) return fail(EXTATTN_EUNSUPPORTED, "unknown dtype");
  int64_t total = 0;
  for (int32_t r = 0; r < num_seqs; ++r) {
    if (prefix[r] < 0) return fail(EXTATTN_EINVAL, "prefix_lens[" + std::to_string(r) + "] < 0");
    if (extend[r] < (extend_min_one ? 1 : 0))
      return fail(EXTATTN_EINVAL, "extend_lens[" + std::to_string(r) + "] out of range");
    if (int64_t(prefix[r]) + extend[r] > INT32_MAX)
      return fail(EXTATTN_EINVAL, "prefix + extend exceeds 2^31-1");
    total += extend[r];
  }
  if (total > INT32_MAX) return fail(EXTATTN_EINVAL, "sum of extend_lens exceeds 2^31-1");
  return EXTATTN_OK;
}

int check_blocks(int32_t num_seqs, const int32_t* prefix, const int32_t* extend, int32_t max_blocks,
                 int64_t num_blocks, int32_t block_size) {
  if (block_size != kBlockSize) return fail(EXTATTN_EUNSUPPORTED, "block_size must be 16");
  if (max_blocks < 1) return fail(EXTATTN_EINVAL, "max_blocks must be >= 1");
  if (num_blocks < 1) return fail(EXTATTN_EINVAL, "num_blocks must be >= 1");
  for (int32_t r = 0; r < num_seqs; ++r) {
    const int64_t need = (int64_t(prefix[r]) + extend[r] + kBlockSize - 1) / kBlockSize;
    if (need > max_blocks)
      return fail(EXTATTN_EINVAL, "request " + std::to_string(r) + " needs more than max_blocks blocks");
  }
  return EXTATTN_OK;
}

}  // namespace

namespace extattn {
int set_error(int code, const char* msg) { return fail(code, msg); }
int set_hip_error(hipError_t e, const char* what) { return hip_fail(e, what); }
}  // namespace extattn

extern "C" {

const char* extattn_last_error(void) { return g_error.c_str(); }

int extattn_read_status(const void* workspace, uint32_t* flags, int32_t* bad_block_reads, int32_t* exact_waves,
                        void* stream) {
  if (!flags || !bad_block_reads || !exact_waves) return fail(EXTATTN_EINVAL, "null pointer");
  if (!workspace) {  // the allocation-free entry point's scratch on the current device
    void* p = nullptr;
    const int rc = noalloc_scratch(&p);
    if (rc != EXTATTN_OK) return rc;
    workspace = p;
  }
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return fail(EXTATTN_EINVAL, "workspace must be 256-byte aligned");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  int32_t words[3] = {0, 0, 0};
  hipError_t e = hipMemcpyAsync(words, workspace, sizeof(words), hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (status)");
  e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize (status)");
  *flags = uint32_t(words[0]);
  *bad_block_reads = words[1];
  *exact_waves = words[2];
  g_error.clear();
  return EXTATTN_OK;
}

int extattn_token_budget_step(int32_t n_running, const int64_t* running_total, const int64_t* running_computed,
                              int32_t n_waiting, const int64_t* waiting_total, const int64_t* waiting_cached,
                              int64_t budget, int32_t* out_index, int64_t* out_prefix, int64_t* out_extend,
                              int32_t capacity, int32_t* n_out, int64_t* budget_left) {
  const char* why = "";
  const int rc = extattn::token_budget_step_impl(n_running, running_total, running_computed, n_waiting, waiting_total,
                                                 waiting_cached, budget, out_index, out_prefix, out_extend, capacity,
                                                 n_out, budget_left, &why);
  if (rc != EXTATTN_OK) return fail(rc, why);
  g_error.clear();
  return EXTATTN_OK;
}

int extattn_mixed_chunk_step(int32_t n_decode, const int64_t* decode_prefix, int64_t chunked_total,
                             int64_t chunked_done, int32_t n_waiting, const int64_t* waiting_total,
                             const int64_t* waiting_cached, int64_t chunk_size, int64_t page_size, int32_t mixed,
                             int32_t* out_kind, int32_t* out_index, int64_t* out_prefix, int64_t* out_extend,
                             int32_t capacity, int32_t* n_out, int64_t* chunk_left, int32_t* next_kind,
                             int32_t* next_index, int64_t* next_done) {
  const char* why = "";
  const int rc = extattn::mixed_chunk_step_impl(n_decode, decode_prefix, chunked_total, chunked_done, n_waiting,
                                                waiting_total, waiting_cached, chunk_size, page_size, mixed, out_kind,
                                                out_index, out_prefix, out_extend, capacity, n_out, chunk_left,
                                                next_kind, next_index, next_done, &why);
  if (rc != EXTATTN_OK) return fail(rc, why);
  g_error.clear();
  return EXTATTN_OK;
}

int extattn_decode_first_with_slack(int64_t ready_decode, int64_t pending_prefill, int64_t chunk_query_len,
                                    int64_t max_batched_tokens, int64_t* p_step, int64_t* d_step, int64_t* limit) {
  const char* why = "";
  const int rc = extattn::decode_first_with_slack_impl(ready_decode, pending_prefill, chunk_query_len,
                                                       max_batched_tokens, p_step, d_step, limit, &why);
  if (rc != EXTATTN_OK) return fail(rc, why);
  g_error.clear();
  return EXTATTN_OK;
}

int extattn_chunk_plan(int64_t n_tokens, int64_t chunk_size, double hit_rate, int64_t* cached,
                       int64_t* effective, int64_t* n_chunks, int64_t* prefix_lens, int64_t* extend_lens,
                       int64_t capacity) {
  const char* why = "";
  const int rc = chunk_plan_impl(n_tokens, chunk_size, hit_rate, cached, effective, n_chunks, prefix_lens,
                                 extend_lens, capacity, &why);
  if (rc != EXTATTN_OK) return fail(rc, why);
  g_error.clear();
  return EXTATTN_OK;
}

int extattn_workspace_bytes(int32_t num_seqs, const int32_t* prefix_lens, const int32_t* extend_lens,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                            size_t* bytes) {
  if (!bytes) return fail(EXTATTN_EINVAL, "bytes must not be null");
  int rc = check_common(num_seqs, prefix_lens, extend_lens, num_q_heads, num_kv_heads, head_dim, dtype, true);
  if (rc != EXTATTN_OK) return rc;
  // the launch plan holds the fused append's items too, so one size serves both calls;
  // it is kept in the plan cache for the attention call that follows
  std::shared_ptr<const LaunchPlan> lp;
  rc = get_launch_plan(num_seqs, prefix_lens, extend_lens, num_q_heads, num_kv_heads, head_dim, dtype, lp);
  if (rc != EXTATTN_OK)
    return fail(rc, rc == EXTATTN_ENOSPC ? "launch too large: partial results exceed 2^31 floats" : "planning failed");
  *bytes = lp->plan.bytes;
  g_error.clear();
  return EXTATTN_OK;
}

int extattn_plan_cache_configure(int32_t max_entries, int64_t max_bytes) {
  if (max_entries < 0 || max_bytes < 0) return fail(EXTATTN_EINVAL, "plan cache bounds must be >= 0");
  plan_cache_configure(max_entries, max_bytes);
  g_error.clear();
  return EXTATTN_OK;
}

int extattn_plan_cache_stats(int64_t* hits, int64_t* misses, int32_t* entries, int64_t* bytes) {
  if (!hits || !misses || !entries || !bytes) return fail(EXTATTN_EINVAL, "null output pointer");
  plan_cache_stats(hits, misses, entries, bytes);
  g_error.clear();
  return EXTATTN_OK;
}

int extattn_plan_cache_clear(void) {
  plan_cache_clear();
  g_error.clear();
  return EXTATTN_OK;
}

size_t extattn_kv_append_workspace_bytes(int32_t num_seqs) {
  if (num_seqs < 0) num_seqs = 0;
  return kHeaderBytes + sizeof(SeqInfo) * size_t(num_seqs);
}

int extattn_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                      const int32_t* block_table, int32_t max_blocks, int64_t num_blocks,
                      const int32_t* prefix_lens, const int32_t* extend_lens, int32_t num_seqs,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t dtype,
                      void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_common(num_seqs, prefix_lens, extend_lens, num_kv_heads, num_kv_heads, head_dim, dtype, false);
  if (rc != EXTATTN_OK) return rc;
  rc = check_blocks(num_seqs, prefix_lens, extend_lens, max_blocks, num_blocks, block_size);
  if (rc != EXTATTN_OK) return rc;
  if (!k_cache || !v_cache || !block_table || !workspace)
    return fail(EXTATTN_EINVAL, "null device pointer");
  const size_t need = extattn_kv_append_workspace_bytes(num_seqs);
  if (workspace_bytes < need) return fail(EXTATTN_ENOSPC, "workspace too small for kv_append");
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return fail(EXTATTN_EINVAL, "workspace must be 256-byte aligned");
  std::vector<unsigned char> blob(need, 0);
  int64_t q_off = 0;
  for (int32_t r = 0; r < num_seqs; ++r) {
    SeqInfo s{int32_t(q_off), prefix_lens[r], extend_lens[r], 0};
    std::memcpy(blob.data() + kHeaderBytes + sizeof(SeqInfo) * r, &s, sizeof(s));
    q_off += extend_lens[r];
  }
  if (q_off == 0) { g_error.clear(); return EXTATTN_OK; }
  if (!k_new || !v_new) return fail(EXTATTN_EINVAL, "null k_new / v_new");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  rc = upload(blob.data(), need, workspace, st);
  if (rc != EXTATTN_OK) return rc;
  KvArgs a{};
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.seqs = reinterpret_cast<const SeqInfo*>(static_cast<unsigned char*>(workspace) + kHeaderBytes);
  a.err = static_cast<int32_t*>(workspace);
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks;
  a.num_seqs = num_seqs;
  a.hkv = num_kv_heads;
  a.head_dim = head_dim;
  a.total_tokens = int32_t(q_off);
  hipError_t e = launch_kv_append(a, dtype, st);
  if (e != hipSuccess) return hip_fail(e, "kv_append launch");
  g_error.clear();
  return EXTATTN_OK;
}

}  // extern "C"

namespace extattn {

// Checks, planning, metadata upload and launches of one extend-attention call;
// with `timed`, the attention kernel records per-item wall-clock stamps.
int extend_call(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                int32_t max_blocks, int64_t num_blocks, const int32_t* prefix_lens, const int32_t* extend_lens,
                int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                int32_t block_size, float scale, int32_t dtype, void* out, float* lse, void* workspace,
                size_t workspace_bytes, void* stream, bool timed, int64_t* stamps, int32_t capacity,
                int32_t* n_items, double* tick_hz, const void* k_new, const void* v_new, MetaUploader upload_fn) {
  const bool fused = k_new != nullptr || v_new != nullptr;
  int rc = check_common(num_seqs, prefix_lens, extend_lens, num_q_heads, num_kv_heads, head_dim, dtype, true);
  if (rc != EXTATTN_OK) return rc;
  rc = check_blocks(num_seqs, prefix_lens, extend_lens, max_blocks, num_blocks, block_size);
  if (rc != EXTATTN_OK) return rc;
  if (!q || !k_cache || !v_cache || !block_table || !out || !workspace)
    return fail(EXTATTN_EINVAL, "null device pointer");
  if (!std::isfinite(scale) || !(scale > 0.0f)) return fail(EXTATTN_EINVAL, "scale must be finite and > 0");
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return fail(EXTATTN_EINVAL, "workspace must be 256-byte aligned");
  if (fused && (!k_new || !v_new)) return fail(EXTATTN_EINVAL, "null k_new / v_new");
  std::shared_ptr<const LaunchPlan> lp;
  rc = get_launch_plan(num_seqs, prefix_lens, extend_lens, num_q_heads, num_kv_heads, head_dim, dtype, lp);
  if (rc != EXTATTN_OK)
    return fail(rc, rc == EXTATTN_ENOSPC ? "launch too large: partial results exceed 2^31 floats" : "planning failed");
  const Plan& plan = lp->plan;
  if (workspace_bytes < plan.bytes)
    return fail(EXTATTN_ENOSPC, "workspace too small: the launch needs " + std::to_string(plan.bytes) + " bytes, " +
                                    std::to_string(workspace_bytes) + " available");
  const int32_t n_launch = int32_t(plan.items.size());
  if (timed) {
    if (!n_items || !tick_hz) return fail(EXTATTN_EINVAL, "null n_items or tick_hz");
    if (dtype != EXTATTN_BF16) return fail(EXTATTN_EUNSUPPORTED, "timed launches exist for bf16 only");
    *n_items = n_launch;
    int dev = 0, khz = 0;
    hipError_t he = hipGetDevice(&dev);
    if (he == hipSuccess) he = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
    if (he != hipSuccess) return hip_fail(he, "wall clock rate");
    *tick_hz = double(khz) * 1e3;
    if (capacity < *n_items) return fail(EXTATTN_ENOSPC, "stamp capacity is smaller than the number of work items");
    if (!stamps) return fail(EXTATTN_EINVAL, "null stamps");
  }

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  rc = upload_fn ? upload_fn(*lp, workspace, st) : upload(lp->blob.data(), lp->blob.size(), workspace, st);
  if (rc != EXTATTN_OK) return rc;

  unsigned char* ws = static_cast<unsigned char*>(workspace);
  AttnArgs a{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.out = out;
  a.lse = lse;
  a.seqs = reinterpret_cast<const SeqInfo*>(ws + plan.off_seqs);
  a.items = reinterpret_cast<const WorkItem*>(ws + plan.off_items);
  a.tasks = reinterpret_cast<const CombineTask*>(ws + plan.off_tasks);
  a.slots = reinterpret_cast<float*>(ws + plan.off_slots);
  a.err = reinterpret_cast<int32_t*>(ws);
  a.zero_page = ws + plan.off_zero;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks;
  a.num_seqs = num_seqs;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.group = num_q_heads / num_kv_heads;
  a.head_dim = head_dim;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.total_rows = int32_t(plan.total_rows);
  a.n_items = n_launch;
  a.n_tasks = int32_t(plan.tasks.size());
  a.stamps = timed ? stamps : nullptr;
  if (fused) {
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_cache_w = const_cast<void*>(k_cache);
    a.v_cache_w = const_cast<void*>(v_cache);
    a.append_done = reinterpret_cast<int32_t*>(ws + kAppendDoneOffset);
    a.n_append = plan.n_append;
  }

  hipError_t e;
  if (dtype == EXTATTN_F32) {
    if (fused) {  // fp32: the append runs as its own launch first, on the same stream
      KvArgs ka{};
      ka.k_new = k_new;
      ka.v_new = v_new;
      ka.k_cache = const_cast<void*>(k_cache);
      ka.v_cache = const_cast<void*>(v_cache);
      ka.block_table = block_table;
      ka.seqs = a.seqs;
      ka.err = a.err;
      ka.num_blocks = num_blocks;
      ka.max_blocks = max_blocks;
      ka.num_seqs = num_seqs;
      ka.hkv = num_kv_heads;
      ka.head_dim = head_dim;
      ka.total_tokens = int32_t(plan.total_rows);
      e = launch_kv_append(ka, dtype, st);
      if (e != hipSuccess) return hip_fail(e, "kv_append launch");
    }
    e = launch_attn_f32(a, st);
    if (e != hipSuccess) return hip_fail(e, "fp32 attention launch");
  } else {
    if (a.n_items > 0) {
      // launches of chunk rows only (and their fused appends) run on the 8-wave chunk
      // kernel; decode / verify rows need the mixed kernel, which takes every item,
      // or, when some request has 33-64 rows and none more, the 4-wave wide kernel
      e = plan.wide ? launch_split_wide(a, st) : plan.n_split > 0 ? launch_attn_bf16(a, st) : launch_chunk_bf16(a, st);
      if (e != hipSuccess) return hip_fail(e, "bf16 attention launch");
    }
    if (a.n_tasks > 0) {
      e = launch_combine(a, dtype, st);
      if (e != hipSuccess) return hip_fail(e, "combine launch");
    }
  }
  g_error.clear();
  return EXTATTN_OK;
}

}  // namespace extattn

extern "C" {

int extattn_extend_attention(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_table, int32_t max_blocks, int64_t num_blocks,
                             const int32_t* prefix_lens, const int32_t* extend_lens, int32_t num_seqs,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, float scale, int32_t dtype, void* out, float* lse,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return extend_call(q, k_cache, v_cache, block_table, max_blocks, num_blocks, prefix_lens, extend_lens, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, block_size, scale, dtype, out, lse, workspace,
                     workspace_bytes, stream, false, nullptr, 0, nullptr, nullptr);
}

int extattn_extend_attention_append(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                    void* v_cache, const int32_t* block_table, int32_t max_blocks,
                                    int64_t num_blocks, const int32_t* prefix_lens, const int32_t* extend_lens,
                                    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, float scale, int32_t dtype, void* out, float* lse,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  if (!k_new || !v_new) return fail(EXTATTN_EINVAL, "null k_new / v_new");
  return extend_call(q, k_cache, v_cache, block_table, max_blocks, num_blocks, prefix_lens, extend_lens, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, block_size, scale, dtype, out, lse, workspace,
                     workspace_bytes, stream, false, nullptr, 0, nullptr, nullptr, k_new, v_new);
}

int extattn_extend_attention_timed(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* block_table, int32_t max_blocks, int64_t num_blocks,
                                   const int32_t* prefix_lens, const int32_t* extend_lens, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, float scale, int32_t dtype, void* out, float* lse,
                                   void* workspace, size_t workspace_bytes, void* stream, int64_t* stamps,
                                   int32_t capacity, int32_t* n_items, double* tick_hz) {
  return extend_call(q, k_cache, v_cache, block_table, max_blocks, num_blocks, prefix_lens, extend_lens, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, block_size, scale, dtype, out, lse, workspace,
                     workspace_bytes, stream, true, stamps, capacity, n_items, tick_hz);
}

}  // extern "C"
