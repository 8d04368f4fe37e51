// Internal definitions shared by the host planner, the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstddef>
#include <cstdint>
#include <memory>
#include <vector>

namespace extattn {

constexpr int kBlockSize = 16;    // tokens per paged-cache block
constexpr int kWaves = 8;         // wave64 per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;  // query rows per wave (one 32x32 MFMA column block)
constexpr int kRowsPerTile = kWaves * 32;  // chunk path: all waves' rows share each K/V tile
constexpr int kChunkKeys = 32;    // chunk path: keys per LDS K/V tile (one 32x32 S^T block)
constexpr int kSplitTile = 32;    // split path: keys per register K/V tile
constexpr int kSplitKeysMin = 1024;  // split path: keys per workgroup (kWaves waves), lower bound
constexpr int kSplitKeysMax = 8192;  // upper bound: a wave's block ids fit one per lane
constexpr int kSplitTargetItems = 256;  // split path aims at this many workgroups (1 per CU on 256 CUs)
constexpr int kChunkTargetItems = 256;  // chunk rows: split key ranges until about this many workgroups (1 per CU)
constexpr int kChunkMinPieceKeys = 1024;  // ... with at least this many keys per piece
constexpr int kCombineRows = 32;         // rows per combine task of split chunk tiles
constexpr int kXcds = 8;  // accelerator dies (own L2 each); a launch's workgroups are dealt to them round-robin
constexpr int kSplitRows = 16;    // split path: rows of one 16-row MFMA block
constexpr int kSplitMaxRows = 32; // split path: at most this many rows (two blocks per wave)
constexpr int kWideWaves = 4;      // wide-split kernel: wave64 per workgroup, one per SIMD, 512 registers each
constexpr int kWideMaxRows = 64;   // ... at most this many rows per split item (four 16-row blocks per wave)
constexpr int kWideKeysMax = 8192; // ... keys per workgroup: a wave's block ids fit two per lane
constexpr int kWideTargetItems = 256;  // ... aims at this many workgroups
// keys per split workgroup of `waves` waves, upper bound
constexpr int split_keys_max(int waves) { return waves == kWideWaves ? kWideKeysMax : kSplitKeysMax; }
constexpr int kFewRows = 2 * kRowsPerWave;  // chunk tiles of at most this many rows are cut into split-length key pieces

// Per-request metadata copied to the workspace.
struct SeqInfo {
  int32_t q_off;   // first query row of the request in q / out
  int32_t prefix;  // P: tokens already in the cache before this chunk
  int32_t extend;  // E: new query tokens
  int32_t pad;
};

enum : int32_t {
  kItemChunk = 0,  // kRowsPerTile rows of one (request, KV head); all waves share LDS K/V tiles
  kItemSplit = 1,  // <= kSplitMaxRows rows (kWideMaxRows in wide launches); each wave takes its own part of the key range
};

// Measurement variant: one record per work item, {start, end} in wall-clock ticks,
// {kind, request}, {start, end} in shader-clock cycles.
constexpr int kStampWords = 6;

// Fused append + attention launches: the first min(items, kAppendProducers) workgroups
// each copy an equal share of the launch's new tokens into the cache before their own
// work item (8 a die with the round-robin deal of workgroups to the 8 dies).
constexpr int kAppendProducers = 64;
constexpr int kAppendDoneOffset = 128;  // byte offset of the append completion counter in the workspace header
// Status words at the start of the workspace (reset by every call's metadata upload):
// word 0 holds flags, word 1 counts invalid block-id reads (wrapping), word 2 counts
// the waves that redid their rows on the exact two-pass path (informational).
constexpr int32_t kStatusBadBlock = 1;     // a block id outside [0, num_blocks) was met
constexpr int32_t kStatusWaitTimeout = 2;  // an attention item stopped waiting for the fused appends

// One workgroup's work. Rows are flattened per (request, KV head) as
// row = pos * group + head_in_group, pos in [0, E), head_in_group in [0, group).
struct WorkItem {
  int32_t kind;
  int32_t seq;
  int32_t kv_head;
  int32_t row0;       // first flattened row
  int32_t nrows;      // rows in this item (<= kRowsPerTile chunk, <= kSplitMaxRows or kWideMaxRows split)
  int32_t key_begin;  // keys [key_begin, key_end); key_begin is a multiple of kChunkKeys
  int32_t key_end;
  int32_t slot;       // < 0: write out/lse directly; else float offset of this item's partial slot
  int32_t task;       // combine task that merges this item's slot, or -1 (direct write)
  int32_t slot_rows;  // rows of the partial slot (a multiple of 16; 0 for direct writes)
  int32_t pad[2];
};

// Merge of the partial results of rows [row0, row0 + nrows) of one (request, KV
// head): rows srow0 .. srow0 + nrows - 1 of the slots at float offsets
// slot0 + i * stride, i in [0, nslots), each slot holding slot_rows rows.
struct CombineTask {
  int32_t seq;
  int32_t kv_head;
  int32_t row0;
  int32_t nrows;
  int32_t slot0;
  int32_t nslots;
  int32_t stride;
  int32_t slot_rows;
  int32_t srow0;
  int32_t pad[3];
};

// A partial slot of `rows` rows: o (normalised, fp32) [rows][D] then lse (natural log) [rows].
inline constexpr size_t slot_floats(int rows, int head_dim) { return size_t(rows) * (head_dim + 1); }

struct AttnArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  void* out;
  float* lse;
  const SeqInfo* seqs;
  const WorkItem* items;
  const CombineTask* tasks;
  float* slots;
  int32_t* err;
  const void* zero_page;  // kZeroPageBytes of zeros in the workspace (stands in for invalid blocks)
  int64_t num_blocks;
  int32_t max_blocks;
  int32_t num_seqs;
  int32_t hq;
  int32_t hkv;
  int32_t group;
  int32_t head_dim;
  float scale;       // softmax scale
  float scale_log2;  // scale * log2(e)
  int32_t total_rows;
  int32_t n_items;
  int32_t n_tasks;
  int64_t* stamps;   // NULL, or [n_items][kStampWords] {start, end, kind, request, clk_start, clk_end}
  // fused append (n_append > 0): workgroups 0 .. n_append-1 first copy their share
  // of k_new / v_new [sum(E), Hkv, D] into the cache, then every wave of them adds 1
  // to *append_done (release); work that reads new keys waits for n_append * waves
  const void* k_new;
  const void* v_new;
  void* k_cache_w;
  void* v_cache_w;
  int32_t* append_done;
  int32_t n_append;
};

struct KvArgs {
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
  const int32_t* block_table;
  const SeqInfo* seqs;
  int32_t* err;
  int64_t num_blocks;
  int32_t max_blocks;
  int32_t num_seqs;
  int32_t hkv;
  int32_t head_dim;
  int32_t total_tokens;
};

// Host plan of one extend_attention call.
struct Plan {
  std::vector<SeqInfo> seqs;
  std::vector<WorkItem> items;
  std::vector<CombineTask> tasks;
  int64_t n_slot_floats = 0;  // size of the partial-slot area
  int32_t split_keys = 0;  // keys per split workgroup (0: no split items)
  int32_t n_append = 0;    // workgroups that also copy new tokens in a fused append launch
  int32_t n_split = 0;     // split items (decode / verify rows) in `items`
  bool wide = false;       // every split item runs on the 4-wave wide-split kernel (up to kWideMaxRows rows)
  int64_t total_rows = 0;
  // byte offsets inside the workspace
  size_t off_zero = 0, off_seqs = 0, off_items = 0, off_tasks = 0, off_slots = 0, bytes = 0, upload_bytes = 0;
};

constexpr size_t kHeaderBytes = 256;  // error word + padding
constexpr size_t kZeroPageBytes = size_t(kBlockSize) * 128 * 4;  // one (block, head) of the largest head_dim, fp32

// plan.cpp
int build_plan(int32_t num_seqs, const int32_t* prefix, const int32_t* extend, int32_t hq, int32_t hkv,
               int32_t head_dim, int32_t dtype, Plan& plan, bool with_append = false);

// plan_cache.cpp. A launch's plan (built with the fused append's items first, so
// one record serves the plain and the fused launch: the plain one starts at item
// n_append) and the workspace image up to plan.upload_bytes.
struct LaunchPlan {
  Plan plan;
  std::vector<unsigned char> blob;
};
constexpr int32_t kPlanCacheEntries = 256;       // default table bounds
constexpr int64_t kPlanCacheBytes = 64ll << 20;
int make_launch_plan(int32_t num_seqs, const int32_t* prefix, const int32_t* extend, int32_t hq, int32_t hkv,
                     int32_t head_dim, int32_t dtype, LaunchPlan& lp);
int get_launch_plan(int32_t num_seqs, const int32_t* prefix, const int32_t* extend, int32_t hq, int32_t hkv,
                    int32_t head_dim, int32_t dtype, std::shared_ptr<const LaunchPlan>& out);
void plan_cache_configure(int32_t max_entries, int64_t max_bytes);

// api.cpp: one extend-attention call (checks, plan, metadata upload, launches).
// `upload` copies the plan's metadata into the workspace on the stream; nullptr
// uses the library's pinned staging pool and copies the whole image.
using MetaUploader = int (*)(const LaunchPlan& lp, void* workspace, hipStream_t stream);
int extend_call(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                int32_t max_blocks, int64_t num_blocks, const int32_t* prefix_lens, const int32_t* extend_lens,
                int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                int32_t block_size, float scale, int32_t dtype, void* out, float* lse, void* workspace,
                size_t workspace_bytes, void* stream, bool timed, int64_t* stamps, int32_t capacity,
                int32_t* n_items, double* tick_hz, const void* k_new = nullptr, const void* v_new = nullptr,
                MetaUploader upload = nullptr);
int set_error(int code, const char* msg);           // thread-local message, returns code
int set_hip_error(hipError_t e, const char* what);  // returns EXTATTN_EHIP

// noalloc.hip: the allocation-free entry point's static device scratch.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
int noalloc_scratch(void** ptr);  // this device's scratch address (looked up once per device)
void plan_cache_stats(int64_t* hits, int64_t* misses, int32_t* entries, int64_t* bytes);
void plan_cache_clear();

// budget.cpp
int token_budget_step_impl(int32_t n_running, const int64_t* running_total, const int64_t* running_computed,
                           int32_t n_waiting, const int64_t* waiting_total, const int64_t* waiting_cached,
                           int64_t budget, int32_t* out_index, int64_t* out_prefix, int64_t* out_extend,
                           int32_t capacity, int32_t* n_out, int64_t* budget_left, const char** why);
int mixed_chunk_step_impl(int32_t n_decode, const int64_t* decode_prefix, int64_t chunked_total,
                          int64_t chunked_done, int32_t n_waiting, const int64_t* waiting_total,
                          const int64_t* waiting_cached, int64_t chunk_size, int64_t page_size, int32_t mixed,
                          int32_t* out_kind, int32_t* out_index, int64_t* out_prefix, int64_t* out_extend,
                          int32_t capacity, int32_t* n_out, int64_t* chunk_left, int32_t* next_kind,
                          int32_t* next_index, int64_t* next_done, const char** why);
int decode_first_with_slack_impl(int64_t ready_decode, int64_t pending_prefill, int64_t chunk_query_len,
                                 int64_t max_batched_tokens, int64_t* p_step, int64_t* d_step, int64_t* limit,
                                 const char** why);

// kernel launchers (one per .hip file)
hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t stream);
hipError_t launch_chunk_bf16(const AttnArgs& a, hipStream_t stream);  // chunk items only
hipError_t launch_split_wide(const AttnArgs& a, hipStream_t stream);  // split items only
hipError_t launch_combine(const AttnArgs& a, int32_t dtype, hipStream_t stream);
hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t stream);
hipError_t launch_kv_append(const KvArgs& a, int32_t dtype, hipStream_t stream);
// Copies `bytes` from `src` (pinned host memory mapped into the device, 16-byte
// aligned) to device memory `dst` with a kernel on `stream`.
hipError_t launch_meta_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);

}  // namespace extattn
