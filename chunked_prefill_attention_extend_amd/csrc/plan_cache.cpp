// Launch-plan cache: the plan of a launch shape (the requests' prefix / extend
// lengths, head counts, head_dim, dtype) is built once and reused while the
// shape repeats.
//
// This is the latency-table RFC's shape table (sections 3.1.3 and 3.1.4: an
// immutable key holding the dynamic shape of one forward, a table filled on
// first use and read afterwards), applied to this library's launch
// configuration instead of to modelled latencies: the key is the launch's
// exact shape, the record its work list, combine tasks and workspace layout,
// and the workspace image the host uploads. Everything that does not change
// the plan (pointers, scale, stream, block tables) stays out of the key.
//
// The table is least-recently-used, bounded by an entry count and a byte
// budget, and shared by all threads (one mutex; records are immutable and
// reference counted, so a caller keeps using a record that another thread
// evicts).
#include <cstring>
#include <list>
#include <memory>
#include <mutex>
#include <vector>

#include "../../include/extattn.h"
#include "internal.hpp"

namespace extattn {
namespace {

struct Entry {
  uint64_t hash;
  std::vector<int32_t> key;
  std::shared_ptr<const LaunchPlan> plan;
  size_t bytes;
};

struct Cache {
  std::mutex mu;
  std::list<Entry> lru;  // most recently used first
  int32_t max_entries = kPlanCacheEntries;
  int64_t max_bytes = kPlanCacheBytes;
  int64_t bytes = 0;
  int64_t hits = 0, misses = 0;

  void trim() {
    while (!lru.empty() && (int64_t(lru.size()) > max_entries || bytes > max_bytes)) {
      bytes -= int64_t(lru.back().bytes);
      lru.pop_back();
    }
  }
};

Cache& cache() {
  static Cache c;
  return c;
}

// FNV-1a over the key's 32-bit words.
uint64_t fnv1a(const std::vector<int32_t>& key) {
  uint64_t h = 1469598103934665603ull;
  for (int32_t v : key) {
    uint32_t u;
    std::memcpy(&u, &v, 4);
    for (int b = 0; b < 4; ++b) {
      h ^= (u >> (8 * b)) & 0xffu;
      h *= 1099511628211ull;
    }
  }
  return h;
}

size_t footprint(const std::vector<int32_t>& key, const LaunchPlan& lp) {
  return sizeof(Entry) + sizeof(LaunchPlan) + key.size() * sizeof(int32_t) + lp.blob.size() +
         lp.plan.seqs.size() * sizeof(SeqInfo) + lp.plan.items.size() * sizeof(WorkItem) +
         lp.plan.tasks.size() * sizeof(CombineTask);
}

}  // namespace

int make_launch_plan(int32_t num_seqs, const int32_t* prefix, const int32_t* extend, int32_t hq, int32_t hkv,
                     int32_t head_dim, int32_t dtype, LaunchPlan& lp) {
  const int rc = build_plan(num_seqs, prefix, extend, hq, hkv, head_dim, dtype, lp.plan, true);
  if (rc != EXTATTN_OK) return rc;
  lp.plan.n_split = 0;
  for (const WorkItem& it : lp.plan.items) lp.plan.n_split += it.kind == kItemSplit ? 1 : 0;
  const Plan& p = lp.plan;
  lp.blob.assign(p.upload_bytes, 0);
  std::memcpy(lp.blob.data() + p.off_seqs, p.seqs.data(), sizeof(SeqInfo) * p.seqs.size());
  if (!p.items.empty()) std::memcpy(lp.blob.data() + p.off_items, p.items.data(), sizeof(WorkItem) * p.items.size());
  if (!p.tasks.empty())
    std::memcpy(lp.blob.data() + p.off_tasks, p.tasks.data(), sizeof(CombineTask) * p.tasks.size());
  return EXTATTN_OK;
}

int get_launch_plan(int32_t num_seqs, const int32_t* prefix, const int32_t* extend, int32_t hq, int32_t hkv,
                    int32_t head_dim, int32_t dtype, std::shared_ptr<const LaunchPlan>& out) {
  std::vector<int32_t> key;
  key.reserve(5 + 2 * size_t(num_seqs));
  key.insert(key.end(), {dtype, hq, hkv, head_dim, num_seqs});
  for (int32_t r = 0; r < num_seqs; ++r) {
    key.push_back(prefix[r]);
    key.push_back(extend[r]);
  }
  const uint64_t h = fnv1a(key);
  Cache& c = cache();
  {
    std::lock_guard<std::mutex> lock(c.mu);
    for (auto it = c.lru.begin(); it != c.lru.end(); ++it) {
      if (it->hash == h && it->key == key) {
        c.lru.splice(c.lru.begin(), c.lru, it);
        ++c.hits;
        out = it->plan;
        return EXTATTN_OK;
      }
    }
    ++c.misses;
  }
  auto lp = std::make_shared<LaunchPlan>();
  const int rc = make_launch_plan(num_seqs, prefix, extend, hq, hkv, head_dim, dtype, *lp);
  if (rc != EXTATTN_OK) return rc;
  out = lp;
  const size_t fp = footprint(key, *lp);
  std::lock_guard<std::mutex> lock(c.mu);
  if (c.max_entries > 0 && int64_t(fp) <= c.max_bytes) {
    // another thread may have added the same shape meanwhile: keep one record
    for (auto it = c.lru.begin(); it != c.lru.end(); ++it) {
      if (it->hash == h && it->key == key) {
        c.bytes -= int64_t(it->bytes);
        c.lru.erase(it);
        break;
      }
    }
    c.lru.push_front(Entry{h, std::move(key), out, fp});
    c.bytes += int64_t(fp);
    c.trim();
  }
  return EXTATTN_OK;
}

void plan_cache_configure(int32_t max_entries, int64_t max_bytes) {
  Cache& c = cache();
  std::lock_guard<std::mutex> lock(c.mu);
  c.max_entries = max_entries;
  c.max_bytes = max_bytes;
  c.trim();
}

void plan_cache_stats(int64_t* hits, int64_t* misses, int32_t* entries, int64_t* bytes) {
  Cache& c = cache();
  std::lock_guard<std::mutex> lock(c.mu);
  if (hits) *hits = c.hits;
  if (misses) *misses = c.misses;
  if (entries) *entries = int32_t(c.lru.size());
  if (bytes) *bytes = c.bytes;
}

void plan_cache_clear() {
  Cache& c = cache();
  std::lock_guard<std::mutex> lock(c.mu);
  c.lru.clear();
  c.bytes = 0;
  c.hits = 0;
  c.misses = 0;
}

}  // namespace extattn
