// Host check of the launch-plan cache (built and run by tests/test_plan_host.py
// with g++, once under the address / undefined-behaviour sanitizers and once
// under the thread sanitizer).
//
//  * a record equals a freshly built plan of the same shape: the same work list,
//    combine tasks, layout, and a workspace image whose descriptor, item and task
//    regions hold exactly those records (zero elsewhere, header included);
//  * a repeated shape hits and returns the same record; any change of a length,
//    of the request order, of the head counts, head_dim or dtype misses;
//  * least-recently-used eviction under the entry bound, nothing kept under a
//    too-small byte bound or with the table off, counters and clear;
//  * several threads looking up and evicting a shared set of shapes at once always
//    get the record of the shape they asked for.
// Exit status 0 when every check passes; the first violation is printed.
#include <atomic>
#include <cstdio>
#include <cstring>
#include <random>
#include <thread>
#include <vector>

#include "../include/extattn.h"
#include "../chunked_prefill_attention_extend_amd/csrc/internal.hpp"

using namespace extattn;

static int fails = 0;
#define CHECK(cond, ...)                \
  do {                                  \
    if (!(cond)) {                      \
      std::printf("FAIL %s: ", #cond);  \
      std::printf(__VA_ARGS__);         \
      std::printf("\n");                \
      ++fails;                          \
      return false;                     \
    }                                   \
  } while (0)

struct Shape {
  std::vector<int32_t> P, E;
  int32_t hq, hkv, d, dtype;
};

static Shape random_shape(std::mt19937& g) {
  static const int heads[][2] = {{32, 8}, {64, 8}, {8, 8}, {28, 4}, {16, 2}};
  Shape s;
  const auto& h = heads[g() % 5];
  s.hq = h[0];
  s.hkv = h[1];
  s.d = (g() & 1) ? 128 : 64;
  s.dtype = (g() % 4) == 0 ? EXTATTN_F32 : EXTATTN_BF16;
  const int n = 1 + int(g() % 10);
  for (int r = 0; r < n; ++r) {
    const int kind = int(g() % 3);
    s.P.push_back(int(g() % 9000));
    s.E.push_back(kind == 0 ? 1 + int(g() % 2000) : (kind == 1 ? 1 + int(g() % 8) : 1));
  }
  return s;
}

static int lookup(const Shape& s, std::shared_ptr<const LaunchPlan>& out) {
  return get_launch_plan(int32_t(s.P.size()), s.P.data(), s.E.data(), s.hq, s.hkv, s.d, s.dtype, out);
}

static bool same_bytes(const void* a, const void* b, size_t n) { return n == 0 || std::memcmp(a, b, n) == 0; }

static void put(std::vector<unsigned char>& dst, size_t off, const void* src, size_t n) {
  if (n) std::memcpy(dst.data() + off, src, n);
}

static bool same_plan(const LaunchPlan& a, const LaunchPlan& b) {
  return a.blob == b.blob && a.plan.bytes == b.plan.bytes && a.plan.n_append == b.plan.n_append &&
         a.plan.items.size() == b.plan.items.size() && a.plan.tasks.size() == b.plan.tasks.size() &&
         a.plan.n_slot_floats == b.plan.n_slot_floats &&
         same_bytes(a.plan.items.data(), b.plan.items.data(), sizeof(WorkItem) * a.plan.items.size()) &&
         same_bytes(a.plan.tasks.data(), b.plan.tasks.data(), sizeof(CombineTask) * a.plan.tasks.size());
}

static bool check_record(const Shape& s, unsigned seed) {
  std::shared_ptr<const LaunchPlan> a, b;
  CHECK(lookup(s, a) == EXTATTN_OK, "seed %u", seed);
  CHECK(lookup(s, b) == EXTATTN_OK, "seed %u", seed);
  CHECK(a.get() == b.get(), "seed %u: a repeated shape returned another record", seed);
  LaunchPlan fresh;
  CHECK(make_launch_plan(int32_t(s.P.size()), s.P.data(), s.E.data(), s.hq, s.hkv, s.d, s.dtype, fresh) ==
            EXTATTN_OK, "seed %u", seed);
  CHECK(same_plan(*a, fresh), "seed %u: record differs from a fresh plan", seed);
  Plan direct;
  CHECK(build_plan(int32_t(s.P.size()), s.P.data(), s.E.data(), s.hq, s.hkv, s.d, s.dtype, direct, true) ==
            EXTATTN_OK, "seed %u", seed);
  CHECK(direct.items.size() == a->plan.items.size() && direct.bytes == a->plan.bytes,
        "seed %u: record differs from the planner's fused-append plan", seed);
  // the workspace image: records where the layout says, zero elsewhere
  const Plan& p = a->plan;
  std::vector<unsigned char> want(p.upload_bytes, 0);
  put(want, p.off_seqs, p.seqs.data(), sizeof(SeqInfo) * p.seqs.size());
  put(want, p.off_items, p.items.data(), sizeof(WorkItem) * p.items.size());
  put(want, p.off_tasks, p.tasks.data(), sizeof(CombineTask) * p.tasks.size());
  CHECK(a->blob == want, "seed %u: workspace image", seed);
  CHECK(p.off_seqs >= kHeaderBytes && p.off_items >= p.off_seqs + sizeof(SeqInfo) * p.seqs.size() &&
            p.off_tasks >= p.off_items + sizeof(WorkItem) * p.items.size() &&
            p.upload_bytes >= p.off_tasks + sizeof(CombineTask) * p.tasks.size() && p.upload_bytes <= p.bytes,
        "seed %u: layout regions overlap", seed);
  return true;
}

static bool check_keys() {
  plan_cache_clear();
  Shape s{{100, 2000, 5}, {1, 300, 1}, 32, 8, 128, EXTATTN_BF16};
  std::shared_ptr<const LaunchPlan> base, x;
  CHECK(lookup(s, base) == EXTATTN_OK, "base");
  auto misses = [&]() {
    int64_t h, m, b;
    int32_t n;
    plan_cache_stats(&h, &m, &n, &b);
    return m;
  };
  const int64_t m0 = misses();
  std::vector<Shape> variants;
  for (int i = 0; i < 3; ++i) {
    Shape v = s;
    v.P[i] += 1;
    variants.push_back(v);
    v = s;
    v.E[i] += 1;
    variants.push_back(v);
  }
  Shape v = s;
  std::swap(v.P[0], v.P[2]);
  std::swap(v.E[0], v.E[2]);
  variants.push_back(v);  // the same requests in another order
  v = s; v.hq = 64; variants.push_back(v);
  v = s; v.hkv = 4; variants.push_back(v);
  v = s; v.d = 64; variants.push_back(v);
  v = s; v.dtype = EXTATTN_F32; variants.push_back(v);
  v = s; v.P.push_back(0); v.E.push_back(1); variants.push_back(v);
  for (size_t i = 0; i < variants.size(); ++i) {
    CHECK(lookup(variants[i], x) == EXTATTN_OK, "variant %zu", i);
    CHECK(x.get() != base.get(), "variant %zu hit the base record", i);
  }
  CHECK(misses() == m0 + int64_t(variants.size()), "every variant must miss");
  CHECK(lookup(s, x) == EXTATTN_OK && x.get() == base.get(), "the base shape must still hit");
  return true;
}

static bool check_bounds() {
  std::mt19937 g(99);
  std::vector<Shape> shapes;
  for (int i = 0; i < 3; ++i) shapes.push_back(random_shape(g));
  shapes[1].P[0] += 1;  // make sure the three differ
  shapes[2].P[0] += 2;
  std::shared_ptr<const LaunchPlan> a, b, c, x;
  int64_t h, m, bytes;
  int32_t n;
  plan_cache_clear();
  plan_cache_configure(2, kPlanCacheBytes);
  CHECK(lookup(shapes[0], a) == 0 && lookup(shapes[1], b) == 0 && lookup(shapes[2], c) == 0, "lookups");
  plan_cache_stats(&h, &m, &n, &bytes);
  CHECK(n == 2 && h == 0 && m == 3 && bytes > 0, "entries %d hits %lld misses %lld", n, (long long)h, (long long)m);
  CHECK(lookup(shapes[2], x) == 0 && x.get() == c.get(), "most recent shape must hit");
  CHECK(lookup(shapes[0], x) == 0 && x.get() != a.get(), "least recent shape must have been evicted");
  CHECK(same_plan(*x, *a), "a rebuilt record equals the evicted one");
  plan_cache_stats(&h, &m, &n, &bytes);
  CHECK(h == 1 && m == 4 && n == 2, "counters after eviction");
  // shrinking evicts at once; a byte bound below one record keeps nothing
  plan_cache_configure(1, kPlanCacheBytes);
  plan_cache_stats(&h, &m, &n, &bytes);
  CHECK(n == 1, "shrink to one entry kept %d", n);
  plan_cache_configure(64, 1);
  plan_cache_stats(&h, &m, &n, &bytes);
  CHECK(n == 0 && bytes == 0, "byte bound of 1 kept %d records", n);
  CHECK(lookup(shapes[1], x) == 0, "lookup");
  plan_cache_stats(&h, &m, &n, &bytes);
  CHECK(n == 0, "a record larger than the byte bound was kept");
  // table off: every lookup plans, nothing is kept, results still right
  plan_cache_clear();
  plan_cache_configure(0, kPlanCacheBytes);
  CHECK(lookup(shapes[1], x) == 0 && lookup(shapes[1], a) == 0 && x.get() != a.get(), "table off");
  CHECK(same_plan(*x, *a), "table off: same plan");
  plan_cache_stats(&h, &m, &n, &bytes);
  CHECK(n == 0 && h == 0 && m == 2, "table off kept %d records, %lld hits", n, (long long)h);
  plan_cache_clear();
  plan_cache_stats(&h, &m, &n, &bytes);
  CHECK(h == 0 && m == 0 && n == 0 && bytes == 0, "clear");
  plan_cache_configure(kPlanCacheEntries, kPlanCacheBytes);
  return true;
}

static bool check_threads() {
  std::mt19937 g(7);
  std::vector<Shape> shapes;
  for (int i = 0; i < 24; ++i) {
    Shape s = random_shape(g);
    s.P[0] = 20000 + i;  // distinct shapes
    shapes.push_back(s);
  }
  std::vector<LaunchPlan> want(shapes.size());
  for (size_t i = 0; i < shapes.size(); ++i)
    make_launch_plan(int32_t(shapes[i].P.size()), shapes[i].P.data(), shapes[i].E.data(), shapes[i].hq,
                     shapes[i].hkv, shapes[i].d, shapes[i].dtype, want[i]);
  plan_cache_clear();
  plan_cache_configure(8, kPlanCacheBytes);  // fewer records than shapes: lookups evict each other
  std::atomic<int> bad{0};
  std::vector<std::thread> th;
  for (int t = 0; t < 6; ++t)
    th.emplace_back([&, t]() {
      std::mt19937 r(1000 + t);
      for (int k = 0; k < 300; ++k) {
        const size_t i = r() % shapes.size();
        std::shared_ptr<const LaunchPlan> x;
        if (lookup(shapes[i], x) != EXTATTN_OK || !same_plan(*x, want[i])) ++bad;
        if (k % 97 == 0 && t == 0) plan_cache_clear();
      }
    });
  for (auto& x : th) x.join();
  plan_cache_configure(kPlanCacheEntries, kPlanCacheBytes);
  CHECK(bad.load() == 0, "%d lookups returned a wrong record", bad.load());
  return true;
}

int main(int argc, char** argv) {
  const bool threads_only = argc > 1 && std::strcmp(argv[1], "threads") == 0;
  int done = 0;
  if (!threads_only) {
    std::mt19937 g(4242);
    for (int i = 0; i < 60 && fails == 0; ++i) {
      const unsigned seed = g();
      std::mt19937 gs(seed);
      if (check_record(random_shape(gs), seed)) ++done;
    }
    if (fails == 0 && check_keys()) ++done;
    if (fails == 0 && check_bounds()) ++done;
  }
  if (fails == 0 && check_threads()) ++done;
  std::printf("%d checks passed, %d failures\n", done, fails);
  return fails == 0 ? 0 : 1;
}
