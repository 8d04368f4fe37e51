// Host check of the launch planner's invariants on random launches (built and run by
// tests/test_plan_host.py with g++ and the address / undefined-behaviour sanitizers).
//
// For every random launch (request mix of chunk, verify and decode rows; GQA group;
// head dim; with and without the fused append) the work list must:
//  * run decode / verify-only launches with 33-64 rows on the wide-split kernel;
//  * cover every (request, KV head, row, key) pair a row attends exactly once, with
//    key ranges that start on 32-key tile boundaries and never pass the row's last
//    visible key's tile;
//  * give every item of a split key range its own partial slot, inside the slot area,
//    and give the slots' rows to combine tasks that cover each row of the range once;
//  * keep split items within the per-wave id budget (kSplitKeysMax keys; kWideKeysMax
//    on the 4-wave wide-split kernel) and the row limit of the kernel that runs them;
//  * give a fused append min(items, kAppendProducers) copying workgroups;
//  * cut chunk tiles into whole rounds of key pieces, with or without split items;
//  * keep the tiles of one chunk group (request, KV head) on a contiguous run of die
//    lanes (list positions modulo kXcds) while every lane still has items.
// Exit status 0 when every launch passes; the first violation is printed.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <set>
#include <tuple>
#include <vector>

#include "../include/extattn.h"
#include "../chunked_prefill_attention_extend_amd/csrc/internal.hpp"

using namespace extattn;

static int fails = 0;
#define CHECK(cond, ...)                         \
  do {                                           \
    if (!(cond)) {                               \
      std::printf("FAIL %s: ", #cond);           \
      std::printf(__VA_ARGS__);                  \
      std::printf("\n");                         \
      ++fails;                                   \
      return false;                              \
    }                                            \
  } while (0)

static bool check_launch(const std::vector<int32_t>& P, const std::vector<int32_t>& E, int hq, int hkv, int d,
                         bool append, unsigned seed) {
  Plan plan;
  const int rc = build_plan(int(P.size()), P.data(), E.data(), hq, hkv, d, EXTATTN_BF16, plan, append);
  CHECK(rc == EXTATTN_OK, "seed %u: build_plan returned %d", seed, rc);
  const int G = hq / hkv;
  const int n = int(P.size());
  // wide-split launches: decode / verify rows only, some past kSplitMaxRows, none past kWideMaxRows
  int max_rows = 0;
  for (int r = 0; r < int(E.size()); ++r) max_rows = std::max(max_rows, E[r] * G);
  CHECK(plan.wide == (max_rows > kSplitMaxRows && max_rows <= kWideMaxRows), "seed %u: wide flag", seed);
  // 1. fused append: the first min(items, kAppendProducers) workgroups copy the new tokens
  const size_t first = 0;
  if (append) {
    CHECK(plan.n_append == int(std::min<size_t>(plan.items.size(), kAppendProducers)), "seed %u: %d producers",
          seed, plan.n_append);
  } else {
    CHECK(plan.n_append == 0, "seed %u", seed);
  }
  // 2. coverage: per (request, head, row) the union of key ranges of its items
  std::map<std::tuple<int, int, int>, std::vector<std::pair<int, int>>> ranges;
  std::vector<std::pair<int64_t, int64_t>> slots;  // [begin, end) in floats
  for (size_t i = first; i < plan.items.size(); ++i) {
    const WorkItem& x = plan.items[i];
    CHECK(x.kind == kItemChunk || x.kind == kItemSplit, "seed %u: kind %d", seed, x.kind);
    CHECK(x.seq >= 0 && x.seq < n && x.kv_head >= 0 && x.kv_head < hkv, "seed %u: item %zu ids", seed, i);
    const int rows = E[x.seq] * G;
    CHECK(x.row0 >= 0 && x.nrows >= 1 && x.row0 + x.nrows <= rows, "seed %u: item %zu rows", seed, i);
    CHECK(x.key_begin >= 0 && x.key_begin < x.key_end && x.key_begin % kChunkKeys == 0,
          "seed %u: item %zu keys [%d, %d)", seed, i, x.key_begin, x.key_end);
    const int kv_len = P[x.seq] + E[x.seq];
    CHECK(x.key_end <= kv_len, "seed %u: item %zu key_end %d > %d", seed, i, x.key_end, kv_len);
    if (x.kind == kItemSplit) {
      const int smax = plan.wide ? kWideMaxRows : kSplitMaxRows;
      CHECK(x.nrows <= smax && rows <= smax && x.row0 == 0, "seed %u: split item %zu rows", seed, i);
      CHECK(x.key_end - x.key_begin <= split_keys_max(plan.wide ? kWideWaves : kWaves),
            "seed %u: split piece of %d keys", seed, x.key_end - x.key_begin);
    } else {
      CHECK(!plan.wide, "seed %u: chunk item %zu in a wide-split launch", seed, i);
      CHECK(x.nrows <= kRowsPerTile && x.row0 % kRowsPerTile == 0, "seed %u: chunk item %zu tile", seed, i);
    }
    if (x.slot >= 0) {
      CHECK(x.task >= 0 && size_t(x.task) < plan.tasks.size(), "seed %u: item %zu task", seed, i);
      const int srows = x.kind == kItemChunk ? (x.nrows + 15) / 16 * 16 : (rows + 15) / 16 * 16;
      CHECK(x.slot_rows == srows, "seed %u: item %zu slot of %d rows, expected %d", seed, i, x.slot_rows, srows);
      CHECK(x.slot % 4 == 0, "seed %u: item %zu slot not 16-byte aligned", seed, i);
      slots.push_back({x.slot, x.slot + int64_t(slot_floats(srows, d))});
    } else {
      CHECK(x.task < 0, "seed %u: direct item %zu has a task", seed, i);
    }
    for (int rr = x.row0; rr < x.row0 + x.nrows; ++rr) ranges[{x.seq, x.kv_head, rr}].push_back({x.key_begin, x.key_end});
  }
  for (int r = 0; r < n; ++r)
    for (int g = 0; g < hkv; ++g)
      for (int rr = 0; rr < E[r] * G; ++rr) {
        auto it = ranges.find({r, g, rr});
        CHECK(it != ranges.end(), "seed %u: request %d head %d row %d not covered", seed, r, g, rr);
        auto v = it->second;
        std::sort(v.begin(), v.end());
        const int need = P[r] + rr / G + 1;  // keys 0 .. P + pos
        int at = 0;
        for (auto& kr : v) {
          CHECK(kr.first == at, "seed %u: request %d head %d row %d: gap or overlap at key %d (next range %d)",
                seed, r, g, rr, at, kr.first);
          at = kr.second;
        }
        CHECK(at >= need, "seed %u: request %d head %d row %d: keys end at %d < %d", seed, r, g, rr, at, need);
        CHECK(at - need < kChunkKeys * 8 + 256, "seed %u: row %d reads far past its keys", seed, rr);
      }
  // 3. slots disjoint and inside the slot area
  std::sort(slots.begin(), slots.end());
  for (size_t i = 0; i < slots.size(); ++i) {
    CHECK(slots[i].first >= 0 && slots[i].second <= plan.n_slot_floats, "seed %u: slot out of the area", seed);
    if (i) CHECK(slots[i - 1].second <= slots[i].first, "seed %u: slots overlap", seed);
  }
  // 4. combine tasks: each (request, head, row) of a split range merged exactly once,
  //    over slots that were written
  std::set<int64_t> slot_starts;
  for (auto& s : slots) slot_starts.insert(s.first);
  std::map<std::tuple<int, int, int>, int> merged;
  for (const CombineTask& t : plan.tasks) {
    CHECK(t.nslots >= 2 && t.nrows >= 1, "seed %u: task with %d slots", seed, t.nslots);
    for (int i = 0; i < t.nslots; ++i)
      CHECK(slot_starts.count(int64_t(t.slot0) + int64_t(i) * t.stride), "seed %u: task reads an unwritten slot", seed);
    CHECK(t.srow0 + t.nrows <= t.slot_rows, "seed %u: task rows past the slot", seed);
    CHECK(int64_t(t.stride) == int64_t(slot_floats(t.slot_rows, d)), "seed %u: task stride %d", seed, t.stride);
    for (int rr = t.row0; rr < t.row0 + t.nrows; ++rr) ++merged[{t.seq, t.kv_head, rr}];
  }
  for (auto& kv : ranges) {
    const bool split = kv.second.size() > 1;
    auto m = merged.find(kv.first);
    const int cnt = m == merged.end() ? 0 : m->second;
    CHECK(cnt == (split ? 1 : 0), "seed %u: row merged %d times (pieces %zu)", seed, cnt, kv.second.size());
  }
  // 4b. chunk tiles are cut into whole rounds of pieces, next to split items too: no
  //     more chunk items than max(kChunkTargetItems, tiles) unless a few-row tile
  //     streams its keys in split-length pieces
  {
    bool few = false;
    int64_t tiles = 0, items = 0;
    for (int r = 0; r < n; ++r) {
      const int64_t rows = int64_t(E[r]) * G;
      if (rows <= (plan.wide ? kWideMaxRows : kSplitMaxRows)) continue;  // split rows
      tiles += (rows + kRowsPerTile - 1) / kRowsPerTile * hkv;
      if (rows % kRowsPerTile != 0 && rows % kRowsPerTile <= kFewRows) few = true;
    }
    for (size_t i = first; i < plan.items.size(); ++i) items += plan.items[i].kind == kItemChunk ? 1 : 0;
    if (!few)
      CHECK(items <= std::max<int64_t>(kChunkTargetItems, tiles), "seed %u: %lld chunk items for %lld tiles", seed,
            (long long)items, (long long)tiles);
  }
  // 5. the lanes: each group's tiles on a contiguous run of lanes (positions taken
  //    modulo kXcds while every lane still has items)
  const size_t body = plan.items.size() - first;
  const size_t full = (body / kXcds) * kXcds;
  std::map<std::pair<int, int>, std::set<size_t>> glanes;
  for (size_t i = first; i < plan.items.size(); ++i) {
    const WorkItem& x = plan.items[i];
    if (x.kind != kItemChunk || x.key_begin != 0 || i - first >= full) continue;
    glanes[{x.seq, x.kv_head}].insert((i - first) % kXcds);
  }
  for (auto& kv : glanes) {
    const auto& ls = kv.second;
    CHECK(*ls.rbegin() - *ls.begin() + 1 == ls.size(), "seed %u: a chunk group's lanes are not contiguous", seed);
  }
  return true;
}

int main(int argc, char** argv) {
  const int launches = argc > 1 ? std::atoi(argv[1]) : 300;
  std::mt19937 rng(12345);
  const int heads[][2] = {{32, 8}, {64, 8}, {8, 8}, {28, 4}, {16, 2}, {64, 1}};
  int done = 0;
  for (int it = 0; it < launches; ++it) {
    const unsigned seed = rng();
    std::mt19937 g(seed);
    const auto& h = heads[g() % 6];
    const int d = (g() & 1) ? 128 : 64;
    const int nreq = 1 + int(g() % 12);
    std::vector<int32_t> P, E;
    for (int r = 0; r < nreq; ++r) {
      const int kind = int(g() % 4);
      const int p = int(g() % (kind == 0 ? 20000 : 9000));
      const int e = kind == 0 ? 1 + int(g() % 3000) : (kind == 1 ? 1 + int(g() % 16) : 1);
      P.push_back(kind == 3 ? 0 : p);
      E.push_back(kind == 3 ? 1 + int(g() % 700) : e);
    }
    if (!check_launch(P, E, h[0], h[1], d, (g() & 3) == 0, seed)) break;
    ++done;
  }
  // launches of decode and verify rows only (wide-split launches among them)
  for (int it = 0; it < launches / 2; ++it) {
    const unsigned seed = rng();
    std::mt19937 g(seed);
    const auto& h = heads[g() % 6];
    const int d = (g() & 1) ? 128 : 64;
    const int nreq = 1 + int(g() % 40);
    const int emax = 1 + int(g() % 8);
    std::vector<int32_t> P, E;
    for (int r = 0; r < nreq; ++r) {
      P.push_back(int(g() % 30000));
      E.push_back(1 + int(g() % emax));
    }
    if (fails || !check_launch(P, E, h[0], h[1], d, (g() & 3) == 0, seed)) break;
    ++done;
  }
  // the pages' workloads
  std::vector<int32_t> P, E;
  for (int i = 0; i < 64; ++i) { P.push_back(511 + int(rng() % 7681)); E.push_back(1); }
  P.push_back(6144); E.push_back(1984);
  if (fails == 0 && check_launch(P, E, 32, 8, 128, false, 1)) ++done;
  if (fails == 0 && check_launch({130048}, {1024}, 64, 8, 128, true, 2)) ++done;
  if (fails == 0 && check_launch({16384}, {8192}, 32, 8, 128, false, 3)) ++done;
  if (fails == 0 && check_launch({0}, {16}, 1, 1, 64, false, 4)) ++done;
  std::printf("%d launches checked, %d failures\n", done, fails);
  return fails == 0 ? 0 : 1;
}
