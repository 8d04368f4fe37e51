// Host-side planning: the chunk plan of one prompt and the work list of one
// extend-attention launch.
#include <algorithm>
#include <array>
#include <cmath>
#include <cstdint>
#include <map>

#include "../../include/extattn.h"
#include "internal.hpp"

namespace extattn {

// Chunk plan (msmodeling chunked-prefill RFC, sections 2.2 and 3.1.3; zdszero
// notes, section "prefill as several resumable extends"): the cached prefix is
// floor(N * hit_rate) with one double multiply; the remaining effective tokens
// are cut into ceil(effective / C) chunks of C tokens, the last one shorter.
int chunk_plan_impl(int64_t n_tokens, int64_t chunk_size, double hit_rate, int64_t* cached,
                    int64_t* effective, int64_t* n_chunks, int64_t* prefix_lens, int64_t* extend_lens,
                    int64_t capacity, const char** why) {
  if (n_tokens < 1) { *why = "n_tokens must be >= 1"; return EXTATTN_EINVAL; }
  if (chunk_size < 1) { *why = "chunk_size must be >= 1"; return EXTATTN_EINVAL; }
  if (!(hit_rate >= 0.0 && hit_rate <= 1.0)) { *why = "hit_rate must lie in [0, 1]"; return EXTATTN_EINVAL; }
  if (!cached || !effective || !n_chunks) { *why = "null output pointer"; return EXTATTN_EINVAL; }
  volatile double product = static_cast<double>(n_tokens) * hit_rate;  // one IEEE multiply, no fusion
  const int64_t c = static_cast<int64_t>(std::floor(product));
  const int64_t eff = n_tokens - c;
  if (eff < 1) { *why = "effective length after prefix-cache hits must be >= 1"; return EXTATTN_EINVAL; }
  const int64_t k = eff / chunk_size + (eff % chunk_size != 0);
  *cached = c;
  *effective = eff;
  *n_chunks = k;
  if (capacity < k) { *why = "capacity is smaller than the number of chunks"; return EXTATTN_ENOSPC; }
  if (!prefix_lens || !extend_lens) { *why = "null plan array"; return EXTATTN_EINVAL; }
  for (int64_t t = 0; t < k; ++t) {
    const int64_t done = std::min(t * chunk_size, eff);
    prefix_lens[t] = c + done;
    extend_lens[t] = std::min(chunk_size, eff - done);
  }
  return EXTATTN_OK;
}

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Lead of the chunk items over the split items in the launch order (percent of the
// split work): see the interleave in build_plan.
constexpr int64_t kChunkLeadPct = 30;

// Launch order of the work items. Workgroups are dealt round-robin to the kXcds
// accelerator dies (workgroup b to die b % kXcds, each die with its own L2) and
// dispatched in order within a die, so the list is built as kXcds lanes, one per
// die, read out round-robin:
//  * the chunk groups (tiles sharing one K/V range), longest first, are laid end
//    to end and dealt to the lanes as contiguous runs of equal length, so that a
//    group's tiles sit on one lane (or a few adjacent ones), consecutive, run side
//    by side and read their K/V into that die's L2 once;
//  * split items (decode / verify rows), longest first, fill the lanes to equal
//    item counts, each to the lane with the most room and then the least work;
//  * within a lane the chunk and split items are interleaved so that both kinds
//    advance through their work at the same rate: chunk rows (matrix-core bound)
//    and decode rows (HBM bound) then run side by side on different CUs from the
//    start instead of the decode rows waiting for the chunk rows' CUs. The chunk
//    items run ahead by kChunkLeadPct percent of the split work, so that the long
//    chunk items are all under way while short split items remain for the end.
// Work is estimated as rows x keys for a chunk item and keys for a split item.
static void order_items(std::vector<std::vector<WorkItem>>& groups, std::vector<WorkItem>& split_items,
                        std::vector<WorkItem>& out) {
  // Items are moved by index (into `pool`: the chunk groups' items, then the split
  // items) and gathered once at the end.
  std::vector<WorkItem> pool;
  std::vector<int64_t> work;
  std::vector<std::pair<uint32_t, uint32_t>> granges;  // [begin, end) in pool
  size_t n_chunk = 0;
  for (const auto& g : groups) n_chunk += g.size();
  const size_t n_total = n_chunk + split_items.size();
  pool.reserve(n_total);
  work.reserve(n_total);
  for (const auto& g : groups) {
    granges.push_back({uint32_t(pool.size()), uint32_t(pool.size() + g.size())});
    for (const WorkItem& x : g) {
      pool.push_back(x);
      work.push_back(int64_t(x.key_end - x.key_begin) * x.nrows);
    }
  }
  for (const WorkItem& x : split_items) {
    pool.push_back(x);
    work.push_back(int64_t(x.key_end - x.key_begin));
  }
  std::vector<uint32_t> idx(n_total);
  for (size_t i = 0; i < n_total; ++i) idx[i] = uint32_t(i);
  auto by_work = [&](uint32_t a, uint32_t b) { return work[a] > work[b]; };
  std::vector<int64_t> gwork(groups.size(), 0);
  for (size_t i = 0; i < groups.size(); ++i) {
    std::stable_sort(idx.begin() + granges[i].first, idx.begin() + granges[i].second, by_work);
    for (uint32_t k = granges[i].first; k < granges[i].second; ++k) gwork[i] += work[k];
  }
  std::vector<size_t> gorder(groups.size());
  for (size_t i = 0; i < gorder.size(); ++i) gorder[i] = i;
  std::stable_sort(gorder.begin(), gorder.end(), [&](size_t a, size_t b) { return gwork[a] > gwork[b]; });
  // The groups, longest first, one after the other, dealt to the lanes as contiguous
  // runs of equal length: a group lands on one lane or on a few adjacent ones, and
  // every lane gets the same number of chunk items (the read-out below only maps
  // list positions to dies while the lanes are equally long).
  std::vector<uint32_t> all_chunk;
  all_chunk.reserve(n_chunk);
  for (size_t gi : gorder)
    all_chunk.insert(all_chunk.end(), idx.begin() + granges[gi].first, idx.begin() + granges[gi].second);
  struct Lane {
    size_t c0 = 0, c1 = 0;  // chunk items all_chunk[c0, c1)
    std::vector<uint32_t> split;
    int64_t cwork = 0, swork = 0;
  };
  std::vector<Lane> lanes(kXcds);
  {
    const size_t per = n_chunk / lanes.size(), extra = n_chunk % lanes.size();
    size_t at = 0;
    for (size_t l = 0; l < lanes.size(); ++l) {
      lanes[l].c0 = at;
      lanes[l].c1 = at + per + (l < extra ? 1 : 0);
      for (size_t k = lanes[l].c0; k < lanes[l].c1; ++k) lanes[l].cwork += work[all_chunk[k]];
      at = lanes[l].c1;
    }
  }
  std::stable_sort(idx.begin() + n_chunk, idx.end(), by_work);
  const int64_t target = int64_t((n_total + lanes.size() - 1) / lanes.size());
  int64_t room[kXcds], swork[kXcds];
  for (int l = 0; l < kXcds; ++l) {
    room[l] = target - int64_t(lanes[l].c1 - lanes[l].c0);
    swork[l] = 0;
    lanes[l].split.reserve(size_t(std::max<int64_t>(room[l], 0)));
  }
  for (size_t k = n_chunk; k < n_total; ++k) {
    const uint32_t x = idx[k];
    int best = 0;
    for (int l = 1; l < kXcds; ++l)
      if (room[l] > room[best] || (room[l] == room[best] && swork[l] < swork[best])) best = l;
    lanes[best].split.push_back(x);
    --room[best];
    swork[best] += work[x];
  }
  for (int l = 0; l < kXcds; ++l) lanes[l].swork = swork[l];
  // interleave within each lane
  std::vector<std::vector<uint32_t>> seq(lanes.size());
  for (size_t l = 0; l < lanes.size(); ++l) {
    const Lane& ln = lanes[l];
    seq[l].reserve(ln.c1 - ln.c0 + ln.split.size());
    size_t ci = ln.c0, si = 0;
    int64_t cdone = 0, sdone = 0;
    while (ci < ln.c1 || si < ln.split.size()) {
      // next item from the list whose dispatched fraction (with the chunk lead) is smaller
      const bool take_chunk =
          si == ln.split.size() ||
          (ci < ln.c1 && __int128(cdone) * ln.swork * (100 - kChunkLeadPct) <= __int128(sdone) * ln.cwork * 100);
      if (take_chunk) {
        cdone += work[all_chunk[ci]];
        seq[l].push_back(all_chunk[ci++]);
      } else {
        sdone += work[ln.split[si]];
        seq[l].push_back(ln.split[si++]);
      }
    }
  }
  // read the lanes out round-robin
  out.clear();
  out.reserve(n_total);
  for (size_t k = 0; out.size() < n_total; ++k)
    for (size_t l = 0; l < seq.size(); ++l)
      if (k < seq[l].size()) out.push_back(pool[seq[l][k]]);
}

// Work list of one launch. Requests whose E * group rows fit two 16-row MFMA
// blocks (decode rows, multi-token verify rows) take the split path: the key range
// is cut into pieces (one workgroup each, one part per wave); each workgroup
// merges its waves' parts and leaves one partial result, and the combine kernel
// merges the workgroups' partials. Longer chunks take the chunk path:
// kRowsPerTile-row tiles over their whole causal key range.
int build_plan(int32_t num_seqs, const int32_t* prefix, const int32_t* extend, int32_t hq, int32_t hkv,
               int32_t head_dim, int32_t dtype, Plan& plan, bool with_append) {
  const int32_t group = hq / hkv;
  plan.seqs.resize(num_seqs);
  plan.items.clear();
  plan.tasks.clear();
  plan.n_slot_floats = 0;
  plan.split_keys = 0;
  plan.n_append = 0;
  int64_t q_off = 0;
  for (int32_t r = 0; r < num_seqs; ++r) {
    plan.seqs[r] = SeqInfo{static_cast<int32_t>(q_off), prefix[r], extend[r], 0};
    q_off += extend[r];
  }
  plan.total_rows = q_off;

  if (dtype == EXTATTN_BF16) {
    std::vector<WorkItem> split_items;
    // Chunk items by group: the tiles of one (request, KV head, key piece) read the
    // same K/V range, so they are launched side by side on one XCD (shared L2).
    std::vector<std::vector<WorkItem>> groups;
    std::map<std::array<int64_t, 3>, size_t> group_of;
    auto add_chunk = [&](const WorkItem& x, int64_t piece_index) {
      const std::array<int64_t, 3> key{x.seq, x.kv_head, piece_index};
      auto f = group_of.find(key);
      if (f == group_of.end()) {
        f = group_of.emplace(key, groups.size()).first;
        groups.emplace_back();
      }
      groups[f->second].push_back(x);
    };
    // Keys per split workgroup: every workgroup pays a fixed start-up (ids, first
    // loads in flight) while it holds its CU alone, so pieces are as long as the
    // work allows while still giving about kSplitTargetItems workgroups; a multiple
    // of kWaves tiles, between kSplitKeysMin and kSplitKeysMax.
    int64_t split_keys = 0, max_rows = 0;
    for (int32_t r = 0; r < num_seqs; ++r) {
      if (int64_t(extend[r]) * group <= kFewRows) split_keys += (int64_t(prefix[r]) + extend[r]) * hkv;
      max_rows = std::max<int64_t>(max_rows, int64_t(extend[r]) * group);
    }
    // Launches of decode / verify rows only, some past the 8-wave split items'
    // kSplitMaxRows rows (and none past kWideMaxRows): every request becomes split
    // items of the 4-wave wide kernel, which reads each context once for up to 64
    // rows.
    plan.wide = max_rows > kSplitMaxRows && max_rows <= kWideMaxRows;
    const int64_t split_max_rows = plan.wide ? kWideMaxRows : kSplitMaxRows;
    const int split_waves = plan.wide ? kWideWaves : kWaves;
    const int64_t kGrain = int64_t(kSplitTile) * split_waves;
    const int64_t target = plan.wide ? kWideTargetItems : kSplitTargetItems;
    int64_t piece = (split_keys + target - 1) / target;
    piece = (piece + kGrain - 1) / kGrain * kGrain;
    piece = std::min<int64_t>(std::max<int64_t>(piece, kSplitKeysMin), split_keys_max(split_waves));
    plan.split_keys = int32_t(piece);
    // Chunk rows: when the chunk tiles alone cannot fill the GPU (short chunks, few
    // heads), each tile's key range is cut into pieces, one workgroup each, and the
    // combine kernel merges the pieces by the page's rule (the one-GPU share of a
    // context-parallel split of the prefix).
    // The tiles take floor(target / tiles) pieces each, so that the pieces fill whole
    // rounds of the CUs, also next to split items (measured on the mixed step, whose
    // 248 tiles then run whole: 0.385-0.390 ms a call against 0.393-0.398 with two
    // pieces a tile and the combine of their partials, kernel span unchanged).
    int64_t chunk_tiles = 0;
    for (int32_t r = 0; r < num_seqs; ++r) {
      const int64_t rows = int64_t(extend[r]) * group;
      if (rows > split_max_rows) chunk_tiles += (rows + kRowsPerTile - 1) / kRowsPerTile * hkv;
    }
    const int64_t chunk_pieces = chunk_tiles == 0 ? 1 : std::max<int64_t>(1, kChunkTargetItems / chunk_tiles);
    for (int32_t r = 0; r < num_seqs; ++r) {
      const int64_t rows = int64_t(extend[r]) * group;
      const int64_t kv_len = int64_t(prefix[r]) + extend[r];
      if (rows <= split_max_rows) {
        const int32_t srows = int32_t((rows + kSplitRows - 1) / kSplitRows * kSplitRows);  // rows of a partial slot
        const int64_t nwg = (kv_len + piece - 1) / piece;
        const int64_t sf = int64_t(slot_floats(srows, head_dim));
        for (int32_t g = 0; g < hkv; ++g) {
          const int64_t slot0 = plan.n_slot_floats;
          const int32_t task = nwg > 1 ? int32_t(plan.tasks.size()) : -1;
          for (int64_t w = 0; w < nwg; ++w) {
            const int64_t kb = w * piece;
            const int64_t ke = std::min<int64_t>(kv_len, kb + piece);
            split_items.push_back(WorkItem{kItemSplit, r, g, 0, int32_t(rows), int32_t(kb), int32_t(ke),
                                           int32_t(nwg > 1 ? slot0 + w * sf : -1), task, nwg > 1 ? srows : 0,
                                           {0, 0}});
          }
          if (nwg > 1) {
            plan.tasks.push_back(CombineTask{r, g, 0, int32_t(rows), int32_t(slot0), int32_t(nwg), int32_t(sf),
                                             srows, 0, {0, 0, 0}});
            plan.n_slot_floats += nwg * sf;
          }
        }
      } else {
        const int64_t ntiles = (rows + kRowsPerTile - 1) / kRowsPerTile;
        for (int32_t g = 0; g < hkv; ++g) {
          for (int64_t t = 0; t < ntiles; ++t) {
            const int64_t row0 = t * kRowsPerTile;
            const int64_t nrows = std::min<int64_t>(kRowsPerTile, rows - row0);
            const int64_t pos_max = (row0 + nrows - 1) / group;
            const int64_t key_end = int64_t(prefix[r]) + pos_max + 1;
            const int64_t ktiles = (key_end + kChunkKeys - 1) / kChunkKeys;
            int64_t pieces = std::max<int64_t>(1, std::min<int64_t>(chunk_pieces, key_end / kChunkMinPieceKeys));
            // tiles of few rows (verify rows past the split path's reach, ragged last
            // tiles) stream their keys like split items: pieces of the split length
            if (nrows <= kFewRows) pieces = std::max<int64_t>(pieces, (key_end + piece - 1) / piece);
            if (pieces == 1) {
              add_chunk(WorkItem{kItemChunk, r, g, int32_t(row0), int32_t(nrows), 0, int32_t(key_end), -1, -1, 0,
                                 {0, 0}},
                        0);
              continue;
            }
            // pieces of about equal tile counts; the last one holds the diagonal. A
            // partial slot holds the tile's rows rounded up to 16 (not a whole tile:
            // a few-row tile may have many pieces)
            const int32_t srows = int32_t((nrows + 15) / 16 * 16);
            const int64_t sf = int64_t(slot_floats(srows, head_dim));
            const int64_t slot0 = plan.n_slot_floats;
            const int32_t task0 = int32_t(plan.tasks.size());
            for (int64_t i = 0; i < pieces; ++i) {
              const int64_t kb = ktiles * i / pieces * kChunkKeys;
              const int64_t ke = i + 1 < pieces ? ktiles * (i + 1) / pieces * kChunkKeys : key_end;
              add_chunk(WorkItem{kItemChunk, r, g, int32_t(row0), int32_t(nrows), int32_t(kb), int32_t(ke),
                                 int32_t(slot0 + i * sf), task0, srows, {0, 0}},
                        i);
            }
            for (int64_t sr = 0; sr < nrows; sr += kCombineRows)
              plan.tasks.push_back(CombineTask{r, g, int32_t(row0 + sr),
                                               int32_t(std::min<int64_t>(kCombineRows, nrows - sr)), int32_t(slot0),
                                               int32_t(pieces), int32_t(sf), srows, int32_t(sr), {0, 0, 0}});
            plan.n_slot_floats += pieces * sf;
          }
        }
      }
    }
    order_items(groups, split_items, plan.items);
    if (with_append) {
      // Fused append: the launch's first workgroups (the heads of every die's
      // dispatch order) copy the new tokens before their own items, so every die
      // dispatches them before any work that waits for them.
      plan.n_append = int32_t(std::min<size_t>(plan.items.size(), kAppendProducers));
      // A launch of at most one workgroup per CU runs all its items at once, so
      // their order in a lane does not matter for the balance: reversed, each
      // lane starts with its shortest items, which then also copy the new tokens.
      const size_t n = plan.items.size();
      if (n <= size_t(kChunkTargetItems))
        for (size_t l = 0; l < size_t(kXcds) && l < n; ++l) {
          size_t lo = l, hi = l + (n - 1 - l) / kXcds * kXcds;
          for (; lo < hi; lo += kXcds, hi -= kXcds) std::swap(plan.items[lo], plan.items[hi]);
        }
    }
  }

  // slot offsets travel as int32 floats
  if (plan.n_slot_floats > INT32_MAX) return EXTATTN_ENOSPC;
  size_t off = kHeaderBytes;
  plan.off_zero = off;
  off += kZeroPageBytes;
  plan.off_seqs = off;
  off = align_up(off + sizeof(SeqInfo) * num_seqs, 256);
  plan.off_items = off;
  off = align_up(off + sizeof(WorkItem) * plan.items.size(), 256);
  plan.off_tasks = off;
  off = align_up(off + sizeof(CombineTask) * plan.tasks.size(), 256);
  plan.upload_bytes = off;
  plan.off_slots = off;
  off = align_up(off + sizeof(float) * size_t(plan.n_slot_floats), 256);
  plan.bytes = off;
  return EXTATTN_OK;
}

}  // namespace extattn
