// Chunk rows on 32-key tiles, shared by the chunk-only kernel and the mixed kernel.
//
// What is computed (zdszero "Chunked Prefill" notes, section "prefill as several
// resumable extends"): query token i of a chunk at global position P + i takes the
// softmax over keys 0 .. P+i of scale * q.k_j and applies it to v_j; the rectangle
// (keys below P, no mask) and the triangle (the chunk's own keys, causal) are swept
// by one running (m, l) state, which is the page's merge rule applied tile by tile.
// A work item that covers a piece of the key range ends in a partial (o, lse) that
// the combine kernel merges by the same rule.
//
// Layout (chunk_item_t<D, RB, WAVES>; the kernels use RB = 1, WAVES = 8):
//  * A workgroup holds 256 flattened rows (position, head-in-group) of one (request,
//    KV head), 32 * RB per wave, so the whole GQA group shares each K/V tile.
//  * Each 32-key step runs three tiles at once: the Q.K products of tile j+2, the
//    softmax weights of tile j+1 and the P.V products of tile j, interleaved so that
//    every MFMA has a share of the exponentials beside it (two waves per SIMD then
//    keep the matrix core and the vector ALU busy together).
//  * K and V tiles go from the paged cache straight into 8-slot LDS rings
//    (global_load_lds_dwordx4), 8 and 6 tiles ahead of their P.V step, with one
//    barrier every two steps that leaves the last four steps' copies in flight; each
//    wave copies one 1 KB piece of every tile.
//  * Scores are the fp32 products of the given bf16 q and k; the weights are
//    2^(s c - m), c = scale * log2(e), one fma and one exp2 per score, so lse is the
//    log-sum-exp of exactly those scores. m is the first tile's exact row max; a wave
//    whose later weights pass 2^64 against it redoes its rows on an exact two-pass
//    path (chunk_rows_exact).
#pragma once

#include <type_traits>

#include "attn_bf16_common.hpp"

namespace extattn {

constexpr int kChunkRing = 8;  // LDS ring slots per operand (K, V) of the chunk kernel

// Bound on one lane's sum of a tile's 16 weights in the fast loop. The running max
// m is fixed by the first tile, so later weights grow with the scores; up to 2^64
// they are exact in fp32 and in bf16, and O and l (at most 2^17 keys of them) stay
// far below the fp32 range.
constexpr float kFastBound = 18446744073709551616.0f;  // 2^64

// A wave's rows computed exactly in two passes over their keys, straight from
// the paged cache (the rare path): the row max first, then the weights
// 2^(s c - m) against it, their fp32 sum and the weighted values. One lane per row.
// Invalid block ids read as zeros, as in the fast loop (which reported them).
template <int D, int RB>
__device__ void chunk_rows_exact(const AttnArgs& a, const WorkItem& it, int wave, int lane) {
  const int rloc = wave * RB * kRowsPerWave + lane;
  if (lane >= RB * kRowsPerWave || rloc >= it.nrows) return;
  const SeqInfo si = a.seqs[it.seq];
  const int G = a.group, g = it.kv_head;
  const int rho = it.row0 + rloc, pos = rho / G, hh = rho - pos * G;
  const int64_t orow = int64_t(si.q_off + pos) * a.hq + g * G + hh;
  const int lim = min(si.prefix + pos, it.key_end - 1);
  const int32_t* bt = a.block_table + int64_t(it.seq) * a.max_blocks;
  const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache);
  const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache);
  const float c2 = a.scale_log2;
  u32x4 qv[D / 8];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + orow * D;
#pragma unroll
    for (int c = 0; c < D / 8; ++c) qv[c] = *reinterpret_cast<const u32x4*>(qp + 8 * c);
  }
  auto lo = [](uint32_t w) { return __uint_as_float(w << 16); };
  auto hi = [](uint32_t w) { return __uint_as_float(w & 0xffff0000u); };
  auto block_base = [&](int j, const uint16_t* cache) -> const uint16_t* {
    const int32_t phys = bt[j / kBlockSize];
    return block_ok(phys, a.num_blocks) ? cache + (int64_t(phys) * a.hkv + g) * (kBlockSize * D) : nullptr;
  };
  auto score = [&](int j) -> float {
    const uint16_t* kb = block_base(j, kc);
    if (!kb) return 0.f;
    const uint16_t* kp = kb + (j % kBlockSize) * D;
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
      const u32x4 kk = *reinterpret_cast<const u32x4*>(kp + 8 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s = fmaf(lo(qv[c][e]), lo(kk[e]), s);
        s = fmaf(hi(qv[c][e]), hi(kk[e]), s);
      }
    }
    return s;
  };
  float mx = -INFINITY;
  for (int j = it.key_begin; j <= lim; ++j) mx = fmaxf(mx, score(j));
  const float m = mx * c2;
  float l = 0.f;
  for (int j = it.key_begin; j <= lim; ++j) l += __builtin_amdgcn_exp2f(fmaf(score(j), c2, -m));
  const float inv = 1.f / l;
  const float lse = (m + __builtin_amdgcn_logf(l)) * kLn2;
  if (it.slot < 0 && a.lse) a.lse[orow] = lse;
  if (it.slot >= 0) a.slots[it.slot + it.slot_rows * D + rloc] = lse;
  // the weighted values, 32 features at a time
#pragma unroll 1
  for (int d0 = 0; d0 < D; d0 += 32) {
    float acc[32];
#pragma unroll
    for (int d = 0; d < 32; ++d) acc[d] = 0.f;
    for (int j = it.key_begin; j <= lim; ++j) {
      const float p = __builtin_amdgcn_exp2f(fmaf(score(j), c2, -m));
      const uint16_t* vb = block_base(j, vc);
      if (vb) {
        const uint16_t* vp = vb + d0 * kBlockSize + (j % kBlockSize);
#pragma unroll
        for (int d = 0; d < 32; ++d) acc[d] = fmaf(p, __uint_as_float(uint32_t(vp[d * kBlockSize]) << 16), acc[d]);
      }
    }
    if (it.slot < 0) {
      uint16_t* op = static_cast<uint16_t*>(a.out) + orow * D + d0;
#pragma unroll
      for (int d = 0; d < 32; d += 4) {
        const u32x2 pk = {pack2(acc[d] * inv, acc[d + 1] * inv), pack2(acc[d + 2] * inv, acc[d + 3] * inv)};
        *reinterpret_cast<u32x2*>(op + d) = pk;
      }
    } else {
      float* sl = a.slots + it.slot + rloc * D + d0;  // rows [slot_rows][D], then lse [slot_rows]
#pragma unroll
      for (int d = 0; d < 32; d += 4)
        *reinterpret_cast<float4*>(sl + d) = float4{acc[d] * inv, acc[d + 1] * inv, acc[d + 2] * inv, acc[d + 3] * inv};
    }
  }
}

template <int D, int RB, int WAVES>
__device__ void chunk_item_t(const AttnArgs& a, const WorkItem& it, unsigned char* smem) {
  constexpr int KT = kChunkKeys;                  // keys per tile
  constexpr int NC = D / 8;                       // 16-byte pieces per K row
  constexpr int KS = D / 16;                      // MFMA k-steps over the head dim
  constexpr int DB = D / 32;                      // 32-feature blocks of O^T
  constexpr int NB = 2 * DB;                      // (16-key half, feature block) P.V products
  constexpr int KT_BYTES = KT * D * 2;            // one K tile (= one V tile)
  constexpr int VSUB = D * kBlockSize * 2;        // one V^T sub-tile (16 keys)
  constexpr int PIECES = KT_BYTES / 1024;         // 1 KB direct loads per tile (K and V each)
  constexpr int NINST = PIECES >= WAVES ? PIECES / WAVES : 1;  // per wave and tile (waves past PIECES copy none)
  constexpr int THREADS = 64 * WAVES;
  constexpr int RING = kChunkRing;                // LDS ring slots per operand (= loop unroll)
  constexpr int KLEAD = 8, VLEAD = 6;             // tiles a copy runs ahead of its step's P.V tile
  // Copies issued in the last OUT steps may still be in flight at a barrier: the two
  // steps after a barrier read K(u+3), K(u+4), V(u+1), V(u+2), issued KLEAD - 2 and
  // VLEAD steps before their reads, so OUT <= min(KLEAD - 4, VLEAD - 2). A K copy
  // overwrites the slot last read 2 steps earlier and a V copy the slot last read
  // 8 - VLEAD steps earlier, each across a barrier (barriers follow odd steps), so
  // KLEAD <= 8 and VLEAD <= 6 with 8 slots.
  constexpr int OUT = (KLEAD - 4 < VLEAD - 2) ? KLEAD - 4 : VLEAD - 2;
  static_assert(KLEAD <= RING && VLEAD <= RING - 2 && KLEAD >= VLEAD && OUT >= 1 && KLEAD % 2 == 0,
                "ring leads");
  constexpr int KBUF = 0, VBUF = RING * KT_BYTES, IDBUF = 2 * RING * KT_BYTES;
  constexpr int PPS = 8 / KS;                     // weight pairs of a row block per interleave slot
  static_assert(KS == NB, "one Q.K and one P.V product per row block and slot");
  static_assert(PIECES % WAVES == 0 || WAVES % PIECES == 0, "pieces must split evenly over the waves");
  static_assert(8 % KS == 0, "pairs split evenly over the slots");

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const SeqInfo si = a.seqs[it.seq];
  const int G = a.group, g = it.kv_head;
  const int kv_len = si.prefix + si.extend;
  // Waves whose 64 rows all lie past the item's rows still copy their share of
  // every tile and keep the barriers, but skip the products (wave-uniform test).
  const bool wave_rows = wave * (RB * kRowsPerWave) < it.nrows;
  const float c2 = a.scale_log2;

  int rloc[RB], lim[RB];
  bool valid[RB];
  int64_t orow[RB];
  u32x4 qf[RB][KS];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    rloc[b] = wave * (RB * kRowsPerWave) + b * kRowsPerWave + l32;
    valid[b] = rloc[b] < it.nrows;
    const int rho = it.row0 + rloc[b];
    const int pos = valid[b] ? rho / G : 0;
    const int hh = valid[b] ? rho - pos * G : 0;
    orow[b] = int64_t(si.q_off + pos) * a.hq + g * G + hh;
    lim[b] = valid[b] ? min(si.prefix + pos, it.key_end - 1) : -1;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + orow[b] * D + hi * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[b][ks] = valid[b] ? *reinterpret_cast<const u32x4*>(qp + ks * 16) : zero4();
      // With one wave per SIMD (two row blocks) Q is only ever an MFMA operand, which
      // may come from the accumulation registers: keep it there, so that the vector
      // registers hold the scores the softmax works on
      if constexpr (RB == 2) asm volatile("" : "+a"(qf[b][ks]));
    }
  }
  // Q's loads are waited for here, once: otherwise the compiler waits for them at
  // their first use in every step (each step's products sit under a branch), and
  // such a wait (vmcnt 0) also drains the tile copies in flight.
  if constexpr (RB == 1) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(qf[0][ks]));
  }
  const int lim_min = min(si.prefix + it.row0 / G, it.key_end - 1);

  const int32_t* bt = a.block_table + int64_t(it.seq) * a.max_blocks;
  const int nblk = (kv_len + kBlockSize - 1) / kBlockSize;
  const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache);
  const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache);

  // LDS operand reads (swizzles as in the helpers' layout description).
  const int k_off0 = key_of_row(l32) * (D * 2) + (((hi ^ (l32 & 15)) & (NC - 1)) << 4);
  const int v_off = l32 * (kBlockSize * 2) + ((hi ^ swz_v(l32)) << 4);
  // This lane's V-ring base, held in a register: the ring sits above 64 KB, so with
  // the ring's offset folded into each read's address the reads would each need an
  // add; from this base every slot and sub-tile offset fits the reads' 16-bit
  // immediate.
  uint32_t vbase = lds_addr(smem + VBUF) + uint32_t(v_off);
  asm volatile("" : "+v"(vbase));

  const int t0 = it.key_begin / KT;
  const int t1 = (it.key_end + KT - 1) / KT;
  const int n = t1 - t0;

  // Block ids go through a 2-window LDS ring (2 x 32 tiles x 2 blocks) filled by direct
  // loads (wave 0); window k covers tiles t0 + 32k .. t0 + 32k + 31 and sits in ring
  // half k & 1. From there each lane holds the 64-bit K and V source addresses of one
  // (tile, 16-key block) entry, lane (tile & 31) * 2 + block, so that a copy needs two
  // readlanes and no scalar arithmetic. Step u copies K of tile u + KLEAD and V of
  // tile u + VLEAD, so the register is refreshed half at a time: the lower half (tiles
  // 32k .. 32k+15) at step 32k - KLEAD, the upper half at step 32k + 16 - KLEAD, each
  // after the last copy that read the entries it replaces. Entries past the sequence end or past the range,
  // and ids outside [0, num_blocks), point at the zero page; the invalid ones are
  // reported as their entries are made.
  int32_t* id_ring = reinterpret_cast<int32_t*>(smem + IDBUF);
  auto fill_ids = [&](int k) {  // window k into ring half k & 1
    if (wave != 0) return;
    const int lb = (t0 + 32 * k) * (KT / kBlockSize) + lane;
    const int src = lb < nblk ? lb : nblk - 1;
    dma4(bt, uint32_t(src) * 4u, lds_addr(id_ring + (k & 1) * 64));
  };
  const unsigned char* kc_g = reinterpret_cast<const unsigned char*>(kc + int64_t(g) * (kBlockSize * D));
  const unsigned char* vc_g = reinterpret_cast<const unsigned char*>(vc + int64_t(g) * (kBlockSize * D));
  const uint64_t blk_bytes = uint64_t(a.hkv) * (kBlockSize * D * 2);
  uint32_t akl = 0, akh = 0, avl = 0, avh = 0;  // this lane's entry: K and V source addresses
  // Entries of window k: lanes of ring half `half` (0: lanes 0..31, 1: lanes 32..63), or all.
  auto make_entries = [&](int k, int half) {
    const int32_t v = id_ring[(k & 1) * 64 + lane];
    const bool mine = half < 0 || (lane >> 5) == half;
    const bool inside = (t0 + 32 * k) * (KT / kBlockSize) + lane < nblk;
    const bool ok = block_ok(v, a.num_blocks);
    const uint64_t bad = __builtin_amdgcn_ballot_w64(mine && inside && !ok);
    if (bad != 0 && wave == 0 && lane == 0) report_bad_blocks(a.err, int(__builtin_popcountll(bad)));
    const bool use = inside && ok && t0 + 32 * k + (lane >> 1) < t1;
    const uint64_t off = uint64_t(uint32_t(use ? v : 0)) * blk_bytes;
    const uint64_t zp = reinterpret_cast<uint64_t>(a.zero_page);
    const uint64_t ka = use ? reinterpret_cast<uint64_t>(kc_g) + off : zp;
    const uint64_t va = use ? reinterpret_cast<uint64_t>(vc_g) + off : zp;
    if (mine) {
      akl = uint32_t(ka);
      akh = uint32_t(ka >> 32);
      avl = uint32_t(va);
      avh = uint32_t(va >> 32);
    }
  };
  auto entry = [&](uint32_t lo, uint32_t hi, int idx) -> const void* {
    const uint32_t l = __builtin_amdgcn_readlane(lo, idx), h = __builtin_amdgcn_readlane(hi, idx);
    return reinterpret_cast<const void*>((uint64_t(h) << 32) | l);
  };
  // Per-lane sources (within a block) and LDS destinations of this wave's pieces
  // x = 0 .. NINST-1 (piece wave + WAVES x of the tile, in 16-key block my_blk[x]).
  uint32_t k_src[NINST], v_src[NINST], k_dst[NINST], v_dst[NINST];
  int my_blk[NINST];
#pragma unroll
  for (int x = 0; x < NINST; ++x) {
    const int i = wave + WAVES * x;
    my_blk[x] = (i % PIECES) / (PIECES / 2);
    const int nn = i * 64 + lane;
    const int r = nn / NC, c = nn % NC;
    k_src[x] = uint32_t(((r & 15) * D + ((c ^ (key_of_row(r & 15) & (NC - 1))) * 8)) * 2);
    const int d = ((i * 64 + lane) % (VSUB / 16)) / 2, cv = lane & 1;
    v_src[x] = uint32_t((d * kBlockSize + ((cv ^ swz_v(d)) * 8)) * 2);
    k_dst[x] = lds_addr(smem + KBUF) + i * 1024;
    v_dst[x] = lds_addr(smem + VBUF) + i * 1024;
  }
  const bool has_piece = PIECES >= WAVES || wave < PIECES;  // compile-time true when every wave has pieces
  auto issue_k = [&](int v, int slot) {  // K of tile t0 + v into ring slot `slot`
    if (!has_piece) return;
#pragma unroll
    for (int x = 0; x < NINST; ++x)
      dma16(entry(akl, akh, (v & 31) * 2 + my_blk[x]), k_src[x], k_dst[x] + slot * KT_BYTES);
  };
  auto issue_v = [&](int v, int slot) {
    if (!has_piece) return;
#pragma unroll
    for (int x = 0; x < NINST; ++x)
      dma16(entry(avl, avh, (v & 31) * 2 + my_blk[x]), v_src[x], v_dst[x] + slot * KT_BYTES);
  };

  f32x16 o[RB][DB];
  float m[RB], l[RB], mneg[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
#pragma unroll
    for (int db = 0; db < DB; ++db) o[b][db] = f32x16{};
    m[b] = 0.f;
    l[b] = 0.f;
    mneg[b] = 0.f;
  }

  auto row_max = [&](const f32x16& s) -> float {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
    return mx;
  };
  // Causal mask of a diagonal tile (and of keys past the range end), both blocks;
  // tiles before j_mask need none (wave-uniform test).
  const int j_mask =
      __builtin_amdgcn_readfirstlane(lim_min >= KT - 1 ? (lim_min - (KT - 1)) / KT + 1 : 0);
  auto mask = [&](int j, f32x16 (&s)[RB]) {
    if (j >= j_mask) {
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        const int t = lim[b] - j * KT - 8 * hi;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (key_of_elem(i, 0) > t) s[b][i] = -INFINITY;
      }
    }
  };
  // Weights 2^(s c - m) of one block as packed bf16, and this lane's fp32 sum of
  // them (taken before the rounding).
  auto weights = [&](const f32x16& s, float mn, u32x4 (&pf)[2], float& ls) {
    float l0 = 0.f, l1 = 0.f;
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[8 * v + 2 * w], c2, mn));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[8 * v + 2 * w + 1], c2, mn));
        pf[v][w] = pack2(p0, p1);
        l0 += p0;
        l1 += p1;
      }
    ls = l0 + l1;
  };
  // Check of a tile's weights before they enter P.V: a lane whose sum passed
  // kFastBound (or overflowed) marks the wave (`ovf`, wave-uniform). Such a wave
  // runs the loop to its end like the others (its results are dropped, so nothing
  // in the loop depends on the mark) and then redoes its rows exactly.
  bool ovf = false;
  auto check = [&](const float (&ls)[RB]) {
    bool big = false;
#pragma unroll
    for (int b = 0; b < RB; ++b) big = big || !(ls[b] <= kFastBound);
    if (__builtin_amdgcn_ballot_w64(big) != 0) ovf = true;
#pragma unroll
    for (int b = 0; b < RB; ++b) l[b] += ls[b];
  };
  // S^T of one tile for both blocks from K ring slot `slot` (compile-time).
  auto qk = [&](auto slot_tag, f32x16 (&s)[RB]) {
    constexpr int slot = decltype(slot_tag)::value;
    const unsigned char* base = smem + KBUF + slot * KT_BYTES;
#pragma unroll
    for (int b = 0; b < RB; ++b) s[b] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 kf = *reinterpret_cast<const u32x4*>(base + (k_off0 ^ (ks << 5)));
#pragma unroll
      for (int b = 0; b < RB; ++b) s[b] = mfma32(kf, qf[b][ks], s[b]);
    }
  };
  // Values of keys past the sequence end must read as zero (their weights are zero,
  // but the cache slots may hold anything and 0 * NaN would poison O). Only the
  // range's last tile reaches past the end; its V tile is cleared in LDS once, after
  // it has landed and before it is read (the caller puts barriers around this).
  const bool tail_clip = (t1 * KT > kv_len);
  auto clip_tail = [&](int slot) {
    unsigned char* base = smem + VBUF + slot * KT_BYTES;
    const int kt = (t1 - 1) * KT;
    for (int piece = tid; piece < 4 * D; piece += THREADS) {
      const int b = piece / (2 * D), d = (piece / 2) % D, h = piece & 1;
      const int key0 = kt + 16 * b + 8 * (h ^ swz_v(d));
      if (key0 + 8 > kv_len) {
        u32x4* pp = reinterpret_cast<u32x4*>(base + b * VSUB + d * (kBlockSize * 2) + h * 16);
        *pp = clip_keys(*pp, key0, kv_len);
      }
    }
  };

  // Fused append: the launch's first workgroups write the new tokens' K/V (keys P
  // and up) into the cache. Tiles below tile P / 32 hold only older keys, in whole cache
  // blocks the appends never touch, so a wave waits for the appends only before it
  // copies tile P / 32 (relative index v_new), if that tile is in its range.
  const int v_new = (si.prefix >> 5) - t0;
  const bool wait_new = a.n_append > 0 && v_new < n;

  // The wave waits once, at the start of the 8-step group whose steps issue that
  // copy (the prologue, when the copy is among the first KLEAD), so the steps hold
  // no test for it; launches without fused appends run a copy of the loop without
  // the group test.
  auto sweep = [&](auto fused_tag) {
    constexpr bool FUSED = decltype(fused_tag)::value;
    constexpr int kIssuePerStep = 2 * NINST;
    // Prologue: ids of windows 0 and 1; K of tiles t0 .. t0+KLEAD-1 and V of t0 ..
    // t0+VLEAD-1, each tile v in ring slot v % RING.
    fill_ids(0);
    fill_ids(1);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    make_entries(0, -1);
    if (FUSED && v_new < KLEAD) wait_appends_wave<WAVES>(a);
    bool wait_pending = FUSED && v_new >= KLEAD;
#pragma unroll
    for (int v = 0; v < KLEAD; ++v) issue_k(v, v);
#pragma unroll
    for (int v = 0; v < VLEAD; ++v) issue_v(v, v);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    if (tail_clip && n <= VLEAD) {  // the last tile's V is already here
      clip_tail((n - 1) % RING);
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    // otherwise its V (copied at step n-1-VLEAD) has landed by the barrier after
    // step bclip (odd, bclip - OUT >= n-1-VLEAD) and is cleared there, before step
    // n-1 reads it
    const int bfirst = n - 1 - VLEAD + OUT;
    const int bclip = (bfirst & 1) ? bfirst : bfirst + 1;
    static_assert(OUT <= VLEAD - 2, "bclip <= n - 2: the clip lands before step n-1");
    f32x16 sa[RB], sb[RB];
    u32x4 pa[RB][2], pb[RB][2];
    float la[RB], lb[RB];
    // The first tile sets m to the rows' exact max (0 for rows with no visible key);
    // the second tile's scores wait for the first step's softmax.
    if (wave_rows) {
      qk(std::integral_constant<int, 0>{}, sa);
      mask(t0, sa);
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        float mx = row_max(sa[b]);
        mx = fmaxf(mx, partner(mx, hi));
        m[b] = (mx == -INFINITY) ? 0.f : mx * c2;
        mneg[b] = -m[b];
        weights(sa[b], mneg[b], pa[b], la[b]);
      }
      qk(std::integral_constant<int, 1>{}, sb);
    }
    // Steps 0 and 1 copy K of tiles KLEAD and KLEAD+1 into the slots of tiles
    // KLEAD-8 and KLEAD-7; with KLEAD = 8 those are tiles 0 and 1, read just above.
    if constexpr (KLEAD > RING - 2) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    // Step u (tile j = t0 + u): on entry tile j's weights are in px / lsx and S(j+1)
    // (raw) is in sy; K(j+2) sits in K slot (u+2)%RING and V(j) in V slot u%RING. The step
    //   checks tile j's weights (see `check`),
    //   runs KS interleave slots, each with the Q.K products of tile j+2 (into sx)
    //     and the P.V products of tile j for both blocks, next to the exps of tile
    //     j+1's weights (masked if diagonal; packed and summed one slot later, into
    //     py / lsy),
    //   issues the copies of K(j+KLEAD) (slot last read in step u-2) and V(j+VLEAD)
    //     (slot last read in step u+VLEAD-8) after its first and second interleave
    //     slots,
    //   and, after odd steps only, waits for the copies issued up to step u-OUT and
    //     meets the other waves. Between a slot's last read and its next copy, and
    //     between a copy and its first read, lie at least one such barrier (see OUT).
    auto step = [&](auto slot_tag, auto mask_tag, int u, f32x16 (&sx)[RB], f32x16 (&sy)[RB], u32x4 (&px)[RB][2],
                    u32x4 (&py)[RB][2], float (&lsx)[RB], float (&lsy)[RB]) {
      constexpr int sl = decltype(slot_tag)::value;  // u % RING
      constexpr bool diag = decltype(mask_tag)::value;  // tile j+1 may need the causal mask
      const int j = t0 + u;
      // entries: the lower half of window (u + KLEAD) / 32 at u = 32 - KLEAD (mod 32),
      // its upper half at u = 16 - KLEAD (mod 32) (from step 48 - KLEAD on; window 0
      // came whole), each after the last copy (of V, VLEAD behind K) that used the
      // entries it replaces; the next
      // window's ids replace the ring half of the window before at u = 0 (mod 32)
      if constexpr (sl % 2 == 0) {
        if ((u & 31) == 32 - KLEAD) make_entries((u + KLEAD) >> 5, 0);
        if ((u & 31) == 16 - KLEAD && u >= 48 - KLEAD) make_entries((u + KLEAD) >> 5, 1);
        if ((u & 31) == 0 && u > 0) fill_ids((u >> 5) + 1);
      }
      auto issue_kc = [&]() { issue_k(u + KLEAD, (sl + KLEAD) % RING); };
      auto issue_vc = [&]() { issue_v(u + VLEAD, (sl + VLEAD) % RING); };
      if (!wave_rows) {
        issue_kc();
        issue_vc();
      }
      if (wave_rows) {
        check(lsx);
        // In the masked steps (tile j+1 at or past j_mask), weights of keys past a row's
        // last key are set to zero as they are made. Element i of a lane holds key
        // 8 hi + key_of_elem(i, 0) of the tile.
        int tmask[RB];
#pragma unroll
        for (int b = 0; b < RB; ++b) tmask[b] = diag ? lim[b] - (j + 1) * KT - 8 * hi : 0;
        __builtin_amdgcn_sched_barrier(0);
        constexpr int slk = (sl + 2) % RING;  // K slot of tile j+2
        const unsigned char* kb = smem + KBUF + slk * KT_BYTES;
        typedef __attribute__((address_space(3))) const unsigned char lds_byte;
        typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
        lds_byte* vb = reinterpret_cast<lds_byte*>(vbase) + sl * KT_BYTES;
        auto kread = [&](int t) -> u32x4 { return *reinterpret_cast<const u32x4*>(kb + (k_off0 ^ (t << 5))); };
        auto vread = [&](int i) -> u32x4 {
          return *reinterpret_cast<lds_u32x4*>(vb + (i / DB) * VSUB + (i % DB) * 32 * (kBlockSize * 2));
        };
        u32x4 kf[KS], vf[NB];
        float e[RB][16];
        float s0[RB], s1[RB];  // this lane's two partial sums of tile j+1's weights
        auto finish = [&](int b, int pp) {  // pack and sum pair pp of block b
          const int v = pp >> 2, w = pp & 3;
          py[b][v][w] = pack2(e[b][2 * pp], e[b][2 * pp + 1]);
          if (pp == 0) {
            s0[b] = e[b][0];
            s1[b] = e[b][1];
          } else {
            s0[b] += e[b][2 * pp];
            s1[b] += e[b][2 * pp + 1];
          }
        };
        kf[0] = kread(0);
        vf[0] = vread(0);
        kf[1] = kread(1);
        vf[1] = vread(1);
#pragma unroll
        for (int t = 0; t < KS; ++t) {
          if (t + 2 < KS) {
            kf[t + 2] = kread(t + 2);
            vf[t + 2] = vread(t + 2);
          }
#pragma unroll
          for (int b = 0; b < RB; ++b) sx[b] = mfma32(kf[t], qf[b][t], t == 0 ? f32x16{} : sx[b]);
#pragma unroll
          for (int b = 0; b < RB; ++b) o[b][t % DB] = mfma32(vf[t], px[b][t / DB], o[b][t % DB]);
#pragma unroll
          for (int b = 0; b < RB; ++b)
#pragma unroll
            for (int q = 0; q < PPS; ++q) {
              const int pp = t * PPS + q, v = pp >> 2, w = pp & 3;
              const int i0 = 8 * v + 2 * w;
              e[b][2 * pp] = __builtin_amdgcn_exp2f(fmaf(sy[b][i0], c2, mneg[b]));
              e[b][2 * pp + 1] = __builtin_amdgcn_exp2f(fmaf(sy[b][i0 + 1], c2, mneg[b]));
              if constexpr (diag) {
                if (key_of_elem(i0, 0) > tmask[b]) e[b][2 * pp] = 0.f;
                if (key_of_elem(i0 + 1, 0) > tmask[b]) e[b][2 * pp + 1] = 0.f;
              }
              // keep the exps in this slot (otherwise they sink towards their uses)
              asm volatile("" : "+v"(e[b][2 * pp]), "+v"(e[b][2 * pp + 1]));
            }
          if (t > 0) {
#pragma unroll
            for (int b = 0; b < RB; ++b)
#pragma unroll
              for (int q = 0; q < PPS; ++q) finish(b, (t - 1) * PPS + q);
          }
          // the step's copies go out after its first two slots, K then V
          if (t == 0) issue_kc();
          if (t == 1) issue_vc();
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int b = 0; b < RB; ++b) {
#pragma unroll
          for (int q = 0; q < PPS; ++q) finish(b, (KS - 1) * PPS + q);
          lsy[b] = s0[b] + s1[b];
        }
      }
      if constexpr (sl % 2 == 1) {
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(OUT * kIssuePerStep) : "memory");
        if (tail_clip && n > VLEAD && u == bclip) {  // V of the last tile has landed
          clip_tail((n - 1) % RING);
          asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        }
      }
    };
    // The step count is rounded up to the RING-way unroll: tiles past the range read
    // the zero page and are masked out entirely. Steps whose tile j+1 lies before
    // j_mask need no mask (all but an item's last few); they run first, in whole groups.
    const int npad = (n + RING - 1) / RING * RING;
    const int nfree = min(npad, max(0, j_mask - t0 - 1) / RING * RING);
    using F = std::false_type;
    using T = std::true_type;
    auto group = [&](auto mask_tag, int u) {
      step(std::integral_constant<int, 0>{}, mask_tag, u, sa, sb, pa, pb, la, lb);
      step(std::integral_constant<int, 1>{}, mask_tag, u + 1, sb, sa, pb, pa, lb, la);
      step(std::integral_constant<int, 2>{}, mask_tag, u + 2, sa, sb, pa, pb, la, lb);
      step(std::integral_constant<int, 3>{}, mask_tag, u + 3, sb, sa, pb, pa, lb, la);
      step(std::integral_constant<int, 4>{}, mask_tag, u + 4, sa, sb, pa, pb, la, lb);
      step(std::integral_constant<int, 5>{}, mask_tag, u + 5, sb, sa, pb, pa, lb, la);
      step(std::integral_constant<int, 6>{}, mask_tag, u + 6, sa, sb, pa, pb, la, lb);
      step(std::integral_constant<int, 7>{}, mask_tag, u + 7, sb, sa, pb, pa, lb, la);
    };
    static_assert(RING == 8, "the loop body runs RING steps");
    // before a group whose steps copy tile v_new (step v_new - KLEAD) or later tiles
    auto wait_before = [&](int u) {
      if (FUSED && wait_pending && v_new < u + RING + KLEAD) {
        wait_appends_wave<WAVES>(a);
        wait_pending = false;
      }
    };
    int u = 0;
    for (; u < nfree; u += RING) {
      wait_before(u);
      group(F{}, u);
    }
    for (; u < npad; u += RING) {
      wait_before(u);
      group(T{}, u);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // drain the copies issued past the end
  };
  if (n > 0) {
    if (wait_new)
      sweep(std::true_type{});
    else
      sweep(std::false_type{});
  }
  if (!ovf) {
#pragma unroll
    for (int b = 0; b < RB; ++b)
      write_row<D>(a, o[b], m[b], l[b], valid[b], hi, orow[b], it.slot, it.slot_rows, rloc[b]);
  } else {
    if (lane == 0) atomicAdd(a.err + 2, 1);
    chunk_rows_exact<D, RB>(a, it, wave, lane);
  }
}

}  // namespace extattn
