// bf16 extend attention on the CDNA4 matrix cores (gfx950).
//
// What is computed (zdszero "Chunked Prefill" notes, section "prefill as
// several resumable extends"): query token i of a chunk at global position
// P + i takes the softmax over keys 0 .. P+i of scale * q.k_j and applies it
// to v_j. Keys below P are the rectangle (never masked), keys P .. P+i the
// triangle (the causal diagonal); both are swept by one running (m, l)
// online-softmax state, which is the page's merge rule applied tile by tile.
// Split key ranges end in a partial (o, lse) that the combine kernel merges
// with the same rule.
//
// Layout of the work (one workgroup = 8 wave64, 2 per SIMD, one per CU):
//  * Rows are (position, head-in-group) pairs of one (request, KV head): the
//    whole GQA group shares each K/V tile.
//  * Chunk items: 256 rows, 32 per wave; 32-key K/V tiles are copied from the
//    paged cache straight into 4-slot LDS rings once per workgroup and read by
//    all 8 waves (one barrier per tile).
//  * Split items (<= 32 rows: decode rows, multi-token verify rows): every
//    wave takes all the rows and reads its own part of the key range straight
//    from HBM into MFMA operand registers (no LDS); the waves' parts are merged
//    in LDS, and a workgroup
//    whose range is part of a longer context leaves a partial result for the
//    combine kernel.
//
// The contraction runs transposed: S^T = K Q^T and O^T = V^T P^T on
// v_mfma_f32_32x32x16_bf16. A lane then owns one query row (column l % 32 of
// every accumulator), so the row max / row sum stay in-lane except for one
// exchange with lane l ^ 32, and the P^T operand of the second product is the
// first product's accumulator converted to bf16 in place. The key order inside
// a 32-key block is permuted (bits 2 and 3 of the row index swapped) so that
// each lane's 8 P^T values cover 8 consecutive keys, which makes the V^T
// operand one 16-byte read of the slot-minor V cache layout.
#include <type_traits>

#include "attn_bf16_common.hpp"

namespace extattn {

template <int D>
__device__ void chunk_item(const AttnArgs& a, const WorkItem& it, unsigned char* smem) {
  constexpr int KT = kChunkKeys;                  // keys per tile (one 32x32 S^T block)
  constexpr int NC = D / 8;                       // 16-byte pieces per K row
  constexpr int KS = D / 16;                      // MFMA k-steps over the head dim
  constexpr int DB = D / 32;                      // 32-feature blocks of O^T
  constexpr int KT_BYTES = KT * D * 2;            // one K tile (= one V tile)
  constexpr int VSUB = D * kBlockSize * 2;        // one V^T sub-tile (16 keys)
  constexpr int PIECES = KT_BYTES / 1024;         // 1 KB direct loads per tile (K and V each)
  constexpr int NINST = (PIECES + kWaves - 1) / kWaves;  // per wave
  constexpr int RING = 4;                         // LDS ring slots per operand
  constexpr int KBUF = 0, VBUF = RING * KT_BYTES; // LDS: K ring, then V ring, then block ids
  constexpr int IDBUF = 2 * RING * KT_BYTES;
  static_assert(PIECES % kWaves == 0 || kWaves % PIECES == 0, "pieces must split evenly over the waves");

  const int tid = threadIdx.x;
  // wave index as a uniform (scalar) value: block bases and LDS destinations stay in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const SeqInfo si = a.seqs[it.seq];
  const int G = a.group, g = it.kv_head;
  const int kv_len = si.prefix + si.extend;
  const int rloc = wave * kRowsPerWave + l32;
  const bool valid = rloc < it.nrows;
  // Waves whose 32 rows all lie past the item's rows (items of few rows: verify rows,
  // ragged last tiles) still copy their share of every K/V tile and keep the
  // barriers, but skip the products and the softmax work (wave-uniform test).
  const bool wave_rows = wave * kRowsPerWave < it.nrows;
  const int rho = it.row0 + rloc;
  const int pos = valid ? rho / G : 0;
  const int hh = valid ? rho - pos * G : 0;
  const int64_t orow = int64_t(si.q_off + pos) * a.hq + g * G + hh;
  const int lim = valid ? min(si.prefix + pos, it.key_end - 1) : -1;
  const int lim_min = min(si.prefix + it.row0 / G, it.key_end - 1);
  const float c2 = a.scale_log2;

  // Query rows enter the products exactly as given (bf16); the softmax scale is
  // applied to the fp32 scores, inside the exponent.
  u32x4 qf[KS];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + orow * D + hi * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = valid ? *reinterpret_cast<const u32x4*>(qp + ks * 16) : zero4();
  }

  const int32_t* bt = a.block_table + int64_t(it.seq) * a.max_blocks;
  const int nblk = (kv_len + kBlockSize - 1) / kBlockSize;
  const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache);
  const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache);

  // K read of k-step ks: row key_of_row(l32), position (2 ks + hi) ^ swz_k(row) =
  // (2 ks) ^ (hi ^ (l32 & 15)); the row base is a multiple of the row size, so
  // the offset is k_off0 ^ (ks << 5).
  const int k_off0 = key_of_row(l32) * (D * 2) + (((hi ^ (l32 & 15)) & (NC - 1)) << 4);
  const int v_off = l32 * (kBlockSize * 2) + ((hi ^ swz_v(l32)) << 4);

  const int t0 = it.key_begin / KT;
  const int t1 = (it.key_end + KT - 1) / KT;
  const int n = t1 - t0;

  // Block ids go through a small LDS ring (64 tiles = 128 ids) filled by direct
  // loads, 32 tiles at a time, so the loop holds no register-destination loads.
  int32_t* id_ring = reinterpret_cast<int32_t*>(smem + IDBUF);
  // Copy the ids of tiles [jt, jt + 32) into ring half (jt - t0) / 32 % 2 (wave 0 only).
  auto fill_ids = [&](int jt) {
    if (wave != 0) return;
    const int lb = jt * (KT / kBlockSize) + lane;  // 64 ids
    const int src = lb < nblk ? lb : nblk - 1;     // stay inside the table row
    const int half = ((jt - t0) / 32) & 1;
    dma4(bt, uint32_t(src) * 4u, lds_addr(id_ring + half * 64));
  };
  // Each wave copies one 1 KB piece of every K and V tile (waves beyond the piece
  // count copy nothing); piece `wave` lies in block my_blk of the tile.
  static_assert(NINST == 1, "one piece per wave and tile");
  const bool has_piece = PIECES >= kWaves || wave < PIECES;  // compile-time true when every wave has one
  const int my_blk = has_piece ? wave / (PIECES / 2) : 0;
  // The ids of a 32-tile window (64 entries) sit one per lane in `idwin`, loaded from
  // the ring once per window and checked there: entries past the sequence end and
  // ids outside [0, num_blocks) become -1 (read the zero page); the invalid ones are
  // counted in the error word (once per window and workgroup).
  int32_t idwin = -1;
  auto load_window = [&](int k) {
    const int32_t v = id_ring[(k & 1) * 64 + lane];
    const bool inside = (t0 + 32 * k) * (KT / kBlockSize) + lane < nblk;
    const bool ok = block_ok(v, a.num_blocks);
    const uint64_t bad = __builtin_amdgcn_ballot_w64(inside && !ok);
    if (bad != 0 && wave == 0 && lane == 0) report_bad_blocks(a.err, int(__builtin_popcountll(bad)));
    // tiles past the range (padding steps) read the zero page even where the
    // sequence still has keys
    const bool in_range = t0 + 32 * k + (lane >> 1) < t1;
    idwin = (inside && ok && in_range) ? v : -1;
  };
  // This wave's block id of tile j (wave-uniform).
  auto read_blk = [&](int j) -> int32_t {
    return __builtin_amdgcn_readlane(idwin, ((j - t0) & 31) * 2 + my_blk);
  };
  // Per-lane byte offsets (within the piece's block) of this wave's direct loads.
  uint32_t k_src[NINST], v_src[NINST];
#pragma unroll
  for (int x = 0; x < NINST; ++x) {
    const int i = wave + kWaves * x;  // 1 KB piece of the tile
    // K: 16-byte slot (i, lane) is row r (key r of the tile), position c; it holds piece c ^ swz_k(r)
    const int n = i * 64 + lane;
    const int r = n / NC, c = n % NC;
    k_src[x] = uint32_t(((r & 15) * D + ((c ^ (key_of_row(r & 15) & (NC - 1))) * 8)) * 2);
    // V: slot (i, lane) is feature row d of sub-tile i / (PIECES / 2), position cv; it holds half cv ^ swz_v(d)
    const int d = ((i * 64 + lane) % (VSUB / 16)) / 2, cv = lane & 1;
    v_src[x] = uint32_t((d * kBlockSize + ((cv ^ swz_v(d)) * 8)) * 2);
  }
  // Copy sources and destinations as scalars computed once: this (request, KV head)'s
  // first block in each cache, the byte stride between blocks, and this wave's LDS
  // piece in K slot 0 / V slot 0 (slots are KT_BYTES apart).
  const unsigned char* kc_g = reinterpret_cast<const unsigned char*>(kc + int64_t(g) * (kBlockSize * D));
  const unsigned char* vc_g = reinterpret_cast<const unsigned char*>(vc + int64_t(g) * (kBlockSize * D));
  const uint32_t blk_bytes = uint32_t(a.hkv) * (kBlockSize * D * 2);  // < 2^32: 32x32 -> 64-bit product below
  const uint32_t k_dst = lds_addr(smem + KBUF) + wave * 1024;
  const uint32_t v_dst = lds_addr(smem + VBUF) + wave * 1024;
  auto src_base = [&](const unsigned char* cache_g, int32_t blk) -> const unsigned char* {
    const unsigned char* p = cache_g + uint64_t(uint32_t(max(blk, 0))) * uint64_t(blk_bytes);
    return blk < 0 ? static_cast<const unsigned char*>(a.zero_page) : p;
  };
  auto issue_k = [&](int32_t blk, int slot) {
    if (has_piece) dma16(src_base(kc_g, blk), k_src[0], k_dst + slot * KT_BYTES);
  };
  auto issue_v = [&](int32_t blk, int slot) {
    if (has_piece) dma16(src_base(vc_g, blk), v_src[0], v_dst + slot * KT_BYTES);
  };

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  // Running max m (log2 units of the scaled scores) and this lane's share of the row
  // sum l. m is the exact row max of the first tile; afterwards it is raised only
  // when a tile's weights grow past kSumBound (rare), so no tile needs a row max.
  float m = 0.f, l = 0.f;
  float mneg = 0.f;  // -m: the weights are 2^(s c - m), one fma and one exp2 per score

  // S^T of one tile from K ring slot `slot` (compile-time). Invalid blocks were
  // loaded from the zero page; keys past the sequence end are masked later.
  auto qk = [&](auto slot_tag, f32x16& s) {
    constexpr int slot = decltype(slot_tag)::value;
    const unsigned char* base = smem + KBUF + slot * KT_BYTES;
    s = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 kf = *reinterpret_cast<const u32x4*>(base + (k_off0 ^ (ks << 5)));
      s = mfma32(kf, qf[ks], s);
    }
  };
  auto row_max = [&](const f32x16& s) -> float {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
    return mx;
  };
  // Causal mask of a diagonal tile (and of keys past the range end). Element i holds
  // key kt + 8 hi + key_of_elem(i, 0), so the test is one threshold against constants.
  // first tile index whose last key passes lim_min (tiles from there on may need masking)
  const int j_mask =
      __builtin_amdgcn_readfirstlane(lim_min >= KT - 1 ? (lim_min - (KT - 1)) / KT + 1 : 0);  // uniform
  auto mask = [&](int j, f32x16& s) {
    const int kt = j * KT;
    if (j >= j_mask) {
      const int t = lim - kt - 8 * hi;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (key_of_elem(i, 0) > t) s[i] = -INFINITY;
    }
  };
  // Scores leave their QK product as raw fp32 dot products s. Weights
  // p = 2^(s c - m), c = scale * log2(e), as packed bf16 for the P.V product, and this
  // lane's fp32 sum of them over the tile, taken before the rounding (lse carries no
  // rounding of the weights; the normaliser is within 2^-9 relative of the rounded
  // weights' sum).
  auto weights = [&](const f32x16& s, u32x4 (&pf)[2], float& ls) {
    float l0 = 0.f, l1 = 0.f;
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[8 * v + 2 * w], c2, mneg));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[8 * v + 2 * w + 1], c2, mneg));
        pf[v][w] = pack2(p0, p1);
        l0 += p0;
        l1 += p1;
      }
    ls = l0 + l1;
  };
  // Check of a tile's weights before they enter P.V: when some lane's sum passed
  // kSumBound (or overflowed), raise m to the rows' exact max over the tile, rescale
  // O and l and redo the tile's weights (the next tile's weights use the new m).
  // Then add the sum to l.
  auto check = [&](const f32x16& s, u32x4 (&pf)[2], float& ls) {
    if (__builtin_amdgcn_ballot_w64(ls > kSumBound) != 0) {
      float mx = row_max(s);
      mx = fmaxf(mx, partner(mx, hi));
      const float d = fmaxf(fmaf(mx, c2, mneg), 0.f);  // masked rows: -inf -> 0
      const float alpha = __builtin_amdgcn_exp2f(-d);
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
      l *= alpha;
      m += d;
      mneg = -m;
      weights(s, pf, ls);
    }
    l += ls;
  };
  // O^T += V^T P^T for one tile from V ring slot `slot` (compile-time).
  auto pv = [&](auto slot_tag, const u32x4 (&pf)[2]) {
    constexpr int slot = decltype(slot_tag)::value;
    const unsigned char* base = smem + VBUF + slot * KT_BYTES;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int b = 0; b < 2; ++b) {  // 16-key block of the tile; this lane's keys 16 b + 8 hi .. +8
        const u32x4 vf = *reinterpret_cast<const u32x4*>(base + v_off + b * VSUB + db * 32 * (kBlockSize * 2));
        o[db] = mfma32(vf, pf[b], o[db]);
      }
  };
  // Values of keys past the sequence end read as zero: their weights are zero but the
  // cache slots may hold anything (0 * NaN would poison O). Only the range's last tile
  // can reach past the end; its V tile is cleared in LDS once, after it has landed
  // and before it is read (the caller puts barriers around this).
  const bool tail_clip = (t1 * KT > kv_len);
  const int j_clip = tail_clip ? t1 - 2 : INT_MIN;  // step whose next tile is the clipped last one
  auto clip_tail = [&](int slot) {
    unsigned char* base = smem + VBUF + slot * KT_BYTES;
    const int kt = (t1 - 1) * KT;
    for (int piece = tid; piece < 4 * D; piece += kThreads) {  // 16-byte pieces of the V tile
      const int b = piece / (2 * D), d = (piece / 2) % D, h = piece & 1;
      const int key0 = kt + 16 * b + 8 * (h ^ swz_v(d));
      if (key0 + 8 > kv_len) {
        u32x4* pp = reinterpret_cast<u32x4*>(base + b * VSUB + d * (kBlockSize * 2) + h * 16);
        *pp = clip_keys(*pp, key0, kv_len);
      }
    }
  };

  if (n > 0) {
    // Pipeline over tiles j = t0 + u: tile j's K sits in K slot u % 4 and its V in
    // V slot u % 4. Every step issues the same number of tile loads (tiles past the
    // end load the zero page), so waiting for "at most one step's worth outstanding"
    // completes everything older; waves without a piece issue none.
    constexpr int kIssuePerStep = 2 * NINST;
    // Prologue: ids of tiles t0 .. t0+63, then K and V of t0 and t0+1, K of t0+2.
    fill_ids(t0);
    fill_ids(t0 + 32);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    load_window(0);
    const int32_t b0 = read_blk(t0);
    issue_k(b0, 0);
    issue_v(b0, 0);
    const int32_t b1 = read_blk(t0 + 1);
    issue_k(b1, 1);
    issue_v(b1, 1);
    int32_t pending = read_blk(t0 + 2);  // tile j+2: K issued, V not yet
    issue_k(pending, 2);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    if (tail_clip && n == 1) {  // the first tile is the last one
      clip_tail(0);
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    f32x16 sa, sb;
    u32x4 pa[2], pb[2];  // packed weights of the tiles whose scores are in sa / sb
    float la = 0.f, lb = 0.f;  // and this lane's sums of them
    // The first tile sets m to the rows' exact max (0 for rows with no visible key).
    if (wave_rows) {
      qk(std::integral_constant<int, 0>{}, sa);
      mask(t0, sa);
      float mx = row_max(sa);
      mx = fmaxf(mx, partner(mx, hi));
      m = (mx == -INFINITY) ? 0.f : mx * c2;
      mneg = -m;
      weights(sa, pa, la);
    }
    // Steady step u (tile j = t0 + u, not the last): S(j) is in scur (masked) and its
    // weights in pcur / lcur, K(j+1) in K slot (u+1)%4, V(j) in V slot u%4. Then
    //   check tile j's weights (rare path: raise m before the next weights),
    //   region A: S(j+1) = QK(j+1) MFMAs, with the copies of K(j+3) and V(j+2) (their
    //     slots were last read two steps ago) issued half way,
    //   mask tile j+1 if diagonal,
    //   region B: O += P(j) V(j) MFMAs interleaved with tile j+1's weights.
    auto step = [&](auto slot_tag, int u, f32x16& scur, f32x16& snext, u32x4 (&pcur)[2], u32x4 (&pnext)[2],
                    float& lcur, float& lnext) {
      constexpr int sl = decltype(slot_tag)::value;  // u % 4
      const int j = t0 + u;
      // ids of tiles j+32 .. j+63 replace those of tiles j-32 .. j-1 (long consumed);
      // the first read (tile j+32, by step u+29) comes after two barriers. u = sl (mod 4),
      // so only step 0 can start a 32-step period and only step 1 a new window.
      if constexpr (sl == 0) {
        if ((u & 31) == 0 && u > 0) fill_ids(j + 32);
      }
      if constexpr (sl == 1) {
        if (((u + 3) & 31) == 0) load_window((u + 3) >> 5);  // tile j+3 starts a new window
      }
      // This step's tile copies (K(j+3), V(j+2); their slots are not read in this step)
      // go out in the middle of region A, after the first QK MFMAs are under way;
      // waves without rows issue them at once.
      auto issue = [&]() {
        const int32_t bk = read_blk(j + 3);
        issue_k(bk, (sl + 3) & 3);
        issue_v(pending, (sl + 2) & 3);
        pending = bk;
      };
      if (!wave_rows) issue();
      if (wave_rows) {
        check(scur, pcur, lcur);
        __builtin_amdgcn_sched_barrier(0);  // regions A and B are scheduled separately
        // region A: the K operand reads run 3 ahead of their MFMAs
        {
          constexpr int sl1 = (sl + 1) & 3;
          const unsigned char* kb = smem + KBUF + sl1 * KT_BYTES;
          u32x4 kf[KS];
#pragma unroll
          for (int ks = 0; ks < 3 && ks < KS; ++ks) kf[ks] = *reinterpret_cast<const u32x4*>(kb + (k_off0 ^ (ks << 5)));
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            if (ks + 3 < KS) kf[ks + 3] = *reinterpret_cast<const u32x4*>(kb + (k_off0 ^ ((ks + 3) << 5)));
            snext = mfma32(kf[ks], qf[ks], ks == 0 ? f32x16{} : snext);
            if (ks == KS / 2 - 1) issue();
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        mask(j + 1, snext);
        __builtin_amdgcn_sched_barrier(0);
        // region B: the V operand reads run 3 ahead; consecutive MFMAs update different
        // O blocks (16-key half b = i / DB, feature block i % DB); tile j+1's weights go
        // next to the MFMAs (exps front-loaded, each pair packed and summed one MFMA later)
        {
          const unsigned char* vb = smem + VBUF + sl * KT_BYTES + v_off;
          auto vread = [&](int i) -> u32x4 {
            return *reinterpret_cast<const u32x4*>(vb + (i / DB) * VSUB + (i % DB) * 32 * (kBlockSize * 2));
          };
          constexpr int NPAIR = 8;
          constexpr int NB = 2 * DB;
          float l0 = 0.f, l1 = 0.f;
          float e[16];
          u32x4 vf[NB];
          auto finish = [&](int pp) {  // pack and sum pair pp (its exps were issued one group earlier)
            const int v = pp >> 2, w = pp & 3;
            pnext[v][w] = pack2(e[2 * pp], e[2 * pp + 1]);
            if (pp == 0) {
              l0 = e[0];
              l1 = e[1];
            } else {
              l0 += e[2 * pp];
              l1 += e[2 * pp + 1];
            }
          };
          // exps of pairs [lo(i), lo(i+1)) go with MFMA i, front-loaded so that the last
          // MFMA has none after it
          auto lo = [](int i) { return i >= NB ? NPAIR : min(NPAIR, (i * NPAIR + NB - 2) / (NB - 1)); };
#pragma unroll
          for (int i = 0; i < 3 && i < NB; ++i) vf[i] = vread(i);
#pragma unroll
          for (int i = 0; i < NB; ++i) {
            if (i + 3 < NB) vf[i + 3] = vread(i + 3);
            o[i % DB] = mfma32(vf[i], pcur[i / DB], o[i % DB]);
#pragma unroll
            for (int pp = lo(i); pp < lo(i + 1); ++pp) {
              const int v = pp >> 2, w = pp & 3;
              e[2 * pp] = __builtin_amdgcn_exp2f(fmaf(snext[8 * v + 2 * w], c2, mneg));
              e[2 * pp + 1] = __builtin_amdgcn_exp2f(fmaf(snext[8 * v + 2 * w + 1], c2, mneg));
            }
            if (i > 0) {
#pragma unroll
              for (int pp = lo(i - 1); pp < lo(i); ++pp) finish(pp);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
          for (int pp = lo(NB - 1); pp < lo(NB); ++pp) finish(pp);
          lnext = l0 + l1;
        }
      }
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(kIssuePerStep) : "memory");
      if (j == j_clip) {  // V(j+1) has landed: clear its keys past the end
        clip_tail((sl + 1) & 3);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      }
    };
    // The last tile: check and P V with the sequence-end clip; nothing to issue.
    auto last = [&](f32x16& scur, u32x4 (&pcur)[2], float& lcur) {
      if (!wave_rows) return;
      check(scur, pcur, lcur);
      pv(std::integral_constant<int, 0>{}, pcur);
    };
    // The step count is rounded up so that the 4-way unrolled loop needs no remainder:
    // tiles past the range's end read the zero page and are masked out entirely.
    const int npad = n + ((1 - n) & 3);  // npad = 1 (mod 4), npad >= n
    for (int u = 0; u + 4 < npad; u += 4) {
      step(std::integral_constant<int, 0>{}, u, sa, sb, pa, pb, la, lb);
      step(std::integral_constant<int, 1>{}, u + 1, sb, sa, pb, pa, lb, la);
      step(std::integral_constant<int, 2>{}, u + 2, sa, sb, pa, pb, la, lb);
      step(std::integral_constant<int, 3>{}, u + 3, sb, sa, pb, pa, lb, la);
    }
    // tile t0 + npad - 1 (npad - 1 is a multiple of 4): S in sa, V in ring slot 0
    last(sa, pa, la);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // drain the loads issued past the end
  }
  write_row<D>(a, o, m, l, valid, hi, orow, it.slot, it.slot_rows, rloc);
}

// ---------------------------------------------------------------------------
// Split items: <= 32 rows (decode rows, multi-token verify rows); each wave
// streams its own part of the key range from HBM straight into MFMA operand
// registers. These run on v_mfma_f32_16x16x32_bf16 with RB = 1 or 2 blocks of 16
// query rows per wave; the RB blocks share every K/V operand, so the context is
// read once whatever the row count. Accumulator element i of lane l belongs to
// query row l % 16 of its block and MFMA row 4 (l / 16) + i; MFMA row r of key
// block b holds key 8 (r / 4) + 4 b + r % 4 of the tile, so each lane's P^T
// operand (4 values from block 0, 4 from block 1) covers 8 consecutive keys.
// With one row block two 32-key tiles are in flight per wave; with two, the
// second block's operands take the registers of the second tile, and the next
// tile is loaded as soon as the current one has been consumed.
// ---------------------------------------------------------------------------
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ inline f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                 c, 0, 0, 0);
}

template <int D, int RB>
__device__ void split_item(const AttnArgs& a, const WorkItem& it, unsigned char* smem) {
  constexpr int KS = D / 32;  // 32-wide k-steps over the head dim
  constexpr int DB = D / 16;  // 16-feature blocks of O^T
  const int tid = threadIdx.x;
  const int lane = tid & 63, l16 = lane & 15, q4 = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const SeqInfo si = a.seqs[it.seq];
  const int G = a.group, g = it.kv_head;
  const int kv_len = si.prefix + si.extend;

  // Row block rb of this lane: row rb * 16 + l16 of the item.
  u32x4 qf[RB][KS];
  int lim[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int rr = rb * kSplitRows + l16;
    const bool valid = rr < it.nrows;
    const int pos = valid ? rr / G : 0;
    const int hh = valid ? rr - pos * G : 0;
    const int64_t orow = int64_t(si.q_off + pos) * a.hq + g * G + hh;
    lim[rb] = valid ? min(si.prefix + pos, it.key_end - 1) : -1;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + orow * D + q4 * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[rb][ks] = valid ? *reinterpret_cast<const u32x4*>(qp + ks * 32) : zero4();
  }
  const int32_t* bt = a.block_table + int64_t(it.seq) * a.max_blocks;
  const int nblk = (kv_len + kBlockSize - 1) / kBlockSize;
  const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache);
  const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache);

  f32x4 o[RB][DB];
  float m[RB], l[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int db = 0; db < DB; ++db) o[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[rb] = -INFINITY;
    l[rb] = 0.f;
  }

  // Keys (within the 32-key tile) this lane loads as MFMA rows of blocks 0 / 1.
  const int kbase = 8 * (l16 >> 2) + (l16 & 3);
  // This wave's tiles [tw0, tw1) of the item's key range.
  const int nt = (it.key_end - it.key_begin + kSplitTile - 1) / kSplitTile;
  const int tw0 = wave * nt / kWaves, tw1 = (wave + 1) * nt / kWaves;
  // All block ids of the wave's range in one load (one per lane), checked once:
  // ids outside [0, num_blocks) become -1 (read the zero page) and are counted;
  // entries past the sequence end are -1 too. No tile load then waits on an id.
  static_assert(kSplitKeysMax / kSplitTile / kWaves * (kSplitTile / kBlockSize) <= 64, "ids of a wave fit one per lane");
  int32_t idw = -1;
  {
    const int lb = (it.key_begin + tw0 * kSplitTile) / kBlockSize + lane;
    const bool inside = lane < (tw1 - tw0) * (kSplitTile / kBlockSize) && lb < nblk;
    const int32_t v = inside ? bt[lb] : -1;
    const bool ok = block_ok(v, a.num_blocks);
    const uint64_t bad = __builtin_amdgcn_ballot_w64(inside && !ok);
    if (bad != 0 && lane == 0) report_bad_blocks(a.err, int(__builtin_popcountll(bad)));
    idw = (inside && ok) ? v : -1;
  }
  const unsigned char* zp = static_cast<const unsigned char*>(a.zero_page);
  auto blk_base = [&](const uint16_t* cache, int32_t blk) -> const uint16_t* {
    return blk < 0 ? reinterpret_cast<const uint16_t*>(zp) : cache + (int64_t(blk) * a.hkv + g) * (kBlockSize * D);
  };
  struct Tile {
    u32x4 kf[2][KS];
    u32x4 vf[DB];
    int kt;
  };
  // Loads are unconditional (invalid blocks and blocks past the end read the zero
  // page); the sequence end is applied when the tile is consumed, so the next
  // tile's loads stay in flight while this one is computed. Every K/V byte is read
  // once here, so the loads carry the non-temporal hint (streamed, not kept in the
  // caches): measured 5.35 TB/s for the decode rows against 4.1 TB/s without it.
  auto load = [&](int jj, Tile& T) {
    const int kt = it.key_begin + jj * kSplitTile;
    // tiles loaded past the wave's range may index past lane 63: any valid id will do
    const int e = (2 * (jj - tw0)) & 63;
    const int32_t s0 = __builtin_amdgcn_readlane(idw, e), s1 = __builtin_amdgcn_readlane(idw, e + 1);
    const uint16_t* kb0 = blk_base(kc, s0);
    const uint16_t* kb1 = blk_base(kc, s1);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int koff = kbase + 4 * b;  // < 32; block koff / 16
      const uint16_t* kp = (koff < kBlockSize ? kb0 : kb1) + (koff % kBlockSize) * D + q4 * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) T.kf[b][ks] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + ks * 32));
    }
    const uint16_t* vp = (q4 < 2 ? blk_base(vc, s0) : blk_base(vc, s1)) + 8 * (q4 & 1);
#pragma unroll
    for (int db = 0; db < DB; ++db) T.vf[db] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp + (db * 16 + l16) * kBlockSize));
    T.kt = kt;
  };
  auto compute = [&](Tile& T) {
    const int kt = T.kt;
    u32x4 pf[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      f32x4 sc[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        sc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) sc[b] = mfma16(T.kf[b][ks], qf[rb][ks], sc[b]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (kt + 8 * q4 + 4 * b + i > lim[rb]) sc[b][i] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[b][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m[rb], mx * a.scale_log2);
      if (mnew > m[rb]) {
        const float alpha = __builtin_amdgcn_exp2f(m[rb] - mnew);
#pragma unroll
        for (int db = 0; db < DB; ++db) o[rb][db] *= alpha;
        l[rb] *= alpha;
        m[rb] = mnew;
      }
      const float msafe = (m[rb] == -INFINITY) ? 0.f : m[rb];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[b][0], a.scale_log2, -msafe));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[b][1], a.scale_log2, -msafe));
        const float p2 = __builtin_amdgcn_exp2f(fmaf(sc[b][2], a.scale_log2, -msafe));
        const float p3 = __builtin_amdgcn_exp2f(fmaf(sc[b][3], a.scale_log2, -msafe));
        l[rb] += (p0 + p1) + (p2 + p3);
        pf[rb][2 * b] = pack2(p0, p1);
        pf[rb][2 * b + 1] = pack2(p2, p3);
      }
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const u32x4 vv = clip_keys(T.vf[db], kt + 8 * q4, kv_len);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) o[rb][db] = mfma16(vv, pf[rb], o[rb][db]);
    }
  };

  if constexpr (RB == 1) {
    // Two tiles in flight. Loads are issued whether or not the tile is used (tiles
    // past the wave's range read the zero page): a load under a branch would make
    // the compiler wait for it where the branches join.
    Tile ta, tb;
    load(tw0, ta);
    for (int jj = tw0; jj < tw1; jj += 2) {
      load(jj + 1, tb);
      compute(ta);
      load(jj + 2, ta);
      if (jj + 1 < tw1) compute(tb);
    }
  } else {
    Tile ta;
    load(tw0, ta);
    for (int jj = tw0; jj < tw1; ++jj) {
      compute(ta);
      load(jj + 1, ta);
    }
  }

  // Merge the waves' partial results through LDS (the page's merge rule over the
  // kWaves parts): part[w][row][d] holds unnormalised o, mls[w][row] = (m, l).
  constexpr int SR = RB * kSplitRows;  // rows per wave and rows of the partial slot
  float* part = reinterpret_cast<float*>(smem);
  float* mls = part + kWaves * SR * D;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float lt = l[rb] + __shfl_xor(l[rb], 16);
    lt += __shfl_xor(lt, 32);
    const int rr = rb * kSplitRows + l16;
    if (rr < it.nrows) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<float4*>(part + (wave * SR + rr) * D + db * 16 + 4 * q4) =
            float4{o[rb][db][0], o[rb][db][1], o[rb][db][2], o[rb][db][3]};
      if (q4 == 0) {
        mls[(wave * SR + rr) * 2] = m[rb];
        mls[(wave * SR + rr) * 2 + 1] = lt;
      }
    }
  }
  __syncthreads();
  constexpr int TPR = D / 4;           // threads per row, 4 features each
  constexpr int RPP = kThreads / TPR;  // rows per pass
  const int c4 = (tid % TPR) * 4;
#pragma unroll
  for (int r0 = 0; r0 < SR; r0 += RPP) {
    const int r = r0 + tid / TPR;
    if (r >= it.nrows) continue;
    float4 acc = {0.f, 0.f, 0.f, 0.f};
    float L = 0.f, M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mls[(w * SR + r) * 2]);
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float lw = mls[(w * SR + r) * 2 + 1];
        if (lw > 0.f) {
          const float f = __builtin_amdgcn_exp2f(mls[(w * SR + r) * 2] - M);
          const float4 ow = *reinterpret_cast<const float4*>(part + (w * SR + r) * D + c4);
          L += f * lw;
          acc.x += f * ow.x;
          acc.y += f * ow.y;
          acc.z += f * ow.z;
          acc.w += f * ow.w;
        }
      }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const float lse_wg = L > 0.f ? (M + __builtin_amdgcn_logf(L)) * kLn2 : -INFINITY;
    const float4 res = float4{acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
    if (it.task < 0) {  // this workgroup covered the whole key range
      const int rpos = r / G;
      const int64_t orow_r = int64_t(si.q_off + rpos) * a.hq + g * G + (r - rpos * G);
      uint16_t* op = static_cast<uint16_t*>(a.out) + orow_r * D + c4;
      u32x2 pk = {pack2(res.x, res.y), pack2(res.z, res.w)};
      *reinterpret_cast<u32x2*>(op) = pk;
      if (c4 == 0 && a.lse) a.lse[orow_r] = lse_wg;
    } else {
      // Leave this workgroup's partial (normalised o, natural-log lse) in its slot;
      // the combine kernel merges the workgroups' partials of the task.
      float* sl = a.slots + it.slot;  // rows [SR][D], then lse [SR]
      *reinterpret_cast<float4*>(sl + r * D + c4) = res;
      if (c4 == 0) sl[SR * D + r] = lse_wg;
    }
  }
}

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2)))
void attn_bf16_kernel(AttnArgs a) {
  constexpr int kChunkLds = 2 * 4 * kChunkKeys * D * 2 + 512;                     // K/V rings + block ids
  constexpr int kSplitLds = kWaves * 2 * kSplitRows * (D + 2) * 4;                 // wave partials (2 row blocks)
  __shared__ __attribute__((aligned(16))) unsigned char smem[kChunkLds > kSplitLds ? kChunkLds : kSplitLds];
  const WorkItem it = a.items[blockIdx.x];
  // measurement variant: the workgroup's start and end (after its last wave) in
  // wall-clock ticks; the start is stored at once so that nothing stays live
  if (a.stamps && threadIdx.x == 0) {
    int64_t* st = a.stamps + 4 * int64_t(blockIdx.x);
    st[0] = int64_t(wall_clock64());
    st[2] = it.kind;
    st[3] = it.seq;
  }
  if (it.kind == kItemAppend) {
    append_item<D, kWaves>(a, it);
  } else {
    if (a.n_append > 0 && it.key_end > a.seqs[it.seq].prefix) wait_appends<kWaves>(a);  // reads new keys
    if (it.kind == kItemChunk)
      chunk_item<D>(a, it, smem);
    else if (it.nrows <= kSplitRows)
      split_item<D, 1>(a, it, smem);
    else
      split_item<D, 2>(a, it, smem);
  }
  if (a.stamps) {
    __syncthreads();
    if (threadIdx.x == 0) a.stamps[4 * int64_t(blockIdx.x) + 1] = int64_t(wall_clock64());
  }
}

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t stream) {
  if (a.n_items <= 0) return hipSuccess;
  if (a.head_dim == 64)
    hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3(unsigned(a.n_items)), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_bf16_kernel<128>, dim3(unsigned(a.n_items)), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace extattn
