// Split items of the bf16 path: decode rows and multi-token verify rows, each
// wave streaming its own part of the key range from HBM (shared by the mixed
// kernel and the 4-wave wide-split kernel).
#pragma once

#include "attn_bf16_common.hpp"

namespace extattn {

// ---------------------------------------------------------------------------
// Split items: <= 32 rows on the 8-wave kernels, <= 64 on the 4-wave wide-split
// kernel (decode rows, multi-token verify rows); each of the W waves streams its
// own part of the key range from HBM. These
// run on v_mfma_f32_16x16x32_bf16 with RB = 1 .. 4 blocks of 16 query rows per
// wave; the RB blocks share every K/V operand, so the context is read once
// whatever the row count. Accumulator element i of lane l belongs to
// query row l % 16 of its block and MFMA row 4 (l / 16) + i; MFMA row r of key
// block b holds key 8 (r / 4) + 4 b + r % 4 of the tile, so each lane's P^T
// operand (4 values from block 0, 4 from block 1) covers 8 consecutive keys.
// At 8 waves (256 registers a wave) each wave copies its next 32-key tile (K and
// V, 16 KB at D = 128) whole into an LDS slot of its own while the current one is
// computed, and reads it back in operand layout. Loaded straight into operand
// registers, a K operand instruction would read 64 bytes of each of 16 keys: half
// of 16 cache lines per instruction, which streams at about half the rate of whole
// lines (27 against 52 GB/s per CU with 64 CUs reading, 5.9 against 6.8 TB/s with
// all of them). The copies read whole lines: 4 keys x 256 B of K or 32 feature rows
// x 32 B of V per instruction, with the non-temporal hint (every byte is read
// once). At 4 waves (512 registers) K and V go straight into
// a register ring of 4 tiles at up to two row blocks and of 2 at three or four.
// ---------------------------------------------------------------------------
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ inline f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                 c, 0, 0, 0);
}

// Position XOR of the 16-byte pieces of key k (0..31) in a split tile's K rows in
// LDS. The 16 keys one operand read touches (MFMA row r holds key 8 (r / 4) + r % 4
// + 4 b) get 16 distinct values at D = 128 (256-byte rows: the value is r), and at
// D = 64 (128-byte rows, two to a 256-byte bank row) 8 distinct values among the
// keys of either parity, so each 16-lane group of a read hits 16 different bank
// groups.
template <int D>
__device__ constexpr int kswz(int k) {
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  return D == 128 ? ((k & 3) | (((k >> 3) & 3) << 2)) : (((k >> 1) & 1) | (((k >> 3) & 3) << 1));
}

// LDS bytes of the 8-wave split path's tile slots (K and V of one 32-key tile a wave).
template <int D>
constexpr int split_slot_lds() { return kWaves * 2 * kSplitTile * D * 2; }

template <int D, int RB, int W>
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
  // At 3-4 row blocks on the wide kernel Q stays in LDS (an image of the operand
  // registers after the merge area, written once by wave rb for block rb) and is
  // read where each product uses it; the registers go to the K/V ring instead.
  constexpr bool QLDS = W == kWideWaves && RB >= 3;
  const uint32_t qimg = lds_addr(smem) + uint32_t(W * RB * kSplitRows * (D + 2) * 4);
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
    if constexpr (QLDS) {
      if (rb == wave) {
        typedef __attribute__((address_space(3))) u32x4 lds_q_t;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          *reinterpret_cast<lds_q_t*>(qimg + uint32_t(((rb * KS + ks) * 64 + lane) * 16)) =
              valid ? *reinterpret_cast<const u32x4*>(qp + ks * 32) : zero4();
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[rb][ks] = valid ? *reinterpret_cast<const u32x4*>(qp + ks * 32) : zero4();
    }
  }
  if constexpr (QLDS) __syncthreads();
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
  const int tw0 = wave * nt / W, tw1 = (wave + 1) * nt / W;
  // All block ids of the wave's range in one or two loads (one per lane each),
  // checked once: ids outside [0, num_blocks) become -1 (read the zero page) and
  // are counted; entries past the sequence end are -1 too. No tile load then
  // waits on an id.
  constexpr int IDS = split_keys_max(W) / kSplitTile / W * (kSplitTile / kBlockSize);  // ids of a wave, at most
  constexpr int IDR = (IDS + 63) / 64;
  static_assert(IDR <= 2, "ids of a wave fit two per lane");
  int32_t idw[IDR];
#pragma unroll
  for (int h = 0; h < IDR; ++h) {
    const int lb = (it.key_begin + tw0 * kSplitTile) / kBlockSize + h * 64 + lane;
    const bool inside = h * 64 + lane < (tw1 - tw0) * (kSplitTile / kBlockSize) && lb < nblk;
    const int32_t v = inside ? bt[lb] : -1;
    const bool ok = block_ok(v, a.num_blocks);
    const uint64_t bad = __builtin_amdgcn_ballot_w64(inside && !ok);
    if (bad != 0 && lane == 0) report_bad_blocks(a.err, int(__builtin_popcountll(bad)));
    idw[h] = (inside && ok) ? v : -1;
  }
  // id of entry e (wave-uniform) of the window
  auto id_at = [&](int e) -> int32_t {
    if constexpr (IDR == 1) return __builtin_amdgcn_readlane(idw[0], e);
    else return e < 64 ? __builtin_amdgcn_readlane(idw[0], e) : __builtin_amdgcn_readlane(idw[1], e - 64);
  };
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
    // tiles loaded past the wave's range may index past the window: any valid id will do
    const int e = (2 * (jj - tw0)) & (64 * IDR - 1);
    const int32_t s0 = id_at(e), s1 = id_at(e + 1);
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
  // 8-wave kernels: the wave's LDS slot (K tile, then V tile) and the per-lane
  // copy sources and operand read addresses. Piece c (16 bytes) of key k of the
  // K tile sits at position c ^ kswz(k) of the key's row, so that the 16 keys
  // one operand read touches fall in 16 different bank groups; the two 16-byte
  // halves of a V row are swapped on bit 3 of the row for the same reason.
  constexpr int NI = D / 16;           // 1 KB copies per K (and per V) tile
  constexpr int KROW = D * 2;          // bytes of a K row
  constexpr int NC = D / 8;            // 16-byte pieces of a K row
  constexpr int KPI = 1024 / KROW;     // keys per K copy
  constexpr int VBLK = kBlockSize * D * 2;  // bytes of one block's V head (and K head)
  const uint32_t kslot = lds_addr(smem) + uint32_t(wave * 2 * NI * 1024);
  const uint32_t vslot = kslot + uint32_t(NI * 1024);
  uint32_t k_src[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int key = i * KPI + lane / NC;  // key of the tile this lane copies, < 32
    k_src[i] = uint32_t((key % kBlockSize) * KROW + (((lane % NC) ^ kswz<D>(key)) << 4));
  }
  const uint32_t v_src0 = uint32_t((lane >> 1) * 32 + (((lane & 1) ^ ((lane >> 4) & 1)) << 4));
  const int key0 = 8 * (l16 >> 2) + (l16 & 3);  // key of MFMA row l16 in block 0
  const uint32_t k_rd = kslot + uint32_t(key0 * KROW + ((q4 ^ kswz<D>(key0)) << 4));
  const uint32_t v_rd = vslot + uint32_t((q4 >> 1) * VBLK + l16 * 32 + (((q4 & 1) ^ ((l16 >> 3) & 1)) << 4));
  // Copy the K (or V) tile of tile jj into its half of the wave's slot: NI direct
  // copies of whole lines.
  auto issue_half = [&](int jj, bool v) {
    const int e = (2 * (jj - tw0)) & (64 * IDR - 1);
    const int32_t s0 = id_at(e), s1 = id_at(e + 1);
    const uint16_t* c = v ? vc : kc;
    const uint16_t* b0 = blk_base(c, s0);
    const uint16_t* b1 = blk_base(c, s1);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (v)
        dma16_nt(i < NI / 2 ? b0 : b1, v_src0 + uint32_t((i % (NI / 2)) * 1024), vslot + uint32_t(i * 1024));
      else
        dma16_nt(i < NI / 2 ? b0 : b1, k_src[i], kslot + uint32_t(i * 1024));
    }
  };
  typedef __attribute__((address_space(3))) const u32x4 lds_cq_t;
  // K operands of tile jj from the slot (its K copies have landed).
  auto read_k = [&](Tile& T, int jj) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint32_t ka = k_rd ^ uint32_t(ks << 6);  // piece 4 ks + q4: bits 6-7 of the row offset
#pragma unroll
      for (int b = 0; b < 2; ++b) T.kf[b][ks] = *reinterpret_cast<lds_cq_t*>(ka + uint32_t(b * 4 * KROW));
    }
    T.kt = it.key_begin + jj * kSplitTile;
  };
  // V operands of tile jj, once its V copies have landed (only the next tile's K
  // copies, issued after them, may still be in flight), then the next tile's V copies
  // into the freed half. Runs between a tile's weights and its P.V products.
  auto fetch_v = [&](Tile& T, int jj) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NI) : "memory");
#pragma unroll
    for (int db = 0; db < DB; ++db) T.vf[db] = *reinterpret_cast<lds_cq_t*>(v_rd + uint32_t(db * 16 * 32));
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    issue_half(jj + 1, true);
  };
  // before_pv(T) runs between the weights and the P.V products (fetch_v on the
  // 8-wave kernel, nothing on the register ring of the wide kernel).
  auto compute = [&](Tile& T, auto&& before_pv) {
    const int kt = T.kt;
    u32x4 pf[RB];
    // With Q in LDS, a block's KS operand pieces are read together, once per tile,
    // the next block's while this block's products run (an opaque address: the
    // compiler must not hoist the reads out of the loop into registers).
    u32x4 qn[KS];
    auto read_q = [&](int rb) {
      uint32_t qa = qimg + uint32_t((rb * KS * 64 + lane) * 16);
      asm volatile("" : "+v"(qa));
      typedef __attribute__((address_space(3))) const u32x4 lds_cq_t;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qn[ks] = *reinterpret_cast<lds_cq_t*>(qa + uint32_t(ks * 64 * 16));
    };
    if constexpr (QLDS) read_q(0);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      f32x4 sc[2];
      u32x4 qq[KS];
      if constexpr (QLDS) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qq[ks] = qn[ks];
        if (rb + 1 < RB) read_q(rb + 1);
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        sc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if constexpr (QLDS)
            sc[b] = mfma16(T.kf[b][ks], qq[ks], sc[b]);
          else
            sc[b] = mfma16(T.kf[b][ks], qf[rb][ks], sc[b]);
        }
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
    before_pv(T);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const u32x4 vv = clip_keys(T.vf[db], kt + 8 * q4, kv_len);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) o[rb][db] = mfma16(vv, pf[rb], o[rb][db]);
    }
  };

  if constexpr (W == kWideWaves) {
    // One wave per SIMD with 512 registers: NT tiles in a ring, NT - 1 of them in
    // flight while one is computed (loads unconditional, as below): 4 tiles at up
    // to 2 row blocks, 2 at 3-4 (a third measured slower at 3 blocks, and spills at 4).
    constexpr int NT = RB <= 2 ? 4 : 2;
    Tile tl[NT];
#pragma unroll
    for (int k = 0; k < NT; ++k) load(tw0 + k, tl[k]);
    for (int jj = tw0; jj < tw1; jj += NT) {
#pragma unroll
      for (int k = 0; k < NT; ++k) {
        if (k == 0 || jj + k < tw1) compute(tl[k], [](Tile&) {});
        load(jj + k + NT, tl[k]);
      }
    }
  } else {
    // Tile jj + 1 is copied into the slot while tile jj is computed from registers,
    // each half as soon as tile jj's operands have left it: K after its reads at the
    // start of the tile, V after its reads before the P.V products. The copies go
    // out in the order K(jj), V(jj), K(jj + 1), V(jj + 1), so each wait leaves
    // exactly the later half's NI copies in flight. The compiler sees none of these
    // copies, so these waits are the only ones: every copy has landed before its half
    // is read, and the reads have returned before the half is overwritten. The
    // copies past the wave's range (any valid block id, or the zero page) are
    // drained before the merge reuses the LDS.
    issue_half(tw0, false);
    issue_half(tw0, true);
    for (int jj = tw0; jj < tw1; ++jj) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NI) : "memory");
      Tile T;
      read_k(T, jj);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue_half(jj + 1, false);
      compute(T, [&](Tile& t) { fetch_v(t, jj); });
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // Merge the waves' partial results through LDS (the page's merge rule over the
  // W parts): part[w][row][d] holds unnormalised o, mls[w][row] = (m, l). The 16-byte
  // piece j of a row sits at j ^ (row % 16): the 16 rows a wave writes at once then
  // fall in 16 different bank groups, and a row is still read whole.
  constexpr int SR = RB * kSplitRows;  // rows per wave and rows of the partial slot
  float* part = reinterpret_cast<float*>(smem);
  float* mls = part + W * SR * D;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float lt = l[rb] + __shfl_xor(l[rb], 16);
    lt += __shfl_xor(lt, 32);
    const int rr = rb * kSplitRows + l16;
    if (rr < it.nrows) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<float4*>(part + (wave * SR + rr) * D + (((db * 4 + q4) ^ (rr & 15)) << 2)) =
            float4{o[rb][db][0], o[rb][db][1], o[rb][db][2], o[rb][db][3]};
      if (q4 == 0) {
        mls[(wave * SR + rr) * 2] = m[rb];
        mls[(wave * SR + rr) * 2 + 1] = lt;
      }
    }
  }
  __syncthreads();
  constexpr int TPR = D / 4;           // threads per row, 4 features each
  constexpr int RPP = 64 * W / TPR;  // rows per pass
  const int c4 = (tid % TPR) * 4;
#pragma unroll
  for (int r0 = 0; r0 < SR; r0 += RPP) {
    const int r = r0 + tid / TPR;
    if (r >= it.nrows) continue;
    float4 acc = {0.f, 0.f, 0.f, 0.f};
    float L = 0.f, M = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, mls[(w * SR + r) * 2]);
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float lw = mls[(w * SR + r) * 2 + 1];
        if (lw > 0.f) {
          const float f = __builtin_amdgcn_exp2f(mls[(w * SR + r) * 2] - M);
          const float4 ow = *reinterpret_cast<const float4*>(part + (w * SR + r) * D + (((c4 >> 2) ^ (r & 15)) << 2));
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

}  // namespace extattn
