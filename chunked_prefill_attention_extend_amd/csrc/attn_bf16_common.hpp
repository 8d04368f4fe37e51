// Device helpers of the bf16 attention kernels: MFMA wrappers, the key order
// inside a 32-key tile, LDS swizzles and direct-to-LDS copies, the row epilogue,
// and the fused append's copy and wait.
#pragma once

#include "device_common.hpp"

namespace extattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLn2 = 0.6931471805599453f;

__device__ inline f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                 c, 0, 0, 0);
}

__device__ inline uint32_t pack2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Key (within a 32-key block) that MFMA row m of the S^T product holds.
__device__ inline int key_of_row(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// Key (within a 32-key block) of accumulator element i in lane half `hi`.
__device__ inline int key_of_elem(int i, int hi) { return ((i >> 3) << 4) + (hi << 3) + (i & 7); }

__device__ inline u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

// Zero the bf16 values of a 16-byte V piece whose keys k0 .. k0+7 reach kv_len
// (branch-free: a per-lane branch here would split the wave's control flow).
__device__ inline u32x4 clip_keys(u32x4 v, int k0, int kv_len) {
  const int n = kv_len - k0;  // keys of the piece that are inside
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t lo = (2 * w < n) ? 0x0000ffffu : 0u;
    const uint32_t hi = (2 * w + 1 < n) ? 0xffff0000u : 0u;
    v[w] &= (lo | hi);
  }
  return v;
}

// Write a finished row: either the final output (bf16) and lse, or a partial
// slot (fp32 o normalised, natural-log lse) for the combine kernel.
template <int D>
__device__ inline void write_row(const AttnArgs& a, const f32x16 (&o)[D / 32], float m, float l, bool valid,
                                 int hi, int64_t orow, int32_t slot, int32_t slot_rows, int rloc) {
  constexpr int DB = D / 32;
  const float lt = l + __shfl_xor(l, 32);
  if (!valid) return;
  if (slot < 0) {
    const float inv = 1.f / lt;
    uint16_t* op = static_cast<uint16_t*>(a.out) + orow * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int d = db * 32 + u * 8 + hi * 4;
        u32x2 pk = {pack2(o[db][4 * u] * inv, o[db][4 * u + 1] * inv),
                    pack2(o[db][4 * u + 2] * inv, o[db][4 * u + 3] * inv)};
        *reinterpret_cast<u32x2*>(op + d) = pk;
      }
    if (hi == 0 && a.lse) a.lse[orow] = (m + __builtin_amdgcn_logf(lt)) * kLn2;
  } else {
    float* sl = a.slots + slot;  // rows [slot_rows][D], then lse [slot_rows]
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int d = db * 32 + u * 8 + hi * 4;
        float4 v = {o[db][4 * u] * inv, o[db][4 * u + 1] * inv, o[db][4 * u + 2] * inv, o[db][4 * u + 3] * inv};
        *reinterpret_cast<float4*>(sl + rloc * D + d) = v;
      }
    if (hi == 0) sl[slot_rows * D + rloc] = lt > 0.f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Chunk items: 256 rows, LDS-shared K/V tiles of 32 keys.
//
// K/V tiles go from the paged cache straight into LDS (global_load_lds_dwordx4:
// each lane's 16 bytes land at the instruction's LDS base + 16 * lane), so no
// registers hold the next tile. Each wave copies one 1 KB piece of every K and
// every V tile. LDS layouts (per ring slot):
//   K: 32 rows (keys) x D bf16; 16-byte piece p of row r sits at position
//      p ^ swz_k(r), swz_k(r) = key_of_row(r % 16) (mod pieces per row).
//   V: two sub-tiles, one per 16-key block, each D rows (features) x 16 keys;
//      half h (8 keys) of row d sits at position h ^ swz_v(d),
//      swz_v(d) = ((d >> 2) ^ (d >> 3)) & 1.
// A piece lies inside one cache block, so every direct load has a uniform base
// address and a 32-bit per-lane offset. Both swizzles keep every aligned group
// of 8 (and of 16) lanes of a 16-byte LDS read on distinct banks. Invalid block
// ids and tiles past the range read a page of zeros; keys past the range are
// masked in the scores, and values past the sequence end are cleared in LDS.
// ---------------------------------------------------------------------------
__device__ inline int swz_v(int d) { return ((d >> 2) ^ (d >> 3)) & 1; }

// Value of lane l ^ 32 (the other lane holding the same query row).
// v_permlane32_swap exchanges lanes 32..63 of its first operand with lanes 0..31
// of its second; either result then holds the partner value in the lane half that
// received it, whether or not both operands share a register.
__device__ inline float partner(float x, int hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  const uint32_t v = hi ? r[0] : r[1];
  return __builtin_bit_cast(float, v);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// LDS byte address of a pointer into the workgroup's shared memory, as a wave-uniform value.
__device__ inline uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)p)));
}

// Direct copies from global memory into LDS: lane l's 16 (or 4) bytes at base + off
// land at LDS address lds + 16 l (4 l). They are issued as inline assembly on purpose:
// the compiler's wait-count pass treats any direct-to-LDS load it sees as a possible
// producer of every later LDS read and then drains all LDS reads before each use
// (s_waitcnt lgkmcnt(0)), which serialises the MFMA operand reads. The kernel orders
// these copies itself (s_waitcnt vmcnt and a barrier before the data is read); loads
// the compiler does not know about only make its own vmcnt waits stricter.
__device__ inline void dma16(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(off), "s"(base) : "memory", "m0");
}
// The same copy with the non-temporal hint, for bytes read exactly once (split
// items): streamed past the caches, 6.9 against 6.1 TB/s for whole-line copies with
// all CUs reading, 55 against 52 GB/s per CU with 64.
__device__ inline void dma16_nt(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(lds), "v"(off), "s"(base) : "memory", "m0");
}
__device__ inline void dma4(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2" ::"s"(lds), "v"(off), "s"(base) : "memory", "m0");
}


// ---------------------------------------------------------------------------
// Fused append. Workgroup p < n_append of the launch first copies groups
// [p NG / n_append, (p+1) NG / n_append) of the NG groups of 16 consecutive new
// tokens of the launch (rows of k_new, request order) into the paged cache: K as
// 16-byte pieces, V as whole 16-slot rows of the slot-minor layout when the group
// fills one cache block (else element by element); then each of its waves adds 1 to
// the completion counter with release semantics at device scope, and the
// workgroup goes on to its own work item. Work that reads new keys waits until
// the counter says that every copying wave is done. The copying workgroups are
// the first of the launch, so every die dispatches its share of them before any
// other workgroup of the launch, and they wait for nothing before they signal: the
// waits end. A wait is still bounded and sets kStatusWaitTimeout in the status
// flags if it gives up.
// ---------------------------------------------------------------------------
template <int D, int WAVES>
__device__ void append_share(const AttnArgs& a, int p) {
  constexpr int PIECES = D / 8;  // 16-byte pieces of a head vector
  constexpr int NT = 64 * WAVES;
  const int tid = threadIdx.x;
  const int total = a.total_rows;
  // whole groups of 16 consecutive new tokens (rows of k_new): groups [gb, ge)
  const int ngroups = (total + kBlockSize - 1) / kBlockSize;
  const int gb = int(int64_t(ngroups) * p / a.n_append), ge = int(int64_t(ngroups) * (p + 1) / a.n_append);
  const uint16_t* kn = static_cast<const uint16_t*>(a.k_new);
  const uint16_t* vn = static_cast<const uint16_t*>(a.v_new);
  uint16_t* kc = static_cast<uint16_t*>(a.k_cache_w);
  uint16_t* vc = static_cast<uint16_t*>(a.v_cache_w);
  const int hkv = a.hkv;
  // physical block and slot of new-token row t (-1: invalid block id, reported once per token)
  auto locate = [&](int t, int& slot) -> int32_t {
    const int r = find_seq(a.seqs, a.num_seqs, t);
    const SeqInfo si = a.seqs[r];
    const int pos = si.prefix + (t - si.q_off);
    slot = pos % kBlockSize;
    return a.block_table[int64_t(r) * a.max_blocks + pos / kBlockSize];
  };
  constexpr int KB = 4;  // K pieces, and V rows / 2, a thread loads before it stores
  for (int grp = gb; grp < ge; ++grp) {
    const int t0 = grp * kBlockSize;
    const int nt = min(kBlockSize, total - t0);
    const int nk = nt * hkv * PIECES, nv = hkv * D;
    // The first batch of the group's K pieces and V rows is loaded before the
    // block lookup, so that the loads overlap the lookup's dependent reads.
    u32x4 kv[KB];
    uint32_t vw[2][kBlockSize / 2];
    auto load_k = [&](int base) {
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const int i = base + k * NT;
        if (i < nk) {
          const int tl = i / (hkv * PIECES), rem = i - tl * (hkv * PIECES);
          kv[k] = *reinterpret_cast<const u32x4*>(kn + (int64_t(t0 + tl) * hkv + rem / PIECES) * D + (rem % PIECES) * 8);
        }
      }
    };
    auto load_v = [&](int base) {  // the group's 16 tokens of (head, feature) rows base, base + NT
      if (nt < kBlockSize) return;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int i = base + k * NT;
        if (i < nv) {
          const int g = i / D, d = i - g * D;
#pragma unroll
          for (int e = 0; e < kBlockSize / 2; ++e)
            vw[k][e] = uint32_t(vn[(int64_t(t0 + 2 * e) * hkv + g) * D + d]) |
                       (uint32_t(vn[(int64_t(t0 + 2 * e + 1) * hkv + g) * D + d]) << 16);
        }
      }
    };
    load_k(tid);
    load_v(tid);
    // the usual case: the group's tokens are slots 0..15 of one cache block
    const int r0 = find_seq(a.seqs, a.num_seqs, t0);
    const SeqInfo s0 = a.seqs[r0];
    const int pos0 = s0.prefix + (t0 - s0.q_off);
    const bool whole = nt == kBlockSize && t0 + kBlockSize <= s0.q_off + s0.extend && pos0 % kBlockSize == 0;
    const int32_t phys0 = whole ? a.block_table[int64_t(r0) * a.max_blocks + pos0 / kBlockSize] : -1;
    const bool whole_ok = whole && block_ok(phys0, a.num_blocks);
    // K: one 16-byte piece per (token, head, piece)
    for (int base = tid; base < nk; base += KB * NT) {
      if (base != tid) load_k(base);
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const int i = base + k * NT;
        if (i >= nk) continue;
        const int tl = i / (hkv * PIECES), rem = i - tl * (hkv * PIECES);
        const int g = rem / PIECES, c = rem % PIECES;
        int slot = tl;
        const int32_t phys = whole ? phys0 : locate(t0 + tl, slot);
        if (!block_ok(phys, a.num_blocks)) {
          if (g == 0 && c == 0) report_bad_blocks(a.err, 1);
          continue;
        }
        *reinterpret_cast<u32x4*>(kc + ((int64_t(phys) * hkv + g) * kBlockSize + slot) * D + c * 8) = kv[k];
      }
    }
    // V (slot-minor): whole 16-slot rows of the block, else element by element
    for (int base = tid; base < nv; base += 2 * NT) {
      if (whole) {
        if (base != tid) load_v(base);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int i = base + k * NT;
          if (i >= nv || !whole_ok) continue;  // invalid ids were reported with K
          const int g = i / D, d = i - g * D;
          u32x4* dst = reinterpret_cast<u32x4*>(vc + ((int64_t(phys0) * hkv + g) * D + d) * kBlockSize);
          dst[0] = u32x4{vw[k][0], vw[k][1], vw[k][2], vw[k][3]};
          dst[1] = u32x4{vw[k][4], vw[k][5], vw[k][6], vw[k][7]};
        }
      } else {
        for (int k = 0; k < 2; ++k) {
          const int i = base + k * NT;
          if (i >= nv) continue;
          const int g = i / D, d = i - g * D;
          for (int tl = 0; tl < nt; ++tl) {
            int slot;
            const int32_t phys = locate(t0 + tl, slot);
            if (!block_ok(phys, a.num_blocks)) continue;
            vc[((int64_t(phys) * hkv + g) * D + d) * kBlockSize + slot] = vn[(int64_t(t0 + tl) * hkv + g) * D + d];
          }
        }
      }
    }
  }
  if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_add(a.append_done, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kWaitSpinLimit = 1 << 20;  // polls, ~0.3 us apart: ~0.3 s

// Lane 0 of the calling wave polls the counter until every append wave is done
// (relaxed loads spaced out, so that hundreds of waiting waves do not flood one
// address; bounded, leaving kStatusWaitTimeout if it gives up).
template <int WAVES>
__device__ inline void poll_appends(const AttnArgs& a) {
  if ((threadIdx.x & 63) == 0) {
    const int target = a.n_append * WAVES;
    int spins = 0;
    while (__hip_atomic_load(a.append_done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(10);
      if (++spins == kWaitSpinLimit) {
        atomicOr(a.err, kStatusWaitTimeout);
        break;
      }
    }
  }
}

// The whole workgroup waits: one lane polls, then one acquire fence makes the
// appended K/V visible before the workgroup's first load.
template <int WAVES>
__device__ void wait_appends(const AttnArgs& a) {
  if (threadIdx.x == 0) {
    poll_appends<WAVES>(a);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

// One wave waits (for its own later loads): its lane 0 polls, then the wave's
// acquire fence.
template <int WAVES>
__device__ void wait_appends_wave(const AttnArgs& a) {
  poll_appends<WAVES>(a);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

}  // namespace extattn
