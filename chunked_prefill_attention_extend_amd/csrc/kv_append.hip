// Append new tokens' K and V to the paged cache.
//
// One workgroup per 16 consecutive new tokens (request order). Their requests,
// physical blocks and slots are looked up once into LDS. K goes to
// k_cache[block][head][slot][:] as 16-byte pieces. V goes to the slot-minor layout
// v_cache[block][head][d][slot]: one thread per (head, feature d); when the 16
// tokens fill one cache block exactly (slots 0..15 of one block, the usual case
// for chunks that start on a block boundary), the thread writes the feature's whole
// 16-slot row with wide stores, else each token's element on its own.
#include "device_common.hpp"

namespace extattn {

template <typename T>
__global__ __launch_bounds__(256) void kv_append_kernel(KvArgs a) {
  constexpr int kEl = 16 / sizeof(T);  // elements per 16-byte piece
  constexpr int kGroup = kBlockSize;   // tokens per workgroup
  __shared__ int32_t s_phys[kGroup];   // physical block of each token, -1: nothing to write
  __shared__ int32_t s_slot[kGroup];
  __shared__ int32_t s_whole;          // the group fills slots 0..15 of one block
  const int t0 = int(blockIdx.x) * kGroup;
  const int D = a.head_dim;
  const int pieces = D / kEl;
  const int tid = int(threadIdx.x);
  if (tid < kGroup) {
    const int token = t0 + tid;
    int32_t phys = -1, slot = 0;
    if (token < a.total_tokens) {
      const int r = find_seq(a.seqs, a.num_seqs, token);
      const SeqInfo s = a.seqs[r];
      const int pos = s.prefix + (token - s.q_off);
      const int32_t p = a.block_table[int64_t(r) * a.max_blocks + pos / kBlockSize];
      if (block_ok(p, a.num_blocks)) {
        phys = p;
        slot = pos % kBlockSize;
      } else {
        report_bad_blocks(a.err, 1);  // one count per token whose block id is invalid
      }
    }
    s_phys[tid] = phys;
    s_slot[tid] = slot;
  }
  if (tid == 0) s_whole = 1;
  __syncthreads();
  if (tid < kGroup && (s_phys[tid] < 0 || s_phys[tid] != s_phys[0] || s_slot[tid] != tid)) s_whole = 0;
  __syncthreads();

  const int hkv = a.hkv;
  const T* kn = static_cast<const T*>(a.k_new);
  const T* vn = static_cast<const T*>(a.v_new);
  T* kc = static_cast<T*>(a.k_cache);
  T* vc = static_cast<T*>(a.v_cache);
  // K: one 16-byte piece per (token, head, piece)
  const int nk = kGroup * hkv * pieces;
  for (int i = tid; i < nk; i += int(blockDim.x)) {
    const int tl = i / (hkv * pieces);
    const int rem = i - tl * (hkv * pieces);
    const int g = rem / pieces, c = rem - g * pieces;
    const int32_t phys = s_phys[tl];
    if (phys < 0) continue;
    const int64_t src = (int64_t(t0 + tl) * hkv + g) * D + c * kEl;
    const int64_t dst = ((int64_t(phys) * hkv + g) * kBlockSize + s_slot[tl]) * D + c * kEl;
    *reinterpret_cast<u32x4*>(kc + dst) = *reinterpret_cast<const u32x4*>(kn + src);
  }
  // V: one (head, feature) row per thread and pass
  const bool whole = s_whole != 0;
  const int32_t phys0 = s_phys[0];
  for (int i = tid; i < hkv * D; i += int(blockDim.x)) {
    const int g = i / D, d = i - g * D;
    if (whole) {
      constexpr int kWords = kGroup * int(sizeof(T)) / 4;  // 32-bit words of the row
      uint32_t w[kWords];
#pragma unroll
      for (int k = 0; k < kWords; ++k) {
        if constexpr (sizeof(T) == 2) {
          const uint16_t lo = vn[(int64_t(t0 + 2 * k) * hkv + g) * D + d];
          const uint16_t hi = vn[(int64_t(t0 + 2 * k + 1) * hkv + g) * D + d];
          w[k] = uint32_t(lo) | (uint32_t(hi) << 16);
        } else {
          w[k] = __float_as_uint(vn[(int64_t(t0 + k) * hkv + g) * D + d]);
        }
      }
      T* p = vc + ((int64_t(phys0) * hkv + g) * D + d) * kBlockSize;
#pragma unroll
      for (int q = 0; q < kWords / 4; ++q)
        *reinterpret_cast<u32x4*>(p + q * (16 / int(sizeof(T)))) = u32x4{w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]};
    } else {
      for (int tl = 0; tl < kGroup; ++tl) {
        const int32_t phys = s_phys[tl];
        if (phys < 0) continue;
        vc[((int64_t(phys) * hkv + g) * D + d) * kBlockSize + s_slot[tl]] =
            vn[(int64_t(t0 + tl) * hkv + g) * D + d];
      }
    }
  }
}

hipError_t launch_kv_append(const KvArgs& a, int32_t dtype, hipStream_t stream) {
  const int64_t blocks = (int64_t(a.total_tokens) + kBlockSize - 1) / kBlockSize;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  if (blocks == 0) return hipSuccess;
  if (dtype == 0)
    hipLaunchKernelGGL(kv_append_kernel<uint16_t>, dim3(unsigned(blocks)), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(kv_append_kernel<float>, dim3(unsigned(blocks)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace extattn
