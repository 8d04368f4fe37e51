// Append new tokens' K and V to the paged cache.
//
// One thread per (token, KV head, 16-byte piece of the head vector). K goes
// to k_cache[block][head][slot][:] as one 16-byte store; V goes to the
// slot-minor layout v_cache[block][head][d][slot], one element per d.
#include "device_common.hpp"

namespace extattn {

template <typename T>
__global__ __launch_bounds__(256) void kv_append_kernel(KvArgs a) {
  constexpr int kEl = 16 / sizeof(T);  // elements per 16-byte piece
  const int pieces = a.head_dim / kEl;
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = int64_t(a.total_tokens) * a.hkv * pieces;
  if (idx >= total) return;
  const int token = int(idx / (int64_t(a.hkv) * pieces));
  const int rem = int(idx % (int64_t(a.hkv) * pieces));
  const int g = rem / pieces;
  const int c = rem % pieces;
  const int r = find_seq(a.seqs, a.num_seqs, token);
  const SeqInfo s = a.seqs[r];
  const int pos = s.prefix + (token - s.q_off);
  const int32_t phys = a.block_table[int64_t(r) * a.max_blocks + pos / kBlockSize];
  if (!block_ok(phys, a.num_blocks)) {
    if (g == 0 && c == 0) atomicAdd(a.err, 1);
    return;
  }
  const int slot = pos % kBlockSize;
  const int D = a.head_dim;
  const T* kn = static_cast<const T*>(a.k_new) + (int64_t(token) * a.hkv + g) * D + c * kEl;
  const T* vn = static_cast<const T*>(a.v_new) + (int64_t(token) * a.hkv + g) * D + c * kEl;
  T* kc = static_cast<T*>(a.k_cache) + ((int64_t(phys) * a.hkv + g) * kBlockSize + slot) * D + c * kEl;
  *reinterpret_cast<u32x4*>(kc) = *reinterpret_cast<const u32x4*>(kn);
  T vals[kEl];
  *reinterpret_cast<u32x4*>(vals) = *reinterpret_cast<const u32x4*>(vn);
  T* vc = static_cast<T*>(a.v_cache) + (int64_t(phys) * a.hkv + g) * int64_t(D) * kBlockSize + slot;
#pragma unroll
  for (int e = 0; e < kEl; ++e) vc[int64_t(c * kEl + e) * kBlockSize] = vals[e];
}

hipError_t launch_kv_append(const KvArgs& a, int32_t dtype, hipStream_t stream) {
  const int el = dtype == 0 ? 8 : 4;
  const int64_t total = int64_t(a.total_tokens) * a.hkv * (a.head_dim / el);
  const int64_t blocks = (total + 255) / 256;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  if (dtype == 0)
    hipLaunchKernelGGL(kv_append_kernel<uint16_t>, dim3(unsigned(blocks)), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(kv_append_kernel<float>, dim3(unsigned(blocks)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace extattn
