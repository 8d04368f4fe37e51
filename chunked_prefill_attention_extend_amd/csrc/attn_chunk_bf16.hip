// bf16 extend attention for launches of chunk rows only (with a fused append or not):
// one workgroup of 8 waves per chunk item (attn_chunk_item.hpp), no decode / verify
// items, so the kernel holds only the chunk code.
#include "attn_chunk_item.hpp"

namespace extattn {

template <int D, int RB, int WAVES>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * WAVES, 64 * WAVES), amdgpu_waves_per_eu(WAVES / 4, WAVES / 4)))
void chunk_bf16_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kChunkRing * kChunkKeys * D * 2 + 512];
  const WorkItem it = a.items[blockIdx.x];
  // measurement variant: the workgroup's start and end in wall-clock ticks
  if (a.stamps && threadIdx.x == 0) {
    int64_t* st = a.stamps + kStampWords * int64_t(blockIdx.x);
    st[0] = int64_t(wall_clock64());
    st[4] = int64_t(clock64());
    st[2] = it.kind;
    st[3] = it.seq;
  }
  if (a.n_append > 0 && int(blockIdx.x) < a.n_append) append_share<D, WAVES>(a, blockIdx.x);
  chunk_item_t<D, RB, WAVES>(a, it, smem);  // waits for the appends before its first new-key copy
  if (a.stamps) {
    __syncthreads();
    if (threadIdx.x == 0) {
      int64_t* st = a.stamps + kStampWords * int64_t(blockIdx.x);
      st[5] = int64_t(clock64());
      st[1] = int64_t(wall_clock64());
    }
  }
}

hipError_t launch_chunk_bf16(const AttnArgs& a, hipStream_t stream) {
  if (a.n_items <= 0) return hipSuccess;
  if (a.head_dim == 64)
    hipLaunchKernelGGL((chunk_bf16_kernel<64, 1, kWaves>), dim3(unsigned(a.n_items)), dim3(kThreads), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((chunk_bf16_kernel<128, 1, kWaves>), dim3(unsigned(a.n_items)), dim3(kThreads), 0,
                       stream, a);
  return hipGetLastError();
}

}  // namespace extattn
