// bf16 extend attention for launches of decode / verify rows only, when some
// request has more rows per KV head than the 8-wave kernels' split items take
// (up to 64: e.g. 8 candidate tokens of a 64-query-head / 8-KV-head model).
//
// What is computed is the same as on the other kernels (zdszero "Chunked
// Prefill" notes, section "prefill as several resumable extends": the softmax
// of a query row over keys 0 .. its position, split key ranges merged by the
// page's rule). Here a workgroup is 4 wave64, one per SIMD, each with up to 512
// registers (the output accumulators in the accumulation registers): a wave
// holds all of the item's rows (one to four 16-row blocks sharing every K/V
// operand) and a ring of K/V register tiles (4 at up to two blocks, 2 at three or
// four), so the context is read once for up to 64 rows.
#include "attn_split_item.hpp"

namespace extattn {

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kWideWaves, 64 * kWideWaves), amdgpu_waves_per_eu(1)))
void split_wide_kernel(AttnArgs a) {
  // wave partials of up to 64 rows, then the Q image of 3-4 row blocks
  constexpr int kLds = kWideWaves * kWideMaxRows * (D + 2) * 4 + kWideMaxRows / 16 * (D / 32) * 1024;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kLds];
  const WorkItem it = a.items[blockIdx.x];
  if (a.stamps && threadIdx.x == 0) {
    int64_t* st = a.stamps + kStampWords * int64_t(blockIdx.x);
    st[0] = int64_t(wall_clock64());
    st[4] = int64_t(clock64());
    st[2] = it.kind;
    st[3] = it.seq;
  }
  if (a.n_append > 0 && int(blockIdx.x) < a.n_append) append_share<D, kWideWaves>(a, blockIdx.x);
  if (a.n_append > 0 && it.key_end > a.seqs[it.seq].prefix) wait_appends<kWideWaves>(a);  // reads new keys
  if (it.nrows <= 16)
    split_item<D, 1, kWideWaves>(a, it, smem);
  else if (it.nrows <= 32)
    split_item<D, 2, kWideWaves>(a, it, smem);
  else if (it.nrows <= 48)
    split_item<D, 3, kWideWaves>(a, it, smem);
  else
    split_item<D, 4, kWideWaves>(a, it, smem);
  if (a.stamps) {
    __syncthreads();
    if (threadIdx.x == 0) {
      int64_t* st = a.stamps + kStampWords * int64_t(blockIdx.x);
      st[5] = int64_t(clock64());
      st[1] = int64_t(wall_clock64());
    }
  }
}

hipError_t launch_split_wide(const AttnArgs& a, hipStream_t stream) {
  if (a.n_items <= 0) return hipSuccess;
  if (a.head_dim == 64)
    hipLaunchKernelGGL(split_wide_kernel<64>, dim3(unsigned(a.n_items)), dim3(64 * kWideWaves), 0, stream, a);
  else
    hipLaunchKernelGGL(split_wide_kernel<128>, dim3(unsigned(a.n_items)), dim3(64 * kWideWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace extattn
