// bf16 extend attention on the CDNA4 matrix cores (gfx950): the mixed kernel, for
// launches that hold decode / verify rows (split items), alone or next to chunk rows.
//
// What is computed (zdszero "Chunked Prefill" notes, section "prefill as
// several resumable extends"): query token i of a chunk at global position
// P + i takes the softmax over keys 0 .. P+i of scale * q.k_j and applies it
// to v_j. A decode row is the case E = 1 (keys 0 .. P). Split key ranges end in
// a partial (o, lse) that the combine kernel merges with the page's merge rule.
//
// Layout of the work (one workgroup = 8 wave64, 2 per SIMD, one per CU):
//  * Rows are (position, head-in-group) pairs of one (request, KV head): the
//    whole GQA group shares each K/V read.
//  * Chunk items run the shared chunk code (attn_chunk_item.hpp).
//  * Split items (<= 32 rows: decode rows, multi-token verify rows): every
//    wave takes all the rows and streams its own part of the key range through
//    an LDS slot of its own (whole-line copies, one tile ahead); the waves'
//    parts are merged in LDS, and a workgroup whose range is part of a longer
//    context leaves a partial result for the combine kernel.
//
// Both paths contract on the matrix cores with the key order inside a 32-key
// block permuted so that each lane's P^T values cover consecutive keys, which
// makes the V^T operand one 16-byte read of the slot-minor V cache layout.
#include <type_traits>

#include "attn_chunk_item.hpp"
#include "attn_split_item.hpp"

namespace extattn {

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2)))
void attn_bf16_kernel(AttnArgs a) {
  constexpr int kChunkLds = 2 * kChunkRing * kChunkKeys * D * 2 + 512;            // K/V rings + block ids
  constexpr int kSplitLds = kWaves * 2 * kSplitRows * (D + 2) * 4;                 // wave partials (2 row blocks)
  __shared__ __attribute__((aligned(16))) unsigned char smem[kChunkLds > kSplitLds ? kChunkLds : kSplitLds];
  static_assert(split_slot_lds<D>() <= (kChunkLds > kSplitLds ? kChunkLds : kSplitLds), "split tile slots fit");
  const WorkItem it = a.items[blockIdx.x];
  // measurement variant: the workgroup's start and end (after its last wave) in
  // wall-clock ticks; the start is stored at once so that nothing stays live
  if (a.stamps && threadIdx.x == 0) {
    int64_t* st = a.stamps + kStampWords * int64_t(blockIdx.x);
    st[0] = int64_t(wall_clock64());
    st[4] = int64_t(clock64());
    st[2] = it.kind;
    st[3] = it.seq;
  }
  if (a.n_append > 0 && int(blockIdx.x) < a.n_append) append_share<D, kWaves>(a, blockIdx.x);
  if (it.kind == kItemChunk) {
    chunk_item_t<D, 1, kWaves>(a, it, smem);  // waits for the appends before its first new-key copy
  } else {
    if (a.n_append > 0 && it.key_end > a.seqs[it.seq].prefix) wait_appends<kWaves>(a);  // reads new keys
    if (it.nrows <= kSplitRows)
      split_item<D, 1, kWaves>(a, it, smem);
    else
      split_item<D, 2, kWaves>(a, it, smem);
  }
  if (a.stamps) {
    __syncthreads();
    if (threadIdx.x == 0) {
      int64_t* st = a.stamps + kStampWords * int64_t(blockIdx.x);
      st[5] = int64_t(clock64());
      st[1] = int64_t(wall_clock64());
    }
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
