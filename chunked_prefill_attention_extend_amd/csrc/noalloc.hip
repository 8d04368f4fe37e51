// Allocation-free extend attention: a static device scratch stands in for the
// caller's workspace, for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid allocation).
//
// The scratch (kNoAllocScratchBytes) lives in the library's code object: every GPU
// the library runs on holds its own copy until the process ends. Its address is
// looked up once per device with hipGetSymbolAddress; host code uses only that
// address, never the array's name. Calls on one GPU share the scratch, so calls
// that overlap on one GPU (two streams, two threads) race.
//
// The metadata of a call (request descriptors, work items, combine tasks) reaches
// the scratch through kernel arguments: a few launches of a small copy kernel on
// the caller's stream, which also clear the status words. No pinned staging is
// used, so the call allocates nothing, host-pinned memory included. The zero page
// that invalid block ids read sits at a fixed offset of the scratch; static device
// storage starts zeroed and no kernel ever stores there, so it is never copied.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <mutex>

#include "../../include/extattn.h"
#include "internal.hpp"

namespace extattn {

__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMetaWords = 480;  // payload of one copy launch (1920 bytes of kernel arguments)

struct MetaChunk {
  uint32_t offset;        // byte offset in the scratch (a multiple of 4)
  uint32_t words;         // 32-bit words to copy
  uint32_t reset_header;  // also clear the status words and the append counter
  uint32_t pad;
  uint32_t data[kMetaWords];
};

__global__ void meta_upload_kernel(unsigned char* base, MetaChunk c) {
  uint32_t* dst = reinterpret_cast<uint32_t*>(base + c.offset);
  for (uint32_t i = threadIdx.x; i < c.words; i += blockDim.x) dst[i] = c.data[i];
  if (c.reset_header)
    for (uint32_t i = threadIdx.x; i < kHeaderBytes / 4; i += blockDim.x) reinterpret_cast<uint32_t*>(base)[i] = 0;
}

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];

// Copies the plan's descriptors [off_seqs, upload_bytes) into the scratch and clears
// its header, in launches of at most kMetaWords words, on `stream`.
int upload_by_arguments(const LaunchPlan& lp, void* ws, hipStream_t stream) {
  const Plan& p = lp.plan;
  const size_t begin = p.off_seqs, end = p.upload_bytes;
  static_assert(kHeaderBytes % 4 == 0, "header of whole words");
  if (begin % 4 != 0 || end % 4 != 0) return set_error(EXTATTN_EHIP, "metadata layout is not word aligned");
  size_t off = begin;
  bool first = true;
  while (first || off < end) {
    MetaChunk c{};
    const size_t n = std::min(end - off, sizeof(c.data));
    c.offset = uint32_t(off);
    c.words = uint32_t(n / 4);
    c.reset_header = first ? 1u : 0u;
    if (n) std::memcpy(c.data, lp.blob.data() + off, n);
    hipLaunchKernelGGL(meta_upload_kernel, dim3(1), dim3(256), 0, stream, static_cast<unsigned char*>(ws), c);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return set_hip_error(e, "metadata copy launch");
    off += n;
    first = false;
  }
  return EXTATTN_OK;
}

}  // namespace

int noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_hip_error(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return set_error(EXTATTN_EHIP, "device index out of range");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return set_hip_error(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress (scratch)");
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return EXTATTN_OK;
}

}  // namespace extattn

extern "C" int extattn_extend_attention_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                                const int32_t* block_table, int32_t max_blocks, int64_t num_blocks,
                                                const int32_t* prefix_lens, const int32_t* extend_lens,
                                                int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                                int32_t head_dim, int32_t block_size, float scale, int32_t dtype,
                                                void* out, float* lse, void* stream) {
  void* ws = nullptr;
  const int rc = extattn::noalloc_scratch(&ws);
  if (rc != EXTATTN_OK) return rc;
  // the plan's size check against the scratch happens in extend_call (EXTATTN_ENOSPC)
  return extattn::extend_call(q, k_cache, v_cache, block_table, max_blocks, num_blocks, prefix_lens, extend_lens,
                              num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, scale, dtype, out, lse, ws,
                              extattn::kNoAllocScratchBytes, stream, false, nullptr, 0, nullptr, nullptr, nullptr,
                              nullptr, extattn::upload_by_arguments);
}
