// Metadata upload by a kernel that reads pinned, device-mapped host memory.
//
// A call's descriptors (request table, work items, combine tasks) are a few tens of
// KB. Copying them with hipMemcpyAsync hands the transfer to a DMA engine, and the
// attention kernel queued behind it then starts only after a cross-engine signal,
// which costs tens of microseconds per call. A kernel on the caller's stream that
// loads the staging buffer over the host link and stores it into the workspace is
// ordered behind the previous kernel and ahead of the next by the stream alone.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.hpp"

namespace extattn {

namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyMaxGroups = 64;

__global__ __launch_bounds__(kCopyThreads) void meta_copy_kernel(const uint4* __restrict__ src,
                                                                  uint4* __restrict__ dst, uint32_t n16,
                                                                  const unsigned char* __restrict__ src_tail,
                                                                  unsigned char* __restrict__ dst_tail,
                                                                  uint32_t tail) {
  const uint32_t stride = gridDim.x * kCopyThreads;
  for (uint32_t i = blockIdx.x * kCopyThreads + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
  if (blockIdx.x == 0 && threadIdx.x < tail) dst_tail[threadIdx.x] = src_tail[threadIdx.x];
}

}  // namespace

hipError_t launch_meta_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16 != 0) return hipErrorInvalidValue;
  if (bytes > size_t(UINT32_MAX)) return hipErrorInvalidValue;
  const uint32_t n16 = uint32_t(bytes / 16), tail = uint32_t(bytes % 16);
  uint32_t groups = (n16 + kCopyThreads - 1) / kCopyThreads;
  if (groups < 1) groups = 1;
  if (groups > kCopyMaxGroups) groups = kCopyMaxGroups;
  const unsigned char* s = static_cast<const unsigned char*>(src);
  unsigned char* d = static_cast<unsigned char*>(dst);
  hipLaunchKernelGGL(meta_copy_kernel, dim3(groups), dim3(kCopyThreads), 0, stream,
                     reinterpret_cast<const uint4*>(s), reinterpret_cast<uint4*>(d), n16, s + size_t(n16) * 16,
                     d + size_t(n16) * 16, tail);
  return hipGetLastError();
}

}  // namespace extattn
