// Device helpers shared by the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include "internal.hpp"

namespace extattn {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Request that owns flattened query row `row` (requests are in q order; the
// last request whose first row is <= row owns it).
__device__ inline int find_seq(const SeqInfo* seqs, int num_seqs, int row) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (seqs[mid].q_off <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ inline bool block_ok(int32_t phys, int64_t num_blocks) {
  return phys >= 0 && int64_t(phys) < num_blocks;
}

// Report n invalid block-id reads in the status words (flag, then count).
__device__ inline void report_bad_blocks(int32_t* status, int n) {
  atomicOr(status, kStatusBadBlock);
  atomicAdd(status + 1, n);
}

}  // namespace extattn
