// fp32 extend attention on the vector ALUs (one wave per query row and head).
//
// The plain definition, evaluated key block by key block with the running
// max / running sum rescale (zdszero notes, section "prefill as several
// resumable extends": o_i as a softmax over keys 0..P+i; the (m, l) merge).
// Lanes own 64 keys at a time for the scores, then own features of the output
// for the P.V accumulation.
#include "device_common.hpp"

namespace extattn {

__device__ inline float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a) {
  constexpr int X = D / 64;
  const int row = blockIdx.x;
  const int h = blockIdx.y;
  const int lane = threadIdx.x;
  const int r = find_seq(a.seqs, a.num_seqs, row);
  const SeqInfo s = a.seqs[r];
  const int pos = row - s.q_off;
  const int lim = s.prefix + pos;  // last key attended (inclusive)
  const int g = h / a.group;
  __shared__ float qs[D];
  const float* qp = static_cast<const float*>(a.q) + (int64_t(row) * a.hq + h) * D;
#pragma unroll
  for (int x = 0; x < X; ++x) qs[lane + 64 * x] = qp[lane + 64 * x];
  __syncthreads();
  const int32_t* bt = a.block_table + int64_t(r) * a.max_blocks;
  const float* kc = static_cast<const float*>(a.k_cache);
  const float* vc = static_cast<const float*>(a.v_cache);
  float m = -INFINITY, l = 0.f, o[X];
#pragma unroll
  for (int x = 0; x < X; ++x) o[x] = 0.f;
  for (int kb = 0; kb <= lim; kb += 64) {
    const int key = kb + lane;
    float sc = -INFINITY;
    if (key <= lim) {
      const int32_t phys = bt[key / kBlockSize];
      if (block_ok(phys, a.num_blocks)) {
        const float* kp = kc + ((int64_t(phys) * a.hkv + g) * kBlockSize + key % kBlockSize) * D;
        float acc = 0.f;
#pragma unroll 8
        for (int d = 0; d < D; ++d) acc = fmaf(qs[d], kp[d], acc);
        sc = acc * a.scale;
      } else {
        sc = 0.f;
        if (key % kBlockSize == 0 && h == 0) report_bad_blocks(a.err, 1);
      }
    }
    const float mnew = fmaxf(m, wave_max(sc));  // lane 0's key kb <= lim, so finite
    const float alpha = expf(m - mnew);
    const float p = key <= lim ? expf(sc - mnew) : 0.f;
    l = l * alpha + wave_sum(p);
#pragma unroll
    for (int x = 0; x < X; ++x) o[x] *= alpha;
    const int nk = min(64, lim - kb + 1);
    for (int j = 0; j < nk; ++j) {
      const float pj = __shfl(p, j);
      const int kj = kb + j;
      const int32_t phys = bt[kj / kBlockSize];
      if (!block_ok(phys, a.num_blocks)) continue;
      const float* vp = vc + (int64_t(phys) * a.hkv + g) * int64_t(D) * kBlockSize + kj % kBlockSize;
#pragma unroll
      for (int x = 0; x < X; ++x) o[x] = fmaf(pj, vp[int64_t(lane + 64 * x) * kBlockSize], o[x]);
    }
    m = mnew;
  }
  const float inv = 1.f / l;
  float* op = static_cast<float*>(a.out) + (int64_t(row) * a.hq + h) * D;
#pragma unroll
  for (int x = 0; x < X; ++x) op[lane + 64 * x] = o[x] * inv;
  if (a.lse && lane == 0) a.lse[int64_t(row) * a.hq + h] = m + logf(l);
}

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t stream) {
  if (a.total_rows <= 0) return hipSuccess;
  if (a.hq > 65535) return hipErrorInvalidValue;
  const dim3 grid(unsigned(a.total_rows), unsigned(a.hq));
  if (a.head_dim == 64)
    hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace extattn
