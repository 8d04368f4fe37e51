// Merge of partial attention results (split key ranges) into the output.
//
// Each partial carries its normalised output o_s and its log-sum-exp lse_s.
// The merge is the online-softmax rule of the zdszero notes (section "prefill
// as several resumable extends", merge equation) applied to any number of
// parts: lse = ln sum_s exp(lse_s), o = sum_s exp(lse_s - lse) o_s. Parts with
// no keys carry lse_s = -inf and weight 0.
#include "device_common.hpp"

namespace extattn {

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

template <int D>
__global__ __launch_bounds__(256) void combine_kernel(AttnArgs a) {
  constexpr int kTpr = D / 4;          // threads per row, 4 features each
  constexpr int kRpp = 256 / kTpr;     // rows per pass
  const CombineTask t = a.tasks[blockIdx.x];
  const SeqInfo s = a.seqs[t.seq];
  const int sub = threadIdx.x % kTpr;
  for (int r = threadIdx.x / kTpr; r < t.nrows; r += kRpp) {
    const int sr = t.srow0 + r;  // row within the slots
    float mx = -INFINITY;
    for (int i = 0; i < t.nslots; ++i) {
      const float* sl = a.slots + int64_t(t.slot0) + int64_t(i) * t.stride;
      mx = fmaxf(mx, sl[t.slot_rows * D + sr]);
    }
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    for (int i = 0; i < t.nslots; ++i) {
      const float* sl = a.slots + int64_t(t.slot0) + int64_t(i) * t.stride;
      const float L = sl[t.slot_rows * D + sr];
      if (L == -INFINITY) continue;
      const float w = expf(L - mx);
      wsum += w;
      const float4 o = *reinterpret_cast<const float4*>(sl + sr * D + sub * 4);
      acc[0] = fmaf(w, o.x, acc[0]);
      acc[1] = fmaf(w, o.y, acc[1]);
      acc[2] = fmaf(w, o.z, acc[2]);
      acc[3] = fmaf(w, o.w, acc[3]);
    }
    const int row = t.row0 + r;
    const int pos = row / a.group;
    const int hh = row % a.group;
    const int64_t orow = int64_t(s.q_off + pos) * a.hq + t.kv_head * a.group + hh;
    const float inv = 1.f / wsum;
    uint16_t* op = static_cast<uint16_t*>(a.out) + orow * D + sub * 4;
    u32x2 packed = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
    *reinterpret_cast<u32x2*>(op) = packed;
    if (sub == 0 && a.lse) a.lse[orow] = mx + logf(wsum);
  }
}

hipError_t launch_combine(const AttnArgs& a, int32_t dtype, hipStream_t stream) {
  (void)dtype;  // partial results exist for the bf16 path only
  if (a.n_tasks <= 0) return hipSuccess;
  if (a.head_dim == 64)
    hipLaunchKernelGGL(combine_kernel<64>, dim3(unsigned(a.n_tasks)), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(combine_kernel<128>, dim3(unsigned(a.n_tasks)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace extattn
