// Weighted combine of the routed expert outputs and the shared expert
// ("DeepSeek-V4-Flash-SI" card, 架构特性: each token's output is the
// routing-weighted sum of its selected experts, plus the shared expert):
//   y[t] = bf16( sum_j w[t,j] * o[pair_pos[t*k + j]] + ysh[t] )
// summed in fp32 in rank order j.  A gather (one thread per 4 columns of one
// token), so the result is deterministic: no atomics.  The shared expert's
// output may come as split-K slices (decode sizes), added in slice order
// before it joins the sum.
#include "moe_internal.h"

namespace moe {

// K = k (compile-time): the k pair positions and weights, then all k rows'
// float4 loads are issued before the first multiply-add, so a thread has
// k + 1 row loads in flight instead of one at a time.
template <int K>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o,
                                                      const float* __restrict__ w,
                                                      const int32_t* __restrict__ pair_pos,
                                                      const float* __restrict__ ysh, int parts,
                                                      uint16_t* __restrict__ y, int64_t T, int H) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;  // one float4 of y
  const int per_row = H / 4;
  const int64_t t = q / per_row;
  if (t >= T) return;
  const int c = (int)(q - t * per_row) * 4;
  int32_t pp[K];
  float wj[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    pp[j] = pair_pos[t * K + j];
    wj[j] = w[t * K + j];
  }
  // the rows of o are read once, a wave taking 1 KB of one row: whole-line
  // non-temporal loads (wload)
  typedef float f4v __attribute__((ext_vector_type(4)));
  f4v v[K];
#pragma unroll
  for (int j = 0; j < K; ++j) v[j] = wload<f4v>(o + (size_t)pp[j] * H + c);
  f4v s = {0.f, 0.f, 0.f, 0.f};
  if (ysh) {   // read once too
    const float* p = ysh + (size_t)t * H + c;
    const size_t stride = (size_t)T * H;
    s = wload<f4v>(p);
    for (int i = 1; i < parts; ++i) {
      const f4v b = wload<f4v>(p + i * stride);
      s.x += b.x; s.y += b.y; s.z += b.z; s.w += b.w;
    }
  }
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int j = 0; j < K; ++j) {
    acc.x = fmaf(wj[j], v[j].x, acc.x);
    acc.y = fmaf(wj[j], v[j].y, acc.y);
    acc.z = fmaf(wj[j], v[j].z, acc.z);
    acc.w = fmaf(wj[j], v[j].w, acc.w);
  }
  if (ysh) {
    acc.x += s.x; acc.y += s.y; acc.z += s.z; acc.w += s.w;
  }
  const uint32_t lo = f32_to_bf16(acc.x) | (f32_to_bf16(acc.y) << 16);
  const uint32_t hi = f32_to_bf16(acc.z) | (f32_to_bf16(acc.w) << 16);
  *reinterpret_cast<uint2*>(y + (size_t)t * H + c) = make_uint2(lo, hi);
}

hipError_t launch_combine(const float* o, const float* topk_w, const int32_t* pair_pos,
                          const float* ysh, int ysh_parts, uint16_t* y, int64_t T, int H, int k,
                          hipStream_t st) {
  const int64_t n = T * (H / 4);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
#define MOE_COMBINE(KK)                                                                      \
  case KK:                                                                                   \
    hipLaunchKernelGGL((combine_kernel<KK>), grid, dim3(256), 0, st, o, topk_w, pair_pos, ysh, \
                       ysh_parts, y, T, H);                                                  \
    break;
  switch (k) {
    MOE_COMBINE(1) MOE_COMBINE(2) MOE_COMBINE(3) MOE_COMBINE(4)
    MOE_COMBINE(5) MOE_COMBINE(6) MOE_COMBINE(7) MOE_COMBINE(8)
    default: return hipErrorInvalidValue;   // 1 <= k <= 8 is checked by the caller
  }
#undef MOE_COMBINE
  return hipGetLastError();
}

}  // namespace moe
