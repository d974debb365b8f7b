// Weighted combine of the routed expert outputs and the shared expert
// ("DeepSeek-V4-Flash-SI" card, 架构特性: each token's output is the
// routing-weighted sum of its selected experts, plus the shared expert):
//   y[t] = bf16( sum_j w[t,j] * o[pair_pos[t*k + j]] + ysh[t] )
// summed in fp32 in rank order j.  A gather (one thread per 4 columns of one
// token), so the result is deterministic: no atomics.
#include "moe_internal.h"

namespace moe {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o,
                                                      const float* __restrict__ w,
                                                      const int32_t* __restrict__ pair_pos,
                                                      const float* __restrict__ ysh,
                                                      uint16_t* __restrict__ y, int64_t T, int H,
                                                      int k) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;  // one float4 of y
  const int per_row = H / 4;
  const int64_t t = q / per_row;
  if (t >= T) return;
  const int c = (int)(q - t * per_row) * 4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const float wj = w[t * k + j];
    const float4 v = *reinterpret_cast<const float4*>(o + (size_t)pair_pos[t * k + j] * H + c);
    acc.x = fmaf(wj, v.x, acc.x);
    acc.y = fmaf(wj, v.y, acc.y);
    acc.z = fmaf(wj, v.z, acc.z);
    acc.w = fmaf(wj, v.w, acc.w);
  }
  if (ysh) {
    const float4 s = *reinterpret_cast<const float4*>(ysh + (size_t)t * H + c);
    acc.x += s.x; acc.y += s.y; acc.z += s.z; acc.w += s.w;
  }
  const uint32_t lo = f32_to_bf16(acc.x) | (f32_to_bf16(acc.y) << 16);
  const uint32_t hi = f32_to_bf16(acc.z) | (f32_to_bf16(acc.w) << 16);
  *reinterpret_cast<uint2*>(y + (size_t)t * H + c) = make_uint2(lo, hi);
}

hipError_t launch_combine(const float* o, const float* topk_w, const int32_t* pair_pos,
                          const float* ysh, uint16_t* y, int64_t T, int H, int k,
                          hipStream_t st) {
  const int64_t n = T * (H / 4);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, o,
                     topk_w, pair_pos, ysh, y, T, H, k);
  return hipGetLastError();
}

}  // namespace moe
