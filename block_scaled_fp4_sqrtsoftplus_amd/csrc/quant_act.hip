// Online FP8 E4M3 activation quantization, one power-of-two (E8M0) scale per
// 128 consecutive elements of a row ("DeepSeek-V4-Flash-SI" card, 架构特性 /
// 低精度计算; 模型训练 table: dynamic FP8 E4M3 with a ue8m0 scale).
//
// Layout: 16 lanes own one 128-element block (8 bf16 = one 16-byte load per
// lane); a 256-thread workgroup covers 16 consecutive blocks of the flattened
// [rows, cols] array, so every load and store is a contiguous run.
#include "moe_internal.h"

namespace moe {

__global__ __launch_bounds__(256) void quant_act_kernel(const uint16_t* __restrict__ x,
                                                        int64_t n_blocks,
                                                        uint8_t* __restrict__ q,
                                                        uint8_t* __restrict__ scale) {
  const int64_t blk = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  const bool live = blk < n_blocks;
  uint4 raw = make_uint4(0, 0, 0, 0);
  if (live) raw = *reinterpret_cast<const uint4*>(x + blk * 128 + sub * 8);
  float v[8];
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
    v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  // reduce over the 16 lanes of the block (xor partners stay inside the group)
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const int e = pow2_scale_exp(amax);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) lo |= e4m3_rne(ldexpf(v[i], -e)) << (8 * i);
#pragma unroll
  for (int i = 0; i < 4; ++i) hi |= e4m3_rne(ldexpf(v[4 + i], -e)) << (8 * i);
  if (live) {
    *reinterpret_cast<uint2*>(q + blk * 128 + sub * 8) = make_uint2(lo, hi);
    if (sub == 0) scale[blk] = (uint8_t)(e + 127);
  }
}

hipError_t launch_quant_act(const uint16_t* x, int64_t rows, int cols, uint8_t* q,
                            uint8_t* scale, hipStream_t st) {
  const int64_t n_blocks = rows * (int64_t)(cols / 128);
  if (n_blocks == 0) return hipSuccess;
  const int64_t grid = (n_blocks + 15) / 16;
  hipLaunchKernelGGL(quant_act_kernel, dim3((unsigned)grid), dim3(256), 0, st, x, n_blocks, q,
                     scale);
  return hipGetLastError();
}

}  // namespace moe
