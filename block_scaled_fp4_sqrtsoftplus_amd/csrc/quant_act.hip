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
  quant_act_block(x, blk, n_blocks, threadIdx.x & 15, q, scale);
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
