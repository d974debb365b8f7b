// MXFP4 -> FP8 expert weights ("DeepSeek-V4-Pro-0813-nvfp4-DSpark" article,
// 阶段一, 关于 MXFP4 的无损种子: the E2M1 nibbles are split and decoded, and
// the block scale is rewritten per 128 elements; the same article names the
// FP8-expert checkpoint option).
//
// Per row and per 128 elements of K: the new E8M0 exponent is the largest of
// the block's four per-32 exponents; every element becomes the E4M3 code
// (round to nearest even, sign kept) of its E2M1 value times 2^(e32 - e128).
// Exact when the four exponents span at most 8 (E4M3's subnormal step 2^-9
// against E2M1's smallest magnitude 0.5); otherwise the smallest values round.
#include "moe_internal.h"

namespace moe {

// |E2M1| of the low three bits of a nibble: 0, 0.5, 1, 1.5, 2, 3, 4, 6
__device__ __forceinline__ float e2m1_mag(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  return e == 0 ? 0.5f * (float)m : __uint_as_float((e + 126u) << 23) * (1.0f + 0.5f * (float)m);
}

// one thread per (row, 128-block): 64 nibble bytes + 4 scale bytes in,
// 128 E4M3 bytes + 1 scale byte out
__global__ __launch_bounds__(256) void cast_fp8_kernel(const uint8_t* __restrict__ w,
                                                       const uint8_t* __restrict__ ws,
                                                       uint8_t* __restrict__ q,
                                                       uint8_t* __restrict__ qs, int64_t rows,
                                                       int K) {
  const int nb = K / 128;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * nb) return;
  const int64_t row = i / nb;
  const int b = (int)(i - row * nb);
  const uint32_t s4 = *reinterpret_cast<const uint32_t*>(ws + row * (K / 32) + 4 * b);
  int e32[4];
  int e128 = -1000;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    e32[j] = (int)((s4 >> (8 * j)) & 0xFFu) - 127;
    e128 = max(e128, e32[j]);
  }
  const uint4* src = reinterpret_cast<const uint4*>(w + row * (K / 2) + 64 * b);
  uint4* dst = reinterpret_cast<uint4*>(q + row * K + 128 * b);
#pragma unroll
  for (int j = 0; j < 4; ++j) {              // 32 elements (one per-32 block) per 16 bytes
    const uint4 in = src[j];
    const float f = ldexpf(1.0f, e32[j] - e128);
    const uint32_t words[4] = {in.x, in.y, in.z, in.w};
    uint32_t out[8];
#pragma unroll
    for (int h = 0; h < 8; ++h) {            // 4 output bytes = 2 input bytes
      const uint32_t two = (words[h >> 1] >> (16 * (h & 1))) & 0xFFFFu;
      uint32_t o = 0;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const uint32_t c = (two >> (4 * n)) & 0xFu;    // element 4h + n: low nibble = even
        const float v = (c & 8u) ? -(e2m1_mag(c) * f) : e2m1_mag(c) * f;
        o |= e4m3_rne(v) << (8 * n);
      }
      out[h] = o;
    }
    dst[2 * j] = make_uint4(out[0], out[1], out[2], out[3]);
    dst[2 * j + 1] = make_uint4(out[4], out[5], out[6], out[7]);
  }
  qs[row * nb + b] = (uint8_t)(e128 + 127);
}

hipError_t launch_cast_fp8(const uint8_t* w, const uint8_t* ws, uint8_t* q, uint8_t* qs,
                           int64_t rows, int K, hipStream_t st) {
  const int64_t n = rows * (K / 128);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(cast_fp8_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, w, ws,
                     q, qs, rows, K);
  return hipGetLastError();
}

}  // namespace moe
