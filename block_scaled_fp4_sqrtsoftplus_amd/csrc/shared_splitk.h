// Decode-sized bf16 shared expert ("DeepSeek-V4-Flash-SI" card, 架构特性: one
// shared expert beside the routed ones, non-expert weights bf16, SwiGLU
// clamped to +-10) as split-K device code, for M <= 64 tokens with H and I
// multiples of 512.  The bodies below run inside stand-alone kernels
// (bf16_gemm.hip) or as extra workgroups of the routing launches (route.hip,
// bf16_gemm.hip), so that at decode sizes the shared expert needs no launch
// and no stream of its own.
//
// Split-K GEMM body: workgroup (bx, s) of NW waves owns a block of weight rows
// and the K slice [512 s, 512 (s+1)).  The slice of the token rows (64 rows,
// rows >= M repeat row M - 1) is staged once in LDS -- 16-byte chunk c of row r
// at slot c ^ (r & 7), so the 16-byte operand reads of 8 consecutive rows hit
// distinct banks -- and shared by all waves; wave (rw, kw) owns two 16-row
// weight tiles (EPI_SWIGLU: the w1 tile and the w3 tile of the same 16 h
// columns; EPI_F32: two consecutive tiles) and the kw-th 1/KW of the slice,
// and issues all of its weight loads at once.  The KW partial sums of a tile
// meet in LDS in a fixed tree; wave kw = 0 writes P[s][t][n] (EPI_SWIGLU:
// g at n, u at N + n, rows of 2N floats).  The S slices are added in slice
// order by shared_swiglu_body (up) or by the combine (down), so results do
// not depend on timing.
#pragma once

#include "moe_internal.h"

namespace moe {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

enum { EPI_F32 = 0, EPI_SWIGLU = 1 };

__device__ __forceinline__ v4f mfma_bf16(const uint4& a, const uint4& b, v4f acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

// Workgroup rows of the split-K body: EPI_SWIGLU h columns (16 per row
// wave), EPI_F32 weight rows (32 per row wave).
template <int EPI, int RW>
constexpr int shared_splitk_rows() {
  return EPI == EPI_SWIGLU ? 16 * RW : 32 * RW;
}

// xs: 64 x 64 16-byte LDS slots (64 KB), also the reduction buffer.
template <int EPI, int NW, int RW>
__device__ __forceinline__ void shared_splitk_body(const uint16_t* __restrict__ X,
                                                   const uint16_t* __restrict__ W,
                                                   const uint16_t* __restrict__ W3,
                                                   float* __restrict__ P, int M, int N, int K,
                                                   int bx, int s, uint4 (*xs)[64]) {
  constexpr int KW = NW / RW;
  constexpr int KSL = kSharedSplitK;
  constexpr int KSW = KSL / KW;             // K per wave
  constexpr int STEPS = KSW / 32;
  constexpr int NT = NW * 64;
  constexpr int CH = KSL / 8;               // 16-byte chunks of a token row's slice
  constexpr int XL = 64 * CH / NT;          // 16-byte staging loads per thread
  static_assert(NW % RW == 0 && STEPS >= 1 && 64 * CH % NT == 0 && CH % 8 == 0 && CH <= 64,
                "split-K shape");
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int rw = wv % RW, kw = wv / RW;
  const int col = lane & 15, grp = lane >> 4;
  const int k0 = s * KSL;
  const uint16_t* wp[2];
  if (EPI == EPI_SWIGLU) {
    const int c = bx * 16 * RW + 16 * rw + col;
    wp[0] = W + (size_t)c * K;
    wp[1] = W3 + (size_t)c * K;
  } else {
    const int r = bx * 32 * RW + 32 * rw + col;
    wp[0] = W + (size_t)r * K;
    wp[1] = W + (size_t)(r + 16) * K;
  }
  const int kb = k0 + kw * KSW + 8 * grp;
  uint4 xv[XL];
#pragma unroll
  for (int it = 0; it < XL; ++it) {
    const int q = it * NT + tid;
    const int row = q / CH, ch = q % CH;
    xv[it] = *reinterpret_cast<const uint4*>(X + (size_t)min(row, M - 1) * K + k0 + 8 * ch);
  }
  uint4 A[STEPS][2];
#pragma unroll
  for (int j = 0; j < STEPS; ++j)
#pragma unroll
    for (int t = 0; t < 2; ++t) A[j][t] = *reinterpret_cast<const uint4*>(wp[t] + kb + 32 * j);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int it = 0; it < XL; ++it) {
    const int q = it * NT + tid;
    const int row = q / CH, ch = q % CH;
    xs[row][ch ^ (row & 7)] = xv[it];
  }
  __syncthreads();
  v4f acc[2][4];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[t][m] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < STEPS; ++j) {
    uint4 B[4];
    const int ch = (kw * KSW + 32 * j) / 8 + grp;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int row = 16 * m + col;
      B[m] = xs[row][ch ^ (row & 7)];
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[t][m] = mfma_bf16(A[j][t], B[m], acc[t][m]);
  }
  if constexpr (KW > 1) {
    // slots of 32 x 64 floats (8 KB): RW * KW / 2 <= 8 of them fit in xs
    __syncthreads();
    float* red = reinterpret_cast<float*>(&xs[0][0]);
#pragma unroll
    for (int half = KW / 2; half >= 1; half >>= 1) {
      if (kw >= half && kw < 2 * half) {
        float* r = red + (size_t)(rw * (KW / 2) + kw - half) * 32 * 64;
        int i = 0;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int v = 0; v < 4; ++v) r[(i++) * 64 + lane] = acc[t][m][v];
      }
      __syncthreads();
      if (kw < half) {
        const float* r = red + (size_t)(rw * (KW / 2) + kw) * 32 * 64;
        int i = 0;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[t][m][v] += r[(i++) * 64 + lane];
      }
      __syncthreads();
    }
  }
  if (kw != 0) return;
  // D layout: lane l holds rows 4 (l / 16) + v of a tile for token l % 16
  const int rowlen = EPI == EPI_SWIGLU ? 2 * N : N;
  float* ps = P + (size_t)s * M * rowlen;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int tok = 16 * m + col;
    if (tok >= M) continue;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int n = EPI == EPI_SWIGLU ? t * N + bx * 16 * RW + 16 * rw + 4 * grp
                                      : bx * 32 * RW + 32 * rw + 16 * t + 4 * grp;
      *reinterpret_cast<float4*>(ps + (size_t)tok * rowlen + n) =
          make_float4(acc[t][m][0], acc[t][m][1], acc[t][m][2], acc[t][m][3]);
    }
  }
}

// h[t][c..c+3] for flat index i = t * (N / 4) + c / 4 (i < M * N / 4): g and u
// summed over the S slices in slice order, then bf16(silu(clip(g)) * clip(u)).
__device__ __forceinline__ void shared_swiglu_body(const float* __restrict__ P, int S, int M,
                                                   int N, float limit, uint16_t* __restrict__ h,
                                                   int i) {
  const int q = N / 4;
  if (i >= M * q) return;
  const int t = i / q, c = 4 * (i % q);
  const size_t stride = (size_t)M * 2 * N;
  const float* p = P + (size_t)t * 2 * N + c;
  float4 g = *reinterpret_cast<const float4*>(p);
  float4 u = *reinterpret_cast<const float4*>(p + N);
  for (int s = 1; s < S; ++s) {
    const float4 a = *reinterpret_cast<const float4*>(p + s * stride);
    const float4 b = *reinterpret_cast<const float4*>(p + s * stride + N);
    g.x += a.x; g.y += a.y; g.z += a.z; g.w += a.w;
    u.x += b.x; u.y += b.y; u.z += b.z; u.w += b.w;
  }
  const float gv[4] = {g.x, g.y, g.z, g.w}, uv[4] = {u.x, u.y, u.z, u.w};
  uint32_t hv[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float gg = fminf(fmaxf(gv[v], -limit), limit);
    const float uu = fminf(fmaxf(uv[v], -limit), limit);
    hv[v] = f32_to_bf16(gg / (1.0f + expf(-gg)) * uu);
  }
  *reinterpret_cast<uint2*>(h + (size_t)t * N + c) =
      make_uint2(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16));
}

}  // namespace moe
