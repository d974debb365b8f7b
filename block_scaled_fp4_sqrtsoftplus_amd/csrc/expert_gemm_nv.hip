// Grouped expert GEMMs for NVFP4 expert weights ("DeepSeek-V4-Pro-0813-nvfp4-
// DSpark" article, 阶段三导出: the same E2M1 nibble grid as MXFP4, with one
// E4M3 scale -- mantissa included -- per 16 elements instead of an E8M0
// scale per 32).
//
// gfx950's block-scaled MFMA takes power-of-two (E8M0) scales per 32
// elements only, so here each weight element is dequantized in registers to
// fp16: E2M1 value x E4M3 scale (at most 2 + 4 significant bits and within
// [2^-10, 2688]: exact in fp16); the activations' FP8 codes are converted to
// fp16 without their scale (exact), each K step's four fp16 MFMAs
// (v_mfma_f32_16x16x32_f16, exact products, fp32 sums) start from zero, and
// the step's result is added to the accumulator times the token's
// power-of-two activation scale (exact scaling).  Work split, weight-row
// tiles and epilogues (clamped SwiGLU + per-128 FP8 requant of h; fp32 or
// bf16 rows) are those of the streaming FP4 kernel: m-tiles of at most 16
// pairs, four waves of 64 weight rows, a four-step register ring of weight,
// scale and activation loads.
//
// K order: the sum over a 128-element K step does not depend on the order,
// so lane group g (lanes 16g..16g+15) takes elements 32g..32g+31 of the step
// -- 16 contiguous bytes of a weight row, 32 of an activation row -- and MFMA
// j (j = 0..3) takes elements 32g + 8j .. +7 of them.
#include "moe_internal.h"

#include <type_traits>

namespace moe {

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float silu_nv(float g) { return g / (1.0f + expf(-g)); }

// 8 E2M1 nibbles (low nibble first) times an fp16 scale -> 8 fp16
__device__ __forceinline__ h8 fp4x8_to_f16(uint32_t w, _Float16 s) {
  const h2 sc = {s, s};
  const h2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * sc;
  const h2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * sc;
  const h2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * sc;
  const h2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * sc;
  return h8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// 8 E4M3 codes (two dwords) -> 8 fp16, unscaled
__device__ __forceinline__ h8 fp8x8_to_f16(uint32_t lo, uint32_t hi) {
  const h2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
  const h2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
  const h2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
  const h2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
  return h8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ bool map_tile_nv(const ExpertGemmArgs& p, int mt_max, int n_tiles,
                                            int& n_tile, int& e, int& m0, int& off_e, int& n_e) {
  const int G = gridDim.x;
  const int b = blockIdx.x;
  const int w = (b & 7) * (G >> 3) + (b >> 3);   // XCD-aware: consecutive ids per XCD
  n_tile = w / mt_max;
  const int mt = w - n_tile * mt_max;
  if (n_tile >= n_tiles) return false;
  if (mt >= p.mtile_off[p.E]) return false;
  int lo = 0, hi = p.E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.mtile_off[mid] <= mt) lo = mid; else hi = mid;
  }
  e = lo;
  m0 = (mt - p.mtile_off[e]) * 16;
  off_e = p.expert_offsets[e];
  n_e = p.expert_offsets[e + 1] - off_e;
  return true;
}

}  // namespace

template <int MODE>
__global__ __launch_bounds__(kGemmThreads) void expert_gemm_nv(ExpertGemmArgs p, int mt_max,
                                                                int n_tiles) {
  __shared__ float red[4][16];
  int n_tile, e, m0, off_e, n_e;
  if (!map_tile_nv(p, mt_max, n_tiles, n_tile, e, m0, off_e, n_e)) return;

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int K = p.K, N = p.N;
  const int S = K / 128;                    // a multiple of 4
  const size_t wrow_bytes = (size_t)K / 2;
  const size_t srow_bytes = (size_t)K / 16;

  const uint8_t* wptr[4];
  const uint8_t* sptr[4];
  int n0;
  bool wave_live = true;
  if (MODE == 1) {
    n0 = n_tile * kG1Cols;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row = n0 + 32 * wv + 16 * (t & 1) + col;
      const uint8_t* base = (t < 2) ? p.w : p.w3;
      const uint8_t* sbase = (t < 2) ? p.w_scale : p.w3_scale;
      wptr[t] = base + ((size_t)e * N + row) * wrow_bytes + grp * 16;
      sptr[t] = sbase + ((size_t)e * N + row) * srow_bytes + grp * 2;
    }
  } else {
    n0 = n_tile * kG2Rows;
    wave_live = (n0 + 64 * wv) < N;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row = wave_live ? (n0 + 64 * wv + 16 * t + col) : 0;
      wptr[t] = p.w + ((size_t)e * N + row) * wrow_bytes + grp * 16;
      sptr[t] = p.w_scale + ((size_t)e * N + row) * srow_bytes + grp * 2;
    }
  }
  const int slot = min(m0 + col, n_e - 1);
  const int64_t brow = (MODE == 1) ? (int64_t)(p.sorted_pairs[off_e + slot] / p.top_k)
                                   : (int64_t)(off_e + slot);
  const uint8_t* bptr = p.a + brow * K + 32 * grp;
  const uint8_t* bsp = p.a_scale + brow * S;

  v4f acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};

  if (wave_live) {
    // ring of four K steps: weight bytes, the two per-16 scale bytes of each
    // weight row this lane covers, activation bytes and scale
    uint4 A[4][4], B[4][2];
    uint32_t SC[4][4], BS[4];
    auto load_step = [&](int s, uint4 (&a)[4], uint32_t (&sc)[4], uint4 (&b)[2], uint32_t& bs) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        a[t] = *reinterpret_cast<const uint4*>(wptr[t] + (size_t)s * 64);
        sc[t] = *reinterpret_cast<const uint16_t*>(sptr[t] + (size_t)s * 8);
      }
      b[0] = *reinterpret_cast<const uint4*>(bptr + (size_t)s * 128);
      b[1] = *reinterpret_cast<const uint4*>(bptr + (size_t)s * 128 + 16);
      bs = bsp[s];
    };
    auto compute = [&](const uint4 (&a)[4], const uint32_t (&sc)[4], const uint4 (&b)[2],
                       uint32_t bs) {
      const float sx = __uint_as_float(bs << 23);   // 2^(bs - 127): E8M0 as an fp32 exponent
      const uint32_t bw[8] = {b[0].x, b[0].y, b[0].z, b[0].w, b[1].x, b[1].y, b[1].z, b[1].w};
      h8 bo[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) bo[j] = fp8x8_to_f16(bw[2 * j], bw[2 * j + 1]);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const h2 ws = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc[t], 1.0f, false);  // E4M3 scales
        const uint32_t aw[4] = {a[t].x, a[t].y, a[t].z, a[t].w};
        v4f part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          part = __builtin_amdgcn_mfma_f32_16x16x32_f16(fp4x8_to_f16(aw[j], j < 2 ? ws[0] : ws[1]),
                                                        bo[j], part, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[t][v] = __builtin_fmaf(part[v], sx, acc[t][v]);
      }
    };
    load_step(0, A[0], SC[0], B[0], BS[0]);
    load_step(1, A[1], SC[1], B[1], BS[1]);
    load_step(2, A[2], SC[2], B[2], BS[2]);
    load_step(3, A[3], SC[3], B[3], BS[3]);
    // loads past the last step re-read step S-1 (cache hits), so that no
    // load sits behind a branch and the waits before each step stay exact
    for (int s0 = 0; s0 < S; s0 += 4) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        compute(A[d], SC[d], B[d], BS[d]);
        load_step(min(s0 + d + 4, S - 1), A[d], SC[d], B[d], BS[d]);
      }
    }
  }

  if (MODE == 1) {
    float h[2][4];
    const float lim = p.limit;
    float amax = 0.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float g = fminf(fmaxf(acc[tt][v], -lim), lim);
        const float u = fminf(fmaxf(acc[tt + 2][v], -lim), lim);
        const float hv = silu_nv(g) * u;
        h[tt][v] = hv;
        amax = fmaxf(amax, fabsf(hv));
      }
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    if (lane < 16) red[wv][lane] = amax;
    __syncthreads();
    const float bmax = fmaxf(fmaxf(red[0][col], red[1][col]), fmaxf(red[2][col], red[3][col]));
    const int ex = pow2_scale_exp(bmax);
    if (m0 + col < n_e) {
      const size_t row = (size_t)(off_e + m0 + col);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        uint32_t word = 0;
#pragma unroll
        for (int v = 0; v < 4; ++v) word |= e4m3_rne(ldexpf(h[tt][v], -ex)) << (8 * v);
        *reinterpret_cast<uint32_t*>(p.hq + row * N + n0 + 32 * wv + 16 * tt + 4 * grp) = word;
      }
      if (wv == 0 && grp == 0) p.hs[row * (N / 128) + n0 / 128] = (uint8_t)(ex + 127);
    }
  } else {
    if (!wave_live || m0 + col >= n_e) return;
    const size_t row = (size_t)(off_e + m0 + col);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const size_t c = (size_t)n0 + 64 * wv + 16 * t + 4 * grp;
      if (p.out_fp32) {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + row * N + c) =
            make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
      } else {
        const uint32_t lo = f32_to_bf16(acc[t][0]) | (f32_to_bf16(acc[t][1]) << 16);
        const uint32_t hi = f32_to_bf16(acc[t][2]) | (f32_to_bf16(acc[t][3]) << 16);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + row * N + c) =
            make_uint2(lo, hi);
      }
    }
  }
}

static unsigned pad8_nv(int64_t g) { return (unsigned)((g + 7) / 8 * 8); }

template <int MODE>
static hipError_t launch_nv(const ExpertGemmArgs& a, int mt_max, hipStream_t st) {
  if (a.K % 512) return hipErrorInvalidValue;
  const int n_tiles = MODE == 1 ? a.N / kG1Cols : (a.N + kG2Rows - 1) / kG2Rows;
  const unsigned grid = pad8_nv((int64_t)n_tiles * mt_max);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((expert_gemm_nv<MODE>), dim3(grid), dim3(kGemmThreads), 0, st, a, mt_max,
                     n_tiles);
  return hipGetLastError();
}

hipError_t launch_expert_gemm1_nv(const ExpertGemmArgs& a, int mt_max, hipStream_t st) {
  return launch_nv<1>(a, mt_max, st);
}
hipError_t launch_expert_gemm2_nv(const ExpertGemmArgs& a, int mt_max, hipStream_t st) {
  return launch_nv<2>(a, mt_max, st);
}

}  // namespace moe
