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
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

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

}  // namespace

// LDS row stride of the staged scale lines: 256 bytes (K = 4096) + 16, so
// that the 16 rows a wave reads at one K offset fall in distinct banks
constexpr int kNvScaleStride = 272;
__shared__ uint32_t nv_lds[4 * 4 * 16 * kNvScaleStride / 4];   // 69632 bytes

// LINE: K <= 4096 -- each wave copies the whole scale lines of its 64 weight
// rows (at most 256 bytes each) to its own LDS area once, and every step
// reads its two bytes per row from there.  Read from HBM a group of steps at
// a time (32 of a line's bytes every four steps), the lines were fetched
// again and again (~25% more HBM reads at decode).  Longer K loads each
// group's scales with the group (see below).
template <int MODE, bool LINE>
__global__ __launch_bounds__(kGemmThreads, 2) void expert_gemm_nv(ExpertGemmArgs p, int mt_max,
                                                                int n_tiles) {
  __shared__ float red[4][16];
  int n_tile, e, m0, off_e, n_e;
  if (!map_expert_tile(p, mt_max, n_tiles, 16, n_tile, e, m0, off_e, n_e)) return;

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int K = p.K, N = p.N;
  const int S = K / 128;                    // a multiple of 4
  const size_t wrow_bytes = (size_t)K / 2;
  const size_t srow_bytes = (size_t)K / 16;

  // weight tile t: 16 rows from a wave-uniform base; two K steps of its
  // rows go out as two whole-line loads (lane (grp, col): row col % 8, then
  // row 8 + col % 8, bytes 64 * (col / 8) + 16 * grp of the line), turned
  // into the steps' operands by line_pair_to_steps
  const uint8_t* wtile[4];
  const uint32_t loff = (uint32_t)((col & 7) * wrow_bytes + 64 * (col >> 3) + 16 * grp);
  const uint8_t* sptr[4];   // + 8 * grp
  const uint8_t* srow[4];   // scale line of the lane's weight row
  int n0;
  bool wave_live = true;
  if (MODE == 1) {
    n0 = n_tile * kG1Cols;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row0 = n0 + 32 * wv + 16 * (t & 1);
      const int row = row0 + col;
      const uint8_t* base = (t < 2) ? p.w : p.w3;
      const uint8_t* sbase = (t < 2) ? p.w_scale : p.w3_scale;
      wtile[t] = base + ((size_t)e * N + row0) * wrow_bytes;
      srow[t] = sbase + ((size_t)e * N + row) * srow_bytes;
      sptr[t] = srow[t] + grp * 8;
    }
  } else {
    n0 = n_tile * kG2Rows;
    wave_live = (n0 + 64 * wv) < N;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row0 = wave_live ? (n0 + 64 * wv + 16 * t) : 0;
      const int row = row0 + col;
      wtile[t] = p.w + ((size_t)e * N + row0) * wrow_bytes;
      srow[t] = p.w_scale + ((size_t)e * N + row) * srow_bytes;
      sptr[t] = srow[t] + grp * 8;
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
    // Register ring of four K steps (weight and activation bytes); the
    // scales come once per group of four steps: lane group g loads the 8
    // scale bytes of step 4i+g of its row (32 contiguous bytes per row), and
    // a 4x4 transpose across the lane groups hands every lane the pair of
    // scales it needs in each of the four steps.
    v4u A[4][4], B[4][2];
    v2u SR[4];
    uint32_t BSW;
    // LINE: [tile][row][byte] scale lines of this wave's rows
    uint8_t* const lds_sc = LINE ? reinterpret_cast<uint8_t*>(nv_lds) + wv * (4 * 16 * kNvScaleStride) : nullptr;
    // steps s, s + 1 (s even): the weight lines of the two steps (rows 0-7 of
    // each tile into a0, rows 8-15 into a1, non-temporal), and each step's
    // activation bytes
    const size_t w8 = 8 * wrow_bytes;
    auto load_pair = [&](int s, v4u (&a0)[4], v4u (&b0)[2], v4u (&a1)[4], v4u (&b1)[2]) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        a0[t] = wload<v4u>(wtile[t] + loff + (size_t)s * 64);
        a1[t] = wload<v4u>(wtile[t] + w8 + loff + (size_t)s * 64);
      }
      b0[0] = *reinterpret_cast<const v4u*>(bptr + (size_t)s * 128);
      b0[1] = *reinterpret_cast<const v4u*>(bptr + (size_t)s * 128 + 16);
      b1[0] = *reinterpret_cast<const v4u*>(bptr + (size_t)s * 128 + 128);
      b1[1] = *reinterpret_cast<const v4u*>(bptr + (size_t)s * 128 + 144);
    };
    auto load_scales = [&](int s0) {
      if constexpr (!LINE) {
#pragma unroll
        for (int t = 0; t < 4; ++t) SR[t] = *reinterpret_cast<const v2u*>(sptr[t] + (size_t)s0 * 8);
      }
      BSW = *reinterpret_cast<const uint32_t*>(bsp + s0);
    };
    // scale pairs of this lane for steps s0..s0+3: ST[t][d] = two fp16
    auto transpose_scales = [&](uint32_t (&st)[4][4]) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        uint32_t r[4];
        r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(SR[t].x, 1.0f, false));
        r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(SR[t].x, 1.0f, true));
        r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(SR[t].y, 1.0f, false));
        r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(SR[t].y, 1.0f, true));
        // lane groups 2,3 of r[0], r[1] <-> lane groups 0,1 of r[2], r[3]
        const auto x02 = __builtin_amdgcn_permlane32_swap(r[0], r[2], false, false);
        const auto x13 = __builtin_amdgcn_permlane32_swap(r[1], r[3], false, false);
        // odd lane groups of the first operand <-> even lane groups of the second
        const auto y01 = __builtin_amdgcn_permlane16_swap(x02[0], x13[0], false, false);
        const auto y23 = __builtin_amdgcn_permlane16_swap(x02[1], x13[1], false, false);
        st[t][0] = y01[0];
        st[t][1] = y01[1];
        st[t][2] = y23[0];
        st[t][3] = y23[1];
      }
    };
    auto compute = [&](const v4u (&a)[4], const uint32_t (&st)[4][4], int d, const v4u (&b)[2],
                       uint32_t bsw) {
      const float sx = __uint_as_float(((bsw >> (8 * d)) & 0xFFu) << 23);  // 2^(code - 127)
      h8 bo[4];
      bo[0] = fp8x8_to_f16(b[0].x, b[0].y);
      bo[1] = fp8x8_to_f16(b[0].z, b[0].w);
      bo[2] = fp8x8_to_f16(b[1].x, b[1].y);
      bo[3] = fp8x8_to_f16(b[1].z, b[1].w);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const h2 ws = __builtin_bit_cast(h2, st[t][d]);
        v4f part = {0.f, 0.f, 0.f, 0.f};
        part = __builtin_amdgcn_mfma_f32_16x16x32_f16(fp4x8_to_f16(a[t].x, ws[0]), bo[0], part, 0, 0, 0);
        part = __builtin_amdgcn_mfma_f32_16x16x32_f16(fp4x8_to_f16(a[t].y, ws[0]), bo[1], part, 0, 0, 0);
        part = __builtin_amdgcn_mfma_f32_16x16x32_f16(fp4x8_to_f16(a[t].z, ws[1]), bo[2], part, 0, 0, 0);
        part = __builtin_amdgcn_mfma_f32_16x16x32_f16(fp4x8_to_f16(a[t].w, ws[1]), bo[3], part, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[t][v] = __builtin_fmaf(part[v], sx, acc[t][v]);
      }
    };
    // one group of four steps; LOAD: refill the ring with the next group
    auto group = [&](int s0, auto load) {
      uint32_t st[4][4];
      if constexpr (LINE) {
        // the lane's pair of scales (scale groups 2 grp, 2 grp + 1) per step
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const uint32_t raw = *reinterpret_cast<const uint16_t*>(
                lds_sc + (t * 16 + col) * kNvScaleStride + 8 * (s0 + d) + 2 * grp);
            st[t][d] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw, 1.0f, false));
          }
      } else {
        transpose_scales(st);
      }
      const uint32_t bsw = BSW;
      if constexpr (decltype(load)::value) load_scales(s0 + 4);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        if ((d & 1) == 0) {
#pragma unroll
          for (int t = 0; t < 4; ++t) line_pair_to_steps(A[d][t], A[d + 1][t]);
        }
        compute(A[d], st, d, B[d], bsw);
        // refill two steps at a time (one weight line pair)
        if constexpr (decltype(load)::value) {
          if (d & 1) load_pair(s0 + 3 + d, A[d - 1], B[d - 1], A[d], B[d]);
        }
        __builtin_amdgcn_sched_barrier(0);   // keep each refill behind its compute
      }
    };
    v4u SL[4][4];
    if constexpr (LINE) {
      // lane group g copies bytes 64 g .. 64 g + 63 of each line; pieces past
      // the line's end clamp to its last 16 bytes (same data, same place)
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          SL[t][j] = *reinterpret_cast<const v4u*>(srow[t] + min(64 * grp + 16 * j, 8 * S - 16));
      __builtin_amdgcn_sched_barrier(0);
    }
    load_scales(0);
    load_pair(0, A[0], B[0], A[1], B[1]);
    __builtin_amdgcn_sched_barrier(0);   // same issue order as in the loop
    load_pair(2, A[2], B[2], A[3], B[3]);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (LINE) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<v4u*>(lds_sc + (t * 16 + col) * kNvScaleStride +
                                  min(64 * grp + 16 * j, 8 * S - 16)) = SL[t][j];
    }
    for (int s0 = 0; s0 < S - 4; s0 += 4) group(s0, std::true_type{});
    group(S - 4, std::false_type{});
  }

  if (MODE == 1) {
    float h[2][4];
    const float lim = p.limit;
    float amax = 0.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float g = clamp_sym(acc[tt][v], lim);
        const float u = clamp_sym(acc[tt + 2][v], lim);
        const float hv = silu_fast(g) * u;
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
        const uint32_t word = e4m3x4_exp(h[tt], ex);
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

// ---------------------------------------------------------------------------
// Larger batches: m-tiles of 64 pairs (K <= 4096)
// ---------------------------------------------------------------------------
// Eight waves of 32 weight rows (GEMM1: 16 h columns, their w1 and w3 rows;
// GEMM2: 32 output columns); the register ring of weight steps as above.
// The m-tile's 64 activation rows of a K step are converted to fp16 once,
// by the staging lanes, into LDS (double buffer; 16-byte chunk c of a row at
// slot c ^ (row & 15), so that the 16 rows a wave reads at one offset hit
// distinct banks), and every wave takes four 16-pair sub-tiles from there:
// each dequantized weight operand feeds four MFMAs.  The waves' scale lines
// (staged as in the LINE streaming kernel) and the 64 tokens' activation
// scales stay in LDS for the tile; one barrier per K step.  Tiles whose
// activation scales all lie in the range fp16 can carry exactly are staged
// with the scales applied and accumulate in the MFMAs; the others stage the
// unscaled codes and scale each step's sums on the VALU (see the kernel).
constexpr int kNvM = 64;
constexpr int kNvMThreads = 512;

template <int MODE>
__global__ __launch_bounds__(kNvMThreads, 1) void expert_gemm_nv_m64(ExpertGemmArgs p,
                                                                      int mt_max, int n_tiles) {
  __shared__ __attribute__((aligned(16))) uint8_t xl[2][kNvM * 256];   // fp16 activations
  __shared__ __attribute__((aligned(16))) uint8_t bsl[kNvM][32];
  __shared__ float red[8][kNvM];
  int n_tile, e, m0, off_e, n_e;
  if (!map_expert_tile_em(p, n_tiles, kNvM, n_tile, e, m0, off_e, n_e)) return;

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int K = p.K, N = p.N;
  const int S = K / 128;                    // a multiple of 4, at most 32
  const size_t wrow_bytes = (size_t)K / 2;
  const size_t srow_bytes = (size_t)K / 16;

  const uint8_t* wptr[2];
  const uint8_t* srow[2];
  int n0;
  if (MODE == 1) {
    n0 = n_tile * kG1Cols;
    const int row = n0 + 16 * wv + col;       // h column: its w1 row (t 0) and w3 row (t 1)
    wptr[0] = p.w + ((size_t)e * N + row) * wrow_bytes + grp * 16;
    wptr[1] = p.w3 + ((size_t)e * N + row) * wrow_bytes + grp * 16;
    srow[0] = p.w_scale + ((size_t)e * N + row) * srow_bytes;
    srow[1] = p.w3_scale + ((size_t)e * N + row) * srow_bytes;
  } else {
    n0 = n_tile * kG2Rows;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int row = min(n0 + 32 * wv + 16 * t + col, N - 1);
      wptr[t] = p.w + ((size_t)e * N + row) * wrow_bytes + grp * 16;
      srow[t] = p.w_scale + ((size_t)e * N + row) * srow_bytes;
    }
  }
  uint8_t* const lds_sc = reinterpret_cast<uint8_t*>(nv_lds) + wv * (32 * kNvScaleStride);

  // staging role: thread (sr, sq) converts bytes 16 sq .. 16 sq + 15 of token
  // row sr of each step (fp16 chunks 2 sq, 2 sq + 1); rows past the expert's
  // last pair repeat that pair's row (computed, dropped)
  const int sr = threadIdx.x >> 3, sq = threadIdx.x & 7;
  const int sslot = min(m0 + sr, n_e - 1);
  const int64_t stok = (MODE == 1) ? (int64_t)(p.sorted_pairs[off_e + sslot] / p.top_k)
                                   : (int64_t)(off_e + sslot);
  const uint8_t* xsrc = p.a + stok * K + 16 * sq;
  const int xc0 = sr * 256 + ((2 * sq) ^ (sr & 15)) * 16;
  const int xc1 = sr * 256 + ((2 * sq + 1) ^ (sr & 15)) * 16;

  // tile-long LDS tables: the 64 tokens' activation scales, this wave's
  // weight scale lines (pieces past a line's end clamp to its last 16
  // bytes: same data, same place)
  {
    const int b0 = min(4 * sq, S - 4);
    *reinterpret_cast<uint32_t*>(&bsl[sr][b0]) =
        *reinterpret_cast<const uint32_t*>(p.a_scale + stok * S + b0);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int pos = min(64 * grp + 16 * j, 8 * S - 16);
        *reinterpret_cast<v4u*>(lds_sc + (16 * t + col) * kNvScaleStride + pos) =
            *reinterpret_cast<const v4u*>(srow[t] + pos);
      }
  }

  // Scaled staging: when every activation scale of the tile is 2^e with
  // -15 <= e <= 7, the staged fp16 values can carry their scale exactly
  // (448 * 2^7 < 65504, and the E4M3 grid step 2^-9 times 2^-15 is still
  // an fp16 subnormal step), so the MFMAs accumulate straight into acc; else
  // the unscaled codes, each step's sums then scaled into acc (exact powers
  // of two) by the VALU.
  bool scaled_ok = true;
  {
    const int b0 = min(4 * sq, S - 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = p.a_scale[stok * S + b0 + j];
      scaled_ok = scaled_ok && c >= 127 - 15 && c <= 127 + 7;
    }
  }
  const bool scaled = __syncthreads_and(scaled_ok);

  v4f acc[2][4];   // [weight tile][16-pair sub-tile]
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[t][m] = v4f{0.f, 0.f, 0.f, 0.f};

  v4u A[4][2];     // weight ring: [step][tile]
  v4u R;           // the 16 activation bytes of the next step to stage
  auto load_w = [&](int s, v4u (&a)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) a[t] = *reinterpret_cast<const v4u*>(wptr[t] + (size_t)s * 64);
  };
  auto load_x = [&](int s) { R = *reinterpret_cast<const v4u*>(xsrc + (size_t)s * 128); };
  // the rows of step s (in R) into LDS buffer buf; SC: times 2^(e_s - 127)
  auto store_x = [&](int buf, int s, auto sc) {
    h8 lo = fp8x8_to_f16(R.x, R.y), hi = fp8x8_to_f16(R.z, R.w);
    if constexpr (decltype(sc)::value) {
      const _Float16 f = (_Float16)__uint_as_float((uint32_t)bsl[sr][s] << 23);
      const h8 fv = {f, f, f, f, f, f, f, f};
      lo = lo * fv;
      hi = hi * fv;
    }
    *reinterpret_cast<h8*>(&xl[buf][xc0]) = lo;
    *reinterpret_cast<h8*>(&xl[buf][xc1]) = hi;
  };
  // one K step from the weight ring slot a and LDS buffer buf: MFMA j of a
  // 16 x 16 tile takes elements 32 grp + 8 j .. +7 of the step
  auto compute = [&](int s, const v4u (&a)[2], int buf, auto sc) {
    h8 wb[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint32_t raw = *reinterpret_cast<const uint16_t*>(
          lds_sc + (16 * t + col) * kNvScaleStride + 8 * s + 2 * grp);
      const h2 ws = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw, 1.0f, false);
      wb[t][0] = fp4x8_to_f16(a[t].x, ws[0]);
      wb[t][1] = fp4x8_to_f16(a[t].y, ws[0]);
      wb[t][2] = fp4x8_to_f16(a[t].z, ws[1]);
      wb[t][3] = fp4x8_to_f16(a[t].w, ws[1]);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int r = 16 * m + col;
      const uint8_t* xr = &xl[buf][r * 256];
      h8 bo[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bo[j] = *reinterpret_cast<const h8*>(xr + ((4 * grp + j) ^ (r & 15)) * 16);
      if constexpr (decltype(sc)::value) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[t][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wb[t][j], bo[j], acc[t][m], 0, 0, 0);
      } else {
        const float sx = __uint_as_float((uint32_t)bsl[r][s] << 23);   // 2^(code - 127)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          v4f part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int j = 0; j < 4; ++j)
            part = __builtin_amdgcn_mfma_f32_16x16x32_f16(wb[t][j], bo[j], part, 0, 0, 0);
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[t][m][v] = __builtin_fmaf(part[v], sx, acc[t][m][v]);
        }
      }
    }
  };
  // one group of four steps; LOAD: refill the weight ring with the next group
  // (two steps at a time: both halves of each 128-byte line back to back)
  auto group = [&](int s0, auto load, auto sc) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int s = s0 + d;
      compute(s, A[d], s & 1, sc);
      store_x((s + 1) & 1, min(s + 1, S - 1), sc);   // step s + 1 (the last step's copy is unused)
      load_x(min(s + 2, S - 1));
      if constexpr (decltype(load)::value) {
        if (d & 1) {
          load_w(s0 + 3 + d, A[d - 1]);
          load_w(s0 + 4 + d, A[d]);
        }
      }
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);   // no work moved across steps
    }
  };

  auto k_loop = [&](auto sc) {
    load_x(0);
    store_x(0, 0, sc);
    load_x(min(1, S - 1));
#pragma unroll
    for (int d = 0; d < 4; ++d) load_w(d, A[d]);
    __syncthreads();
    for (int s0 = 0; s0 < S - 4; s0 += 4) group(s0, std::true_type{}, sc);
    group(S - 4, std::false_type{}, sc);
  };
  if (scaled)
    k_loop(std::true_type{});
  else
    k_loop(std::false_type{});

  // lane holds acc[t][m][v] = output (weight row 4 grp + v of tile t, token
  // 16 m + col)
  if (MODE == 1) {
    const float lim = p.limit;
    float h[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float a = 0.f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float g = clamp_sym(acc[0][m][v], lim);
        const float u = clamp_sym(acc[1][m][v], lim);
        h[m][v] = silu_fast(g) * u;
        a = fmaxf(a, fabsf(h[m][v]));
      }
      a = fmaxf(a, __shfl_xor(a, 16));
      a = fmaxf(a, __shfl_xor(a, 32));
      if (lane < 16) red[wv][16 * m + col] = a;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int tok = 16 * m + col;
      if (m0 + tok >= n_e) continue;
      float bmax = red[0][tok];
#pragma unroll
      for (int w = 1; w < 8; ++w) bmax = fmaxf(bmax, red[w][tok]);
      const int ex = pow2_scale_exp(bmax);
      const size_t row = (size_t)(off_e + m0 + tok);
      const uint32_t word = e4m3x4_exp(h[m], ex);
      *reinterpret_cast<uint32_t*>(p.hq + row * N + n0 + 16 * wv + 4 * grp) = word;
      if (wv == 0 && grp == 0) p.hs[row * (N / 128) + n0 / 128] = (uint8_t)(ex + 127);
    }
  } else {
    if (n0 + 32 * wv >= N) return;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int tok = 16 * m + col;
      if (m0 + tok >= n_e) continue;
      const size_t row = (size_t)(off_e + m0 + tok);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const size_t c = (size_t)n0 + 32 * wv + 16 * t + 4 * grp;
        if (p.out_fp32) {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + row * N + c) =
              make_float4(acc[t][m][0], acc[t][m][1], acc[t][m][2], acc[t][m][3]);
        } else {
          const uint32_t lo = f32_to_bf16(acc[t][m][0]) | (f32_to_bf16(acc[t][m][1]) << 16);
          const uint32_t hi = f32_to_bf16(acc[t][m][2]) | (f32_to_bf16(acc[t][m][3]) << 16);
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + row * N + c) =
              make_uint2(lo, hi);
        }
      }
    }
  }
}

static unsigned pad8_nv(int64_t g) { return (unsigned)((g + 7) / 8 * 8); }

template <int MODE>
static hipError_t launch_nv(const ExpertGemmArgs& a, int bm, int mt_max, hipStream_t st) {
  if (a.K % 512) return hipErrorInvalidValue;
  const int n_tiles = MODE == 1 ? a.N / kG1Cols : (a.N + kG2Rows - 1) / kG2Rows;
  const unsigned grid = pad8_nv((int64_t)n_tiles * mt_max);
  if (grid == 0) return hipSuccess;
  if (bm == kNvM) {
    if (a.K > 4096) return hipErrorInvalidValue;
    hipLaunchKernelGGL((expert_gemm_nv_m64<MODE>), dim3(grid), dim3(kNvMThreads), 0, st, a,
                       mt_max, n_tiles);
  } else if (bm != 16) {
    return hipErrorInvalidValue;
  } else if (a.K <= 4096)
    hipLaunchKernelGGL((expert_gemm_nv<MODE, true>), dim3(grid), dim3(kGemmThreads), 0, st, a,
                       mt_max, n_tiles);
  else
    hipLaunchKernelGGL((expert_gemm_nv<MODE, false>), dim3(grid), dim3(kGemmThreads), 0, st, a,
                       mt_max, n_tiles);
  return hipGetLastError();
}

hipError_t launch_expert_gemm1_nv(const ExpertGemmArgs& a, int bm, int mt_max, hipStream_t st) {
  return launch_nv<1>(a, bm, mt_max, st);
}
hipError_t launch_expert_gemm2_nv(const ExpertGemmArgs& a, int bm, int mt_max, hipStream_t st) {
  return launch_nv<2>(a, bm, mt_max, st);
}

}  // namespace moe
