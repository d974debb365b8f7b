// Grouped expert GEMMs for W4AFP8 expert weights ("DeepSeek-V4-Flash-0731-
// W4AFP8-mt" card, 量化方式 and 权重约定: signed INT4, two per byte along K,
// one float32 scale per 128 elements of K; FP8 E4M3 activations).
//
// A K step is 128 elements: one weight scale group and one activation
// block.  The INT4 code q of nibble n (two's complement) enters the FP8 MFMA
// as the E4M3 byte u = n ^ 8 = q + 8 in 0..15.  E4M3 codes 0..15 encode
// exactly u * 2^-9 (subnormals below 8, exponent field 1 from 8 up), so with
// a block scale of 2^9 on that operand the step's MFMA gives
// sum_k (q_k + 8) x_k.  One more MFMA per step, against a constant operand of
// code 0x88 (-8 * 2^-9), gives -8 sum_k x_k per token, which enters the
// step's weight MFMAs as their accumulator input, so that they return
// sum_k q_k x_k; the row's float32 group scale then multiplies that into the
// accumulator.
// The products u * x are exact (4 x 4 significant bits) and the per-step
// sums are fp32, as in the other expert GEMMs.
//
// MFMA roles are swapped relative to the FP4 kernels: A = activations (rows
// = the m-tile's 16 pairs, their E8M0 scale per 128 as A's block scale),
// B = weights (columns = 16 weight rows), so that the four results a lane
// holds share one weight row and one group scale.  Lane l (c = l % 16,
// g = l / 16) supplies token c and weight row c of the tile; lane group g
// takes elements 32g .. 32g+31 of the step: 16 bytes of the weight row and
// 32 bytes of the activation row.  The unpacked weight bytes come out as
// the even elements of each 8 followed by the odd ones, and the activation
// bytes are permuted the same way (both operands share the MFMA's K slots,
// so any common order sums the same products).  D: lane l holds
// D[4g + v][c] -- token 4g + v, weight row c.
//
// Work split, m-tiles of 16 pairs, 4 waves x 64 weight rows, the register
// ring of four K steps, the per-group scale loads and the XCD-aware tile map
// follow the NVFP4 expert GEMMs; K must be a multiple of 512.
#include "moe_internal.h"

#include <type_traits>

namespace moe {

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// The MFMA groups below (E8M0 block scales sa on A, sb on B) leave 2 wait
// states between the VALU instructions that build the operands and the
// first MFMA (the compiler cannot insert them in front of an asm; without
// them the MFMA read a stale B register), and the scale registers and the
// results untouched for 32 wait states after the last, as in the FP4
// kernels.

// Five MFMAs for one 16-pair step: c = a . neg8 from zero (neg8: E4M3 code
// 0x88 = -8 * 2^-9, so with the 2^9 block scale c = -8 sum x per token), then
// d[t] = a . b[t] + c for the four weight tiles; the corrected sums come out
// of the matrix pipe (as in mfma_w4x12 below).
__device__ __forceinline__ void mfma_w4x5(const v8i& a, const v8i& neg8, const v8i (&b)[4], int sa,
                                          int sb, v4f& c, v4f (&d)[4]) {
#define W4X5_ROW(T)                                                                        \
  "v_mfma_scale_f32_16x16x128_f8f6f4 %[d" #T "], %[a], %[b" #T "], %[c], %[s], %[t] op_sel_hi:[0,0,0]\n\t"
  asm volatile(
      "s_nop 1\n\t"
      "v_mfma_scale_f32_16x16x128_f8f6f4 %[c], %[a], %[e], 0, %[s], %[t] op_sel_hi:[0,0,0]\n\t"
      "s_nop 1\n\t"
      W4X5_ROW(0) W4X5_ROW(1) W4X5_ROW(2) W4X5_ROW(3)
      "s_nop 15\n\t"
      "s_nop 15"
      : [c] "=&v"(c), [d0] "=&v"(d[0]), [d1] "=&v"(d[1]), [d2] "=&v"(d[2]), [d3] "=&v"(d[3])
      : [a] "v"(a), [e] "v"(neg8), [b0] "v"(b[0]), [b1] "v"(b[1]), [b2] "v"(b[2]),
        [b3] "v"(b[3]), [s] "v"(sa), [t] "v"(sb));
#undef W4X5_ROW
}

// Twelve MFMAs: for the four activation operands a[m] (block scales sa[m]),
// c[m] = a[m] . neg8 from zero (neg8: E4M3 code 0x88 = -8 * 2^-9, so with
// the 2^9 block scale c[m] = -8 sum x per token), then d0[m] = a[m] . b0 +
// c[m] and d1[m] = a[m] . b1 + c[m]: the step's sums with the correction
// already applied, taken as the MFMAs' accumulator input (exactly the
// registers the correction MFMA wrote, which the matrix pipe interlocks like
// an accumulation chain; a 32-wait-state gap there measured slower and gave
// the same bits).  One 2-wait-state lead, one 32-wait-state guard for the
// group.  Result: the same bits as subtracting c[m] from the two sums
// afterwards, one VALU op less per result and step, and GEMM2's kernel
// (which spilled with the subtraction) within its registers.
__device__ __forceinline__ void mfma_w4x12(const v8i (&a)[4], const v8i& neg8, const v8i& b0,
                                           const v8i& b1, const int (&sa)[4], int sb,
                                           v4f (&c)[4], v4f (&d0)[4], v4f (&d1)[4]) {
#define W4X12_CORR(M)                                                                      \
  "v_mfma_scale_f32_16x16x128_f8f6f4 %[c" #M "], %[a" #M "], %[e], 0, %[s" #M "], %[t] op_sel_hi:[0,0,0]\n\t"
#define W4X12_ROW(M)                                                                      \
  "v_mfma_scale_f32_16x16x128_f8f6f4 %[x" #M "], %[a" #M "], %[b0], %[c" #M "], %[s" #M "], %[t] op_sel_hi:[0,0,0]\n\t" \
  "v_mfma_scale_f32_16x16x128_f8f6f4 %[y" #M "], %[a" #M "], %[b1], %[c" #M "], %[s" #M "], %[t] op_sel_hi:[0,0,0]\n\t"
  asm volatile(
      "s_nop 1\n\t"
      W4X12_CORR(0) W4X12_CORR(1) W4X12_CORR(2) W4X12_CORR(3)
      "s_nop 1\n\t"
      W4X12_ROW(0) W4X12_ROW(1) W4X12_ROW(2) W4X12_ROW(3)
      "s_nop 15\n\t"
      "s_nop 15"
      : [c0] "=&v"(c[0]), [c1] "=&v"(c[1]), [c2] "=&v"(c[2]), [c3] "=&v"(c[3]),
        [x0] "=&v"(d0[0]), [x1] "=&v"(d0[1]), [x2] "=&v"(d0[2]), [x3] "=&v"(d0[3]),
        [y0] "=&v"(d1[0]), [y1] "=&v"(d1[1]), [y2] "=&v"(d1[2]), [y3] "=&v"(d1[3])
      : [a0] "v"(a[0]), [a1] "v"(a[1]), [a2] "v"(a[2]), [a3] "v"(a[3]), [e] "v"(neg8),
        [b0] "v"(b0), [b1] "v"(b1), [s0] "v"(sa[0]), [s1] "v"(sa[1]), [s2] "v"(sa[2]),
        [s3] "v"(sa[3]), [t] "v"(sb));
#undef W4X12_CORR
#undef W4X12_ROW
}

// 32 INT4 codes (16 bytes of a weight row) -> the E4M3 bytes q + 8 of the
// B operand: dword 2i holds elements 8i, 8i+2, 8i+4, 8i+6, dword 2i+1 the
// odd ones 8i+1 .. 8i+7
__device__ __forceinline__ v8i int4_operand(const v4u& w) {
  const uint32_t y0 = w.x ^ 0x88888888u, y1 = w.y ^ 0x88888888u;
  const uint32_t y2 = w.z ^ 0x88888888u, y3 = w.w ^ 0x88888888u;
  return v8i{(int)(y0 & 0x0F0F0F0Fu), (int)((y0 >> 4) & 0x0F0F0F0Fu),
             (int)(y1 & 0x0F0F0F0Fu), (int)((y1 >> 4) & 0x0F0F0F0Fu),
             (int)(y2 & 0x0F0F0F0Fu), (int)((y2 >> 4) & 0x0F0F0F0Fu),
             (int)(y3 & 0x0F0F0F0Fu), (int)((y3 >> 4) & 0x0F0F0F0Fu)};
}

// 16 activation bytes (elements 0..15 in order) -> the same slot order:
// dword 2i the even elements 8i, 8i+2, 8i+4, 8i+6, dword 2i+1 the odd ones
__device__ __forceinline__ v4u act_slots16(const v4u& b) {
  return v4u{__builtin_amdgcn_perm(b.y, b.x, 0x06040200u), __builtin_amdgcn_perm(b.y, b.x, 0x07050301u),
             __builtin_amdgcn_perm(b.w, b.z, 0x06040200u), __builtin_amdgcn_perm(b.w, b.z, 0x07050301u)};
}

// 32 activation bytes (elements 0..31 in order) -> the same slot order
__device__ __forceinline__ v8i act_operand(const v4u& b0, const v4u& b1) {
  const uint32_t a[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
  v8i r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[2 * i] = (int)__builtin_amdgcn_perm(a[2 * i + 1], a[2 * i], 0x06040200u);
    r[2 * i + 1] = (int)__builtin_amdgcn_perm(a[2 * i + 1], a[2 * i], 0x07050301u);
  }
  return r;
}

constexpr int kW4ScaleB = 127 + 9;        // E8M0 2^9: undoes the 2^-9 of the INT4 bytes

}  // namespace

// LINE: K <= 4096 -- each weight row's whole scale line (at most 128 bytes)
// is loaded once, a quarter per lane group, and each group of four steps
// takes its four scales from the lane group holding them (ds_bpermute).
// Read a piece at a time over the K loop, the line was fetched again and
// again (~25% more HBM reads at decode).  Longer K loads each group's four
// scales with the group.
template <int MODE, bool LINE>
__global__ __launch_bounds__(kGemmThreads, 2) void expert_gemm_w4(ExpertGemmArgs p, int mt_max,
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

  // weight tile t: 16 rows from a wave-uniform base; two K steps of its
  // rows go out as two whole-line loads (lane (grp, col): row col % 8, then
  // row 8 + col % 8, bytes 64 * (col / 8) + 16 * grp of the line), turned
  // into the steps' operands by line_pair_to_steps
  const uint8_t* wtile[4];
  const uint32_t loff = (uint32_t)((col & 7) * wrow_bytes + 64 * (col >> 3) + 16 * grp);
  const float* sptr[4];
  int n0;
  bool wave_live = true;
  if (MODE == 1) {
    n0 = n_tile * kG1Cols;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row0 = n0 + 32 * wv + 16 * (t & 1);
      const int row = row0 + col;
      const uint8_t* base = (t < 2) ? p.w : p.w3;
      const float* sbase = reinterpret_cast<const float*>((t < 2) ? p.w_scale : p.w3_scale);
      wtile[t] = base + ((size_t)e * N + row0) * wrow_bytes;
      sptr[t] = sbase + ((size_t)e * N + row) * S;
    }
  } else {
    n0 = n_tile * kG2Rows;
    wave_live = (n0 + 64 * wv) < N;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row0 = wave_live ? (n0 + 64 * wv + 16 * t) : 0;
      const int row = row0 + col;
      wtile[t] = p.w + ((size_t)e * N + row0) * wrow_bytes;
      sptr[t] = reinterpret_cast<const float*>(p.w_scale) + ((size_t)e * N + row) * S;
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
    // register ring of four K steps (weight and activation bytes); the
    // group scales and the activation scale bytes come once per four steps
    v4u A[4][4], B[4][2];
    v4u SW[4];                 // !LINE: float32 scales of steps s0..s0+3, per tile
    v4u SL[4][2];              // LINE: scales of steps 8 grp .. 8 grp + 7, per tile
    uint32_t BSW;              // activation scale bytes of steps s0..s0+3
    const v8i neg8 = {(int)0x88888888u, (int)0x88888888u, (int)0x88888888u, (int)0x88888888u,
                      (int)0x88888888u, (int)0x88888888u, (int)0x88888888u, (int)0x88888888u};
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
        for (int t = 0; t < 4; ++t) SW[t] = *reinterpret_cast<const v4u*>(sptr[t] + s0);
      }
      BSW = *reinterpret_cast<const uint32_t*>(bsp + s0);
    };
    auto compute = [&](const v4u (&a)[4], const v4u (&sw)[4], int d, const v4u (&b)[2],
                       uint32_t bsw) {
      const int sa = (int)((bsw >> (8 * d)) & 0xFFu);
      const v8i xa = act_operand(b[0], b[1]);
      v8i wb[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) wb[t] = int4_operand(a[t]);
      v4f c, part[4];
      mfma_w4x5(xa, neg8, wb, sa, kW4ScaleB, c, part);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float s = __uint_as_float(sw[t][d]);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[t][v] = __builtin_fmaf(part[t][v], s, acc[t][v]);
      }
    };
    // one group of four steps; LOAD: refill the ring with the next group
    auto group = [&](int s0, auto load) {
      v4u sw[4];
      if constexpr (LINE) {
        const int src = (16 * (s0 >> 3) + col) * 4;   // lane group s0 / 8 holds them
        const bool hi = (s0 & 4) != 0;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int d = 0; d < 4; ++d)
            sw[t][d] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)(hi ? SL[t][1][d] : SL[t][0][d]));
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) sw[t] = SW[t];
      }
      const uint32_t bsw = BSW;
      if constexpr (decltype(load)::value) load_scales(s0 + 4);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        if ((d & 1) == 0) {
#pragma unroll
          for (int t = 0; t < 4; ++t) line_pair_to_steps(A[d][t], A[d + 1][t]);
        }
        compute(A[d], sw, d, B[d], bsw);
        // refill two steps at a time (one weight line pair)
        if constexpr (decltype(load)::value) {
          if (d & 1) load_pair(s0 + 3 + d, A[d - 1], B[d - 1], A[d], B[d]);
        }
        __builtin_amdgcn_sched_barrier(0);   // keep each refill behind its compute
      }
    };
    if constexpr (LINE) {
      // steps past the last one clamp to it (in bounds, never used)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        SL[t][0] = *reinterpret_cast<const v4u*>(sptr[t] + min(8 * grp, S - 4));
        SL[t][1] = *reinterpret_cast<const v4u*>(sptr[t] + min(8 * grp + 4, S - 4));
      }
    }
    load_scales(0);
    load_pair(0, A[0], B[0], A[1], B[1]);
    __builtin_amdgcn_sched_barrier(0);   // same issue order as in the loop
    load_pair(2, A[2], B[2], A[3], B[3]);
    __builtin_amdgcn_sched_barrier(0);
    for (int s0 = 0; s0 < S - 4; s0 += 4) group(s0, std::true_type{});
    group(S - 4, std::false_type{});
  }

  // lane holds acc[t][v] = output (token 4 * grp + v, weight row col of tile t)
  if (MODE == 1) {
    float h[2][4];
    float amax[4];
    const float lim = p.limit;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      amax[v] = 0.f;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const float g = clamp_sym(acc[tt][v], lim);
        const float u = clamp_sym(acc[tt + 2][v], lim);
        const float hv = silu_fast(g) * u;
        h[tt][v] = hv;
        amax[v] = fmaxf(amax[v], fabsf(hv));
      }
      // over the 16 weight rows of the lane group
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) amax[v] = fmaxf(amax[v], __shfl_xor(amax[v], m));
    }
    if (col == 0) {
#pragma unroll
      for (int v = 0; v < 4; ++v) red[wv][4 * grp + v] = amax[v];
    }
    __syncthreads();
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int tok = 4 * grp + v;
      if (m0 + tok >= n_e) continue;
      const float bmax = fmaxf(fmaxf(red[0][tok], red[1][tok]), fmaxf(red[2][tok], red[3][tok]));
      const int ex = pow2_scale_exp(bmax);
      const size_t row = (size_t)(off_e + m0 + tok);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        p.hq[row * N + n0 + 32 * wv + 16 * tt + col] = (uint8_t)e4m3x1(ldexpf(h[tt][v], -ex));
      if (wv == 0 && col == 0) p.hs[row * (N / 128) + n0 / 128] = (uint8_t)(ex + 127);
    }
  } else {
    if (!wave_live) return;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int tok = 4 * grp + v;
      if (m0 + tok >= n_e) continue;
      const size_t row = (size_t)(off_e + m0 + tok);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const size_t c = (size_t)n0 + 64 * wv + 16 * t + col;
        if (p.out_fp32)
          reinterpret_cast<float*>(p.out)[row * N + c] = acc[t][v];
        else
          reinterpret_cast<uint16_t*>(p.out)[row * N + c] = (uint16_t)f32_to_bf16(acc[t][v]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Larger batches: m-tiles of 64 pairs (K <= 4096)
// ---------------------------------------------------------------------------
// Eight waves of 32 weight rows (GEMM1: 16 h columns, their w1 and w3 rows;
// GEMM2: 32 output columns), the register ring of weight steps as above.
// The m-tile's 64 activation rows of a K step are staged once in LDS, already
// in the MFMA's slot order (double buffer; 16-byte chunks xor-swizzled by
// row, so that the 16 rows a wave reads at one offset hit distinct banks;
// permuting once while staging instead of in every wave's operand reads:
// -5% time) and every wave takes four 16-pair
// sub-tiles from there: each unpacked weight operand feeds four MFMAs.  The
// waves' float32 scale lines (rows padded to 33) and the 64 tokens'
// activation scales stay in LDS for the whole tile; one barrier per K step.
constexpr int kW4M = 64;
constexpr int kW4MThreads = 512;

template <int MODE>
__global__ __launch_bounds__(kW4MThreads, 2) void expert_gemm_w4_m64(ExpertGemmArgs p,
                                                                      int mt_max, int n_tiles) {
  __shared__ __attribute__((aligned(16))) uint8_t xl[2][kW4M * 128];
  __shared__ float wsl[8][32][33];
  __shared__ __attribute__((aligned(16))) uint8_t bsl[kW4M][32];
  __shared__ float red[8][kW4M];
  int n_tile, e, m0, off_e, n_e;
  if (!map_expert_tile_em(p, n_tiles, kW4M, n_tile, e, m0, off_e, n_e)) return;

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int K = p.K, N = p.N;
  const int S = K / 128;                    // a multiple of 4, at most 32
  const size_t wrow_bytes = (size_t)K / 2;

  const uint8_t* wptr[2];
  const float* srow[2];
  int n0;
  if (MODE == 1) {
    n0 = n_tile * kG1Cols;
    const int row = n0 + 16 * wv + col;       // h column: its w1 row (t 0) and w3 row (t 1)
    wptr[0] = p.w + ((size_t)e * N + row) * wrow_bytes + grp * 16;
    wptr[1] = p.w3 + ((size_t)e * N + row) * wrow_bytes + grp * 16;
    srow[0] = reinterpret_cast<const float*>(p.w_scale) + ((size_t)e * N + row) * S;
    srow[1] = reinterpret_cast<const float*>(p.w3_scale) + ((size_t)e * N + row) * S;
  } else {
    n0 = n_tile * kG2Rows;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int row = min(n0 + 32 * wv + 16 * t + col, N - 1);
      wptr[t] = p.w + ((size_t)e * N + row) * wrow_bytes + grp * 16;
      srow[t] = reinterpret_cast<const float*>(p.w_scale) + ((size_t)e * N + row) * S;
    }
  }

  // staging role: thread (sr, sq) moves the 16-byte chunk sq of token row sr
  // of each step; rows past the expert's last pair repeat that pair's row
  // (computed, dropped)
  const int sr = threadIdx.x >> 3, sq = threadIdx.x & 7;
  const int sslot = min(m0 + sr, n_e - 1);
  const int64_t stok = (MODE == 1) ? (int64_t)(p.sorted_pairs[off_e + sslot] / p.top_k)
                                   : (int64_t)(off_e + sslot);
  const uint8_t* xsrc = p.a + stok * K + 16 * sq;
  const int xc = sr * 128 + (sq ^ (sr & 7)) * 16;

  // tile-long LDS tables: the 64 tokens' activation scales and this wave's
  // weight scale lines (positions past S clamp to S - 4: same data)
  {
    const int b0 = min(4 * sq, S - 4);
    *reinterpret_cast<uint32_t*>(&bsl[sr][b0]) =
        *reinterpret_cast<const uint32_t*>(p.a_scale + stok * S + b0);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int f0 = min(8 * grp, S - 4), f1 = min(8 * grp + 4, S - 4);
      const v4u a0 = *reinterpret_cast<const v4u*>(srow[t] + f0);
      const v4u a1 = *reinterpret_cast<const v4u*>(srow[t] + f1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wsl[wv][16 * t + col][f0 + j] = __uint_as_float(a0[j]);
        wsl[wv][16 * t + col][f1 + j] = __uint_as_float(a1[j]);
      }
    }
  }

  v4f acc[2][4];   // [weight tile][16-pair sub-tile]
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[t][m] = v4f{0.f, 0.f, 0.f, 0.f};

  const v8i neg8 = {(int)0x88888888u, (int)0x88888888u, (int)0x88888888u, (int)0x88888888u,
                    (int)0x88888888u, (int)0x88888888u, (int)0x88888888u, (int)0x88888888u};
  v4u A[4][2];     // weight ring: [step][tile]
  v4u R;           // the chunk of the next step to stage
  auto load_w = [&](int s, v4u (&a)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) a[t] = *reinterpret_cast<const v4u*>(wptr[t] + (size_t)s * 64);
  };
  auto load_x = [&](int s) { R = *reinterpret_cast<const v4u*>(xsrc + (size_t)s * 128); };
  auto store_x = [&](int buf) { *reinterpret_cast<v4u*>(&xl[buf][xc]) = act_slots16(R); };

  // one K step from the weight ring slot a and LDS buffer buf
  auto compute = [&](int s, const v4u (&a)[2], int buf) {
    const v8i b0 = int4_operand(a[0]), b1 = int4_operand(a[1]);
    const float sw0 = wsl[wv][col][s], sw1 = wsl[wv][16 + col][s];
    v8i xa[4];
    int sa[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint8_t* xr = &xl[buf][(16 * m + col) * 128];
      const v4u lo = *reinterpret_cast<const v4u*>(xr + ((2 * grp) ^ (col & 7)) * 16);
      const v4u hi = *reinterpret_cast<const v4u*>(xr + ((2 * grp + 1) ^ (col & 7)) * 16);
      xa[m] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                  (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      sa[m] = bsl[16 * m + col][s];
    }
    v4f c[4], d0[4], d1[4];
    mfma_w4x12(xa, neg8, b0, b1, sa, kW4ScaleB, c, d0, d1);
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        acc[0][m][v] = __builtin_fmaf(d0[m][v], sw0, acc[0][m][v]);
        acc[1][m][v] = __builtin_fmaf(d1[m][v], sw1, acc[1][m][v]);
      }
  };
  // one group of four steps; LOAD: refill the weight ring with the next group
  // (two steps at a time: both halves of each 128-byte line back to back)
  auto group = [&](int s0, auto load) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int s = s0 + d;
      compute(s, A[d], s & 1);
      store_x((s + 1) & 1);                 // step s + 1 (the last step's copy is unused)
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

  load_x(0);
  store_x(0);
  load_x(min(1, S - 1));
#pragma unroll
  for (int d = 0; d < 4; ++d) load_w(d, A[d]);
  __syncthreads();
  for (int s0 = 0; s0 < S - 4; s0 += 4) group(s0, std::true_type{});
  group(S - 4, std::false_type{});

  // lane holds acc[t][m][v] = output (token 16 m + 4 grp + v, weight row col
  // of tile t)
  if (MODE == 1) {
    const float lim = p.limit;
    float h[4][4];
    float amax[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float g = clamp_sym(acc[0][m][v], lim);
        const float u = clamp_sym(acc[1][m][v], lim);
        h[m][v] = silu_fast(g) * u;
        float a = fabsf(h[m][v]);
#pragma unroll
        for (int k = 1; k < 16; k <<= 1) a = fmaxf(a, __shfl_xor(a, k));
        amax[m][v] = a;
      }
    if (col == 0) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[wv][16 * m + 4 * grp + v] = amax[m][v];
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int tok = 16 * m + 4 * grp + v;
        if (m0 + tok >= n_e) continue;
        float bmax = red[0][tok];
#pragma unroll
        for (int w = 1; w < 8; ++w) bmax = fmaxf(bmax, red[w][tok]);
        const int ex = pow2_scale_exp(bmax);
        const size_t row = (size_t)(off_e + m0 + tok);
        p.hq[row * N + n0 + 16 * wv + col] = (uint8_t)e4m3x1(ldexpf(h[m][v], -ex));
        if (wv == 0 && col == 0) p.hs[row * (N / 128) + n0 / 128] = (uint8_t)(ex + 127);
      }
  } else {
    if (n0 + 32 * wv >= N) return;
    // the output addresses are formed only now (an opaque copy of the row
    // base keeps the compiler from computing them before the K loop and
    // holding them through it)
    int rbase = off_e + m0;
    asm volatile("" : "+s"(rbase));
    const size_t c0 = (size_t)n0 + 32 * wv + col;   // + 16 t
    if (p.out_fp32) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int tok = 16 * m + 4 * grp + v;
          if (m0 + tok >= n_e) continue;
          float* o = reinterpret_cast<float*>(p.out) + (size_t)(rbase + tok) * N + c0;
          o[0] = acc[0][m][v];
          o[16] = acc[1][m][v];
        }
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int tok = 16 * m + 4 * grp + v;
          if (m0 + tok >= n_e) continue;
          uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + (size_t)(rbase + tok) * N + c0;
          o[0] = (uint16_t)f32_to_bf16(acc[0][m][v]);
          o[16] = (uint16_t)f32_to_bf16(acc[1][m][v]);
        }
    }
  }
}

static unsigned pad8_w4(int64_t g) { return (unsigned)((g + 7) / 8 * 8); }

template <int MODE>
static hipError_t launch_w4(const ExpertGemmArgs& a, int bm, int mt_max, hipStream_t st) {
  if (a.K % 512) return hipErrorInvalidValue;
  const int n_tiles = MODE == 1 ? a.N / kG1Cols : (a.N + kG2Rows - 1) / kG2Rows;
  const unsigned grid = pad8_w4((int64_t)n_tiles * mt_max);
  if (grid == 0) return hipSuccess;
  if (bm == kW4M) {
    if (a.K > 4096) return hipErrorInvalidValue;
    hipLaunchKernelGGL((expert_gemm_w4_m64<MODE>), dim3(grid), dim3(kW4MThreads), 0, st, a,
                       mt_max, n_tiles);
  } else if (bm != 16) {
    return hipErrorInvalidValue;
  } else if (a.K <= 4096)
    hipLaunchKernelGGL((expert_gemm_w4<MODE, true>), dim3(grid), dim3(kGemmThreads), 0, st, a,
                       mt_max, n_tiles);
  else
    hipLaunchKernelGGL((expert_gemm_w4<MODE, false>), dim3(grid), dim3(kGemmThreads), 0, st, a,
                       mt_max, n_tiles);
  return hipGetLastError();
}

hipError_t launch_expert_gemm1_w4(const ExpertGemmArgs& a, int bm, int mt_max, hipStream_t st) {
  return launch_w4<1>(a, bm, mt_max, st);
}
hipError_t launch_expert_gemm2_w4(const ExpertGemmArgs& a, int bm, int mt_max, hipStream_t st) {
  return launch_w4<2>(a, bm, mt_max, st);
}

}  // namespace moe
