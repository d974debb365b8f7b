// Grouped expert GEMMs on gfx950 block-scaled MFMA.
//
// What is computed ("DeepSeek-V4-Flash-SI" card, 架构特性: SwiGLU clamped to
// +-10; 低精度计算: FP4 E2M1 weights with an E8M0 scale per 32, FP8 E4M3
// activations with a power-of-two scale per 128):
//   GEMM1 (per expert e, for its pairs in sorted order)
//     g = deq(xq[tok]) . deq(w1[e])^T,  u = deq(xq[tok]) . deq(w3[e])^T
//     h = silu(clip(g)) * clip(u)  -> FP8 E4M3 + E8M0 per 128 of I  (hq, hs)
//   GEMM2
//     o = deq(hq) . deq(w2[e])^T   -> fp32 or bf16 rows in sorted order
//
// Instruction: v_mfma_scale_f32_16x16x128_f8f6f4 with A = FP4 weights
// (cbsz = 4) and B = FP8 activations (blgp = 0). Operand layout (measured on
// gfx950 with one-hot operands):
//   A: lane l holds row l%16, K elements 32*(l/16) .. +31 in 16 bytes, the
//      even element in the low nibble -- exactly 16 consecutive bytes of a
//      checkpoint row [N, K/2], and its E8M0 scale is the row's per-32 scale
//      of that K block;
//   B: lane l holds column l%16, K elements 16*(l/16) .. +15 in bytes 0-15
//      and 64 + 16*(l/16) .. +15 in bytes 16-31; its scale covers K block
//      l/16 -- for per-128 activation scales all four lane groups carry the
//      same byte;
//   D: lane l holds D[4*(l/16) + v][l%16], v = 0..3.
// So one K step is 128 elements: 64 weight bytes and 128 activation bytes
// per row, and the FP8 activation block scale lines up with the step.
//
// Scale operands: a streaming kernel built on the compiler builtin, whose
// scale registers the compiler reused right after the MFMA, gave rows 1-15 of
// the 16x16 tile a wrong scale (row 0 right).  Isolated probes that
// overwrite an A, B or scale register with the very next VALU instruction
// show no effect, so the exact condition is not pinned down; the kernels
// therefore issue the instruction from inline assembly and keep its scale
// registers and accumulators untouched for 32 wait states after it
// (mfma_fp4_fp8 below, and once per K step in the tile kernel).  Before it,
// the asm leaves the 2 wait states the compiler puts between a VALU write of
// a source register and the MFMA, which it cannot do in front of an asm.
//
// Work decomposition: a workgroup (4 waves) owns one m-tile of one expert
// (16 * MT pairs) and one n-tile of weight rows; it streams its weight rows
// once over the whole K with 16-byte loads straight into the MFMA operand
// registers (each weight byte is used by exactly one lane). Activation rows
// are gathered per token; with MT > 1 they are staged once per K step in LDS
// and shared by the four waves. m-tiles are enumerated through a device-side
// prefix over experts (mtile_off), so expert counts never travel to the host.
// Workgroup ids are remapped so that the tiles of one weight n-tile that land
// on the same XCD (ids are dealt round-robin over the 8 XCDs) are processed
// together there, and share that XCD's L2.  The 128-pair tile kernel
// (prefill) is persistent instead: one workgroup per CU walks a share of the
// tiles in the same XCD-local, expert-major order.
#include "moe_internal.h"

#include <algorithm>
#include <atomic>
#include <type_traits>

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));

// acc += (A * 2^(sa-127)) x (B * 2^(sb-127)) per 32-element K block; A is 32
// FP4 values per lane (cbsz 4), B 32 FP8 values per lane (blgp 0), scale
// bytes in bits 0-7 of sa / sb (op_sel 0).  Issued from inline assembly so
// that the 32 wait states after it are guaranteed: no instruction of this
// wave can overwrite a scale (or data) register the instruction may still be
// reading, and its result is final before any later VALU read.
__device__ __forceinline__ v4f mfma_fp4_fp8(const uint4& a, const uint4& b0, const uint4& b1,
                                            v4f acc, int sa, int sb) {
  v4i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w};
  v8i bv = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
            (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
  asm volatile(
      "s_nop 1\n\t"
      "v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0] cbsz:4\n\t"
      "s_nop 15\n\t"
      "s_nop 15"
      : "+v"(acc)
      : "v"(av), "v"(bv), "v"(sa), "v"(sb));
  return acc;
}

// FP8 weights (E4M3, cbsz 0): A is 32 bytes per lane laid out like the FP8
// activation operand (bytes 0-15: K = 16*(l/16) + j, bytes 16-31:
// K = 64 + 16*(l/16) + j); one scale per 128 for all four lane groups.
__device__ __forceinline__ v4f mfma_fp8_fp8(const uint4& a0, const uint4& a1, const uint4& b0,
                                            const uint4& b1, v4f acc, int sa, int sb) {
  v8i av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
  v8i bv = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
            (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
  asm volatile(
      "s_nop 1\n\t"
      "v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]\n\t"
      "s_nop 15\n\t"
      "s_nop 15"
      : "+v"(acc)
      : "v"(av), "v"(bv), "v"(sa), "v"(sb));
  return acc;
}

// The MT MFMAs of one weight tile in a K step of the generic kernel (FP4
// weights: A = 16 bytes, cbsz 4; FP8 weights: A = 32 bytes, cbsz 0), from one
// asm statement; the last of a step (the _g variants) closes it with 32 wait
// states and takes every scale register of the step (k0..k3: the weight
// tiles') as an input, so that none is reused before them.  (Plain device
// functions: templates called from the kernel's lambdas fail overload
// resolution in the host compilation pass.)
#define GEN_MFMA(M, CB)                                                                         \
  "v_mfma_scale_f32_16x16x128_f8f6f4 %[c" #M "], %[a], %[b" #M "], %[c" #M "], %[sa], %[s" #M \
  "] op_sel_hi:[0,0,0]" CB "\n\t"
#define GEN_GUARD "s_nop 15\n\ts_nop 15"
#define GEN_KA [k0] "v"(ka[0]), [k1] "v"(ka[1]), [k2] "v"(ka[2]), [k3] "v"(ka[3])
#define GEN_DEF1(NAME, AT, CB, G)                                                              \
  __device__ __forceinline__ void NAME(v4f* acc, const AT& av, const v8i* bv, uint32_t sa,    \
                                       const uint32_t* sb, const uint32_t* ka) {              \
    asm volatile("s_nop 1\n\t" GEN_MFMA(0, CB) G                                             \
                 : [c0] "+v"(acc[0])                                                          \
                 : [a] "v"(av), [b0] "v"(bv[0]), [sa] "v"(sa), [s0] "v"(sb[0]), GEN_KA);      \
  }
#define GEN_DEF4(NAME, AT, CB, G)                                                              \
  __device__ __forceinline__ void NAME(v4f* acc, const AT& av, const v8i* bv, uint32_t sa,    \
                                       const uint32_t* sb, const uint32_t* ka) {              \
    asm volatile("s_nop 1\n\t" GEN_MFMA(0, CB) GEN_MFMA(1, CB) GEN_MFMA(2, CB) GEN_MFMA(3, CB) G \
                 : [c0] "+v"(acc[0]), [c1] "+v"(acc[1]), [c2] "+v"(acc[2]), [c3] "+v"(acc[3])  \
                 : [a] "v"(av), [b0] "v"(bv[0]), [b1] "v"(bv[1]), [b2] "v"(bv[2]),             \
                   [b3] "v"(bv[3]), [sa] "v"(sa), [s0] "v"(sb[0]), [s1] "v"(sb[1]),            \
                   [s2] "v"(sb[2]), [s3] "v"(sb[3]), GEN_KA);                                 \
  }
GEN_DEF1(gen_fp4_1, v4i, " cbsz:4", "")
GEN_DEF1(gen_fp4_1_g, v4i, " cbsz:4", GEN_GUARD)
GEN_DEF1(gen_fp8_1, v8i, "", "")
GEN_DEF1(gen_fp8_1_g, v8i, "", GEN_GUARD)
GEN_DEF4(gen_fp4_4, v4i, " cbsz:4", "")
GEN_DEF4(gen_fp4_4_g, v4i, " cbsz:4", GEN_GUARD)
GEN_DEF4(gen_fp8_4, v8i, "", "")
GEN_DEF4(gen_fp8_4_g, v8i, "", GEN_GUARD)
#undef GEN_DEF1
#undef GEN_DEF4
#undef GEN_MFMA
#undef GEN_GUARD
#undef GEN_KA

template <int MODE, int MT, bool FP8W = false>
__global__ __launch_bounds__(kGemmThreads) void expert_gemm_kernel(ExpertGemmArgs p, int mt_max,
                                                                    int n_tiles) {
  constexpr int BM = 16 * MT;
  constexpr int LDS_ROW = 144;  // 128 activation bytes + 16 pad (bank spread)
  constexpr bool STAGED = MT > 1;
  __shared__ __attribute__((aligned(16))) uint8_t bsm[STAGED ? 2 : 1][STAGED ? BM : 1][LDS_ROW];
  __shared__ float red[4][BM];

  int n_tile, e, m0, off_e, n_e;
  if (!map_expert_tile(p, mt_max, n_tiles, BM, n_tile, e, m0, off_e, n_e)) return;

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int col = lane & 15;   // token slot within a 16-column sub-tile
  const int grp = lane >> 4;   // K group
  const int K = p.K, N = p.N;
  const int S = K / 128;
  // FP4: K/2 bytes per row and a scale per 32 (this lane's K block: + grp);
  // FP8: K bytes per row and one scale per 128 (per K step)
  const size_t wrow_bytes = FP8W ? (size_t)K : (size_t)K / 2;
  const size_t srow_bytes = FP8W ? (size_t)K / 128 : (size_t)K / 32;
  const int sgrp = FP8W ? 0 : grp;

  // ---- weight rows of this wave (4 MFMA row tiles) ----
  const uint8_t* wptr[4];
  const uint8_t* sptr[4];
  bool wave_live = true;
  int n0;
  if (MODE == 1) {
    n0 = n_tile * kG1Cols;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row = n0 + 32 * wv + 16 * (t & 1) + col;
      const uint8_t* base = (t < 2) ? p.w : p.w3;
      const uint8_t* sbase = (t < 2) ? p.w_scale : p.w3_scale;
      wptr[t] = base + ((size_t)e * N + row) * wrow_bytes + grp * 16;
      sptr[t] = sbase + ((size_t)e * N + row) * srow_bytes + sgrp;
    }
  } else {
    n0 = n_tile * kG2Rows;
    wave_live = (n0 + 64 * wv) < N;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row = wave_live ? (n0 + 64 * wv + 16 * t + col) : 0;
      wptr[t] = p.w + ((size_t)e * N + row) * wrow_bytes + grp * 16;
      sptr[t] = p.w_scale + ((size_t)e * N + row) * srow_bytes + sgrp;
    }
  }

  // ---- activation rows (this lane's token column in each sub-tile); slots
  // past the expert's last pair read that last pair's row, results dropped
  auto act_row = [&](int slot) -> int64_t {
    slot = min(slot, n_e - 1);
    return (MODE == 1) ? (int64_t)(p.sorted_pairs[off_e + slot] / p.top_k) : (int64_t)(off_e + slot);
  };
  const uint8_t* bptr[MT];
  const uint8_t* bsp[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int64_t row = act_row(m0 + 16 * m + col);
    bptr[m] = p.a + row * K + 16 * grp;
    bsp[m] = p.a_scale + row * (K / 128);
  }
  // LDS staging (MT > 1): thread i copies 16 bytes of token row i/8 (+32)
  constexpr int ST_ROUNDS = STAGED ? (BM * 8) / kGemmThreads : 1;
  const uint8_t* st_src[ST_ROUNDS];
  const int st_chunk = threadIdx.x & 7;
#pragma unroll
  for (int r = 0; r < ST_ROUNDS; ++r)
    st_src[r] = p.a + act_row(m0 + (threadIdx.x >> 3) + 32 * r) * K + 16 * st_chunk;

  v4f acc[4][MT];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[t][m] = v4f{0.f, 0.f, 0.f, 0.f};

  // Two-stage register ring, unrolled so that no register is ever copied:
  // stage X holds one K step's weight bytes, scale bytes and (unstaged)
  // activation bytes, all written by loads only.
  struct Stage {
    uint4 a[4][FP8W ? 2 : 1];
    uint32_t sa[4];
    uint4 b[MT][2];
    uint32_t sb[MT];
    uint4 st[ST_ROUNDS];
  };
  Stage X0, X1;
  auto load = [&](int s, Stage& x) {
    if (wave_live) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if constexpr (FP8W) {
          x.a[t][0] = *reinterpret_cast<const uint4*>(wptr[t] + (size_t)s * 128);
          x.a[t][1] = *reinterpret_cast<const uint4*>(wptr[t] + (size_t)s * 128 + 64);
          x.sa[t] = sptr[t][s];
        } else {
          x.a[t][0] = *reinterpret_cast<const uint4*>(wptr[t] + (size_t)s * 64);
          x.sa[t] = sptr[t][(size_t)s * 4];
        }
      }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      x.sb[m] = bsp[m][s];
      if constexpr (!STAGED) {
        x.b[m][0] = *reinterpret_cast<const uint4*>(bptr[m] + (size_t)s * 128);
        x.b[m][1] = *reinterpret_cast<const uint4*>(bptr[m] + (size_t)s * 128 + 64);
      }
    }
    if constexpr (STAGED) {
#pragma unroll
      for (int r = 0; r < ST_ROUNDS; ++r)
        x.st[r] = *reinterpret_cast<const uint4*>(st_src[r] + (size_t)s * 128);
    }
  };
  auto stage_store = [&](int buf, const Stage& x) {
#pragma unroll
    for (int r = 0; r < ST_ROUNDS; ++r)
      *reinterpret_cast<uint4*>(&bsm[buf][(threadIdx.x >> 3) + 32 * r][16 * st_chunk]) = x.st[r];
  };
  auto compute = [&](int buf, Stage& x) {
    if constexpr (STAGED) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        x.b[m][0] = *reinterpret_cast<const uint4*>(&bsm[buf][16 * m + col][16 * grp]);
        x.b[m][1] = *reinterpret_cast<const uint4*>(&bsm[buf][16 * m + col][64 + 16 * grp]);
      }
    }
    if (wave_live) {
      // one asm statement per weight tile, one 32-wait-state guard per step
      // (the last statement, which holds every scale register of the step)
      typedef typename std::conditional<FP8W, v8i, v4i>::type AV;
      v8i bv[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m)
        bv[m] = v8i{(int)x.b[m][0].x, (int)x.b[m][0].y, (int)x.b[m][0].z, (int)x.b[m][0].w,
                    (int)x.b[m][1].x, (int)x.b[m][1].y, (int)x.b[m][1].z, (int)x.b[m][1].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        AV av;
        if constexpr (FP8W)
          av = AV{(int)x.a[t][0].x, (int)x.a[t][0].y, (int)x.a[t][0].z, (int)x.a[t][0].w,
                  (int)x.a[t][FP8W ? 1 : 0].x, (int)x.a[t][FP8W ? 1 : 0].y,
                  (int)x.a[t][FP8W ? 1 : 0].z, (int)x.a[t][FP8W ? 1 : 0].w};
        else
          av = AV{(int)x.a[t][0].x, (int)x.a[t][0].y, (int)x.a[t][0].z, (int)x.a[t][0].w};
        if constexpr (FP8W && MT == 1) (t == 3 ? gen_fp8_1_g : gen_fp8_1)(acc[t], av, bv, x.sa[t], x.sb, x.sa);
        else if constexpr (FP8W) (t == 3 ? gen_fp8_4_g : gen_fp8_4)(acc[t], av, bv, x.sa[t], x.sb, x.sa);
        else if constexpr (MT == 1) (t == 3 ? gen_fp4_1_g : gen_fp4_1)(acc[t], av, bv, x.sa[t], x.sb, x.sa);
        else (t == 3 ? gen_fp4_4_g : gen_fp4_4)(acc[t], av, bv, x.sa[t], x.sb, x.sa);
      }
    }
  };
  // one K step: compute from x (its activations in LDS buffer `buf` when
  // staged), then refill x with step s + 2 (clamped to the last step, whose
  // reload is harmless) and stage step s + 1 for the next round
  auto step = [&](int s, int buf, Stage& x, Stage& other) {
    compute(buf, x);
    if constexpr (STAGED) {
      if (s + 1 < S) stage_store(buf ^ 1, other);
      __syncthreads();
    }
    load(min(s + 2, S - 1), x);
  };

  load(0, X0);
  load(min(1, S - 1), X1);
  if constexpr (STAGED) {
    stage_store(0, X0);
    __syncthreads();
  }
  for (int s = 0; s < S; s += 2) {
    step(s, 0, X0, X1);
    if (s + 1 < S) step(s + 1, 1, X1, X0);
  }

  if (MODE == 1) {
    // ---- clamped SwiGLU, per-128 FP8 requant of h over this tile's 128 columns ----
    float h[MT][2][4];
    const float lim = p.limit;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float amax = 0.f;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float g = clamp_sym(acc[tt][m][v], lim);
          const float u = clamp_sym(acc[tt + 2][m][v], lim);
          const float hv = silu_fast(g) * u;
          h[m][tt][v] = hv;
          amax = fmaxf(amax, fabsf(hv));
        }
      amax = fmaxf(amax, __shfl_xor(amax, 16));
      amax = fmaxf(amax, __shfl_xor(amax, 32));
      if (lane < 16) red[wv][16 * m + lane] = amax;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int tokc = 16 * m + col;
      const float amax = fmaxf(fmaxf(red[0][tokc], red[1][tokc]), fmaxf(red[2][tokc], red[3][tokc]));
      const int ex = pow2_scale_exp(amax);
      const int slot = m0 + tokc;
      if (slot < n_e) {
        const size_t row = (size_t)(off_e + slot);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const uint32_t word = e4m3x4_exp(h[m][tt], ex);
          *reinterpret_cast<uint32_t*>(p.hq + row * N + n0 + 32 * wv + 16 * tt + 4 * grp) = word;
        }
        if (wv == 0 && grp == 0) p.hs[row * (N / 128) + n0 / 128] = (uint8_t)(ex + 127);
      }
    }
  } else {
    if (!wave_live) return;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int slot = m0 + 16 * m + col;
      if (slot >= n_e) continue;
      const size_t row = (size_t)(off_e + slot);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const size_t c = (size_t)n0 + 64 * wv + 16 * t + 4 * grp;
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

// ---------------------------------------------------------------------------
// Streaming variant for m-tiles of at most 16 pairs (decode) when K is
// 1024, 2048 or 4096: every wave keeps four K steps of weight and
// activation loads in flight in a register ring (no register copies, no
// branches around the loads, so the waits before each step's MFMAs cover
// only that step), and reads each weight row's scales once.  Weights go
// out as whole 128-byte lines (two K steps of 8 rows per load, non-
// temporal) and two cross-lane moves per register pair turn a tile's two
// line loads into its two steps' MFMA operands (line_pair_to_steps).  Lanes
// whose pair slot lies past the expert's last pair read that last pair's
// row: their columns are computed and dropped.
// ---------------------------------------------------------------------------
template <int MODE, int S>
__global__ __launch_bounds__(kGemmThreads) void expert_gemm_stream(ExpertGemmArgs p, int mt_max,
                                                                    int n_tiles) {
  __shared__ float red[4][16];
  int n_tile, e, m0, off_e, n_e;
  if (!map_expert_tile(p, mt_max, n_tiles, 16, n_tile, e, m0, off_e, n_e)) return;

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;
  const int grp = lane >> 4;
  constexpr int K = S * 128;                // S in {8, 16, 32}
  const int N = p.N;
  constexpr int SD = S / 4;                 // scale dwords per lane group
  const size_t wrow_bytes = (size_t)K / 2;
  const size_t srow_bytes = (size_t)K / 32;

  // Tile t of the wave is 16 weight rows from row0; its MFMA operand lane
  // (grp, col) is row row0 + col.  The line loads: lane (grp, col) reads row
  // row0 + col % 8 (first load) or row0 + 8 + col % 8 (second), bytes
  // 64 * (col / 8) + 16 * grp of the line, so each load covers 8 whole lines.
  const uint8_t* wtile[4];  // wave-uniform: row row0 of tile t
  const uint8_t* sptr[4];
  int n0;
  bool wave_live = true;
  // lane offset of the first line load (the second is 8 rows further)
  const uint32_t loff = (uint32_t)((col & 7) * wrow_bytes + 64 * (col >> 3) + 16 * grp);
  if (MODE == 1) {
    n0 = n_tile * kG1Cols;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row0 = n0 + 32 * wv + 16 * (t & 1);
      const uint8_t* base = (t < 2) ? p.w : p.w3;
      const uint8_t* sbase = (t < 2) ? p.w_scale : p.w3_scale;
      wtile[t] = base + ((size_t)e * N + row0) * wrow_bytes;
      sptr[t] = sbase + ((size_t)e * N + row0 + col) * srow_bytes;
    }
  } else {
    n0 = n_tile * kG2Rows;
    wave_live = (n0 + 64 * wv) < N;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row0 = wave_live ? (n0 + 64 * wv + 16 * t) : 0;
      wtile[t] = p.w + ((size_t)e * N + row0) * wrow_bytes;
      sptr[t] = p.w_scale + ((size_t)e * N + row0 + col) * srow_bytes;
    }
  }
  const int slot = min(m0 + col, n_e - 1);
  const int64_t brow = (MODE == 1) ? (int64_t)(p.sorted_pairs[off_e + slot] / p.top_k)
                                   : (int64_t)(off_e + slot);
  const uint8_t* bptr = p.a + brow * K + 16 * grp;
  const uint8_t* bsp = p.a_scale + brow * (K / 128);

  v4f acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};

  if (wave_live) {
    // Ring of four K steps of weight and activation bytes.  Weight scales:
    // the four lane groups of a row load the row's whole scale line once (K/32
    // bytes, a quarter each, back to back), and each step takes its byte from
    // the lane group holding it with a cross-lane permute.  Activation
    // scales: one 4-byte load per four steps (4 per-128 scales of the token).
    uint4 A[4][4], B[4][2];
    uint32_t SR[4][SD];
    uint32_t SB0, SB1;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint8_t* src = sptr[t] + grp * S;
      if constexpr (SD >= 4) {
#pragma unroll
        for (int j = 0; j < SD / 4; ++j) {
          const uint4 v = *reinterpret_cast<const uint4*>(src + 16 * j);
          SR[t][4 * j] = v.x; SR[t][4 * j + 1] = v.y; SR[t][4 * j + 2] = v.z; SR[t][4 * j + 3] = v.w;
        }
      } else {
        const uint2 v = *reinterpret_cast<const uint2*>(src);
        SR[t][0] = v.x; SR[t][1] = v.y;
      }
    }
    // steps s and s + 1 (s even) together: the 128-byte line of the two
    // steps of tile t's rows 0-7 into a0[t], of rows 8-15 into a1[t]
    // (line_pair_to_steps makes them step s's and step s + 1's operands)
    const size_t w8 = 8 * wrow_bytes;
    auto load_pair = [&](int s, uint4 (&a0)[4], uint4 (&b0)[2], uint4 (&a1)[4], uint4 (&b1)[2]) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        a0[t] = wload16(wtile[t] + loff + s * 64);
        a1[t] = wload16(wtile[t] + w8 + loff + s * 64);
      }
      b0[0] = *reinterpret_cast<const uint4*>(bptr + (size_t)s * 128);
      b0[1] = *reinterpret_cast<const uint4*>(bptr + (size_t)s * 128 + 64);
      b1[0] = *reinterpret_cast<const uint4*>(bptr + (size_t)s * 128 + 128);
      b1[1] = *reinterpret_cast<const uint4*>(bptr + (size_t)s * 128 + 192);
    };
    auto load_sb = [&](int q) { return *reinterpret_cast<const uint32_t*>(bsp + (size_t)q * 4); };
    // four K steps s = 4q + d (q of parity PAR); with LOADS also the next
    // group's activation scales and a refill of each pair of ring slots right
    // after their use.  The loads of a step pair are issued as a group, in
    // step order, in the prologue and here (scheduling barriers keep the
    // compiler from regrouping them), so the wait before a step's MFMAs
    // leaves the later steps in flight.
    auto four_steps = [&](auto loads, auto par, int q, uint32_t sbc, uint32_t& sbn) {
      constexpr bool LOADS = decltype(loads)::value;
      constexpr int PAR = decltype(par)::value;
      if constexpr (LOADS) sbn = load_sb(q + 1);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        if ((d & 1) == 0) {
#pragma unroll
          for (int t = 0; t < 4; ++t) line_pair_to_steps(A[d][t], A[d + 1][t]);
        }
        // byte 4s + grp of the row's scales sits in lane group (4s)/S,
        // dword s % SD, byte grp
        const int s = 4 * q + d;
        const int src_lane = col + 16 * (s / SD);
        const int dw = (4 * PAR + d) % SD;
        const int sb = (int)(sbc >> (8 * d));          // the MFMA reads bits 0-7
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int w = __shfl((int)SR[t][dw], src_lane);
          acc[t] = mfma_fp4_fp8(A[d][t], B[d][0], B[d][1], acc[t], w >> (8 * grp), sb);
        }
        if constexpr (LOADS) {
          if (d & 1) {
            __builtin_amdgcn_sched_barrier(0);
            load_pair(4 * q + d + 3, A[d - 1], B[d - 1], A[d], B[d]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    };
    using yes = std::integral_constant<bool, true>;
    using no = std::integral_constant<bool, false>;
    using even = std::integral_constant<int, 0>;
    using odd = std::integral_constant<int, 1>;
    SB0 = load_sb(0);
    load_pair(0, A[0], B[0], A[1], B[1]);
    __builtin_amdgcn_sched_barrier(0);
    load_pair(2, A[2], B[2], A[3], B[3]);
    __builtin_amdgcn_sched_barrier(0);
    constexpr int Q = S / 4;  // even, >= 2
    for (int q = 0; q < Q - 2; q += 2) {
      four_steps(yes{}, even{}, q, SB0, SB1);
      four_steps(yes{}, odd{}, q + 1, SB1, SB0);
    }
    four_steps(yes{}, even{}, Q - 2, SB0, SB1);
    four_steps(no{}, odd{}, Q - 1, SB1, SB0);
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
// Streaming variant for FP8 expert weights (E4M3 rows of K bytes, one E8M0
// scale per 128) and m-tiles of at most 16 pairs: each K step reads whole
// 128-byte weight lines (both operand halves back to back); four steps of
// weight and activation loads stay in flight in a register ring; the weight
// and activation scales of four steps arrive as one dword per row / token.
// ---------------------------------------------------------------------------
template <int MODE, int S>
__global__ __launch_bounds__(kGemmThreads) void expert_gemm_stream8(ExpertGemmArgs p, int mt_max,
                                                                     int n_tiles) {
  __shared__ float red[4][16];
  int n_tile, e, m0, off_e, n_e;
  if (!map_expert_tile(p, mt_max, n_tiles, 16, n_tile, e, m0, off_e, n_e)) return;

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  constexpr int K = S * 128;                // S in {8, 16, 32}
  const int N = p.N;

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
      wptr[t] = base + ((size_t)e * N + row) * K + grp * 16;
      sptr[t] = sbase + ((size_t)e * N + row) * S;
    }
  } else {
    n0 = n_tile * kG2Rows;
    wave_live = (n0 + 64 * wv) < N;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row = wave_live ? (n0 + 64 * wv + 16 * t + col) : 0;
      wptr[t] = p.w + ((size_t)e * N + row) * K + grp * 16;
      sptr[t] = p.w_scale + ((size_t)e * N + row) * S;
    }
  }
  const int slot = min(m0 + col, n_e - 1);
  const int64_t brow = (MODE == 1) ? (int64_t)(p.sorted_pairs[off_e + slot] / p.top_k)
                                   : (int64_t)(off_e + slot);
  const uint8_t* bptr = p.a + brow * K + 16 * grp;
  const uint8_t* bsp = p.a_scale + brow * S;

  v4f acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};

  if (wave_live) {
    uint4 A[4][4][2], B[4][2];
    uint32_t SW0[4], SW1[4], SB0, SB1;
    auto load_step = [&](int s, uint4 (&a)[4][2], uint4 (&b)[2]) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        a[t][0] = *reinterpret_cast<const uint4*>(wptr[t] + (size_t)s * 128);
        a[t][1] = *reinterpret_cast<const uint4*>(wptr[t] + (size_t)s * 128 + 64);
      }
      b[0] = *reinterpret_cast<const uint4*>(bptr + (size_t)s * 128);
      b[1] = *reinterpret_cast<const uint4*>(bptr + (size_t)s * 128 + 64);
    };
    // scales of steps 4q .. 4q+3: byte d of a dword per weight row / token
    auto load_sc = [&](int q, uint32_t (&sw)[4], uint32_t& sb) {
#pragma unroll
      for (int t = 0; t < 4; ++t) sw[t] = *reinterpret_cast<const uint32_t*>(sptr[t] + 4 * q);
      sb = *reinterpret_cast<const uint32_t*>(bsp + 4 * q);
    };
    auto four_steps = [&](auto loads, int q, const uint32_t (&swc)[4], uint32_t sbc,
                          uint32_t (&swn)[4], uint32_t& sbn) {
      constexpr bool LOADS = decltype(loads)::value;
      if constexpr (LOADS) load_sc(q + 1, swn, sbn);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int sb = (int)(sbc >> (8 * d));
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[t] = mfma_fp8_fp8(A[d][t][0], A[d][t][1], B[d][0], B[d][1], acc[t],
                                (int)(swc[t] >> (8 * d)), sb);
        if constexpr (LOADS) {
          __builtin_amdgcn_sched_barrier(0);
          load_step(4 * q + d + 4, A[d], B[d]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    using yes = std::integral_constant<bool, true>;
    using no = std::integral_constant<bool, false>;
    load_sc(0, SW0, SB0);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      load_step(d, A[d], B[d]);
      __builtin_amdgcn_sched_barrier(0);
    }
    constexpr int Q = S / 4;  // even, >= 2
    for (int q = 0; q < Q - 2; q += 2) {
      four_steps(yes{}, q, SW0, SB0, SW1, SB1);
      four_steps(yes{}, q + 1, SW1, SB1, SW0, SB0);
    }
    four_steps(yes{}, Q - 2, SW0, SB0, SW1, SB1);
    four_steps(no{}, Q - 1, SW1, SB1, SW0, SB0);
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
// Tile variant for m-tiles of 128 pairs (prefill) when K is 1024, 2048 or
// 4096: a tile is 128 pairs x 256 weight rows; each of the four waves owns 4
// weight tiles (64 rows) streamed into registers through a four-step ring.
// The 128 activation rows of a K step are loaded three steps ahead into
// registers, written to one of four LDS buffers two steps before their use,
// and read by all four waves.  The 128 tokens' per-128 activation scales and
// the 256 weight rows' per-32 scale lines sit in LDS (double-buffered across
// tiles).  Per K step a wave issues 32 MFMAs in four asm blocks of 8 (two
// 16-token sub-tiles x four weight tiles); each block also reads the next
// block's activations from LDS, and the last one the next step's first
// operands, the next group's scales (every fourth step) and writes the
// staged activations, all in the shadow of its MFMAs.  Scale operands are
// held from the step's first block to its last, which closes with the wait
// states that protect them and the accumulators (one guard per step).
// Accumulators live in AGPRs.  The grid is persistent (expert_gemm_tile).
//
// LDS activation layout: token t's 16-byte chunk c (bytes 16c..16c+15 of the
// step) sits at slot c ^ (t & 7) of the token's 128-byte line.  With that
// xor the 16-byte reads of a wave (16 consecutive tokens x 4 chunks) run at
// the LDS's full rate (measured on gfx950: about twice the rate of the
// unswizzled and of other xor layouts).  For the reading lane (token
// 16m + col, chunks grp and 4 + grp) the slot does not depend on m, and the
// two chunks sit 64 bytes apart (xor), so every read of the step is one of
// two per-lane base addresses plus an immediate offset
// (buffer * 16384 + m * 2048).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int tile_slot(int t, int c) { return c ^ (t & 7); }

constexpr int kTileBuf = 128 * 128;   // bytes of one activation buffer

// Scale operands: one dword per token sub-tile (bytes = the four K steps of
// a group) and one per weight tile (the lane's K block of those four steps,
// see the transposed scale-line layout in the kernel).  The MFMA takes byte
// Q of both: op_sel (low bit) and op_sel_hi (high bit) select the byte of
// each scale operand (measured on gfx950).
// (FP4 weights: A operand format cbsz 4; FP8 weights: cbsz 0)
#define TILE_OPSEL_0 "op_sel:[0,0,0] op_sel_hi:[0,0,0]"
#define TILE_OPSEL_1 "op_sel:[1,1,0] op_sel_hi:[0,0,0]"
#define TILE_OPSEL_2 "op_sel:[0,0,0] op_sel_hi:[1,1,0]"
#define TILE_OPSEL_3 "op_sel:[1,1,0] op_sel_hi:[1,1,0]"
#define TILE_MFMA(C, A, B, S, T, OPS)                                                         \
  "v_mfma_scale_f32_16x16x128_f8f6f4 %[" C "], %[" A "], %[" B "], %[" C "], %[" S "], %[" T \
  "] " OPS "\n\t"
#define TILE_MFMA4(C0, C1, C2, C3, B, T, OPS)                                                 \
  TILE_MFMA(C0, "a0", B, "s0", T, OPS) TILE_MFMA(C1, "a1", B, "s1", T, OPS)                   \
  TILE_MFMA(C2, "a2", B, "s2", T, OPS) TILE_MFMA(C3, "a3", B, "s3", T, OPS)
// the asm statement BODY(op_sel of step Q, weight format) with outputs
// OUTS, inputs INS
#define TILE_Q_ASM(BODY, OUTS, INS)                                                       \
  if constexpr (F8) {                                                                     \
    if constexpr (Q == 0) asm volatile(BODY(TILE_OPSEL_0) : OUTS : INS);                  \
    else if constexpr (Q == 1) asm volatile(BODY(TILE_OPSEL_1) : OUTS : INS);             \
    else if constexpr (Q == 2) asm volatile(BODY(TILE_OPSEL_2) : OUTS : INS);             \
    else asm volatile(BODY(TILE_OPSEL_3) : OUTS : INS);                                   \
  } else {                                                                                \
    if constexpr (Q == 0) asm volatile(BODY(TILE_OPSEL_0 " cbsz:4") : OUTS : INS);        \
    else if constexpr (Q == 1) asm volatile(BODY(TILE_OPSEL_1 " cbsz:4") : OUTS : INS);   \
    else if constexpr (Q == 2) asm volatile(BODY(TILE_OPSEL_2 " cbsz:4") : OUTS : INS);   \
    else asm volatile(BODY(TILE_OPSEL_3 " cbsz:4") : OUTS : INS);                         \
  }

#define TILE_ACC_OUT                                                                        \
  [c0] "+a"(c0[0]), [c1] "+a"(c0[1]), [c2] "+a"(c0[2]), [c3] "+a"(c0[3]), [d0] "+a"(c1[0]), \
      [d1] "+a"(c1[1]), [d2] "+a"(c1[2]), [d3] "+a"(c1[3]), [x0] "=&v"(x0), [x1] "=&v"(x1), \
      [y0] "=&v"(y0), [y1] "=&v"(y1)
#define TILE_OPND_IN                                                                         \
  [a0] "v"(a[0]), [a1] "v"(a[1]), [a2] "v"(a[2]), [a3] "v"(a[3]), [b0] "v"(b0), [b1] "v"(b1), \
      [s0] "v"(sa[0]), [s1] "v"(sa[1]), [s2] "v"(sa[2]), [s3] "v"(sa[3]), [lo] "v"(lo),       \
      [hi] "v"(hi)

// Activations of two sub-tiles (tokens 16*m + col and 16*(m+1) + col) of the
// buffer at byte offset BOFF: operand b = {chunk grp, chunk 4 + grp}.
template <int OFF>
__device__ __forceinline__ void tile_read2(v8i& b0, v8i& b1, uint32_t lo, uint32_t hi) {
  v4i x0, x1, y0, y1;
  asm volatile(
      "ds_read_b128 %0, %4 offset:%6\n\t"
      "ds_read_b128 %1, %5 offset:%6\n\t"
      "ds_read_b128 %2, %4 offset:%7\n\t"
      "ds_read_b128 %3, %5 offset:%7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x0), "=&v"(x1), "=&v"(y0), "=&v"(y1)
      : "v"(lo), "v"(hi), "n"(OFF), "n"(OFF + 2048));
  b0 = v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
  b1 = v8i{y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
}

// 8 MFMAs of step Q on (b0, b1) -- two token sub-tiles x four weight tiles --
// while reading the next two sub-tiles at OFF into (n0, n1); the block ends
// once the reads have landed.  No wait states: the caller keeps the scale
// registers and accumulators untouched until the step's last block, which
// closes with them.
#define TILE_READ_BODY(OPS)                                                         \
  "ds_read_b128 %[x0], %[lo] offset:%[o0]\n\t"                                      \
  "ds_read_b128 %[x1], %[hi] offset:%[o0]\n\t"                                      \
  "ds_read_b128 %[y0], %[lo] offset:%[o1]\n\t"                                      \
  "ds_read_b128 %[y1], %[hi] offset:%[o1]\n\t"                                      \
  TILE_MFMA4("c0", "c1", "c2", "c3", "b0", "t0", OPS)                               \
  TILE_MFMA4("d0", "d1", "d2", "d3", "b1", "t1", OPS) "s_waitcnt lgkmcnt(0)"
#define TILE_READ_IN TILE_OPND_IN, [t0] "v"(sb0), [t1] "v"(sb1), [o0] "n"(OFF), [o1] "n"(OFF + 2048)
template <int OFF, int Q, bool F8 = false>
__device__ __forceinline__ void tile_mfma8_read(v4f (&c0)[4], v4f (&c1)[4],
                                                const typename std::conditional<F8, v8i, v4i>::type (&a)[4],
                                                const v8i& b0, const v8i& b1, const int (&sa)[4],
                                                int sb0, int sb1, v8i& n0, v8i& n1, uint32_t lo,
                                                uint32_t hi) {
  v4i x0, x1, y0, y1;
  TILE_Q_ASM(TILE_READ_BODY, TILE_ACC_OUT, TILE_READ_IN);
  n0 = v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
  n1 = v8i{y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
}

// Scales of a group of four K steps: the token scale dwords of the 8
// sub-tiles (bytes s..s+3 of token 16*m + col's line: tok + m * TROW) and
// the weight scale dwords of the lane's row in each of the four weight tiles
// (wrow + t * WROW; the lane's K block, steps s..s+3).
template <int TROW, int WROW>
__device__ __forceinline__ void tile_read_scales(uint32_t (&tw)[8], uint32_t (&ww)[4], uint32_t tok,
                                                 uint32_t wrow) {
  asm volatile(
      "ds_read_b32 %0, %12\n\t"
      "ds_read_b32 %1, %12 offset:%14\n\t"
      "ds_read_b32 %2, %12 offset:%15\n\t"
      "ds_read_b32 %3, %12 offset:%16\n\t"
      "ds_read_b32 %4, %12 offset:%17\n\t"
      "ds_read_b32 %5, %12 offset:%18\n\t"
      "ds_read_b32 %6, %12 offset:%19\n\t"
      "ds_read_b32 %7, %12 offset:%20\n\t"
      "ds_read_b32 %8, %13\n\t"
      "ds_read_b32 %9, %13 offset:%21\n\t"
      "ds_read_b32 %10, %13 offset:%22\n\t"
      "ds_read_b32 %11, %13 offset:%23\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(tw[0]), "=&v"(tw[1]), "=&v"(tw[2]), "=&v"(tw[3]), "=&v"(tw[4]), "=&v"(tw[5]),
        "=&v"(tw[6]), "=&v"(tw[7]), "=&v"(ww[0]), "=&v"(ww[1]), "=&v"(ww[2]), "=&v"(ww[3])
      : "v"(tok), "v"(wrow), "n"(TROW), "n"(2 * TROW), "n"(3 * TROW), "n"(4 * TROW),
        "n"(5 * TROW), "n"(6 * TROW), "n"(7 * TROW), "n"(WROW), "n"(2 * WROW), "n"(3 * WROW));
}

// The last 8 MFMAs of step Q (sub-tiles 6, 7) with the next step's LDS work
// in their shadow: after the first four, the reads of the next step's first
// two sub-tiles (buffer offset OFFN) into n0, n1, and the LDS stores of this
// thread's staged activation registers r (at wa + WOFF + 1024 * j); with SC
// also the next group's scales, as tile_read_scales (into tw, ww, registers
// of their own: the MFMAs after the reads still use the current ones).
// Every scale register of the step is an input, so that none is reused
// before the closing 32 wait states; then the LDS wait.
#define TILE_LAST_LDS                                \
  "ds_read_b128 %[x0], %[lo] offset:%[o0]\n\t"       \
  "ds_read_b128 %[x1], %[hi] offset:%[o0]\n\t"       \
  "ds_read_b128 %[y0], %[lo] offset:%[o1]\n\t"       \
  "ds_read_b128 %[y1], %[hi] offset:%[o1]\n\t"       \
  "ds_write_b128 %[wa], %[r0] offset:%[w0]\n\t"      \
  "ds_write_b128 %[wa], %[r1] offset:%[w1]\n\t"      \
  "ds_write_b128 %[wa], %[r2] offset:%[w2]\n\t"      \
  "ds_write_b128 %[wa], %[r3] offset:%[w3]\n\t"
#define TILE_LAST_SCALES                              \
  "ds_read_b32 %[tw0], %[tok]\n\t"                    \
  "ds_read_b32 %[tw1], %[tok] offset:%[q1]\n\t"       \
  "ds_read_b32 %[tw2], %[tok] offset:%[q2]\n\t"       \
  "ds_read_b32 %[tw3], %[tok] offset:%[q3]\n\t"       \
  "ds_read_b32 %[tw4], %[tok] offset:%[q4]\n\t"       \
  "ds_read_b32 %[tw5], %[tok] offset:%[q5]\n\t"       \
  "ds_read_b32 %[tw6], %[tok] offset:%[q6]\n\t"       \
  "ds_read_b32 %[tw7], %[tok] offset:%[q7]\n\t"       \
  "ds_read_b32 %[ww0], %[wrow]\n\t"                   \
  "ds_read_b32 %[ww1], %[wrow] offset:%[p1]\n\t"      \
  "ds_read_b32 %[ww2], %[wrow] offset:%[p2]\n\t"      \
  "ds_read_b32 %[ww3], %[wrow] offset:%[p3]\n\t"
#define TILE_LAST_CLOSE "s_nop 15\n\ts_nop 15\n\ts_waitcnt lgkmcnt(0)"
#define TILE_LAST_BODY(OPS)                                              \
  "s_nop 1\n\t" TILE_MFMA4("c0", "c1", "c2", "c3", "b0", "t6", OPS)       \
  TILE_LAST_LDS TILE_MFMA4("d0", "d1", "d2", "d3", "b1", "t7", OPS) TILE_LAST_CLOSE
#define TILE_LAST_SC_BODY(OPS)                                           \
  "s_nop 1\n\t" TILE_MFMA4("c0", "c1", "c2", "c3", "b0", "t6", OPS)       \
  TILE_LAST_LDS TILE_LAST_SCALES                                         \
  TILE_MFMA4("d0", "d1", "d2", "d3", "b1", "t7", OPS) TILE_LAST_CLOSE
#define TILE_LAST_IN                                                                           \
  TILE_OPND_IN, [t6] "v"(sb[6]), [t7] "v"(sb[7]), [k0] "v"(sb[0]), [k1] "v"(sb[1]),            \
      [k2] "v"(sb[2]), [k3] "v"(sb[3]), [k4] "v"(sb[4]), [k5] "v"(sb[5]), [o0] "n"(OFFN),      \
      [o1] "n"(OFFN + 2048), [wa] "v"(wa), [r0] "v"(r[0]), [r1] "v"(r[1]), [r2] "v"(r[2]),     \
      [r3] "v"(r[3]), [w0] "n"(WOFF), [w1] "n"(WOFF + 1024), [w2] "n"(WOFF + 2048),             \
      [w3] "n"(WOFF + 3072)
#define TILE_LAST_SC_OUT                                                                      \
  TILE_ACC_OUT, [tw0] "=&v"(tw[0]), [tw1] "=&v"(tw[1]), [tw2] "=&v"(tw[2]), [tw3] "=&v"(tw[3]), \
      [tw4] "=&v"(tw[4]), [tw5] "=&v"(tw[5]), [tw6] "=&v"(tw[6]), [tw7] "=&v"(tw[7]),         \
      [ww0] "=&v"(ww[0]), [ww1] "=&v"(ww[1]), [ww2] "=&v"(ww[2]), [ww3] "=&v"(ww[3])
#define TILE_LAST_SC_IN                                                                    \
  TILE_LAST_IN, [tok] "v"(tok), [wrow] "v"(wrow), [q1] "n"(TROW), [q2] "n"(2 * TROW),      \
      [q3] "n"(3 * TROW), [q4] "n"(4 * TROW), [q5] "n"(5 * TROW), [q6] "n"(6 * TROW),      \
      [q7] "n"(7 * TROW), [p1] "n"(WROW), [p2] "n"(2 * WROW), [p3] "n"(3 * WROW)
template <int OFFN, int WOFF, bool SC, int TROW, int WROW, int Q, bool F8 = false>
__device__ __forceinline__ void tile_mfma8_last_pf(v4f (&c0)[4], v4f (&c1)[4],
                                                   const typename std::conditional<F8, v8i, v4i>::type (&a)[4],
                                                   const v8i& b0, const v8i& b1,
                                                   const int (&sa)[4], const int (&sb)[8],
                                                   v8i& n0, v8i& n1, uint32_t lo, uint32_t hi,
                                                   const v4i (&r)[4], uint32_t wa,
                                                   uint32_t (&tw)[8], uint32_t (&ww)[4],
                                                   uint32_t tok, uint32_t wrow) {
  v4i x0, x1, y0, y1;
  if constexpr (SC) {
    TILE_Q_ASM(TILE_LAST_SC_BODY, TILE_LAST_SC_OUT, TILE_LAST_SC_IN);
  } else {
    TILE_Q_ASM(TILE_LAST_BODY, TILE_ACC_OUT, TILE_LAST_IN);
    (void)tw; (void)ww; (void)tok; (void)wrow;
  }
  n0 = v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
  n1 = v8i{y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
}
#undef TILE_LAST_LDS
#undef TILE_LAST_SCALES
#undef TILE_LAST_CLOSE
#undef TILE_LAST_BODY
#undef TILE_LAST_SC_BODY
#undef TILE_LAST_IN
#undef TILE_LAST_SC_OUT
#undef TILE_LAST_SC_IN
#undef TILE_READ_BODY
#undef TILE_READ_IN
#undef TILE_ACC_OUT
#undef TILE_OPND_IN
#undef TILE_Q_ASM
#undef TILE_MFMA4
#undef TILE_MFMA
#undef TILE_OPSEL_0
#undef TILE_OPSEL_1
#undef TILE_OPSEL_2
#undef TILE_OPSEL_3

// Workgroup barrier once this wave's LDS writes are done; no memory access
// is moved across it (outstanding global loads stay in flight).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// Load of a T from global memory (the address space spelt out, so that the
// compiler emits a global load even where it cannot trace the pointer).
template <class T>
__device__ __forceinline__ T gload(const void* p) {
  return *(const __attribute__((address_space(1))) T*)p;
}

// One tile of the persistent tile kernel: expert e, first weight row n0,
// first pair slot m0 among the expert's n_e sorted pairs starting at off_e.
struct TileSel {
  int e, n0, m0, off_e, n_e;
};

// Expert-major tile order: the tiles of one expert are consecutive, m-tile
// fastest (an n-slice of its weights is used by all of its m-tiles back to
// back, and its activation rows by all n-slices close in time); each XCD
// (workgroups are dealt to the 8 XCDs round-robin) takes one contiguous
// eighth of the tiles, so that the workgroups sharing an L2 share weights
// and activations.  Tile u of that order is decoded here
// from LDS copies of the m-tile prefix (mt) and the expert offsets (eo):
// e is the number of entries mt[i] * n_tiles <= u, minus one, counted by the
// whole wave at once.  Wave-uniform.
__device__ __forceinline__ TileSel decode_tile(const int* mt, const int* eo, int E, int n_tiles,
                                               int rows_per_tile, int u, int lane) {
  int cnt = 0;
#pragma unroll
  for (int i0 = 0; i0 <= kMaxExperts; i0 += 64) {
    const int i = i0 + lane;
    const int v = mt[min(i, E)];  // unconditional: the reads overlap
    cnt += __popcll(__ballot((i <= E) & (v * n_tiles <= u)));
  }
  TileSel t;
  t.e = __builtin_amdgcn_readfirstlane(cnt - 1);
  const int mt0 = __builtin_amdgcn_readfirstlane(mt[t.e]);
  const int m_e = __builtin_amdgcn_readfirstlane(mt[t.e + 1]) - mt0;
  const int local = u - mt0 * n_tiles;
  const int n_tile = local / m_e;
  t.n0 = n_tile * rows_per_tile;
  t.m0 = (local - n_tile * m_e) * 128;
  t.off_e = __builtin_amdgcn_readfirstlane(eo[t.e]);
  t.n_e = __builtin_amdgcn_readfirstlane(eo[t.e + 1]) - t.off_e;
  return t;
}

// Persistent tile kernel: one workgroup per CU walks its share of the tiles
// (XCD x = blockIdx % 8 takes the x-th eighth of the expert-major tile list,
// its workgroups every R-th tile of it) as one continuous stream of K steps:
// the weight ring, the activation staging and the scale lines of the next
// tile are loaded while the current tile finishes, so that its epilogue and
// the next tile's first loads overlap instead of following each other.
// F8: FP8 weights ([N, K] E4M3 bytes, one scale per row and K step) instead
// of MXFP4; their 32-byte A operands run through a two-step ring, so that
// the registers stay those of the four-step ring of 16-byte FP4 operands.
template <int MODE, int S, bool F8 = false>
__global__ __launch_bounds__(kGemmThreads, 1) void expert_gemm_tile(ExpertGemmArgs p,
                                                                     int n_tiles) {
  constexpr int MT = 8, BM = 128;
  constexpr int K = S * 128;
  static_assert(S % 4 == 0 && S >= 8, "K steps in groups of four, at least two groups");
  constexpr int RD = F8 ? 2 : 4;                // weight ring depth (steps)
  constexpr int WROWB = F8 ? K : K / 2;         // weight bytes per row
  constexpr int SROWB = F8 ? S : K / 32;        // weight scale bytes per row
  constexpr int WLINE = F8 ? S + 16 : 4 * S + 16;  // weight scale line in LDS, padded (banks)
  typedef typename std::conditional<F8, v8i, v4i>::type AT;
  constexpr int NROWS = MODE == 1 ? kG1Cols : kG2Rows;
  __shared__ __attribute__((aligned(1024))) uint8_t act[4 * kTileBuf];
  __shared__ __attribute__((aligned(16))) uint8_t bsc[2][BM][S];
  __shared__ __attribute__((aligned(16))) uint8_t wsc[2][4][64][WLINE];
  __shared__ float red[4][BM];
  __shared__ int tab_mt[kMaxExperts + 1];
  __shared__ int tab_eo[kMaxExperts + 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int N = p.N, E = p.E;

  for (int i = tid; i <= E; i += kGemmThreads) {
    tab_mt[i] = p.mtile_off[i];
    tab_eo[i] = p.expert_offsets[i];
  }
  __syncthreads();

  // tiles of this workgroup: u = lo + r + j * R, j = 0 .. n_my - 1
  const int total = __builtin_amdgcn_readfirstlane(tab_mt[E]) * n_tiles;
  const int share = (total + 7) >> 3;
  const int R = gridDim.x >> 3;
  const int r = blockIdx.x >> 3;
  const int lo = (blockIdx.x & 7) * share;
  const int hi = min(lo + share, total);
  const int n_my = hi - lo > r ? (hi - lo - r + R - 1) / R : 0;
  if (n_my <= 0) return;
  auto tile_u = [&](int j) { return lo + r + j * R; };
  auto decode = [&](int u) { return decode_tile(tab_mt, tab_eo, E, n_tiles, NROWS, u, lane); };

  // Weight rows of this wave in a tile, as wave-uniform bases (row 16*t +
  // col of the wave's 64 at lane offset col * K/2 + 16 * grp).  Waves past N
  // in GEMM2 read rows 0..63 of the expert and skip the MFMAs: unconditional
  // loads keep every wave's load count the same.
  auto tile_bases = [&](const TileSel& ts, const uint8_t* (&wb)[4], const uint8_t* (&sb)[4]) {
    bool live = true;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      int row0;
      const uint8_t* wbase = p.w;
      const uint8_t* sbase = p.w_scale;
      if (MODE == 1) {
        row0 = ts.n0 + 32 * wv + 16 * (t & 1);
        if (t >= 2) {
          wbase = p.w3;
          sbase = p.w3_scale;
        }
      } else {
        live = ts.n0 + 64 * wv < N;
        row0 = live ? ts.n0 + 64 * wv + 16 * t : 16 * t;
      }
      const size_t rr = (size_t)ts.e * N + row0;
      wb[t] = wbase + rr * WROWB;
      sb[t] = sbase + rr * SROWB;
    }
    return live;
  };
  const uint32_t wlo = (uint32_t)(col * WROWB + 16 * grp);

  // activation staging: this thread moves 4 x 16 bytes per step, for tile
  // tokens 32*wv + 8*j + lane/8 (j = 0..3), landing at slot lane%8 of the
  // token's line, i.e. chunk tile_slot(token, lane%8) of the step (the map
  // is an involution on the chunk index)
  const int a_slot = tile_slot(lane >> 3, lane & 7);
  auto stage_tok = [&](int j) { return 32 * wv + 8 * j + (lane >> 3); };
  // sorted-pair slot of tile token t (slots past the expert's last pair
  // read that last pair's row; their results are dropped)
  auto pair_slot = [&](const TileSel& ts, int t) { return ts.off_e + min(ts.m0 + t, ts.n_e - 1); };
  const int sdst = (32 * wv + (lane >> 3)) * 128 + 16 * (lane & 7);  // + 1024 * j
  auto stage_load = [&](const uint8_t* const (&src)[4], int s, v4i (&rg)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) rg[j] = gload<v4i>(src[j] + (size_t)s * 128);
  };
  auto stage_store = [&](int q, const v4i (&rg)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<v4i*>(act + q * kTileBuf + sdst + 1024 * j) = rg[j];
  };
  AT A[RD][4];  // weight ring: [step % RD][tile]
  auto load_a = [&](const uint8_t* const (&wb)[4], int s, AT (&a)[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if constexpr (F8) {
        // the two 64-byte halves of the row's step line back to back
        const v4i lo = gload<v4i>(wb[t] + wlo + s * 128);
        const v4i hi = gload<v4i>(wb[t] + wlo + s * 128 + 64);
        a[t] = AT{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      } else {
        a[t] = gload<v4i>(wb[t] + wlo + s * 64);
      }
    }
  };

  // Weight scale lines in LDS, transposed per group of four K steps: the
  // line's 16 bytes of steps 4g..4g+3 (byte 4*q + kb: step q, K block kb)
  // are stored as byte 4*kb + q, so that the lane of K block grp reads the
  // four steps' scales of its block as one dword (the MFMA's op_sel then
  // picks the step's byte).  Thread (wv, lane) copies the 16-byte groups
  // L = 4*i + grp (i = 0 .. NG-1) of the wave's 64 row lines (NG groups
  // each): row 16*(L / NG) + col, group L % NG.
  constexpr int NG = S / 4;                 // 16-byte groups per line
  constexpr int CPS = NG >= 4 ? NG / 4 : 1;  // groups a thread copies per preparation step
  struct WLine { v4i c[CPS]; };
  auto sel4 = [](const uint8_t* const (&b)[4], int t) {
    return t == 0 ? b[0] : t == 1 ? b[1] : t == 2 ? b[2] : b[3];
  };
  auto wgroup_src = [&](const uint8_t* const (&sbp)[4], int i) {
    const int L = 4 * i + grp;
    return sel4(sbp, L / NG) + col * (K / 32) + 16 * (L % NG);
  };
  auto wline_load = [&](const uint8_t* const (&sbp)[4], int i0) {
    WLine w;
#pragma unroll
    for (int k = 0; k < CPS; ++k) w.c[k] = i0 + k < NG ? gload<v4i>(wgroup_src(sbp, i0 + k)) : v4i{0, 0, 0, 0};
    return w;
  };
  // FP8: one scale byte per row and step, no transpose (the four lane groups
  // read the same dword); lane (grp, col) copies row 16*grp + col's line
  typedef typename std::conditional<S == 8, v2i, v4i>::type F8Chunk;
  constexpr int F8N = S == 8 ? 1 : S / 16;
  struct F8Line { F8Chunk c[F8N]; };
  auto f8line_load = [&](const uint8_t* const (&sbp)[4]) {
    F8Line w;
    const uint8_t* src = sel4(sbp, grp) + col * S;
#pragma unroll
    for (int k = 0; k < F8N; ++k) w.c[k] = gload<F8Chunk>(src + k * sizeof(F8Chunk));
    return w;
  };
  auto f8line_store = [&](int b, const F8Line& w) {
#pragma unroll
    for (int k = 0; k < F8N; ++k)
      reinterpret_cast<F8Chunk*>(&wsc[b][wv][16 * grp + col][0])[k] = w.c[k];
  };
  // 4x4 byte transpose of a 16-byte group (dword q, byte kb -> dword kb, byte q)
  auto transpose16 = [](const v4i& d) {
    const uint32_t lo01 = __builtin_amdgcn_perm((uint32_t)d[1], (uint32_t)d[0], 0x05010400u);
    const uint32_t hi01 = __builtin_amdgcn_perm((uint32_t)d[1], (uint32_t)d[0], 0x07030602u);
    const uint32_t lo23 = __builtin_amdgcn_perm((uint32_t)d[3], (uint32_t)d[2], 0x05010400u);
    const uint32_t hi23 = __builtin_amdgcn_perm((uint32_t)d[3], (uint32_t)d[2], 0x07030602u);
    return v4i{(int)__builtin_amdgcn_perm(lo23, lo01, 0x05040100u),
               (int)__builtin_amdgcn_perm(lo23, lo01, 0x07060302u),
               (int)__builtin_amdgcn_perm(hi23, hi01, 0x05040100u),
               (int)__builtin_amdgcn_perm(hi23, hi01, 0x07060302u)};
  };
  auto wline_store = [&](int b, int i0, const WLine& w) {
#pragma unroll
    for (int k = 0; k < CPS; ++k) {
      if (i0 + k >= NG) break;
      const int L = 4 * (i0 + k) + grp;
      *reinterpret_cast<v4i*>(&wsc[b][wv][16 * (L / NG) + col][16 * (L % NG)]) = transpose16(w.c[k]);
    }
  };
  typedef typename std::conditional<S == 32, v4i, typename std::conditional<S == 16, v2i, int>::type>::type TChunk;
  auto tline_src = [&](int row) { return p.a_scale + (size_t)row * S + (tid & 1) * (S / 2); };
  auto tline_store = [&](int b, const TChunk& v) {
    *reinterpret_cast<TChunk*>(&bsc[b][tid >> 1][(tid & 1) * (S / 2)]) = v;
  };

  // ---- first tile: scale lines and the start of the pipeline ----
  TileSel cur = decode(tile_u(0));
  const uint8_t* wb[4];
  const uint8_t* sb[4];
  bool live = tile_bases(cur, wb, sb);
  const uint8_t* ssrc[4];
  {
    int rows[4];
    int srow;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ps = pair_slot(cur, stage_tok(j));
      rows[j] = MODE == 1 ? p.sorted_pairs[ps] / p.top_k : ps;
    }
    {
      const int ps = pair_slot(cur, tid >> 1);
      srow = MODE == 1 ? p.sorted_pairs[ps] / p.top_k : ps;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) ssrc[j] = p.a + (size_t)rows[j] * K + 16 * a_slot;
    tline_store(0, gload<TChunk>(tline_src(srow)));
    if constexpr (F8) {
      f8line_store(0, f8line_load(sb));
    } else {
#pragma unroll
      for (int i0 = 0; i0 < NG; i0 += CPS) wline_store(0, i0, wline_load(sb, i0));
    }
  }

  v4f acc[MT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[m][t] = v4f{0.f, 0.f, 0.f, 0.f};

  // Activations run three steps ahead: buffers 0 and 1 are written here and
  // step 2 waits in registers; the first group's scales and the first two
  // sub-tiles of step 0 are read before the loop, later ones by the step
  // before (in the shadow of its last MFMAs).
  v4i R2[2][4];
  load_a(wb, 0, A[0]);
  stage_load(ssrc, 0, R2[0]);
  load_a(wb, 1, A[1]);
  stage_load(ssrc, 1, R2[1]);
  if constexpr (RD == 4) {
    load_a(wb, 2, A[2 % RD]);
    load_a(wb, 3, A[3 % RD]);
  }
  stage_store(0, R2[0]);
  stage_store(1, R2[1]);
  stage_load(ssrc, 2, R2[0]);

  const int rslot = tile_slot(col, grp);
  const uint32_t rd_lo = lds_addr(act) + col * 128 + 16 * rslot;
  const uint32_t rd_hi = rd_lo ^ 64u;
  const uint32_t st_wa = lds_addr(act) + sdst;
  uint32_t sbw[MT];  // token scales of the group's four steps, per sub-tile
  uint32_t saw[4];   // weight scales of the lane's K block for those steps, per weight tile
  v8i x0, x1;
  lds_barrier();
  tile_read_scales<16 * S, 16 * WLINE>(sbw, saw, lds_addr(&bsc[0][col][0]),
                                       lds_addr(&wsc[0][wv][col][F8 ? 0 : 4 * grp]));
  tile_read2<0>(x0, x1, rd_lo, rd_hi);

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;

  for (int jt = 0; jt < n_my; ++jt) {
    const int cb = jt & 1, nb = cb ^ 1;  // scale buffers of this and the next tile
    const uint32_t sc_tok = lds_addr(&bsc[cb][col][0]);
    const uint32_t sc_w = lds_addr(&wsc[cb][wv][col][F8 ? 0 : 4 * grp]);

    const uint32_t nsc_tok = lds_addr(&bsc[nb][col][0]);
    const uint32_t nsc_w = lds_addr(&wsc[nb][wv][col][F8 ? 0 : 4 * grp]);

    // One K step from buffer Q (compile-time) and ring slot Q; its operands
    // for sub-tiles 0, 1 (x0, x1) and, at Q == 0, the group's scales were
    // read by the step before.  The last block also writes the activations
    // of step s + 2 to their buffer and, at Q == 3, reads the next group's
    // scales (the next tile's first group after its last step).
    auto compute = [&](int s, auto qc, auto lastc) {
      constexpr int Q = decltype(qc)::value;
      constexpr bool LAST = decltype(lastc)::value;  // s == S - 1
      constexpr int WB = ((Q + 2) & 3) * kTileBuf;
      if (!live) {
        stage_store((Q + 2) & 3, R2[Q & 1]);
        return;
      }
      // the MFMAs take byte Q of these (op_sel)
      const int sa[4] = {(int)saw[0], (int)saw[1], (int)saw[2], (int)saw[3]};
      const int sbv[8] = {(int)sbw[0], (int)sbw[1], (int)sbw[2], (int)sbw[3],
                          (int)sbw[4], (int)sbw[5], (int)sbw[6], (int)sbw[7]};
      constexpr int B = Q * kTileBuf;
      constexpr int BN = ((Q + 1) & 3) * kTileBuf;
      v8i y0, y1;
      // one guard per step: every scale register of the step stays live
      // until the last block, which closes with the wait states
      tile_mfma8_read<B + 2 * 2048, Q, F8>(acc[0], acc[1], A[Q % RD], x0, x1, sa, sbv[0], sbv[1], y0, y1,
                                    rd_lo, rd_hi);
      tile_mfma8_read<B + 4 * 2048, Q, F8>(acc[2], acc[3], A[Q % RD], y0, y1, sa, sbv[2], sbv[3], x0, x1,
                                    rd_lo, rd_hi);
      tile_mfma8_read<B + 6 * 2048, Q, F8>(acc[4], acc[5], A[Q % RD], x0, x1, sa, sbv[4], sbv[5], y0, y1,
                                    rd_lo, rd_hi);
      const uint32_t tok = LAST ? nsc_tok : sc_tok + s + 1;
      const uint32_t wrow = LAST ? nsc_w : sc_w + (F8 ? 1 : 4) * (s + 1);
      tile_mfma8_last_pf<BN, WB, Q == 3, 16 * S, 16 * WLINE, Q, F8>(acc[6], acc[7], A[Q % RD], y0, y1, sa,
                                                             sbv, x0, x1, rd_lo, rd_hi,
                                                             R2[Q & 1], st_wa, sbw, saw, tok,
                                                             wrow);
    };

    // The next tile (this one again after the last: its loads then only
    // re-read valid rows), prepared in the first steps: P0 decode and pair
    // rows, P1-P4 weight scale lines (stored one step after their load),
    // P4 token scale line (stored at P5) and activation row pointers.
    TileSel nxt;
    const uint8_t* nwb[4];
    const uint8_t* nsb[4];
    bool nlive;
    const uint8_t* nss[4];
    int nraw[4], nraw_s;
    WLine wtmp[2];  // loaded at P into [(P-1)&1], stored at P+1
    F8Line ftmp;    // FP8: loaded at P1, stored at P2
    TChunk ttmp;
    auto prep_load = [&](auto pc) {
      constexpr int P = decltype(pc)::value;
      if constexpr (P == 0) {
        nxt = decode(tile_u(jt + 1 < n_my ? jt + 1 : jt));
        nlive = tile_bases(nxt, nwb, nsb);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int ps = pair_slot(nxt, stage_tok(j));
          nraw[j] = MODE == 1 ? gload<int>(p.sorted_pairs + ps) : ps;
        }
        const int ps = pair_slot(nxt, tid >> 1);
        nraw_s = MODE == 1 ? gload<int>(p.sorted_pairs + ps) : ps;
      } else if constexpr (P >= 1 && P <= 4) {
        if constexpr (F8) {
          if constexpr (P == 1) ftmp = f8line_load(nsb);
        } else {
          wtmp[(P - 1) & 1] = wline_load(nsb, (P - 1) * CPS);
        }
        if constexpr (P == 4) {
          ttmp = gload<TChunk>(tline_src(MODE == 1 ? nraw_s / p.top_k : nraw_s));
#pragma unroll
          for (int j = 0; j < 4; ++j)
            nss[j] = p.a + (size_t)(MODE == 1 ? nraw[j] / p.top_k : nraw[j]) * K + 16 * a_slot;
        }
      }
    };
    auto prep_store = [&](auto pc) {
      constexpr int P = decltype(pc)::value;
      if constexpr (F8) {
        if constexpr (P == 2) f8line_store(nb, ftmp);
      } else if constexpr (P >= 2 && P <= 5) {
        wline_store(nb, (P - 2) * CPS, wtmp[P & 1]);
      }
      if constexpr (P == 5) tline_store(nb, ttmp);
    };

    // Step s: barrier; activation loads for step s+3 into registers;
    // compute(s) from buffer s%4 and ring slot s%RD, writing step s+2's
    // activations (loaded during step s-1) to buffer (s+2)%4 (last read in
    // step s-2, before the barrier of step s-1); weight loads for step s+RD
    // into the ring slot.  Steps past the tile's last come from the next
    // tile.  PREP: compile-time index of the next tile's preparation work;
    // MID: a step of the middle loop (s + 4 < S).
#define TILE_STEP(s, QC, PREP, MID)                                              \
  do {                                                                           \
    constexpr int q_ = QC::value;                                                \
    lds_barrier();                                                               \
    if ((MID) || (s) + 3 < S) stage_load(ssrc, (s) + 3, R2[(q_ + 1) & 1]);       \
    else stage_load(nss, (s) + 3 - S, R2[(q_ + 1) & 1]);                         \
    prep_load(std::integral_constant<int, PREP>{});                              \
    compute((s), QC{}, std::integral_constant<bool, !(MID) && (s) == S - 1>{});  \
    if ((MID) || (s) + RD < S) load_a(wb, (s) + RD, A[q_ % RD]);                 \
    else load_a(nwb, (s) + RD - S, A[q_ % RD]);                                  \
    prep_store(std::integral_constant<int, PREP>{});                             \
  } while (0)
    TILE_STEP(0, I0, 0, 0);
    TILE_STEP(1, I1, 1, 0);
    TILE_STEP(2, I2, 2, 0);
    TILE_STEP(3, I3, 3, 0);
    TILE_STEP(4, I0, 4, 0);
    TILE_STEP(5, I1, 5, 0);
    TILE_STEP(6, I2, 6, 0);
    TILE_STEP(7, I3, 7, 0);
    for (int s0 = 8; s0 < S - 4; s0 += 4) {
      TILE_STEP(s0, I0, -1, 1);
      TILE_STEP(s0 + 1, I1, -1, 1);
      TILE_STEP(s0 + 2, I2, -1, 1);
      TILE_STEP(s0 + 3, I3, -1, 1);
    }
    if constexpr (S > 8) {
      TILE_STEP(S - 4, I0, -1, 0);
      TILE_STEP(S - 3, I1, -1, 0);
      TILE_STEP(S - 2, I2, -1, 0);
      TILE_STEP(S - 1, I3, -1, 0);
    }
#undef TILE_STEP
    // the epilogue reads the accumulators only after the last block's wait
    // states (the MFMAs are invisible to the compiler's hazard tracking)
    asm volatile(""
                 : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]),
                   "+a"(acc[1][0]), "+a"(acc[1][1]), "+a"(acc[1][2]), "+a"(acc[1][3]),
                   "+a"(acc[2][0]), "+a"(acc[2][1]), "+a"(acc[2][2]), "+a"(acc[2][3]),
                   "+a"(acc[3][0]), "+a"(acc[3][1]), "+a"(acc[3][2]), "+a"(acc[3][3]));
    asm volatile(""
                 : "+a"(acc[4][0]), "+a"(acc[4][1]), "+a"(acc[4][2]), "+a"(acc[4][3]),
                   "+a"(acc[5][0]), "+a"(acc[5][1]), "+a"(acc[5][2]), "+a"(acc[5][3]),
                   "+a"(acc[6][0]), "+a"(acc[6][1]), "+a"(acc[6][2]), "+a"(acc[6][3]),
                   "+a"(acc[7][0]), "+a"(acc[7][1]), "+a"(acc[7][2]), "+a"(acc[7][3]));

    const int m0 = cur.m0, off_e = cur.off_e, n_e = cur.n_e, n0 = cur.n0;
    if (MODE == 1) {
      // clamped SwiGLU, per-128 FP8 requant of h over this tile's 128 columns
      const float lim = p.limit;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        float amax = 0.f;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float g = clamp_sym(acc[m][tt][v], lim);
            const float u = clamp_sym(acc[m][tt + 2][v], lim);
            const float hv = silu_fast(g) * u;
            acc[m][tt][v] = hv;                       // h kept in the w1 slots
            amax = fmaxf(amax, fabsf(hv));
          }
        amax = fmaxf(amax, __shfl_xor(amax, 16));
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        if (lane < 16) red[wv][16 * m + lane] = amax;
      }
      __syncthreads();
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int tokc = 16 * m + col;
        const float amax =
            fmaxf(fmaxf(red[0][tokc], red[1][tokc]), fmaxf(red[2][tokc], red[3][tokc]));
        const int ex = pow2_scale_exp(amax);
        const int slot = m0 + tokc;
        if (slot < n_e) {
          const size_t row = (size_t)(off_e + slot);
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const uint32_t word = e4m3x4_exp(acc[m][tt], ex);
            *reinterpret_cast<uint32_t*>(p.hq + row * N + n0 + 32 * wv + 16 * tt + 4 * grp) = word;
          }
          if (wv == 0 && grp == 0) p.hs[row * (N / 128) + n0 / 128] = (uint8_t)(ex + 127);
        }
      }
    } else if (live) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int slot = m0 + 16 * m + col;
        if (slot >= n_e) continue;
        const size_t row = (size_t)(off_e + slot);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const size_t c = (size_t)n0 + 64 * wv + 16 * t + 4 * grp;
          if (p.out_fp32) {
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + row * N + c) =
                make_float4(acc[m][t][0], acc[m][t][1], acc[m][t][2], acc[m][t][3]);
          } else {
            const uint32_t lo2 = f32_to_bf16(acc[m][t][0]) | (f32_to_bf16(acc[m][t][1]) << 16);
            const uint32_t hi2 = f32_to_bf16(acc[m][t][2]) | (f32_to_bf16(acc[m][t][3]) << 16);
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + row * N + c) =
                make_uint2(lo2, hi2);
          }
        }
      }
    }

    // next tile
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[m][t] = v4f{0.f, 0.f, 0.f, 0.f};
    // the zeroed accumulators settle before the next tile's first MFMA
    asm volatile("s_nop 1"
                 : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]),
                   "+a"(acc[1][0]), "+a"(acc[1][1]), "+a"(acc[1][2]), "+a"(acc[1][3]),
                   "+a"(acc[2][0]), "+a"(acc[2][1]), "+a"(acc[2][2]), "+a"(acc[2][3]),
                   "+a"(acc[3][0]), "+a"(acc[3][1]), "+a"(acc[3][2]), "+a"(acc[3][3]));
    asm volatile("s_nop 1"
                 : "+a"(acc[4][0]), "+a"(acc[4][1]), "+a"(acc[4][2]), "+a"(acc[4][3]),
                   "+a"(acc[5][0]), "+a"(acc[5][1]), "+a"(acc[5][2]), "+a"(acc[5][3]),
                   "+a"(acc[6][0]), "+a"(acc[6][1]), "+a"(acc[6][2]), "+a"(acc[6][3]),
                   "+a"(acc[7][0]), "+a"(acc[7][1]), "+a"(acc[7][2]), "+a"(acc[7][3]));
    cur = nxt;
    live = nlive;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      wb[t] = nwb[t];
      sb[t] = nsb[t];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) ssrc[j] = nss[j];
  }
}

static inline unsigned pad8(int64_t g) { return (unsigned)((g + 7) / 8 * 8); }

// Workgroups of a persistent launch: the device's CU count, rounded down to a
// multiple of 8 (the XCD count), at least 8.
static int persistent_workgroups() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 8;
    n = std::max(8, cus / 8 * 8);
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int MODE>
static hipError_t launch_mode(const ExpertGemmArgs& a, int bm, int mt_max, hipStream_t st) {
  const int n_tiles = MODE == 1 ? a.N / kG1Cols : (a.N + kG2Rows - 1) / kG2Rows;
  const unsigned grid = pad8((int64_t)n_tiles * mt_max);
  if (grid == 0) return hipSuccess;
  if (a.fp8w && bm == 128) {
    if (a.K != 1024 && a.K != 2048 && a.K != 4096) return hipErrorInvalidValue;
    if (a.E > kMaxExperts) return hipErrorInvalidValue;
    const unsigned pgrid = std::min(grid, (unsigned)persistent_workgroups());
    if (a.K == 4096)
      hipLaunchKernelGGL((expert_gemm_tile<MODE, 32, true>), dim3(pgrid), dim3(kGemmThreads), 0, st,
                         a, n_tiles);
    else if (a.K == 2048)
      hipLaunchKernelGGL((expert_gemm_tile<MODE, 16, true>), dim3(pgrid), dim3(kGemmThreads), 0, st,
                         a, n_tiles);
    else
      hipLaunchKernelGGL((expert_gemm_tile<MODE, 8, true>), dim3(pgrid), dim3(kGemmThreads), 0, st,
                         a, n_tiles);
    return hipGetLastError();
  }
  if (a.fp8w) {
    if (bm == 16 && a.K == 4096)
      hipLaunchKernelGGL((expert_gemm_stream8<MODE, 32>), dim3(grid), dim3(kGemmThreads), 0, st, a,
                         mt_max, n_tiles);
    else if (bm == 16 && a.K == 2048)
      hipLaunchKernelGGL((expert_gemm_stream8<MODE, 16>), dim3(grid), dim3(kGemmThreads), 0, st, a,
                         mt_max, n_tiles);
    else if (bm == 16 && a.K == 1024)
      hipLaunchKernelGGL((expert_gemm_stream8<MODE, 8>), dim3(grid), dim3(kGemmThreads), 0, st, a,
                         mt_max, n_tiles);
    else if (bm == 16)
      hipLaunchKernelGGL((expert_gemm_kernel<MODE, 1, true>), dim3(grid), dim3(kGemmThreads), 0, st,
                         a, mt_max, n_tiles);
    else if (bm == 64)
      hipLaunchKernelGGL((expert_gemm_kernel<MODE, 4, true>), dim3(grid), dim3(kGemmThreads), 0, st,
                         a, mt_max, n_tiles);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  }
  if (bm == 128) {
    if (a.K != 1024 && a.K != 2048 && a.K != 4096) return hipErrorInvalidValue;
    if (a.E > kMaxExperts) return hipErrorInvalidValue;
    // persistent: at most one workgroup per CU (the LDS use allows no more)
    const unsigned pgrid = std::min(grid, (unsigned)persistent_workgroups());
    if (a.K == 4096)
      hipLaunchKernelGGL((expert_gemm_tile<MODE, 32>), dim3(pgrid), dim3(kGemmThreads), 0, st, a,
                         n_tiles);
    else if (a.K == 2048)
      hipLaunchKernelGGL((expert_gemm_tile<MODE, 16>), dim3(pgrid), dim3(kGemmThreads), 0, st, a,
                         n_tiles);
    else
      hipLaunchKernelGGL((expert_gemm_tile<MODE, 8>), dim3(pgrid), dim3(kGemmThreads), 0, st, a,
                         n_tiles);
  } else if (bm == 16 && a.K == 4096) {
    hipLaunchKernelGGL((expert_gemm_stream<MODE, 32>), dim3(grid), dim3(kGemmThreads), 0, st, a,
                       mt_max, n_tiles);
  } else if (bm == 16 && a.K == 2048) {
    hipLaunchKernelGGL((expert_gemm_stream<MODE, 16>), dim3(grid), dim3(kGemmThreads), 0, st, a,
                       mt_max, n_tiles);
  } else if (bm == 16 && a.K == 1024) {
    hipLaunchKernelGGL((expert_gemm_stream<MODE, 8>), dim3(grid), dim3(kGemmThreads), 0, st, a,
                       mt_max, n_tiles);
  } else if (bm == 16) {
    hipLaunchKernelGGL((expert_gemm_kernel<MODE, 1>), dim3(grid), dim3(kGemmThreads), 0, st, a,
                       mt_max, n_tiles);
  } else {
    hipLaunchKernelGGL((expert_gemm_kernel<MODE, 4>), dim3(grid), dim3(kGemmThreads), 0, st, a,
                       mt_max, n_tiles);
  }
  return hipGetLastError();
}

hipError_t launch_expert_gemm1(const ExpertGemmArgs& a, int bm, int mt_max, hipStream_t st) {
  return launch_mode<1>(a, bm, mt_max, st);
}
hipError_t launch_expert_gemm2(const ExpertGemmArgs& a, int bm, int mt_max, hipStream_t st) {
  return launch_mode<2>(a, bm, mt_max, st);
}

}  // namespace moe
