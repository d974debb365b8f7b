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
// Work decomposition: a workgroup (4 waves) owns one m-tile of one expert
// (16 * MT pairs) and one n-tile of weight rows; it streams its weight rows
// once over the whole K with 16-byte loads straight into the MFMA operand
// registers (each weight byte is used by exactly one lane). Activation rows
// are gathered per token; with MT > 1 they are staged once per K step in LDS
// and shared by the four waves. m-tiles are enumerated through a device-side
// prefix over experts (mtile_off), so expert counts never travel to the host.
// Workgroup ids are remapped so that the tiles of one weight n-tile that land
// on the same XCD (ids are dealt round-robin over the 8 XCDs) are processed
// together there, and share that XCD's L2.
#include "moe_internal.h"

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4f mfma_fp4_fp8(const uint4& a, const uint4& b0, const uint4& b1,
                                            v4f acc, int sa, int sb) {
  v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  v8i bv = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
            (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 4, 0, 0, sa, 0, sb);
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

// Maps the workgroup to (n_tile, expert, m0); returns false when idle.
__device__ __forceinline__ bool map_tile(const ExpertGemmArgs& p, int mt_max, int n_tiles, int bm,
                                         int& n_tile, int& e, int& m0, int& off_e, int& n_e) {
  const int G = gridDim.x;
  const int b = blockIdx.x;
  const int w = (b & 7) * (G >> 3) + (b >> 3);
  n_tile = w / mt_max;
  const int mt = w - n_tile * mt_max;
  if (n_tile >= n_tiles) return false;
  const int total = p.mtile_off[p.E];
  if (mt >= total) return false;
  int lo = 0, hi = p.E;  // mtile_off[lo] <= mt < mtile_off[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.mtile_off[mid] <= mt) lo = mid; else hi = mid;
  }
  e = lo;
  m0 = (mt - p.mtile_off[e]) * bm;
  off_e = p.expert_offsets[e];
  n_e = p.expert_offsets[e + 1] - off_e;
  return true;
}

template <int MODE, int MT>
__global__ __launch_bounds__(kGemmThreads) void expert_gemm_kernel(ExpertGemmArgs p, int mt_max,
                                                                    int n_tiles) {
  constexpr int BM = 16 * MT;
  constexpr int LDS_ROW = 144;  // 128 activation bytes + 16 pad (bank spread)
  __shared__ __attribute__((aligned(16))) uint8_t bsm[MT > 1 ? 2 : 1][MT > 1 ? BM : 1][LDS_ROW];
  __shared__ float red[4][BM];

  int n_tile, e, m0, off_e, n_e;
  if (!map_tile(p, mt_max, n_tiles, BM, n_tile, e, m0, off_e, n_e)) return;

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int col = lane & 15;   // token slot within a 16-column sub-tile
  const int grp = lane >> 4;   // K group
  const int K = p.K, N = p.N;
  const int steps = K / 128;
  const size_t wrow_bytes = (size_t)K / 2;
  const size_t srow_bytes = (size_t)K / 32;

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
      sptr[t] = sbase + ((size_t)e * N + row) * srow_bytes;
    }
  } else {
    n0 = n_tile * kG2Rows;
    wave_live = (n0 + 64 * wv) < N;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row = wave_live ? (n0 + 64 * wv + 16 * t + col) : 0;
      wptr[t] = p.w + ((size_t)e * N + row) * wrow_bytes + grp * 16;
      sptr[t] = p.w_scale + ((size_t)e * N + row) * srow_bytes;
    }
  }

  // ---- activation rows of the MT sub-tiles (this lane's token column) ----
  const uint8_t* bptr[MT];
  const uint8_t* bsp[MT];
  bool bval[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int slot = m0 + 16 * m + col;
    bval[m] = slot < n_e;
    int64_t row = 0;
    if (bval[m]) row = (MODE == 1) ? (int64_t)(p.sorted_pairs[off_e + slot] / p.top_k)
                                   : (int64_t)(off_e + slot);
    bptr[m] = p.a + row * K;
    bsp[m] = p.a_scale + row * (K / 128);
  }

  v4f acc[4][MT];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[t][m] = v4f{0.f, 0.f, 0.f, 0.f};

  // staging loader for MT > 1: thread i copies 16 bytes of one token row
  int st_tok[MT > 1 ? 2 : 1], st_chunk = threadIdx.x & 7;
  const uint8_t* st_src[MT > 1 ? 2 : 1];
  bool st_val[MT > 1 ? 2 : 1];
  if constexpr (MT > 1) {
#pragma unroll
    for (int r = 0; r < (BM * 8 + kGemmThreads - 1) / kGemmThreads && r < 2; ++r) {
      const int tok = (threadIdx.x >> 3) + 32 * r;
      st_tok[r] = tok;
      const int slot = m0 + tok;
      st_val[r] = tok < BM && slot < n_e;
      int64_t row = 0;
      if (st_val[r]) row = (MODE == 1) ? (int64_t)(p.sorted_pairs[off_e + slot] / p.top_k)
                                       : (int64_t)(off_e + slot);
      st_src[r] = p.a + row * K + 16 * st_chunk;
    }
  }
  constexpr int ST_ROUNDS = MT > 1 ? ((BM * 8 + kGemmThreads - 1) / kGemmThreads) : 0;

  if (wave_live || MT > 1) {
    uint4 a_cur[4], a_nxt[4];
    uint32_t s_cur[4], s_nxt[4];
    uint4 b_cur[MT][2], b_nxt[MT][2];
    int bs_cur[MT], bs_nxt[MT];
    uint4 st_reg[2];

    auto load_a = [&](int s, uint4* a, uint32_t* sc) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        a[t] = *reinterpret_cast<const uint4*>(wptr[t] + (size_t)s * 64);
        sc[t] = *reinterpret_cast<const uint32_t*>(sptr[t] + (size_t)s * 4);
      }
    };
    auto load_b_direct = [&](int s, uint4 (*b)[2], int* bs) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (bval[m]) {
          b[m][0] = *reinterpret_cast<const uint4*>(bptr[m] + (size_t)s * 128 + 16 * grp);
          b[m][1] = *reinterpret_cast<const uint4*>(bptr[m] + (size_t)s * 128 + 64 + 16 * grp);
          bs[m] = bsp[m][s];
        } else {
          b[m][0] = make_uint4(0, 0, 0, 0);
          b[m][1] = make_uint4(0, 0, 0, 0);
          bs[m] = 127;
        }
      }
    };
    auto load_bs = [&](int s, int* bs) {
#pragma unroll
      for (int m = 0; m < MT; ++m) bs[m] = bval[m] ? (int)bsp[m][s] : 127;
    };
    auto stage_load = [&](int s) {
#pragma unroll
      for (int r = 0; r < ST_ROUNDS; ++r)
        st_reg[r] = st_val[r] ? *reinterpret_cast<const uint4*>(st_src[r] + (size_t)s * 128)
                              : make_uint4(0, 0, 0, 0);
    };
    auto stage_store = [&](int buf) {
#pragma unroll
      for (int r = 0; r < ST_ROUNDS; ++r)
        if (st_tok[r] < BM)
          *reinterpret_cast<uint4*>(&bsm[buf][st_tok[r]][16 * st_chunk]) = st_reg[r];
    };
    auto read_b_lds = [&](int buf, uint4 (*b)[2]) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        b[m][0] = *reinterpret_cast<const uint4*>(&bsm[buf][16 * m + col][16 * grp]);
        b[m][1] = *reinterpret_cast<const uint4*>(&bsm[buf][16 * m + col][64 + 16 * grp]);
      }
    };
    auto compute = [&](const uint4* a, const uint32_t* sc, uint4 (*b)[2], const int* bs) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int sa = (int)((sc[t] >> (8 * grp)) & 0xFFu);
#pragma unroll
        for (int m = 0; m < MT; ++m)
          acc[t][m] = mfma_fp4_fp8(a[t], b[m][0], b[m][1], acc[t][m], sa, bs[m]);
      }
    };

    if constexpr (MT == 1) {
      load_a(0, a_cur, s_cur);
      load_b_direct(0, b_cur, bs_cur);
      for (int s = 0; s < steps; ++s) {
        if (s + 1 < steps) {
          load_a(s + 1, a_nxt, s_nxt);
          load_b_direct(s + 1, b_nxt, bs_nxt);
        }
        compute(a_cur, s_cur, b_cur, bs_cur);
#pragma unroll
        for (int t = 0; t < 4; ++t) { a_cur[t] = a_nxt[t]; s_cur[t] = s_nxt[t]; }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          b_cur[m][0] = b_nxt[m][0]; b_cur[m][1] = b_nxt[m][1]; bs_cur[m] = bs_nxt[m];
        }
      }
    } else {
      stage_load(0);
      stage_store(0);
      if (wave_live) load_a(0, a_cur, s_cur);
      load_bs(0, bs_cur);
      __syncthreads();
      for (int s = 0; s < steps; ++s) {
        const int buf = s & 1;
        if (s + 1 < steps) {
          stage_load(s + 1);
          if (wave_live) load_a(s + 1, a_nxt, s_nxt);
          load_bs(s + 1, bs_nxt);
        }
        if (wave_live) {
          read_b_lds(buf, b_cur);
          compute(a_cur, s_cur, b_cur, bs_cur);
        }
        if (s + 1 < steps) stage_store(buf ^ 1);
        __syncthreads();
#pragma unroll
        for (int t = 0; t < 4; ++t) { a_cur[t] = a_nxt[t]; s_cur[t] = s_nxt[t]; }
#pragma unroll
        for (int m = 0; m < MT; ++m) bs_cur[m] = bs_nxt[m];
      }
    }
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
          const float g = fminf(fmaxf(acc[tt][m][v], -lim), lim);
          const float u = fminf(fmaxf(acc[tt + 2][m][v], -lim), lim);
          const float hv = silu_f(g) * u;
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
          uint32_t word = 0;
#pragma unroll
          for (int v = 0; v < 4; ++v) word |= e4m3_rne(ldexpf(h[m][tt][v], -ex)) << (8 * v);
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

static inline unsigned pad8(int64_t g) { return (unsigned)((g + 7) / 8 * 8); }

template <int MODE>
static hipError_t launch_mode(const ExpertGemmArgs& a, int bm, int mt_max, hipStream_t st) {
  const int n_tiles = MODE == 1 ? a.N / kG1Cols : (a.N + kG2Rows - 1) / kG2Rows;
  const unsigned grid = pad8((int64_t)n_tiles * mt_max);
  if (grid == 0) return hipSuccess;
  if (bm == 16) {
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
