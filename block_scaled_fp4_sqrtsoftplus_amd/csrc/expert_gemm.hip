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
// Scale operands: the instruction reads its per-lane E8M0 scale registers
// over several cycles after issue (measured: a scale register rewritten by
// the very next VALU instruction gave rows 1-15 of the 16x16 tile the new
// value, row 0 the old one), and the compiler neither holds such writes back
// nor keeps a scale register untouched after its last use.  So the
// instruction is issued from inline assembly followed by 32 wait states
// (mfma_fp4_fp8 below), after which scale registers may be reused freely.
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

#include <type_traits>

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

typedef int v4i __attribute__((ext_vector_type(4)));

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
      "v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0] cbsz:4\n\t"
      "s_nop 15\n\t"
      "s_nop 15"
      : "+v"(acc)
      : "v"(av), "v"(bv), "v"(sa), "v"(sb));
  return acc;
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

// Expert-major tile order for large m-tiles: the tiles of one expert are
// consecutive, m-tile fastest (an n-slice of its weights is used by all of
// its m-tiles back to back, and its activation rows by all n-slices close in
// time), and each XCD (workgroups are dispatched to the 8 XCDs round-robin)
// takes one contiguous eighth of the real tiles, so that the workgroups
// sharing an L2 share weights and activations.
__device__ __forceinline__ bool map_tile_grouped(const ExpertGemmArgs& p, int n_tiles, int bm,
                                                 int& n_tile, int& e, int& m0, int& off_e,
                                                 int& n_e) {
  const int b = blockIdx.x;
  const int total = p.mtile_off[p.E] * n_tiles;
  const int share = (total + 7) >> 3;
  const int r = b >> 3;
  const int u = (b & 7) * share + r;
  if (r >= share || u >= total) return false;
  int lo = 0, hi = p.E;  // mtile_off[lo] * n_tiles <= u < mtile_off[hi] * n_tiles
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.mtile_off[mid] * n_tiles <= u) lo = mid; else hi = mid;
  }
  e = lo;
  const int m_e = p.mtile_off[e + 1] - p.mtile_off[e];
  const int local = u - p.mtile_off[e] * n_tiles;
  n_tile = local / m_e;
  m0 = (local - n_tile * m_e) * bm;
  off_e = p.expert_offsets[e];
  n_e = p.expert_offsets[e + 1] - off_e;
  return true;
}

template <int MODE, int MT>
__global__ __launch_bounds__(kGemmThreads) void expert_gemm_kernel(ExpertGemmArgs p, int mt_max,
                                                                    int n_tiles) {
  constexpr int BM = 16 * MT;
  constexpr int LDS_ROW = 144;  // 128 activation bytes + 16 pad (bank spread)
  constexpr bool STAGED = MT > 1;
  __shared__ __attribute__((aligned(16))) uint8_t bsm[STAGED ? 2 : 1][STAGED ? BM : 1][LDS_ROW];
  __shared__ float red[4][BM];

  int n_tile, e, m0, off_e, n_e;
  if (!map_tile(p, mt_max, n_tiles, BM, n_tile, e, m0, off_e, n_e)) return;

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int col = lane & 15;   // token slot within a 16-column sub-tile
  const int grp = lane >> 4;   // K group
  const int K = p.K, N = p.N;
  const int S = K / 128;
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
      sptr[t] = sbase + ((size_t)e * N + row) * srow_bytes + grp;
    }
  } else {
    n0 = n_tile * kG2Rows;
    wave_live = (n0 + 64 * wv) < N;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row = wave_live ? (n0 + 64 * wv + 16 * t + col) : 0;
      wptr[t] = p.w + ((size_t)e * N + row) * wrow_bytes + grp * 16;
      sptr[t] = p.w_scale + ((size_t)e * N + row) * srow_bytes + grp;
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
    uint4 a[4];
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
        x.a[t] = *reinterpret_cast<const uint4*>(wptr[t] + (size_t)s * 64);
        x.sa[t] = sptr[t][(size_t)s * 4];
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
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int m = 0; m < MT; ++m)
          acc[t][m] = mfma_fp4_fp8(x.a[t], x.b[m][0], x.b[m][1], acc[t][m], (int)x.sa[t], (int)x.sb[m]);
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

// ---------------------------------------------------------------------------
// Streaming variant for m-tiles of at most 16 pairs (decode) when K is
// 1024, 2048 or 4096: every wave keeps four K steps of weight and
// activation loads in flight in a register ring (no register copies, no
// branches around the loads, so the waits before each step's MFMAs cover
// only that step), and reads each weight row's scales once.  Lanes whose pair slot lies past the expert's last pair read that
// last pair's row: their columns are computed and dropped.
// ---------------------------------------------------------------------------
template <int MODE, int S>
__global__ __launch_bounds__(kGemmThreads) void expert_gemm_stream(ExpertGemmArgs p, int mt_max,
                                                                    int n_tiles) {
  __shared__ float red[4][16];
  int n_tile, e, m0, off_e, n_e;
  if (!map_tile(p, mt_max, n_tiles, 16, n_tile, e, m0, off_e, n_e)) return;

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  constexpr int K = S * 128;                // S in {8, 16, 32}
  const int N = p.N;
  constexpr int SD = S / 4;                 // scale dwords per lane group
  const size_t wrow_bytes = (size_t)K / 2;
  const size_t srow_bytes = (size_t)K / 32;

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
    // steps s and s + 1 (s even) together: the two 64-byte halves of each
    // weight row's 128-byte line are requested back to back, so the second
    // request meets the first one's line fill instead of missing again
    auto load_pair = [&](int s, uint4 (&a0)[4], uint4 (&b0)[2], uint4 (&a1)[4], uint4 (&b1)[2]) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        a0[t] = *reinterpret_cast<const uint4*>(wptr[t] + (size_t)s * 64);
        a1[t] = *reinterpret_cast<const uint4*>(wptr[t] + (size_t)s * 64 + 64);
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
        const float g = fminf(fmaxf(acc[tt][v], -lim), lim);
        const float u = fminf(fmaxf(acc[tt + 2][v], -lim), lim);
        const float hv = silu_f(g) * u;
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

// ---------------------------------------------------------------------------
// Tile variant for m-tiles of 128 pairs (prefill) when K is 1024, 2048 or
// 4096.  Each of the four waves owns 4 weight tiles (64 rows) streamed into
// registers through a four-step ring (each weight row's scale line read
// once, as in the streaming kernel).  The 128 activation rows of a K step are
// loaded two steps ahead into registers, written to one of four LDS buffers
// at the end of the step before their use, and read by all four waves; the
// 128 tokens' per-128 activation scales sit in LDS for the whole tile.  Per
// K step a wave issues 32 MFMAs in four asm blocks of 8 (two 16-token
// sub-tiles x four weight tiles), each closed by the wait states that
// protect its operands.  Accumulators live in AGPRs.
//
// LDS activation layout: token t's 16-byte chunk c (bytes 16c..16c+15 of the
// step) sits at slot c ^ (t & 7) ^ ((t >> 3) & 1) of the token's 128-byte
// line, so that the 16-byte reads of 16 consecutive tokens (same c) hit
// distinct banks.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int tile_slot(int t, int c) { return c ^ (t & 7) ^ ((t >> 3) & 1); }

// Two 16-token sub-tiles (B operands b0/b1, scales sb0/sb1) against four
// weight tiles (a[0..3], scales sa0..sa3).
__device__ __forceinline__ void mfma8_fp4_fp8(v4f (&c0)[4], v4f (&c1)[4], const v4i (&a)[4],
                                              const v8i& b0, const v8i& b1, int sa0, int sa1,
                                              int sa2, int sa3, int sb0, int sb1) {
  asm(
      "v_mfma_scale_f32_16x16x128_f8f6f4 %0, %8, %12, %0, %14, %18 op_sel_hi:[0,0,0] cbsz:4\n\t"
      "v_mfma_scale_f32_16x16x128_f8f6f4 %1, %9, %12, %1, %15, %18 op_sel_hi:[0,0,0] cbsz:4\n\t"
      "v_mfma_scale_f32_16x16x128_f8f6f4 %2, %10, %12, %2, %16, %18 op_sel_hi:[0,0,0] cbsz:4\n\t"
      "v_mfma_scale_f32_16x16x128_f8f6f4 %3, %11, %12, %3, %17, %18 op_sel_hi:[0,0,0] cbsz:4\n\t"
      "v_mfma_scale_f32_16x16x128_f8f6f4 %4, %8, %13, %4, %14, %19 op_sel_hi:[0,0,0] cbsz:4\n\t"
      "v_mfma_scale_f32_16x16x128_f8f6f4 %5, %9, %13, %5, %15, %19 op_sel_hi:[0,0,0] cbsz:4\n\t"
      "v_mfma_scale_f32_16x16x128_f8f6f4 %6, %10, %13, %6, %16, %19 op_sel_hi:[0,0,0] cbsz:4\n\t"
      "v_mfma_scale_f32_16x16x128_f8f6f4 %7, %11, %13, %7, %17, %19 op_sel_hi:[0,0,0] cbsz:4\n\t"
      "s_nop 15\n\t"
      "s_nop 15"
      : "+a"(c0[0]), "+a"(c0[1]), "+a"(c0[2]), "+a"(c0[3]),
        "+a"(c1[0]), "+a"(c1[1]), "+a"(c1[2]), "+a"(c1[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(b0), "v"(b1),
        "v"(sa0), "v"(sa1), "v"(sa2), "v"(sa3), "v"(sb0), "v"(sb1));
}

// Workgroup barrier once this wave's LDS writes are done; no memory access
// is moved across it (outstanding global loads stay in flight).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int MODE, int S>
__global__ __launch_bounds__(kGemmThreads, 1) void expert_gemm_tile(ExpertGemmArgs p, int mt_max,
                                                                     int n_tiles) {
  constexpr int MT = 8, BM = 128;
  constexpr int K = S * 128;
  constexpr int SD = S / 4;
  static_assert(S % 4 == 0 && S >= 8, "K steps in groups of four, at least two groups");
  // four activation buffers (one per step of a group of four)
  __shared__ __attribute__((aligned(1024))) uint8_t act0[BM * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t act1[BM * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t act2[BM * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t act3[BM * 128];
  __shared__ __attribute__((aligned(16))) uint8_t bsc[BM][S];
  __shared__ float red[4][BM];
  (void)mt_max;

  int n_tile, e, m0, off_e, n_e;
  if (!map_tile_grouped(p, n_tiles, BM, n_tile, e, m0, off_e, n_e)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int N = p.N;
  const size_t wrow_bytes = (size_t)K / 2;
  const size_t srow_bytes = (size_t)K / 32;

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

  // activation source row of tile token t (slots past the expert's last pair
  // read that last pair's row; their results are dropped)
  auto src_row = [&](int t) -> int64_t {
    const int slot = min(m0 + t, n_e - 1);
    return (MODE == 1) ? (int64_t)(p.sorted_pairs[off_e + slot] / p.top_k)
                       : (int64_t)(off_e + slot);
  };

  // Activation staging: this thread moves 4 x 16 bytes per step, for tokens
  // 32*wv + 8*j + lane/8 (j = 0..3), landing at slot lane%8 of the token's
  // line, i.e. chunk slot ^ (t & 7) ^ ((t >> 3) & 1) of the step (the map is
  // an involution on the chunk index)
  const uint8_t* ssrc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = 32 * wv + 8 * j + (lane >> 3);
    ssrc[j] = p.a + src_row(t) * K + 16 * tile_slot(t, lane & 7);
  }
  const int sdst = (32 * wv + (lane >> 3)) * 128 + 16 * (lane & 7);  // + 1024 * j
  v4i R[2][4];
  auto stage_load = [&](int s, v4i (&r)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = *reinterpret_cast<const v4i*>(ssrc[j] + (size_t)s * 128);
  };
  auto stage_store = [&](uint8_t* buf, const v4i (&r)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<v4i*>(buf + sdst + 1024 * j) = r[j];
  };

  // token scales of the whole tile into LDS: thread tid copies half of
  // token tid/2's scale line
  {
    const int st_tok = tid >> 1, st_half = tid & 1;
    const uint8_t* src = p.a_scale + src_row(st_tok) * S + st_half * (S / 2);
    uint8_t* dst = &bsc[st_tok][st_half * (S / 2)];
    if constexpr (S == 32) {
      *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
    } else if constexpr (S == 16) {
      *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(src);
    } else {
      *reinterpret_cast<uint32_t*>(dst) = *reinterpret_cast<const uint32_t*>(src);
    }
  }

  // weight scale lines (a quarter per lane group)
  uint32_t SR[4][SD];
  {
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
  }

  v4f acc[MT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[m][t] = v4f{0.f, 0.f, 0.f, 0.f};

  v4i A[4][4];  // weight ring: [step % 4][tile]
  // (waves without weight rows load row 0 too: unconditional loads keep the
  // compiler's load counting exact)
  auto load_a = [&](int s, v4i (&a)[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) a[t] = *reinterpret_cast<const v4i*>(wptr[t] + (size_t)s * 64);
  };

  // one K step: activations from `buf`, weights from ring slot `a`; the
  // four steps of a group share one dword of token scales per sub-tile
  uint32_t sbw[MT];
  auto compute = [&](int s, const uint8_t* buf, const v4i (&a)[4]) {
    if (!wave_live) return;
    if ((s & 3) == 0) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
        sbw[m] = *reinterpret_cast<const uint32_t*>(&bsc[16 * m + col][s]);
    }
    const int src_lane = col + 16 * (s / SD);
    int sa[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint32_t w = SR[t][0];
#pragma unroll
      for (int j = 1; j < SD; ++j) w = ((s & (SD - 1)) == j) ? SR[t][j] : w;
      sa[t] = __shfl((int)w, src_lane) >> (8 * grp);
    }
    const int sh = 8 * (s & 3);
#pragma unroll
    for (int m = 0; m < MT; m += 2) {
      v8i b[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int t = 16 * (m + h) + col;
        const v4i lo = *reinterpret_cast<const v4i*>(buf + t * 128 + 16 * tile_slot(t, grp));
        const v4i hi = *reinterpret_cast<const v4i*>(buf + t * 128 + 16 * tile_slot(t, 4 + grp));
        b[h] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      mfma8_fp4_fp8(acc[m], acc[m + 1], a, b[0], b[1], sa[0], sa[1], sa[2], sa[3],
                    (int)(sbw[m] >> sh), (int)(sbw[m + 1] >> sh));
    }
  };

  // Pipeline, step s: barrier; activation loads for step s+2; compute(s)
  // from buffer s%4 and ring slot s%4; weight loads for step s+4 into that
  // slot; step s+1's activations (loaded during step s-1) written to buffer
  // (s+1)%4, last read in step s-3.  Nothing past the last step is loaded.
  uint8_t* const bufs[4] = {act0, act1, act2, act3};
  load_a(0, A[0]);
  stage_load(0, R[0]);
  load_a(1, A[1]);
  stage_load(1, R[1]);
  load_a(2, A[2]);
  load_a(3, A[3]);
  stage_store(act0, R[0]);
#define TILE_STEP(s, q)                                   \
  do {                                                    \
    lds_barrier();                                        \
    if ((s) + 2 < S) stage_load((s) + 2, R[(q) & 1]);     \
    compute((s), bufs[q], A[q]);                          \
    if ((s) + 4 < S) load_a((s) + 4, A[q]);               \
    if ((s) + 1 < S) stage_store(bufs[((q) + 1) & 3], R[((q) + 1) & 1]); \
  } while (0)
  for (int s0 = 0; s0 < S - 4; s0 += 4) {
    TILE_STEP(s0, 0);
    TILE_STEP(s0 + 1, 1);
    TILE_STEP(s0 + 2, 2);
    TILE_STEP(s0 + 3, 3);
  }
  TILE_STEP(S - 4, 0);
  TILE_STEP(S - 3, 1);
  TILE_STEP(S - 2, 2);
  TILE_STEP(S - 1, 3);
#undef TILE_STEP

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
          const float g = fminf(fmaxf(acc[m][tt][v], -lim), lim);
          const float u = fminf(fmaxf(acc[m][tt + 2][v], -lim), lim);
          const float hv = silu_f(g) * u;
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
      const float amax = fmaxf(fmaxf(red[0][tokc], red[1][tokc]), fmaxf(red[2][tokc], red[3][tokc]));
      const int ex = pow2_scale_exp(amax);
      const int slot = m0 + tokc;
      if (slot < n_e) {
        const size_t row = (size_t)(off_e + slot);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          uint32_t word = 0;
#pragma unroll
          for (int v = 0; v < 4; ++v) word |= e4m3_rne(ldexpf(acc[m][tt][v], -ex)) << (8 * v);
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
              make_float4(acc[m][t][0], acc[m][t][1], acc[m][t][2], acc[m][t][3]);
        } else {
          const uint32_t lo = f32_to_bf16(acc[m][t][0]) | (f32_to_bf16(acc[m][t][1]) << 16);
          const uint32_t hi = f32_to_bf16(acc[m][t][2]) | (f32_to_bf16(acc[m][t][3]) << 16);
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
  if (bm == 128) {
    if (a.K != 1024 && a.K != 2048 && a.K != 4096) return hipErrorInvalidValue;
    if (a.K == 4096)
      hipLaunchKernelGGL((expert_gemm_tile<MODE, 32>), dim3(grid), dim3(kGemmThreads), 0, st, a,
                         mt_max, n_tiles);
    else if (a.K == 2048)
      hipLaunchKernelGGL((expert_gemm_tile<MODE, 16>), dim3(grid), dim3(kGemmThreads), 0, st, a,
                         mt_max, n_tiles);
    else
      hipLaunchKernelGGL((expert_gemm_tile<MODE, 8>), dim3(grid), dim3(kGemmThreads), 0, st, a,
                         mt_max, n_tiles);
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
