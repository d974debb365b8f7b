// bf16 GEMMs of the layer: the router logits (the gate stays bf16: the
// PTPC-FP8 article's 排除清单 excludes *ffn.gate* from quantization) and the
// shared expert ("DeepSeek-V4-Flash-SI" card: 1 shared expert, non-expert
// weights bf16, SwiGLU clamped to +-10).
//
// C[t][n] = sum_k X[t][k] * W[n][k] with v_mfma_f32_16x16x32_bf16: weight rows
// are the A operand (lane l: row l%16, 8 consecutive K), token rows the B
// operand (lane l: token l%16, the same 8 K); fp32 accumulation.  Each wave
// owns TPW 16-row weight tiles and streams them over the whole K with 16-byte
// loads straight into operand registers; token rows (MT 16-row sub-tiles) are
// read the same way and are shared through L2.
//   EPI_F32    out[t][n] fp32 (router logits, shared down projection)
//   EPI_SWIGLU tiles 0..TPW/2-1 read w1 rows, the rest w3 rows of the same
//              columns; out[t][n] = bf16(silu(clip(g)) * clip(u))
#include "moe_internal.h"
#include "shared_splitk.h"

#include <type_traits>

namespace moe {

typedef int v4i __attribute__((ext_vector_type(4)));

template <int EPI, int TPW, int MT>
__global__ __launch_bounds__(256) void bf16_gemm_kernel(const uint16_t* __restrict__ X,
                                                        const uint16_t* __restrict__ W,
                                                        const uint16_t* __restrict__ W3,
                                                        void* __restrict__ out, int64_t M, int N,
                                                        int K, float limit) {
  constexpr int BM = 16 * MT;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  // rows (EPI_F32) or h columns (EPI_SWIGLU) covered by this wave
  constexpr int WROWS = EPI == EPI_SWIGLU ? 8 * TPW : 16 * TPW;
  const int n0 = blockIdx.x * 4 * WROWS + wv * WROWS;
  if (n0 >= N) return;  // whole wave idle; no barriers in this kernel

  const uint16_t* wp[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    int row;
    const uint16_t* base;
    if (EPI == EPI_SWIGLU) {
      row = n0 + 16 * (t % (TPW / 2)) + col;
      base = t < TPW / 2 ? W : W3;
    } else {
      row = n0 + 16 * t + col;
      base = W;
    }
    if (row >= N) row = N - 1;  // partial tile: duplicate a valid row, discarded below
    wp[t] = base + (size_t)row * K + 8 * grp;
  }
  const uint16_t* xp[MT];
  bool xv[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int64_t r = m0 + 16 * m + col;
    xv[m] = r < M;
    xp[m] = X + (size_t)(xv[m] ? r : 0) * K + 8 * grp;
  }

  v4f acc[TPW][MT];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[t][m] = v4f{0.f, 0.f, 0.f, 0.f};

  const int steps = K / 32;
  uint4 a_cur[TPW], a_nxt[TPW], b_cur[MT], b_nxt[MT];
#pragma unroll
  for (int t = 0; t < TPW; ++t) a_cur[t] = *reinterpret_cast<const uint4*>(wp[t]);
#pragma unroll
  for (int m = 0; m < MT; ++m)
    b_cur[m] = xv[m] ? *reinterpret_cast<const uint4*>(xp[m]) : make_uint4(0, 0, 0, 0);
  for (int s = 0; s < steps; ++s) {
    if (s + 1 < steps) {
#pragma unroll
      for (int t = 0; t < TPW; ++t)
        a_nxt[t] = *reinterpret_cast<const uint4*>(wp[t] + (size_t)(s + 1) * 32);
#pragma unroll
      for (int m = 0; m < MT; ++m)
        b_nxt[m] = xv[m] ? *reinterpret_cast<const uint4*>(xp[m] + (size_t)(s + 1) * 32)
                         : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[t][m] = mfma_bf16(a_cur[t], b_cur[m], acc[t][m]);
#pragma unroll
    for (int t = 0; t < TPW; ++t) a_cur[t] = a_nxt[t];
#pragma unroll
    for (int m = 0; m < MT; ++m) b_cur[m] = b_nxt[m];
  }

  // D layout: lane l holds D[4*(l/16)+v][l%16] = C[token l%16][row 4*(l/16)+v]
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int64_t r = m0 + 16 * m + col;
    if (r >= M) continue;
    if (EPI == EPI_F32) {
      float* o = static_cast<float*>(out) + (size_t)r * N;
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int c = n0 + 16 * t + 4 * grp;
        if ((N & 3) == 0) {
          if (c < N)
            *reinterpret_cast<float4*>(o + c) =
                make_float4(acc[t][m][0], acc[t][m][1], acc[t][m][2], acc[t][m][3]);
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (c + v < N) o[c + v] = acc[t][m][v];
        }
      }
    } else {
      uint16_t* o = static_cast<uint16_t*>(out) + (size_t)r * N;
#pragma unroll
      for (int t = 0; t < TPW / 2; ++t) {
        const int c = n0 + 16 * t + 4 * grp;
        uint32_t hv[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float g = fminf(fmaxf(acc[t][m][v], -limit), limit);
          const float u = fminf(fmaxf(acc[t + TPW / 2][m][v], -limit), limit);
          hv[v] = f32_to_bf16(g / (1.0f + expf(-g)) * u);
        }
        if (c < N) *reinterpret_cast<uint2*>(o + c) = make_uint2(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Decode-sized variant (M <= 64 tokens, K a multiple of 1024): the weights
// are the whole traffic, so parallelism comes from splitting K.  A
// workgroup of 8 waves owns 16 weight rows (EPI_F32) or 16 h columns, i.e.
// one w1 tile and one w3 tile (EPI_SWIGLU), and all M tokens; wave w streams
// the K slice [w K/8, (w+1) K/8) with a four-step register ring, and the
// eight partial sums are added in LDS in a fixed order (a three-level tree),
// so results do not depend on timing.
// ---------------------------------------------------------------------------
template <int EPI, int MT>
__global__ __launch_bounds__(512) void bf16_skinny_kernel(const uint16_t* __restrict__ X,
                                                          const uint16_t* __restrict__ W,
                                                          const uint16_t* __restrict__ W3,
                                                          void* __restrict__ out, int M, int N,
                                                          int K, float limit) {
  constexpr int NT = EPI == EPI_SWIGLU ? 2 : 1;
  constexpr int NACC = NT * MT * 4;
  __shared__ float red[4][NACC][64];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int KW = K / 8;
  const int k0 = wv * KW;
  const int steps = KW / 32;  // multiple of 4

  const uint16_t* wp[NT];
  const int row = min(n0 + col, N - 1);
#pragma unroll
  for (int t = 0; t < NT; ++t) wp[t] = (t == 0 ? W : W3) + (size_t)row * K + k0 + 8 * grp;
  const uint16_t* xp[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) xp[m] = X + (size_t)min(16 * m + col, M - 1) * K + k0 + 8 * grp;

  v4f acc[NT][MT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[t][m] = v4f{0.f, 0.f, 0.f, 0.f};

  uint4 A[4][NT], B[4][MT];
  auto load = [&](int s, uint4 (&a)[NT], uint4 (&b)[MT]) {
#pragma unroll
    for (int t = 0; t < NT; ++t) a[t] = *reinterpret_cast<const uint4*>(wp[t] + (size_t)s * 32);
#pragma unroll
    for (int m = 0; m < MT; ++m) b[m] = *reinterpret_cast<const uint4*>(xp[m] + (size_t)s * 32);
  };
  auto four = [&](auto loads, int s0) {
    constexpr bool LOADS = decltype(loads)::value;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[t][m] = mfma_bf16(A[d][t], B[d][m], acc[t][m]);
      if constexpr (LOADS) {
        __builtin_amdgcn_sched_barrier(0);
        load(s0 + d + 4, A[d], B[d]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  using yes = std::integral_constant<bool, true>;
  using no = std::integral_constant<bool, false>;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    load(d, A[d], B[d]);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int s0 = 0; s0 < steps - 4; s0 += 4) four(yes{}, s0);
  four(no{}, steps - 4);

  // deterministic tree: 8 -> 4 -> 2 -> 1 partial sums
  auto put = [&](int slot) {
    int i = 0;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[slot][i++][lane] = acc[t][m][v];
  };
  auto add = [&](int slot) {
    int i = 0;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[t][m][v] += red[slot][i++][lane];
  };
  for (int half = 4; half >= 1; half >>= 1) {
    if (wv >= half && wv < 2 * half) put(wv - half);
    __syncthreads();
    if (wv < half) add(wv);
    __syncthreads();
  }
  if (wv != 0) return;

  // D layout: lane l holds D[4*(l/16)+v][l%16] = C[token l%16][row 4*(l/16)+v]
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int r = 16 * m + col;
    if (r >= M) continue;
    const int c = n0 + 4 * grp;
    if (EPI == EPI_F32) {
      float* o = static_cast<float*>(out) + (size_t)r * N;
      if ((N & 3) == 0) {
        if (c < N) *reinterpret_cast<float4*>(o + c) = make_float4(acc[0][m][0], acc[0][m][1], acc[0][m][2], acc[0][m][3]);
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (c + v < N) o[c + v] = acc[0][m][v];
      }
    } else {
      uint16_t* o = static_cast<uint16_t*>(out) + (size_t)r * N;
      uint32_t hv[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float g = fminf(fmaxf(acc[0][m][v], -limit), limit);
        const float u = fminf(fmaxf(acc[1][m][v], -limit), limit);
        hv[v] = f32_to_bf16(g / (1.0f + expf(-g)) * u);
      }
      if (c < N) *reinterpret_cast<uint2*>(o + c) = make_uint2(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16));
    }
  }
}

template <int EPI>
static hipError_t launch_skinny(const uint16_t* X, const uint16_t* W, const uint16_t* W3, void* out,
                                int M, int N, int K, float limit, hipStream_t st) {
  const dim3 grid((unsigned)((N + 15) / 16));
  switch ((M + 15) / 16) {
    case 1: hipLaunchKernelGGL((bf16_skinny_kernel<EPI, 1>), grid, dim3(512), 0, st, X, W, W3, out, M, N, K, limit); break;
    case 2: hipLaunchKernelGGL((bf16_skinny_kernel<EPI, 2>), grid, dim3(512), 0, st, X, W, W3, out, M, N, K, limit); break;
    case 3: hipLaunchKernelGGL((bf16_skinny_kernel<EPI, 3>), grid, dim3(512), 0, st, X, W, W3, out, M, N, K, limit); break;
    default: hipLaunchKernelGGL((bf16_skinny_kernel<EPI, 4>), grid, dim3(512), 0, st, X, W, W3, out, M, N, K, limit); break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Decode-sized shared expert on its own stream (the split-K bodies of
// shared_splitk.h): the skinny kernel above gives every workgroup all of K
// for 16 weight rows, so the token rows are re-read from L2 twice (up) or four
// times (down) per weight byte and only 128 workgroups run the up projection;
// split-K runs 256 workgroups at H = 4096, I = 2048 (up: 64 h columns x 8
// slices, down: 64 rows x 4 slices), the token slice read once per workgroup.
// ---------------------------------------------------------------------------
template <int EPI, int RW>
__global__ __launch_bounds__(512) void bf16_splitk_kernel(const uint16_t* __restrict__ X,
                                                          const uint16_t* __restrict__ W,
                                                          const uint16_t* __restrict__ W3,
                                                          float* __restrict__ P, int M, int N,
                                                          int K) {
  __shared__ uint4 xs[64][64];
  shared_splitk_body<EPI, 8, RW>(X, W, W3, P, M, N, K, blockIdx.x, blockIdx.y, xs);
}

__global__ __launch_bounds__(256) void splitk_swiglu_kernel(const float* __restrict__ P, int S,
                                                            int M, int N, float limit,
                                                            uint16_t* __restrict__ h) {
  shared_swiglu_body(P, S, M, N, limit, h, blockIdx.x * 256 + threadIdx.x);
}

__global__ __launch_bounds__(256) void splitk_sum_kernel(const float* __restrict__ P, int S, int M,
                                                         int N, float* __restrict__ y) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= M * (N / 4)) return;
  const size_t stride = (size_t)M * N;
  const float* p = P + 4 * (size_t)i;
  float4 a = *reinterpret_cast<const float4*>(p);
  for (int s = 1; s < S; ++s) {
    const float4 b = *reinterpret_cast<const float4*>(p + s * stride);
    a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
  }
  *reinterpret_cast<float4*>(y + 4 * (size_t)i) = a;
}

// Shared-expert up projection riding in the router launch (blocks = 0: none).
struct SharedUpArgs {
  const uint16_t* w1;
  const uint16_t* w3;
  float* part;
  int I;
  int blocks;
};

// ---------------------------------------------------------------------------
// Router logits of a small batch (M <= 64 tokens): the gate matrix is only
// E x H bf16 (2 MB at E = 256), so the whole read must be in flight at once.
// Workgroup (nb, ks) of 8 waves owns 16 experts and the K slice
// [ks K/KS, (ks+1) K/KS); each wave loads its 1/8 of that slice in one go
// (no loop), the 8 partial sums meet in a fixed-order LDS tree, and the
// workgroup writes partial[ks][t][e].  The top-k kernel adds the KS partials
// in ks order, so the logits do not depend on timing.  With q, the same
// workgroups also quantize x to FP8 (the layer's next step, which reads the
// same rows): 32 blocks of 128 per workgroup and pass, one launch fewer.
// Workgroups are numbered ks * ceil(N / 16) + nb; with sh.blocks > 0 the
// workgroups after the router's run the shared expert's split-K up
// projection (it reads the same x), which then needs no launch of its own.
// ---------------------------------------------------------------------------
template <int MT, int STEPS>
__global__ __launch_bounds__(512) void router_splitk_kernel(const uint16_t* __restrict__ X,
                                                            const uint16_t* __restrict__ W,
                                                            float* __restrict__ partial, int M,
                                                            int N, int K, int KS,
                                                            uint8_t* __restrict__ q,
                                                            uint8_t* __restrict__ qscale,
                                                            SharedUpArgs sh) {
  constexpr int NACC = MT * 4;
  __shared__ uint4 lds[64][64];   // the router's reduction tree, or the split-K token slice
  const int gx = (N + 15) / 16;
  const int rb = blockIdx.x;
  if (rb >= gx * KS) {
    const int b = rb - gx * KS, nbx = sh.I / shared_splitk_rows<EPI_SWIGLU, 4>();
    shared_splitk_body<EPI_SWIGLU, 8, 4>(X, sh.w1, sh.w3, sh.part, M, sh.I, K, b % nbx, b / nbx,
                                         lds);
    return;
  }
  float (*red)[NACC][64] = reinterpret_cast<float (*)[NACC][64]>(&lds[0][0]);
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int n0 = (rb % gx) * 16;
  const int ks = rb / gx;
  if (q) {
    const int64_t n_blocks = (int64_t)M * (K / 128);
    const int64_t stride = (int64_t)gx * KS * 32;
    for (int64_t b = (int64_t)rb * 32 + (threadIdx.x >> 4); b < n_blocks; b += stride)
      quant_act_block(X, b, n_blocks, threadIdx.x & 15, q, qscale);
  }
  const int k0 = ks * (K / KS) + wv * STEPS * 32;
  const uint16_t* wp = W + (size_t)min(n0 + col, N - 1) * K + k0 + 8 * grp;
  uint4 A[STEPS], B[STEPS][MT];
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    A[s] = *reinterpret_cast<const uint4*>(wp + s * 32);
#pragma unroll
    for (int m = 0; m < MT; ++m)
      B[s][m] = *reinterpret_cast<const uint4*>(X + (size_t)min(16 * m + col, M - 1) * K + k0 +
                                                8 * grp + s * 32);
  }
  v4f acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < STEPS; ++s)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = mfma_bf16(A[s], B[s][m], acc[m]);
  for (int half = 4; half >= 1; half >>= 1) {
    if (wv >= half && wv < 2 * half) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[wv - half][4 * m + v][lane] = acc[m][v];
    }
    __syncthreads();
    if (wv < half) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[m][v] += red[wv][4 * m + v][lane];
    }
    __syncthreads();
  }
  if (wv != 0) return;
  float* out = partial + (size_t)ks * M * N;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int r = 16 * m + col;
    if (r >= M) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int c = n0 + 4 * grp + v;
      if (c < N) out[(size_t)r * N + c] = acc[m][v];
    }
  }
}

// ---------------------------------------------------------------------------
// Large-M tile kernel: 128 tokens x 128 weight rows per workgroup, K in steps
// of 64.  Both operands go through double-buffered LDS (each row's 128-byte
// step line with its 16-byte chunk c at slot c ^ (row & 7), so that the
// 16-byte operand reads of 16 consecutive rows hit distinct banks); the four
// waves split the tile 2 x 2 (64 tokens x 64 rows each, 32 MFMAs per step).
// Lines are loaded into registers two steps ahead (two register sets, the
// K loop unrolled by two so that the set is a compile-time choice: 3-6%
// over one step ahead) and written to the other buffer at the end of the
// step before theirs; one barrier per step.
//   EPI_F32    rows n0..n0+127 of W, out[t][n] fp32
//   EPI_SWIGLU LDS rows 0..63 = w1 rows c0..c0+63, rows 64..127 = w3 rows of
//              the same columns; wave (wm, wn) takes columns c0 + 32 wn ..
//              +31 of both, so g and u of an output meet in one lane.
// Requires N % 128 == 0 (EPI_F32) or N % 64 == 0 (EPI_SWIGLU), K % 64 == 0.
// Split K (EPI_F32): workgroup z covers K elements z*kc .. z*kc + kc - 1
// (kc % 64 == 0) and writes its partial sums to out + z*M*N.
// ---------------------------------------------------------------------------
constexpr int kBfTileLine = 128;            // bytes of a row's K step (64 bf16)
constexpr int kBfTileBuf = 128 * kBfTileLine;

template <int EPI>
__global__ __launch_bounds__(256, 2) void bf16_tile_kernel(const uint16_t* __restrict__ X,
                                                           const uint16_t* __restrict__ W,
                                                           const uint16_t* __restrict__ W3,
                                                           void* __restrict__ out, int64_t M, int N,
                                                           int K, int kc, float limit) {
  __shared__ __attribute__((aligned(1024))) uint8_t As[2][kBfTileBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t Bs[2][kBfTileBuf];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int wm = wv & 1, wn = wv >> 1;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.y * 128;
  const int nb = blockIdx.x;
  const size_t row_bytes = (size_t)K * 2;

  // staging: load j of thread tid moves chunk c = tid % 8 of row
  // r = tid / 8 + 32 j of both operands (eight threads cover a row's 128-byte
  // step line, so one wave's load touches 8 lines), chunk c to LDS slot
  // c ^ (r & 7)
  const int sc = tid & 7;
  const size_t kofs = (size_t)blockIdx.z * kc * 2 + 16 * sc;   // this split's first K byte
  const uint8_t* wsrc[4];
  const uint8_t* xsrc[4];
  uint32_t soff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = (tid >> 3) + 32 * j;
    if (EPI == EPI_SWIGLU) {
      const int c = nb * 64 + (r & 63);
      wsrc[j] = reinterpret_cast<const uint8_t*>(r < 64 ? W : W3) + (size_t)c * row_bytes + kofs;
    } else {
      wsrc[j] = reinterpret_cast<const uint8_t*>(W) + (size_t)(nb * 128 + r) * row_bytes + kofs;
    }
    const int64_t xr = m0 + r < M ? m0 + r : M - 1;   // rows past M repeat row M-1 (dropped)
    xsrc[j] = reinterpret_cast<const uint8_t*>(X) + (size_t)xr * row_bytes + kofs;
    soff[j] = r * kBfTileLine + 16 * (sc ^ (r & 7));
  }
  // (native vector types: loops of struct copies would go through memory)
  // two staging sets: step s's lines in set s & 1, loaded two steps ahead
  v4i ga[2][4], gb[2][4];
  auto gload = [&](int s, auto setc) {
    constexpr int SET = decltype(setc)::value;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ga[SET][j] = *reinterpret_cast<const v4i*>(wsrc[j] + (size_t)s * kBfTileLine);
      gb[SET][j] = *reinterpret_cast<const v4i*>(xsrc[j] + (size_t)s * kBfTileLine);
    }
  };
  auto lstore = [&](auto bufc) {   // buffer BUF from set BUF
    constexpr int BUF = decltype(bufc)::value;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      *reinterpret_cast<v4i*>(&As[BUF][soff[j]]) = ga[BUF][j];
      *reinterpret_cast<v4i*>(&Bs[BUF][soff[j]]) = gb[BUF][j];
    }
  };

  // operand rows of this wave in the LDS tile
  int arow[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
    arow[t] = EPI == EPI_SWIGLU ? (t < 2 ? 32 * wn + 16 * t : 64 + 32 * wn + 16 * (t - 2))
                                : 64 * wn + 16 * t;
  const int lo = 16 * (grp ^ (col & 7));      // chunk grp of a row line (row & 7 == col & 7)
  const int hi = lo ^ 64;                     // chunk grp + 4

  v4f acc[4][4];   // [weight tile][token sub-tile]
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[t][m] = v4f{0.f, 0.f, 0.f, 0.f};

  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  const int steps = kc / 64;
  // step s from buffer BUF = s & 1 (compile-time in the unrolled pair): the
  // lines of step s + 2 are loaded into set BUF once step s's lines (that
  // set) are in LDS, and step s + 1's (set BUF ^ 1) are written to the other
  // buffer at the end
  auto step = [&](int s, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    __syncthreads();                  // buffer BUF written, buffer BUF^1 free
    if (s + 2 < steps) gload(s + 2, bufc);
    bf16x8 a0[4], a1[4], b0[4], b1[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint8_t* r = &As[BUF][(arow[t] + col) * kBfTileLine];
      a0[t] = *reinterpret_cast<const bf16x8*>(r + lo);
      a1[t] = *reinterpret_cast<const bf16x8*>(r + hi);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint8_t* r = &Bs[BUF][(64 * wm + 16 * m + col) * kBfTileLine];
      b0[m] = *reinterpret_cast<const bf16x8*>(r + lo);
      b1[m] = *reinterpret_cast<const bf16x8*>(r + hi);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        acc[t][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[t], b0[m], acc[t][m], 0, 0, 0);
        acc[t][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[t], b1[m], acc[t][m], 0, 0, 0);
      }
    if (s + 1 < steps) lstore(std::integral_constant<int, BUF ^ 1>{});
  };
  gload(0, C0{});
  if (steps > 1) gload(1, C1{});
  lstore(C0{});
  int s = 0;
  for (; s + 1 < steps; s += 2) {
    step(s, C0{});
    step(s + 1, C1{});
  }
  if (s < steps) step(s, C0{});

  // D layout: lane l holds D[4*(l/16)+v][l%16] = C[token l%16][row 4*(l/16)+v]
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int64_t r = m0 + 64 * wm + 16 * m + col;
    if (r >= M) continue;
    if (EPI == EPI_F32) {
      float* o = static_cast<float*>(out) + (size_t)blockIdx.z * M * N + (size_t)r * N;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int c = nb * 128 + 64 * wn + 16 * t + 4 * grp;
        *reinterpret_cast<float4*>(o + c) =
            make_float4(acc[t][m][0], acc[t][m][1], acc[t][m][2], acc[t][m][3]);
      }
    } else {
      uint16_t* o = static_cast<uint16_t*>(out) + (size_t)r * N;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int c = nb * 64 + 32 * wn + 16 * t + 4 * grp;
        uint32_t hv[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float g = fminf(fmaxf(acc[t][m][v], -limit), limit);
          const float u = fminf(fmaxf(acc[t + 2][m][v], -limit), limit);
          hv[v] = f32_to_bf16(g / (1.0f + expf(-g)) * u);
        }
        *reinterpret_cast<uint2*>(o + c) = make_uint2(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16));
      }
    }
  }
}

// tokens from which the tile kernel is used
constexpr int64_t kBfTileMinM = 256;

template <int EPI, int TPW>
static hipError_t launch_bf16(const uint16_t* X, const uint16_t* W, const uint16_t* W3, void* out,
                              int64_t M, int N, int K, float limit, hipStream_t st) {
  if (M == 0) return hipSuccess;
  if (M <= 64 && K % 1024 == 0) return launch_skinny<EPI>(X, W, W3, out, (int)M, N, K, limit, st);
  if (M >= kBfTileMinM && K % 64 == 0 && N % (EPI == EPI_SWIGLU ? 64 : 128) == 0) {
    const dim3 grid((unsigned)(N / (EPI == EPI_SWIGLU ? 64 : 128)), (unsigned)((M + 127) / 128));
    hipLaunchKernelGGL((bf16_tile_kernel<EPI>), grid, dim3(256), 0, st, X, W, W3, out, M, N, K, K,
                       limit);
    return hipGetLastError();
  }
  constexpr int WROWS = EPI == EPI_SWIGLU ? 8 * TPW : 16 * TPW;
  const unsigned gx = (unsigned)((N + 4 * WROWS - 1) / (4 * WROWS));
  if (M <= 16) {
    hipLaunchKernelGGL((bf16_gemm_kernel<EPI, TPW, 1>), dim3(gx, (unsigned)((M + 15) / 16)),
                       dim3(256), 0, st, X, W, W3, out, M, N, K, limit);
  } else {
    hipLaunchKernelGGL((bf16_gemm_kernel<EPI, TPW, 4>), dim3(gx, (unsigned)((M + 63) / 64)),
                       dim3(256), 0, st, X, W, W3, out, M, N, K, limit);
  }
  return hipGetLastError();
}

hipError_t launch_router_gemm(const uint16_t* x, const uint16_t* wg, float* logits, int64_t T,
                              int H, int E, hipStream_t st) {
  return launch_bf16<EPI_F32, 1>(x, wg, nullptr, logits, T, E, H, 0.f, st);
}

// Large batches: the tile kernel has only (E / 128) x (T / 128) workgroups
// (64 for T = 4096, E = 256), so the K loop is split until about 512
// workgroups run; the partial sums are added in split order by the top-k
// kernel.
int router_tile_splits(int64_t T, int H, int E) {
  if (T < kBfTileMinM || H % 64 || E % 128) return 1;
  const int64_t base = (int64_t)(E / 128) * ((T + 127) / 128);
  int ks = 1;
  while (ks < 8 && base * ks < 512 && H % (2 * ks * 64) == 0) ks *= 2;
  return ks;
}

hipError_t launch_router_tile_split(const uint16_t* x, const uint16_t* wg, float* partial,
                                    int64_t T, int H, int E, int splits, hipStream_t st) {
  const dim3 grid((unsigned)(E / 128), (unsigned)((T + 127) / 128), (unsigned)splits);
  hipLaunchKernelGGL((bf16_tile_kernel<EPI_F32>), grid, dim3(256), 0, st, x, wg, nullptr, partial,
                     T, E, H, H / splits, 0.f);
  return hipGetLastError();
}

int router_splits(int64_t T, int H) {
  // per-wave K steps of 32: 1, 2 or 4 are instantiated
  const int unit = kRouterSplits * 8 * 32;
  const int steps = H / unit;
  const bool ok = H % unit == 0 && (steps == 1 || steps == 2 || steps == 4);
  return (T >= 1 && T <= 64 && ok) ? kRouterSplits : 1;
}

hipError_t launch_router_partial(const uint16_t* x, const uint16_t* wg, float* partial, int64_t T,
                                 int H, int E, uint8_t* q, uint8_t* scale, const SharedFused* sf,
                                 hipStream_t st) {
  const int KS = kRouterSplits;
  const int steps = H / KS / 8 / 32;   // per wave
  SharedUpArgs sh{};
  if (sf) {
    sh = SharedUpArgs{sf->w1, sf->w3, sf->part, sf->I,
                      (sf->I / shared_splitk_rows<EPI_SWIGLU, 4>()) * (H / kSharedSplitK)};
  }
  const dim3 grid((unsigned)((E + 15) / 16 * KS + sh.blocks));
  const int M = (int)T;
#define MOE_ROUTER_LAUNCH(MT, ST) \
  hipLaunchKernelGGL((router_splitk_kernel<MT, ST>), grid, dim3(512), 0, st, x, wg, partial, M, E, H, KS, \
                     q, scale, sh)
  const int mt = (M + 15) / 16;
  if (steps == 2) {
    if (mt == 1) MOE_ROUTER_LAUNCH(1, 2); else if (mt == 2) MOE_ROUTER_LAUNCH(2, 2);
    else if (mt == 3) MOE_ROUTER_LAUNCH(3, 2); else MOE_ROUTER_LAUNCH(4, 2);
  } else if (steps == 4) {
    if (mt == 1) MOE_ROUTER_LAUNCH(1, 4); else if (mt == 2) MOE_ROUTER_LAUNCH(2, 4);
    else if (mt == 3) MOE_ROUTER_LAUNCH(3, 4); else MOE_ROUTER_LAUNCH(4, 4);
  } else {  // steps == 1 (router_splits admits only 1, 2, 4)
    if (mt == 1) MOE_ROUTER_LAUNCH(1, 1); else if (mt == 2) MOE_ROUTER_LAUNCH(2, 1);
    else if (mt == 3) MOE_ROUTER_LAUNCH(3, 1); else MOE_ROUTER_LAUNCH(4, 1);
  }
#undef MOE_ROUTER_LAUNCH
  return hipGetLastError();
}

bool shared_split_ok(int64_t T, int H, int I) {
  return T >= 1 && T <= 64 && H % kSharedSplitK == 0 && I % kSharedSplitK == 0;
}

int64_t shared_part_floats(int64_t T, int H, int I) {
  if (!shared_split_ok(T, H, I)) return 0;
  const int64_t up = (int64_t)(H / kSharedSplitK) * T * 2 * I;
  const int64_t down = (int64_t)(I / kSharedSplitK) * T * H;
  return up > down ? up : down;
}

hipError_t launch_shared_up(const uint16_t* x, const uint16_t* w1, const uint16_t* w3,
                            uint16_t* h, float* part, int64_t T, int H, int I, float limit,
                            hipStream_t st) {
  if (!part || !shared_split_ok(T, H, I))
    return launch_bf16<EPI_SWIGLU, 2>(x, w1, w3, h, T, I, H, limit, st);
  const int S = H / kSharedSplitK, M = (int)T;
  hipLaunchKernelGGL((bf16_splitk_kernel<EPI_SWIGLU, 4>), dim3((unsigned)(I / 64), (unsigned)S),
                     dim3(512), 0, st, x, w1, w3, part, M, I, H);
  hipLaunchKernelGGL(splitk_swiglu_kernel, dim3((unsigned)((M * (I / 4) + 255) / 256)), dim3(256),
                     0, st, part, S, M, I, limit, h);
  return hipGetLastError();
}

hipError_t launch_shared_down(const uint16_t* h, const uint16_t* w2, float* ysh, float* part,
                              int64_t T, int H, int I, hipStream_t st) {
  if (!part || !shared_split_ok(T, H, I))
    return launch_bf16<EPI_F32, 1>(h, w2, nullptr, ysh, T, H, I, 0.f, st);
  const int S = I / kSharedSplitK, M = (int)T;
  hipLaunchKernelGGL((bf16_splitk_kernel<EPI_F32, 2>), dim3((unsigned)(H / 64), (unsigned)S),
                     dim3(512), 0, st, h, w2, nullptr, part, M, H, I);
  hipLaunchKernelGGL(splitk_sum_kernel, dim3((unsigned)((M * (H / 4) + 255) / 256)), dim3(256), 0,
                     st, part, S, M, H, ysh);
  return hipGetLastError();
}

}  // namespace moe
