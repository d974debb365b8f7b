// Internal declarations shared by the HIP sources of the library: kernel
// launchers (host functions, one per kernel family) and small device helpers.
// Nothing here is part of the public C ABI (include/moe_fp4.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t h16) {
  return __uint_as_float(h16 << 16);
}

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Smallest integer e with a <= 448 * 2^e for a finite a >= 0, clamped to
// [-127, 127]; a == 0 (and any a below 2^-126) gives -127.  Exact: with
// a = 1.m * 2^(E-127), 448 = 1.75 * 2^8, so e = E - 135 when the mantissa is
// at most 0.75 (0x600000) and E - 134 otherwise.
__device__ __forceinline__ int pow2_scale_exp(float a) {
  uint32_t u = __float_as_uint(a);
  int E = (int)(u >> 23);
  if (E == 0) return -127;
  int e = ((u & 0x7FFFFFu) <= 0x600000u) ? E - 135 : E - 134;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// E4M3FN code of s, |s| <= 448, round to nearest even, sign kept (software).
__device__ __forceinline__ uint32_t e4m3_rne(float s) {
  uint32_t u = __float_as_uint(s);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a >= 0x3C800000u) {               // |s| >= 2^-6: normal E4M3 range
    uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
    code = r - (120u << 3);             // rebias 127 -> 7
    code = code > 0x7Eu ? 0x7Eu : code;
  } else {                              // subnormal step 2^-9
    code = (uint32_t)rintf(__uint_as_float(a) * 512.0f);
  }
  return code | sign;
}

// E4M3FN codes of four floats with |x| <= 448 in bytes 0..3, by the gfx950
// conversion instruction: round to nearest even, sign kept -- the same code
// as e4m3_rne for every float of that range (compared exhaustively on the
// device).
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}
// ... of x[0..3] * 2^-ex (x a float[4] or a 4-vector)
template <class V>
__device__ __forceinline__ uint32_t e4m3x4_exp(const V& x, int ex) {
  return e4m3x4(ldexpf(x[0], -ex), ldexpf(x[1], -ex), ldexpf(x[2], -ex), ldexpf(x[3], -ex));
}
__device__ __forceinline__ uint32_t e4m3x1(float a) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, 0.f, 0, false) & 0xFFu;
}

// SwiGLU's gate, silu(g) = g / (1 + e^-g), in fp32 with the hardware
// exponential and reciprocal (a few ulp; g -> -inf gives -0, g -> +inf g).
__device__ __forceinline__ float silu_fast(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// x clamped to [-lim, lim] (lim > 0, +inf allowed) in one instruction.
__device__ __forceinline__ float clamp_sym(float x, float lim) {
  return __builtin_amdgcn_fmed3f(x, -lim, lim);
}

// Load of bytes that are read exactly once per call (streamed weights, the
// combine's expert rows): a non-temporal global load (the nt bit).
// Measured on MI355X: a 2 GiB read in 1 KB-contiguous wave loads streams at
// 6.2-6.3 TB/s with ordinary loads and 7.0-7.1 TB/s with nt; loads of 8 rows
// x 128 bytes (whole lines) 5.7 -> 6.5 TB/s; but loads that take half of
// each 128-byte line (the other half by a later load) drop from 5.4 to 4.3
// TB/s with nt.  So only loads that cover whole lines use it.
template <class T>
__device__ __forceinline__ T wload(const void* p) {
  return __builtin_nontemporal_load((const __attribute__((address_space(1))) T*)p);
}
__device__ __forceinline__ uint4 wload16(const void* p) {
  typedef unsigned u4v __attribute__((ext_vector_type(4)));
  const u4v v = wload<u4v>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Two line loads of a 16-row weight tile: x0 lane (g, c) holds row c % 8,
// x1 lane (g, c) row 8 + c % 8, both at bytes 64 * (c / 8) + 16 * g of the
// rows' 128-byte line (K steps s, s + 1 of a 4-bit operand; bytes 0-63 and
// 64-127 of one step of an 8-bit one).  The MFMA operand of step s needs row
// c, bytes 16 * g in lane (g, c); that of step s + 1 row c, bytes 64 + 16 * g.
// So step s is x0's lanes 0-7 of each 16-lane row with x1's lanes 0-7 moved
// up by 8, and step s + 1 is x1's lanes 8-15 with x0's lanes 8-15 moved down
// by 8: one DPP row shift per dword, the bank mask picking the moved half.
// V: any 4 x 32-bit vector with .x .y .z .w.
constexpr int kDppRowShr8 = 0x118, kDppRowShl8 = 0x108;
__device__ __forceinline__ uint32_t dpp_up8(uint32_t keep, uint32_t from) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)keep, (int)from, kDppRowShr8, 0xF, 0xC, false);
}
__device__ __forceinline__ uint32_t dpp_down8(uint32_t keep, uint32_t from) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)keep, (int)from, kDppRowShl8, 0xF, 0x3, false);
}
template <class V>
__device__ __forceinline__ void line_pair_to_steps(V& x0, V& x1) {
  V s0 = x0, s1 = x1;
  s0.x = dpp_up8(x0.x, x1.x); s0.y = dpp_up8(x0.y, x1.y);
  s0.z = dpp_up8(x0.z, x1.z); s0.w = dpp_up8(x0.w, x1.w);
  s1.x = dpp_down8(x1.x, x0.x); s1.y = dpp_down8(x1.y, x0.y);
  s1.z = dpp_down8(x1.z, x0.z); s1.w = dpp_down8(x1.w, x0.w);
  x0 = s0;
  x1 = s1;
}

// FP8 E4M3 quantization of the 128-element block blk of a bf16 array (one
// power-of-two scale per block, smallest with amax <= 448 * 2^e): 16 lanes
// (sub = 0..15, consecutive lanes of one wave) take 8 elements each.  Blocks
// at or past n_blocks compute on zeros and store nothing.
__device__ __forceinline__ void quant_act_block(const uint16_t* __restrict__ x, int64_t blk,
                                                int64_t n_blocks, int sub, uint8_t* __restrict__ q,
                                                uint8_t* __restrict__ scale) {
  const bool live = blk < n_blocks;
  uint4 raw = make_uint4(0, 0, 0, 0);
  if (live) raw = *reinterpret_cast<const uint4*>(x + blk * 128 + sub * 8);
  float v[8];
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
    v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  // reduce over the 16 lanes of the block (xor partners stay inside the group)
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const int e = pow2_scale_exp(amax);
  const uint32_t lo = e4m3x4(ldexpf(v[0], -e), ldexpf(v[1], -e), ldexpf(v[2], -e), ldexpf(v[3], -e));
  const uint32_t hi = e4m3x4(ldexpf(v[4], -e), ldexpf(v[5], -e), ldexpf(v[6], -e), ldexpf(v[7], -e));
  if (live) {
    *reinterpret_cast<uint2*>(q + blk * 128 + sub * 8) = make_uint2(lo, hi);
    if (sub == 0) scale[blk] = (uint8_t)(e + 127);
  }
}

// ---------------------------------------------------------------------------
// Tiling constants of the grouped expert GEMMs
// ---------------------------------------------------------------------------
constexpr int kGemmThreads = 256;     // 4 waves
constexpr int kG1Cols = 128;          // h columns per GEMM1 workgroup (one FP8 block)
constexpr int kG2Rows = 256;          // output columns per GEMM2 workgroup
constexpr int kMaxExperts = 512;      // largest expert count a configuration may have

// ---------------------------------------------------------------------------
// Launchers (return hipGetLastError() after enqueueing)
// ---------------------------------------------------------------------------

hipError_t launch_quant_act(const uint16_t* x, int64_t rows, int cols, uint8_t* q,
                            uint8_t* scale, hipStream_t st);

// Decode-sized shared expert carried by the routing launches of moe_layer
// (score routing through the split-K router, shared_split_ok(T, H, I), and
// P <= kFusedMaxPairs): the router launch also runs the split-K up
// projection, the top-k launch adds its slices and applies the clamped
// SwiGLU into h, the permutation launch runs the split-K down projection into
// part, and the combine adds the I / 512 down slices.  One stream, no fork.
struct SharedFused {
  const uint16_t* w1;   // [I, H] bf16
  const uint16_t* w3;   // [I, H] bf16
  const uint16_t* w2;   // [H, I] bf16
  uint16_t* h;          // [M, I] bf16
  float* part;          // shared_part_floats(M, H, I) floats
  int M, H, I;
  float limit;
};

// logits[t, e] = sum_h x[t, h] * wg[e, h]  (bf16 in, fp32 out)
hipError_t launch_router_gemm(const uint16_t* x, const uint16_t* wg, float* logits, int64_t T,
                              int H, int E, hipStream_t st);

// Router logits of a small batch as kRouterSplits partial sums over K:
// partial[ks][t][e]; router_splits() says whether this path applies (T <= 64
// and H a multiple of kRouterSplits * 512), else it returns 1.
constexpr int kRouterSplits = 8;
int router_splits(int64_t T, int H);
// With q (may be null) the same launch also quantizes x to q / scale (as
// launch_quant_act); with sf (may be null) it also runs the shared expert's
// split-K up projection into sf->part.
hipError_t launch_router_partial(const uint16_t* x, const uint16_t* wg, float* partial, int64_t T,
                                 int H, int E, uint8_t* q, uint8_t* scale, const SharedFused* sf,
                                 hipStream_t st);
// Large batches (T >= 256, H % 64 == 0, E % 128 == 0): the bf16 tile GEMM
// with K split router_tile_splits(T, H, E) ways (1 = no split), partial sums
// partial[ks][t][e].
int router_tile_splits(int64_t T, int H, int E);
hipError_t launch_router_tile_split(const uint16_t* x, const uint16_t* wg, float* partial,
                                    int64_t T, int H, int E, int splits, hipStream_t st);

// Scores + top-k from logits given as `splits` partial sums [splits][T][E]
// (added in split order); logits_out (or NULL) receives their sum.  With sf
// (may be null) the same launch also turns the shared expert's up slices in
// sf->part into sf->h.
hipError_t launch_score_topk(const float* logits, int splits, float* logits_out, const float* bias,
                             int64_t T, int E, int k, float route_scale, int32_t* topk_idx,
                             float* topk_w, const SharedFused* sf, hipStream_t st);

hipError_t launch_hash_route(const int64_t* token_ids, int64_t T, int E, int k,
                             float route_scale, uint64_t seed, int32_t* topk_idx, float* topk_w,
                             hipStream_t st);

// Stable counting sort of the P = T*k pairs by expert; with mtile_off (may
// be null) also the m-tile prefix for tiles of bm pairs.
size_t permute_scratch_bytes(int64_t P, int E);
hipError_t launch_permute(const int32_t* topk_idx, int64_t P, int E, int32_t* expert_offsets,
                          int32_t* sorted_pairs, int32_t* pair_pos, void* scratch, int bm,
                          int32_t* mtile_off, hipStream_t st);

// Permutation + m-tile prefix (tiles of bm pairs) of a small batch
// (P <= kFusedMaxPairs, E <= 512) in one workgroup; with sf (may be null)
// the launch's other workgroups run the shared expert's split-K down
// projection (sf->h x w2^T) into sf->part.
constexpr int kFusedMaxPairs = 2048;
hipError_t launch_perm_fused(const int32_t* topk_idx, int P, int E, int bm, int32_t* offsets,
                             int32_t* sorted_pairs, int32_t* pair_pos, int32_t* mtile_off,
                             const SharedFused* sf, hipStream_t st);

// Tile prefix of the grouped GEMMs: mtile_off[e] = sum_{e'<e} ceil(n_e'/bm).
hipError_t launch_tile_prefix(const int32_t* expert_offsets, int E, int bm, int32_t* mtile_off,
                              hipStream_t st);

struct ExpertGemmArgs {
  const uint8_t* a;          // FP8 rows: xq [T, K] (GEMM1) or hq [P, K] (GEMM2)
  const uint8_t* a_scale;    // [rows, K/128]
  const uint8_t* w;          // GEMM1: w1; GEMM2: w2
  const uint8_t* w_scale;
  const uint8_t* w3;         // GEMM1 only
  const uint8_t* w3_scale;
  const int32_t* expert_offsets;
  const int32_t* sorted_pairs;
  const int32_t* mtile_off;
  int E, K, N, top_k;        // N = I (GEMM1) or H (GEMM2); K = H or I
  int64_t P;
  float limit;               // GEMM1: SwiGLU clamp
  uint8_t* hq;               // GEMM1 out
  uint8_t* hs;
  void* out;                 // GEMM2 out
  int out_fp32;
  int fp8w;                  // weights: 0 MXFP4 ([N, K/2] + [N, K/32]), 1 FP8 ([N, K] + [N, K/128])
                             // (NVFP4 and W4AFP8 have launchers of their own)
};

// Grouped-GEMM workgroup -> (n_tile, expert, m0) for grids of n_tiles x
// mt_max workgroups (XCD-aware: workgroup b runs on XCD b % 8, and each
// XCD takes a contiguous run of tiles); false when the workgroup is idle.
// The expert of m-tile mt is the largest e < E with mtile_off[e] <= mt: the
// number of prefix entries at most mt, less one (an expert with no tiles
// shares its entry with the next, so that index is never an empty expert).
// Each lane of the wave compares up to nine entries (E <= 512), all loads
// issued at once: one round of loads instead of a chain of dependent ones
// before the weight stream can start.  Wave-uniform control flow required.
__device__ __forceinline__ bool map_expert_tile(const ExpertGemmArgs& p, int mt_max, int n_tiles,
                                                int bm, int& n_tile, int& e, int& m0, int& off_e,
                                                int& n_e) {
  const int G = gridDim.x;
  const int b = blockIdx.x;
  const int w = (b & 7) * (G >> 3) + (b >> 3);
  n_tile = w / mt_max;
  const int mt = w - n_tile * mt_max;
  if (n_tile >= n_tiles) return false;
  const int lane = threadIdx.x & 63;
  int v[9];
#pragma unroll
  for (int j = 0; j < 9; ++j) v[j] = p.mtile_off[min(lane + 64 * j, p.E)];
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < 9; ++j) cnt += __popcll(__ballot(lane + 64 * j <= p.E && v[j] <= mt));
  // all E + 1 entries at most mt: mt is past the last tile (mtile_off[E] is
  // the tile count), so the workgroup is idle -- no separate load of it
  if (cnt > p.E) return false;
  e = cnt - 1;
  m0 = (mt - __builtin_amdgcn_readfirstlane(p.mtile_off[e])) * bm;
  off_e = p.expert_offsets[e];
  n_e = p.expert_offsets[e + 1] - off_e;
  return true;
}

// Expert-major variant (the 64-pair kernels of the NVFP4 and W4AFP8 formats):
// the tile list runs over (expert, n-tile, m-tile of the expert) in that
// order and is dealt to the 8 XCDs in contiguous eighths (workgroup ids go
// round-robin over the XCDs), so the workgroups an XCD runs at one time
// cover a few experts: an expert's m-tiles of one n-tile run together (its
// weights come into that XCD's L2 once) and its n-tiles follow one another
// (its activation rows stay there).  Workgroups past the list (the grid is
// sized for the host's upper bound of m-tiles) return false.
__device__ __forceinline__ bool map_expert_tile_em(const ExpertGemmArgs& p, int n_tiles, int bm,
                                                   int& n_tile, int& e, int& m0, int& off_e,
                                                   int& n_e) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63;
  int v[9];
#pragma unroll
  for (int j = 0; j < 9; ++j) v[j] = p.mtile_off[min(lane + 64 * j, p.E)];
  const int total = __builtin_amdgcn_readfirstlane(p.mtile_off[p.E]) * n_tiles;
  const int share = (total + 7) >> 3;   // <= gridDim.x / 8: the grid covers the bound
  const int r = b >> 3;
  const int u = (b & 7) * share + r;
  if (r >= share || u >= total) return false;
  // the expert: the last entry e with mtile_off[e] * n_tiles <= u (empty
  // experts share their offset with the next one and are passed over)
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < 9; ++j) cnt += __popcll(__ballot(lane + 64 * j <= p.E && v[j] * n_tiles <= u));
  e = cnt - 1;
  const int mt0 = __builtin_amdgcn_readfirstlane(p.mtile_off[e]);
  const int m_e = __builtin_amdgcn_readfirstlane(p.mtile_off[e + 1]) - mt0;
  const int local = u - mt0 * n_tiles;
  n_tile = local / m_e;
  m0 = (local - n_tile * m_e) * bm;
  off_e = p.expert_offsets[e];
  n_e = p.expert_offsets[e + 1] - off_e;
  return true;
}

// bm = tokens per workgroup tile (16 or 64); mt_max = upper bound of m-tiles.
hipError_t launch_expert_gemm1(const ExpertGemmArgs& a, int bm, int mt_max, hipStream_t st);
hipError_t launch_expert_gemm2(const ExpertGemmArgs& a, int bm, int mt_max, hipStream_t st);
// NVFP4 weights (E4M3 scale per 16), K % 512 == 0; m-tiles of bm = 16 pairs,
// or 64 when K <= 4096.
hipError_t launch_expert_gemm1_nv(const ExpertGemmArgs& a, int bm, int mt_max, hipStream_t st);
hipError_t launch_expert_gemm2_nv(const ExpertGemmArgs& a, int bm, int mt_max, hipStream_t st);
// W4AFP8 weights (INT4 + float32 scale per 128), K % 512 == 0; m-tiles of
// bm = 16 pairs, or 64 when K <= 4096.
hipError_t launch_expert_gemm1_w4(const ExpertGemmArgs& a, int bm, int mt_max, hipStream_t st);
hipError_t launch_expert_gemm2_w4(const ExpertGemmArgs& a, int bm, int mt_max, hipStream_t st);

// MXFP4 [rows, K/2] + [rows, K/32] -> FP8 E4M3 [rows, K] + E8M0 [rows, K/128].
hipError_t launch_cast_fp8(const uint8_t* w, const uint8_t* ws, uint8_t* q, uint8_t* qs,
                           int64_t rows, int K, hipStream_t st);

// Shared expert (bf16): h = bf16(clamped_swiglu(x w1^T, x w3^T)) [T, I];
// ysh = h w2^T [T, H] fp32.  `part` holds shared_part_floats(T, H, I) floats
// of split-K partial sums (decode-sized batches; 0 floats, and unused,
// otherwise).  shared_split_ok: T <= 64, H and I multiples of the K slice.
constexpr int kSharedSplitK = 512;
bool shared_split_ok(int64_t T, int H, int I);
int64_t shared_part_floats(int64_t T, int H, int I);
hipError_t launch_shared_up(const uint16_t* x, const uint16_t* w1, const uint16_t* w3,
                            uint16_t* h, float* part, int64_t T, int H, int I, float limit,
                            hipStream_t st);
hipError_t launch_shared_down(const uint16_t* h, const uint16_t* w2, float* ysh, float* part,
                              int64_t T, int H, int I, hipStream_t st);

// y[t] = bf16(sum_j w[t,j] * o[pair_pos[t*k+j]] + ysh[t]); o fp32 [P, H];
// ysh (may be null) given as ysh_parts slices of T * H floats, added in
// slice order.
hipError_t launch_combine(const float* o, const float* topk_w, const int32_t* pair_pos,
                          const float* ysh, int ysh_parts, uint16_t* y, int64_t T, int H, int k,
                          hipStream_t st);

}  // namespace moe
