// Routing kernels ("DeepSeek-V4-Flash-SI" card, 架构特性 MoE paragraph: top-6
// of the routed experts per token, sqrtsoftplus scores, hash routing in the
// first layers, routing scale 1.5).
//
//  score_topk  one workgroup of 4 waves per token; thread i owns experts i,
//              i + 256; the score s = sqrt(ln(1 + e^z)) is evaluated in double
//              and rounded to fp32; key = s + bias; k rounds of a wave arg-max
//              (larger key first, lower expert id on equal keys) built from two
//              DPP wave reductions each, per wave and then over the waves'
//              candidates; weights s_j / sum(s) * scale in fp32 with the sum
//              taken in rank order (IEEE division).
//  hash_route  one thread per token: SplitMix64 (Steele, Lea, Flood, OOPSLA
//              2014) from (seed << 32) ^ token_id; r mod E with r at or above
//              2^64 - (2^64 mod E) rejected, repeats skipped, first k kept.
//  permute     stable counting sort of the pairs p = t*k + j by expert:
//              per-chunk histograms -> one scan (expert-major, chunk-minor)
//              -> per-chunk stable scatter (one wave walks its chunk in order,
//              ranking equal experts among lanes with a ballot), so the
//              result is deterministic and needs no atomics on positions.
#include "moe_internal.h"
#include "shared_splitk.h"

namespace moe {

extern "C" __device__ unsigned int __ockl_wfred_max_u32(unsigned int);
extern "C" __device__ unsigned int __ockl_wfred_min_u32(unsigned int);

// Order-preserving map of a finite fp32 key to uint32 (larger key -> larger
// integer; equal keys -> equal integers, as +0 and -0 cannot both occur:
// keys are s + b with s > 0).  Every finite key maps above 0x007FFFFF, so 0
// marks a retired or absent expert.
__device__ __forceinline__ uint32_t key_order(float k) {
  const uint32_t u = __float_as_uint(k);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One 256-thread workgroup per token: thread i owns experts i and i + 256,
// so each lane evaluates at most two scores (the double-precision chain is
// the kernel's latency); each wave selects its own top k, and wave 0 selects
// the token's top k from the 4k candidates -- the same order, since the
// token's top k is among the union of the waves' top k.  Workgroups from T
// on (a decode-sized layer with the shared expert) finish the shared
// expert's up projection instead: slices summed in order, clamped SwiGLU.
struct SharedSwigluArgs {
  const float* part;
  uint16_t* h;
  int S, M, I;
  float limit;
};

__global__ __launch_bounds__(256) void score_topk_kernel(const float* __restrict__ logits,
                                                         int splits, float* __restrict__ logits_out,
                                                         const float* __restrict__ bias,
                                                         int64_t T, int E, int k,
                                                         float route_scale,
                                                         int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w,
                                                         SharedSwigluArgs sh) {
  if ((int64_t)blockIdx.x >= T) {
    shared_swiglu_body(sh.part, sh.S, sh.M, sh.I, sh.limit, sh.h,
                       (int)(blockIdx.x - T) * 256 + (int)threadIdx.x);
    return;
  }
  __shared__ uint32_t cand_key[4][8];
  __shared__ int32_t cand_e[4][8];
  __shared__ float cand_s[4][8];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int64_t t = blockIdx.x;
  const float* z = logits + t * E;
  const size_t split_stride = (size_t)T * E;
  float s[2];
  uint32_t ok[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int ex = (int)threadIdx.x + 256 * i;
    if (ex < E) {
      float zf;
      if (splits == kRouterSplits) {
        // all partial loads in flight first, then the fixed-order sum
        float part[kRouterSplits];
#pragma unroll
        for (int q = 0; q < kRouterSplits; ++q) part[q] = z[q * split_stride + ex];
        zf = part[0];
#pragma unroll
        for (int q = 1; q < kRouterSplits; ++q) zf += part[q];
      } else {
        zf = z[ex];
        for (int q = 1; q < splits; ++q) zf += z[q * split_stride + ex];
      }
      if (logits_out) logits_out[t * E + ex] = zf;
      const double zd = (double)zf;
      s[i] = (float)sqrt(log1p(exp(zd)));
      ok[i] = key_order(bias ? s[i] + bias[ex] : s[i]);
    } else {
      s[i] = 0.f;
      ok[i] = 0u;
    }
  }
  // this wave's top k: k rounds of a wave arg-max (largest key, then the
  // lowest expert id), the winner retired by its owner
  for (int j = 0; j < k; ++j) {
    const int i = ok[1] > ok[0] ? 1 : 0;          // equal keys: the lower id (slot 0)
    const uint32_t bk = ok[i];
    const uint32_t be = bk ? (uint32_t)(threadIdx.x + 256 * i) : 0xFFFFFFFFu;
    const uint32_t m = __ockl_wfred_max_u32(bk);
    const uint32_t win = __ockl_wfred_min_u32(bk == m ? be : 0xFFFFFFFFu);
    const int wl = (int)(win & 63);               // owner lane: win = 64 wv + wl (+ 256)
    float ws = 0.f;
    if (m != 0u) {
      ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(win >= 256 ? s[1] : s[0]), wl));
      if (lane == wl) ok[win >= 256 ? 1 : 0] = 0u;
    }
    if (lane == 0) {
      cand_key[wv][j] = m;
      cand_e[wv][j] = m ? (int32_t)win : 0x7FFFFFFF;
      cand_s[wv][j] = ws;
    }
  }
  __syncthreads();
  if (wv != 0) return;
  // the token's top k among the 4k candidates (lane l < 4k holds one)
  const bool has = lane < 4 * k;
  uint32_t ck = has ? cand_key[lane / k][lane % k] : 0u;
  const int32_t ce = has ? cand_e[lane / k][lane % k] : 0x7FFFFFFF;
  const float cs = has ? cand_s[lane / k][lane % k] : 0.f;
  int sel_e[8];
  float sel_s[8];
  for (int j = 0; j < k; ++j) {
    const uint32_t m = __ockl_wfred_max_u32(ck);
    const int win = (int)__ockl_wfred_min_u32(ck == m ? (uint32_t)ce : 0xFFFFFFFFu);
    sel_e[j] = win;
    // the lane holding the winner (unique: experts are distinct)
    const uint64_t hold = __ballot(ck == m && ce == win);
    const int hl = (int)__builtin_ctzll(hold);
    sel_s[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cs), hl));
    if (lane == hl) ck = 0u;
  }
  if (lane == 0) {
    float total = 0.f;
    for (int j = 0; j < k; ++j) total = total + sel_s[j];
    for (int j = 0; j < k; ++j) {
      topk_idx[t * k + j] = sel_e[j];
      topk_w[t * k + j] = (sel_s[j] / total) * route_scale;
    }
  }
}

hipError_t launch_score_topk(const float* logits, int splits, float* logits_out, const float* bias,
                             int64_t T, int E, int k, float route_scale, int32_t* topk_idx,
                             float* topk_w, const SharedFused* sf, hipStream_t st) {
  if (T == 0) return hipSuccess;
  SharedSwigluArgs sh{};
  int64_t extra = 0;
  if (sf) {
    sh = SharedSwigluArgs{sf->part, sf->h, sf->H / kSharedSplitK, sf->M, sf->I, sf->limit};
    extra = ((int64_t)sf->M * (sf->I / 4) + 255) / 256;
  }
  hipLaunchKernelGGL(score_topk_kernel, dim3((unsigned)(T + extra)), dim3(256), 0, st, logits,
                     splits, logits_out, bias, T, E, k, route_scale, topk_idx, topk_w, sh);
  return hipGetLastError();
}

__device__ __forceinline__ uint64_t splitmix64_next(uint64_t& state) {
  state += 0x9E3779B97F4A7C15ull;
  uint64_t z = state;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__global__ __launch_bounds__(256) void hash_route_kernel(const int64_t* __restrict__ ids,
                                                         int64_t T, int E, int k, float w,
                                                         uint64_t seed, uint64_t reject_at,
                                                         int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  uint64_t state = (seed << 32) ^ (uint64_t)ids[t];
  int chosen[8];
  int n = 0;
  // rejection of repeats/out-of-range draws; terminates with probability 1
  // and in practice within a few draws (k <= min(8, E))
  while (n < k) {
    const uint64_t r = splitmix64_next(state);
    if (reject_at != 0 && r >= reject_at) continue;
    const int ex = (int)(r % (uint64_t)E);
    bool dup = false;
    for (int i = 0; i < n; ++i) dup |= (chosen[i] == ex);
    if (!dup) chosen[n++] = ex;
  }
  for (int j = 0; j < k; ++j) {
    topk_idx[t * k + j] = chosen[j];
    topk_w[t * k + j] = w;
  }
}

hipError_t launch_hash_route(const int64_t* ids, int64_t T, int E, int k, float route_scale,
                             uint64_t seed, int32_t* topk_idx, float* topk_w, hipStream_t st) {
  if (T == 0) return hipSuccess;
  // 2^64 - (2^64 mod E); 0 stands for "no rejection" (E a power of two)
  const uint64_t rem = (uint64_t)((((unsigned __int128)1) << 64) % (unsigned)E);
  const uint64_t reject_at = rem == 0 ? 0 : (uint64_t)0 - rem;
  const float w = route_scale / (float)k;
  hipLaunchKernelGGL(hash_route_kernel, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, st, ids,
                     T, E, k, w, seed, reject_at, topk_idx, topk_w);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Permutation
// ---------------------------------------------------------------------------
// Mask of the lanes holding the same value as this lane: one ballot per
// distinct value present in the wave (the lowest unresolved lane's value is
// read as a scalar and compared by every lane), instead of 64 shuffles.
__device__ __forceinline__ uint64_t lanes_with_same(int v) {
  uint64_t same = 0;
  uint64_t todo = __ballot(1);
  while (todo) {
    const int leader = __builtin_ctzll(todo);
    const int lv = __builtin_amdgcn_readlane(v, leader);
    const uint64_t m = __ballot(v == lv);
    if (v == lv) same = m;
    todo &= ~m;
  }
  return same;
}
constexpr int kPermChunk = 1024;  // pairs per chunk (16 waves of 64)

size_t permute_scratch_bytes(int64_t P, int E) {
  const int64_t chunks = (P + kPermChunk - 1) / kPermChunk;
  return (size_t)chunks * E * sizeof(int32_t);
}

// counts[c * E + e] = pairs of chunk c routed to e
__global__ __launch_bounds__(256) void perm_hist_kernel(const int32_t* __restrict__ idx, int64_t P,
                                                        int E, int32_t* __restrict__ counts) {
  __shared__ int32_t h[512];
  const int64_t c = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += 256) h[e] = 0;
  __syncthreads();
  const int64_t lo = c * kPermChunk;
  const int64_t hi = min(P, lo + kPermChunk);
  for (int64_t p = lo + threadIdx.x; p < hi; p += 256) atomicAdd(&h[idx[p]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) counts[c * E + e] = h[e];
}

// inclusive scan of one value per thread over the first 512 threads of the
// workgroup (threads past 512 take part in the barriers; their result is
// meaningless): a shuffle scan inside each wave, then each wave adds the
// totals of the waves below it -- two barriers (a Hillis-Steele scan in LDS
// took eighteen).  wtot: 8 ints of LDS.
__device__ __forceinline__ int32_t block_scan512(int32_t* wtot, int32_t v) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t u = __shfl_up(v, off);
    if (lane >= off) v += u;
  }
  if (lane == 63 && wv < 8) wtot[wv] = v;
  __syncthreads();
  int32_t below = 0;
  for (int w = 0; w < wv && w < 8; ++w) below += wtot[w];
  __syncthreads();
  return v + below;
}

// One workgroup: expert totals, exclusive scan -> expert_offsets, then each
// chunk's base per expert, written over the counts (expert-major order);
// with mtile_off, also the grouped GEMMs' m-tile prefix for tiles of bm.
__global__ __launch_bounds__(512) void perm_scan_kernel(int32_t* __restrict__ counts, int chunks,
                                                        int E, int32_t* __restrict__ offsets,
                                                        int bm, int32_t* __restrict__ mtile_off) {
  __shared__ int32_t tot[8];
  const int e = threadIdx.x;
  // the chunk column of expert e in batches of 16 independent loads (one
  // dependent load per chunk would make the kernel latency-bound)
  constexpr int NB = 16;
  int32_t sum = 0;
  if (e < E)
    for (int c0 = 0; c0 < chunks; c0 += NB) {
      int32_t v[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) v[j] = c0 + j < chunks ? counts[(size_t)(c0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < NB; ++j) sum += v[j];
    }
  const int32_t incl = block_scan512(tot, sum);
  if (e < E) {
    int32_t base = incl - sum;  // exclusive
    offsets[e] = base;
    if (e == E - 1) offsets[E] = incl;
    for (int c0 = 0; c0 < chunks; c0 += NB) {
      int32_t v[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) v[j] = c0 + j < chunks ? counts[(size_t)(c0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        if (c0 + j < chunks) counts[(size_t)(c0 + j) * E + e] = base;
        base += v[j];
      }
    }
  }
  if (mtile_off) {
    const int32_t t = e < E ? (sum + bm - 1) / bm : 0;
    const int32_t ti = block_scan512(tot, t);
    if (e < E) {
      mtile_off[e] = ti - t;
      if (e == E - 1) mtile_off[E] = ti;
    }
  }
}

// One workgroup of 16 waves per chunk; wave w ranks the w-th 64 pairs of the
// chunk.  A pair's position is its expert's base for the chunk, plus the
// counts of its expert in the chunk's lower waves (per-wave counts in LDS,
// summed per expert over the waves), plus the number of lower lanes of its
// wave with the same expert -- the stable order, with all 16 rounds of 64
// in flight at once.
__global__ __launch_bounds__(1024) void perm_scatter_kernel(const int32_t* __restrict__ idx,
                                                            int64_t P, int E,
                                                            const int32_t* __restrict__ base,
                                                            int32_t* __restrict__ sorted_pairs,
                                                            int32_t* __restrict__ pair_pos) {
  constexpr int W = kPermChunk / 64;
  __shared__ int32_t cnt[W][512];
  const int64_t c = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < W * 512; i += 1024) (&cnt[0][0])[i] = 0;
  const int64_t p = c * kPermChunk + (int64_t)w * 64 + lane;
  const bool live = p < P;
  const int ex = live ? idx[p] : -1;
  const uint64_t same = lanes_with_same(ex);
  const int rank = __popcll(same & ((1ull << lane) - 1ull));
  __syncthreads();
  // the highest lane of each expert's group in this wave records the count
  if (live && (same >> lane) == 1ull) cnt[w][ex] = __popcll(same);
  __syncthreads();
  // exclusive running sum over the waves, per expert, from the chunk's base
  for (int e = threadIdx.x; e < E; e += 1024) {
    int32_t run = base[c * E + e];
#pragma unroll
    for (int v = 0; v < W; ++v) {
      const int32_t n = cnt[v][e];
      cnt[v][e] = run;
      run += n;
    }
  }
  __syncthreads();
  if (live) {
    const int32_t pos = cnt[w][ex] + rank;
    sorted_pairs[pos] = (int32_t)p;
    pair_pos[p] = pos;
  }
}

hipError_t launch_permute(const int32_t* topk_idx, int64_t P, int E, int32_t* expert_offsets,
                          int32_t* sorted_pairs, int32_t* pair_pos, void* scratch, int bm,
                          int32_t* mtile_off, hipStream_t st) {
  const int64_t chunks = (P + kPermChunk - 1) / kPermChunk;
  int32_t* counts = static_cast<int32_t*>(scratch);
  if (chunks > 0) {
    hipLaunchKernelGGL(perm_hist_kernel, dim3((unsigned)chunks), dim3(256), 0, st, topk_idx, P, E,
                       counts);
  }
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(512), 0, st, counts, (int)chunks, E,
                     expert_offsets, bm, mtile_off);
  if (chunks > 0) {
    hipLaunchKernelGGL(perm_scatter_kernel, dim3((unsigned)chunks), dim3(1024), 0, st, topk_idx,
                       P, E, counts, sorted_pairs, pair_pos);
  }
  return hipGetLastError();
}

// mtile_off[e] = sum_{e' < e} ceil(n_e' / bm), e = 0..E
__global__ __launch_bounds__(512) void tile_prefix_kernel(const int32_t* __restrict__ offsets,
                                                          int E, int bm,
                                                          int32_t* __restrict__ mtile_off) {
  __shared__ int32_t wtot[8];
  const int e = threadIdx.x;
  int32_t c = 0;
  if (e < E) c = (offsets[e + 1] - offsets[e] + bm - 1) / bm;
  const int32_t incl = block_scan512(wtot, c);
  if (e < E) {
    mtile_off[e] = incl - c;
    if (e == E - 1) mtile_off[E] = incl;
  }
}

hipError_t launch_tile_prefix(const int32_t* expert_offsets, int E, int bm, int32_t* mtile_off,
                              hipStream_t st) {
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(512), 0, st, expert_offsets, E, bm,
                     mtile_off);
  return hipGetLastError();
}


// ---------------------------------------------------------------------------
// Small batches (P = T*k <= kFusedMaxPairs): the permutation and the grouped
// GEMMs' m-tile prefix in one workgroup of 16 waves -- expert histogram,
// exclusive scan, stable scatter, m-tile prefix -- one launch instead of
// four.  Same result as the multi-kernel path: counts come from LDS
// histograms, and the scatter keeps pair order within each expert (wave w
// owns the w-th contiguous chunk of pairs; its base per expert is the sum of
// the lower chunks' counts).  Workgroups from 1 on (a decode-sized layer with
// the shared expert) run its split-K down projection: 64 weight rows (two
// row waves, eight K waves each) x one 512-slice of I per workgroup, 256
// workgroups at H = 4096, I = 2048 (four row waves and 128 workgroups:
// 0.5 us slower).
// ---------------------------------------------------------------------------
constexpr int kFusedWaves = 16;

struct SharedDownArgs {
  const uint16_t* h;
  const uint16_t* w2;
  float* part;
  int M, H, I;
  int blocks;
};

__global__ __launch_bounds__(kFusedWaves * 64) void perm_fused_kernel(
    const int32_t* __restrict__ topk_idx, int P, int E, int bm, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_pairs, int32_t* __restrict__ pair_pos,
    int32_t* __restrict__ mtile_off, SharedDownArgs sh) {
  // 64 KB: the permutation's pair and count arrays (40 KB), or the split-K token slice
  __shared__ uint4 lds[64][64];
  if (blockIdx.x > 0) {
    const int b = blockIdx.x - 1, nbx = sh.H / shared_splitk_rows<EPI_F32, 2>();
    shared_splitk_body<EPI_F32, kFusedWaves, 2>(sh.h, sh.w2, nullptr, sh.part, sh.M, sh.H, sh.I,
                                                b % nbx, b / nbx, lds);
    return;
  }
  int32_t* sel = reinterpret_cast<int32_t*>(&lds[0][0]);   // [kFusedMaxPairs]
  // [kFusedWaves][512]: per-wave counts, then per-wave bases
  int32_t (*wcnt)[512] = reinterpret_cast<int32_t (*)[512]>(sel + kFusedMaxPairs);
  __shared__ int32_t tot[8];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  for (int p = threadIdx.x; p < P; p += kFusedWaves * 64) sel[p] = topk_idx[p];
  for (int i = threadIdx.x; i < kFusedWaves * 512; i += kFusedWaves * 64) (&wcnt[0][0])[i] = 0;
  __syncthreads();

  // per-wave histograms over contiguous pair chunks
  const int chunk = (P + kFusedWaves - 1) / kFusedWaves;
  const int p_lo = min(P, wv * chunk), p_hi = min(P, p_lo + chunk);
  for (int p = p_lo + lane; p < p_hi; p += 64) atomicAdd(&wcnt[wv][sel[p]], 1);
  __syncthreads();

  // expert totals, then one exclusive scan of (count << 16 | m-tiles): both
  // totals stay below 2^16 (P <= 2048, m-tiles <= P / bm + E)
  const int e = threadIdx.x;  // E <= 512 < 1024 threads
  int32_t sum = 0;
  if (e < E)
    for (int w = 0; w < kFusedWaves; ++w) sum += wcnt[w][e];
  const int32_t c = (e < E) ? (sum + bm - 1) / bm : 0;
  const int32_t packed = (sum << 16) | c;
  const int32_t incl = block_scan512(tot, packed);
  if (e < E) {
    const int32_t excl = incl - packed;
    int32_t base = excl >> 16;
    offsets[e] = base;
    mtile_off[e] = excl & 0xFFFF;
    if (e == E - 1) {
      offsets[E] = incl >> 16;
      mtile_off[E] = incl & 0xFFFF;
    }
    for (int w = 0; w < kFusedWaves; ++w) {
      const int32_t n = wcnt[w][e];
      wcnt[w][e] = base;
      base += n;
    }
  }
  __syncthreads();

  // stable scatter, each wave over its chunk in order
  for (int r0 = p_lo; r0 < p_hi; r0 += 64) {
    const int p = r0 + lane;
    const bool live = p < p_hi;
    const int ex = live ? sel[p] : -1;
    const uint64_t same = lanes_with_same(ex);
    const int rank = __popcll(same & ((1ull << lane) - 1ull));
    if (live) {
      const int pos = wcnt[wv][ex] + rank;
      sorted_pairs[pos] = p;
      pair_pos[p] = pos;
    }
    // wave-synchronous: every lane has read its base before the highest
    // lane of each expert advances it
    if (live && (same >> lane) == 1ull) wcnt[wv][ex] += __popcll(same);
  }
}

hipError_t launch_perm_fused(const int32_t* topk_idx, int P, int E, int bm, int32_t* offsets,
                             int32_t* sorted_pairs, int32_t* pair_pos, int32_t* mtile_off,
                             const SharedFused* sf, hipStream_t st) {
  SharedDownArgs sh{};
  if (sf) {
    sh = SharedDownArgs{sf->h, sf->w2, sf->part, sf->M, sf->H, sf->I,
                        (sf->H / shared_splitk_rows<EPI_F32, 2>()) * (sf->I / kSharedSplitK)};
  }
  hipLaunchKernelGGL(perm_fused_kernel, dim3((unsigned)(1 + sh.blocks)), dim3(kFusedWaves * 64), 0,
                     st, topk_idx, P, E, bm, offsets, sorted_pairs, pair_pos, mtile_off, sh);
  return hipGetLastError();
}

}  // namespace moe
