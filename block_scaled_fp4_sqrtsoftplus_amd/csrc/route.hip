// Routing kernels ("DeepSeek-V4-Flash-SI" card, 架构特性 MoE paragraph: top-6
// of the routed experts per token, sqrtsoftplus scores, hash routing in the
// first layers, routing scale 1.5).
//
//  score_topk  one wave per token; lane l owns experts l, l+64, ...; the score
//              s = sqrt(ln(1 + e^z)) is evaluated in double and rounded to fp32;
//              key = s + bias; k rounds of a wave arg-max (larger key first,
//              lower expert id on equal keys); weights s_j / sum(s) * scale in
//              fp32 with the sum taken in rank order (IEEE division).
//  hash_route  one thread per token: SplitMix64 (Steele, Lea, Flood, OOPSLA
//              2014) from (seed << 32) ^ token_id; r mod E with r at or above
//              2^64 - (2^64 mod E) rejected, repeats skipped, first k kept.
//  permute     stable counting sort of the pairs p = t*k + j by expert:
//              per-chunk histograms -> one scan (expert-major, chunk-minor)
//              -> per-chunk stable scatter (one wave walks its chunk in order,
//              ranking equal experts among lanes with a ballot), so the
//              result is deterministic and needs no atomics on positions.
#include "moe_internal.h"

namespace moe {

constexpr int kMaxExpertsPerLane = 8;  // E <= 512

__global__ __launch_bounds__(256) void score_topk_kernel(const float* __restrict__ logits,
                                                         const float* __restrict__ bias,
                                                         int64_t T, int E, int k,
                                                         float route_scale,
                                                         int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* z = logits + t * E;
  float s[kMaxExpertsPerLane], key[kMaxExpertsPerLane];
#pragma unroll
  for (int i = 0; i < kMaxExpertsPerLane; ++i) {
    const int ex = lane + 64 * i;
    if (ex < E) {
      const double zd = (double)z[ex];
      s[i] = (float)sqrt(log1p(exp(zd)));
      key[i] = bias ? s[i] + bias[ex] : s[i];
    } else {
      s[i] = 0.f;
      key[i] = -INFINITY;
    }
  }
  int sel_e[8];
  float sel_s[8];
  for (int j = 0; j < k; ++j) {
    // lane-local best (ascending expert order makes '>' keep the lower id)
    float bk = -INFINITY;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kMaxExpertsPerLane; ++i) {
      const int ex = lane + 64 * i;
      if (ex < E && (key[i] > bk || (key[i] == bk && ex < be))) { bk = key[i]; be = ex; }
    }
    // wave arg-max: (key desc, expert asc) is a total order, so the butterfly
    // gives every lane the same winner
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ok = __shfl_xor(bk, off);
      const int oe = __shfl_xor(be, off);
      if (ok > bk || (ok == bk && oe < be)) { bk = ok; be = oe; }
    }
    sel_e[j] = be;
    // owner lane retires the winner and publishes its unbiased score
    float ws = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxExpertsPerLane; ++i) {
      if (lane + 64 * i == be) { ws = s[i]; key[i] = -INFINITY; }
    }
    sel_s[j] = __shfl(ws, be & 63);
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

hipError_t launch_score_topk(const float* logits, const float* bias, int64_t T, int E, int k,
                             float route_scale, int32_t* topk_idx, float* topk_w,
                             hipStream_t st) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(score_topk_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, st, logits,
                     bias, T, E, k, route_scale, topk_idx, topk_w);
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
constexpr int kPermChunk = 1024;  // pairs per chunk (one wave walks 16 rounds of 64)

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

// One workgroup: expert totals, exclusive scan -> expert_offsets, then each
// chunk's base per expert, written over the counts (expert-major order).
__global__ __launch_bounds__(512) void perm_scan_kernel(int32_t* __restrict__ counts, int chunks,
                                                        int E, int32_t* __restrict__ offsets) {
  __shared__ int32_t tot[512];
  const int e = threadIdx.x;
  int32_t sum = 0;
  if (e < E)
    for (int c = 0; c < chunks; ++c) sum += counts[(size_t)c * E + e];
  tot[e] = sum;
  __syncthreads();
  // inclusive scan over experts (Hillis-Steele, 512 entries)
  for (int off = 1; off < 512; off <<= 1) {
    const int32_t v = e >= off ? tot[e - off] : 0;
    __syncthreads();
    tot[e] += v;
    __syncthreads();
  }
  if (e < E) {
    int32_t base = tot[e] - sum;  // exclusive
    offsets[e] = base;
    if (e == E - 1) offsets[E] = tot[e];
    for (int c = 0; c < chunks; ++c) {
      const int32_t n = counts[(size_t)c * E + e];
      counts[(size_t)c * E + e] = base;
      base += n;
    }
  }
}

// One wave per chunk: walk the chunk 64 pairs at a time in order; a lane's
// position is its expert's running base plus the number of lower lanes with
// the same expert in this round.
__global__ __launch_bounds__(64) void perm_scatter_kernel(const int32_t* __restrict__ idx,
                                                          int64_t P, int E,
                                                          const int32_t* __restrict__ base,
                                                          int32_t* __restrict__ sorted_pairs,
                                                          int32_t* __restrict__ pair_pos) {
  __shared__ int32_t run[512];
  const int64_t c = blockIdx.x;
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) run[e] = base[c * E + e];
  __syncthreads();
  const int64_t lo = c * kPermChunk;
  const int64_t hi = min(P, lo + kPermChunk);
  for (int64_t r0 = lo; r0 < hi; r0 += 64) {
    const int64_t p = r0 + lane;
    const bool live = p < hi;
    const int ex = live ? idx[p] : -1;
    // lanes with the same expert: compare against every lane's value
    uint64_t same = 0;
    for (int j = 0; j < 64; ++j) {
      const int oj = __shfl(ex, j);
      same |= (uint64_t)(oj == ex) << j;
    }
    const uint64_t lower = same & ((1ull << lane) - 1ull);
    const int rank = __popcll(lower);
    const int cnt = __popcll(same);
    int32_t pos = 0;
    if (live) pos = run[ex] + rank;
    __syncthreads();
    if (live) {
      sorted_pairs[pos] = (int32_t)p;
      pair_pos[p] = pos;
      // the highest lane of each expert advances that expert's running base
      if ((same >> lane) == 1ull) run[ex] += cnt;
    }
    __syncthreads();
  }
}

hipError_t launch_permute(const int32_t* topk_idx, int64_t P, int E, int32_t* expert_offsets,
                          int32_t* sorted_pairs, int32_t* pair_pos, void* scratch,
                          hipStream_t st) {
  const int64_t chunks = (P + kPermChunk - 1) / kPermChunk;
  int32_t* counts = static_cast<int32_t*>(scratch);
  if (chunks > 0) {
    hipLaunchKernelGGL(perm_hist_kernel, dim3((unsigned)chunks), dim3(256), 0, st, topk_idx, P, E,
                       counts);
  }
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(512), 0, st, counts, (int)chunks, E,
                     expert_offsets);
  if (chunks > 0) {
    hipLaunchKernelGGL(perm_scatter_kernel, dim3((unsigned)chunks), dim3(64), 0, st, topk_idx, P,
                       E, counts, sorted_pairs, pair_pos);
  }
  return hipGetLastError();
}

// mtile_off[e] = sum_{e' < e} ceil(n_e' / bm), e = 0..E
__global__ __launch_bounds__(512) void tile_prefix_kernel(const int32_t* __restrict__ offsets,
                                                          int E, int bm,
                                                          int32_t* __restrict__ mtile_off) {
  __shared__ int32_t tot[512];
  const int e = threadIdx.x;
  int32_t c = 0;
  if (e < E) c = (offsets[e + 1] - offsets[e] + bm - 1) / bm;
  tot[e] = c;
  __syncthreads();
  for (int off = 1; off < 512; off <<= 1) {
    const int32_t v = e >= off ? tot[e - off] : 0;
    __syncthreads();
    tot[e] += v;
    __syncthreads();
  }
  if (e < E) {
    mtile_off[e] = tot[e] - c;
    if (e == E - 1) mtile_off[E] = tot[e];
  }
}

hipError_t launch_tile_prefix(const int32_t* expert_offsets, int E, int bm, int32_t* mtile_off,
                              hipStream_t st) {
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(512), 0, st, expert_offsets, E, bm,
                     mtile_off);
  return hipGetLastError();
}

}  // namespace moe
