// Host side of the C ABI declared in include/moe_fp4.h: argument validation
// (pure host code, run before any HIP call), workspace carve-up and the launch
// sequence of each entry point.  All launches go to the caller's stream; no
// call synchronises or copies to the host.
#include "moe_fp4.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <functional>
#include <mutex>
#include <new>

#include "moe_internal.h"

namespace {

using namespace moe;

constexpr size_t kAlign = 256;

size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

moe_status check_cfg(const moe_config* c) {
  if (!c) return MOE_ERR_NULL_ARG;
  if (c->tokens < 0) return MOE_ERR_BAD_SHAPE;
  if (c->hidden < 128 || c->hidden > 16384 || c->hidden % 128) return MOE_ERR_BAD_SHAPE;
  if (c->inter < 128 || c->inter > 16384 || c->inter % 128) return MOE_ERR_BAD_SHAPE;
  if (c->n_experts < 1 || c->n_experts > 512) return MOE_ERR_BAD_SHAPE;
  if (c->top_k < 1 || c->top_k > 8 || c->top_k > c->n_experts) return MOE_ERR_BAD_SHAPE;
  if (c->tokens * (int64_t)c->top_k >= (int64_t(1) << 31)) return MOE_ERR_BAD_SHAPE;
  if (!std::isfinite(c->route_scale)) return MOE_ERR_BAD_SHAPE;
  if (!(c->swiglu_limit > 0.f)) return MOE_ERR_BAD_SHAPE;  // NaN fails too; +inf allowed
  if (c->route_mode != MOE_ROUTE_SQRTSOFTPLUS && c->route_mode != MOE_ROUTE_HASH)
    return MOE_ERR_BAD_SHAPE;
  if (c->expert_format != MOE_EXPERTS_MXFP4 && c->expert_format != MOE_EXPERTS_FP8 &&
      c->expert_format != MOE_EXPERTS_NVFP4 && c->expert_format != MOE_EXPERTS_W4AFP8)
    return MOE_ERR_BAD_SHAPE;
  if ((c->expert_format == MOE_EXPERTS_NVFP4 || c->expert_format == MOE_EXPERTS_W4AFP8) &&
      (c->hidden % 512 || c->inter % 512))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Sequential carve-up of a workspace; with base == nullptr it only measures.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <class T>
  T* take(size_t count) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += up(count * sizeof(T));
    return p;
  }
};

struct RouteWs {
  int32_t* perm_scratch;
  float* logits;
  int32_t* mtile_off;  // m-tile prefix written by the single-workgroup routing
};
// Partial sums the router GEMM leaves for the top-k kernel to add (1: the
// logits themselves).
int router_partials(const moe_config& c) {
  const int small = router_splits(c.tokens, c.hidden);
  return small > 1 ? small : router_tile_splits(c.tokens, c.hidden, c.n_experts);
}

RouteWs carve_route(Carver& cv, const moe_config& c) {
  const int64_t P = c.tokens * c.top_k;
  RouteWs r;
  r.perm_scratch = cv.take<int32_t>(permute_scratch_bytes(P, c.n_experts) / sizeof(int32_t) + 1);
  // logits, or their split partial sums
  r.logits = cv.take<float>(c.route_mode == MOE_ROUTE_SQRTSOFTPLUS
                                ? (size_t)c.tokens * c.n_experts * router_partials(c)
                                : 0);
  r.mtile_off = cv.take<int32_t>(c.n_experts + 1);
  return r;
}

struct FfnWs {
  int32_t* mtile_off;
  uint8_t* hq;
  uint8_t* hs;
};
FfnWs carve_ffn(Carver& cv, const moe_config& c) {
  const int64_t P = c.tokens * c.top_k;
  FfnWs f;
  f.mtile_off = cv.take<int32_t>(c.n_experts + 1);
  f.hq = cv.take<uint8_t>((size_t)P * c.inter);
  f.hs = cv.take<uint8_t>((size_t)P * (c.inter / 128));
  return f;
}

struct LayerWs {
  RouteWs route;
  moe_routing routing;
  uint8_t* xq;
  uint8_t* xs;
  FfnWs ffn;
  float* o;
  uint16_t* hsh;
  float* ysh;
  float* shpart;
};
LayerWs carve_layer(Carver& cv, const moe_config& c) {
  const int64_t P = c.tokens * c.top_k;
  LayerWs l;
  l.route = carve_route(cv, c);
  l.routing.topk_idx = cv.take<int32_t>(P);
  l.routing.topk_w = cv.take<float>(P);
  l.routing.expert_offsets = cv.take<int32_t>(c.n_experts + 1);
  l.routing.sorted_pairs = cv.take<int32_t>(P);
  l.routing.pair_pos = cv.take<int32_t>(P);
  l.xq = cv.take<uint8_t>((size_t)c.tokens * c.hidden);
  l.xs = cv.take<uint8_t>((size_t)c.tokens * (c.hidden / 128));
  l.ffn = carve_ffn(cv, c);
  l.o = cv.take<float>((size_t)P * c.hidden);
  l.hsh = cv.take<uint16_t>((size_t)c.tokens * c.inter);
  l.ysh = cv.take<float>((size_t)c.tokens * c.hidden);
  l.shpart = cv.take<float>((size_t)shared_part_floats(c.tokens, c.hidden, c.inter));
  return l;
}

// Device architecture check, cached per device (0 unknown, 1 gfx950, 2 other).
std::atomic<int> g_arch[64];

moe_status check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= 64) return MOE_ERR_ARCH;
  int v = g_arch[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_ERR_HIP;
    v = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch[dev].store(v, std::memory_order_relaxed);
  }
  return v == 1 ? MOE_OK : MOE_ERR_ARCH;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// One side stream per device (default priority, created on first use and kept
// for the process) on which moe_layer runs the shared expert, which needs only
// x.  It forks from and joins back to the caller's stream through two events;
// the per-device mutex keeps the fork/join pairs of concurrent calls from
// interleaving.
struct SideStream {
  std::mutex mu;
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool ready = false;
};
SideStream g_side[64];

// Batches from which moe_layer starts the shared expert early: before the
// top-k and permutation (score routing) or before quantization (hash).
constexpr int64_t kEarlyForkTokens = 256;

moe_status side_stream(SideStream*& out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_ERR_HIP;
  out = &g_side[dev];
  return MOE_OK;
}

moe_status side_init_locked(SideStream& s) {
  if (s.ready) return MOE_OK;
  if (hipStreamCreateWithFlags(&s.stream, hipStreamNonBlocking) != hipSuccess) return MOE_ERR_HIP;
  // device-side ordering only: no timing, no system-scope fence on record
  const unsigned flags = hipEventDisableTiming | hipEventDisableSystemFence;
  if (hipEventCreateWithFlags(&s.fork, flags) != hipSuccess) return MOE_ERR_HIP;
  if (hipEventCreateWithFlags(&s.join, flags) != hipSuccess) return MOE_ERR_HIP;
  s.ready = true;
  return MOE_OK;
}

#define MOE_TRY(expr)                                   \
  do {                                                  \
    hipError_t _e = (expr);                             \
    if (_e != hipSuccess) return MOE_ERR_HIP;           \
  } while (0)

moe_status check_routing_ptrs(const moe_routing* r) {
  if (!r->topk_idx || !r->topk_w || !r->expert_offsets || !r->sorted_pairs || !r->pair_pos)
    return MOE_ERR_NULL_ARG;
  if (!aligned16(r->topk_idx) || !aligned16(r->topk_w) || !aligned16(r->expert_offsets) ||
      !aligned16(r->sorted_pairs) || !aligned16(r->pair_pos))
    return MOE_ERR_MISALIGNED;
  return MOE_OK;
}

moe_status check_weights(const moe_expert_weights* w) {
  if (!w) return MOE_ERR_NULL_ARG;
  const void* ps[6] = {w->w1, w->w1_scale, w->w3, w->w3_scale, w->w2, w->w2_scale};
  for (const void* p : ps)
    if (!p) return MOE_ERR_NULL_ARG;
  for (const void* p : ps)
    if (!aligned16(p)) return MOE_ERR_MISALIGNED;
  return MOE_OK;
}

// Tokens per m-tile of the grouped GEMMs, from the mean pairs per expert:
// 16 (decode-like), 128 (prefill-like, when both K are 1024, 2048 or 4096),
// else 64.
int choose_bm(const moe_config& c) {
  const int64_t P = c.tokens * c.top_k;
  if (P <= (int64_t)32 * c.n_experts) return 16;
  if (c.expert_format == MOE_EXPERTS_NVFP4 || c.expert_format == MOE_EXPERTS_W4AFP8)
    return (c.hidden <= 4096 && c.inter <= 4096) ? 64 : 16;   // 64-pair tiles need K <= 4096
  auto tiled = [](int k) { return k == 1024 || k == 2048 || k == 4096; };
  return (tiled(c.hidden) && tiled(c.inter)) ? 128 : 64;   // MXFP4 and FP8 tile kernels
}

// Routing (S1-S3).  Small batches run the single-workgroup permutation
// kernel, larger ones the histogram / scan / scatter kernels; either also
// writes the grouped GEMMs' m-tile prefix to `mtile_off` (when given), and
// the return flag says whether it did.
moe_status enqueue_route(const moe_config& c, const uint16_t* x, const uint16_t* wg,
                         const float* bias, const int64_t* ids, const float* logits_in,
                         float* logits_out, const moe_routing& r, const RouteWs& ws,
                         hipStream_t st, int32_t* mtile_off = nullptr, bool* tiles_done = nullptr,
                         uint8_t* xq = nullptr, uint8_t* xs = nullptr,
                         const SharedFused* sf = nullptr,
                         const std::function<moe_status()>* after_router = nullptr) {
  const int64_t T = c.tokens, P = T * c.top_k;
  if (tiles_done) *tiles_done = false;
  // called once the router GEMM (or the hash routing) is enqueued
  auto routed = [&]() -> moe_status { return after_router ? (*after_router)() : MOE_OK; };
  moe_status rs;
  // the shared expert rides only in the split-K router / fused permutation launches
  if (sf && !(c.route_mode == MOE_ROUTE_SQRTSOFTPLUS && !logits_in &&
              router_tile_splits(T, c.hidden, c.n_experts) == 1 &&
              router_splits(T, c.hidden) > 1 && P > 0 && P <= kFusedMaxPairs))
    return MOE_ERR_UNSUPPORTED;
  if (c.route_mode == MOE_ROUTE_HASH) {
    MOE_TRY(launch_hash_route(ids, T, c.n_experts, c.top_k, c.route_scale, c.hash_seed,
                              r.topk_idx, r.topk_w, st));
    if ((rs = routed()) != MOE_OK) return rs;
  } else if (logits_in) {
    if ((rs = routed()) != MOE_OK) return rs;
    MOE_TRY(launch_score_topk(logits_in, 1, logits_out, bias, T, c.n_experts, c.top_k,
                              c.route_scale, r.topk_idx, r.topk_w, nullptr, st));
  } else if (router_tile_splits(T, c.hidden, c.n_experts) > 1) {
    const int ks = router_tile_splits(T, c.hidden, c.n_experts);
    MOE_TRY(launch_router_tile_split(x, wg, ws.logits, T, c.hidden, c.n_experts, ks, st));
    if ((rs = routed()) != MOE_OK) return rs;
    MOE_TRY(launch_score_topk(ws.logits, ks, logits_out, bias, T, c.n_experts, c.top_k,
                              c.route_scale, r.topk_idx, r.topk_w, nullptr, st));
  } else if (router_splits(T, c.hidden) > 1) {
    MOE_TRY(launch_router_partial(x, wg, ws.logits, T, c.hidden, c.n_experts, xq, xs, sf, st));
    if ((rs = routed()) != MOE_OK) return rs;
    MOE_TRY(launch_score_topk(ws.logits, router_splits(T, c.hidden), logits_out, bias, T,
                              c.n_experts, c.top_k, c.route_scale, r.topk_idx, r.topk_w, sf,
                              st));
  } else {
    float* dst = logits_out ? logits_out : ws.logits;
    MOE_TRY(launch_router_gemm(x, wg, dst, T, c.hidden, c.n_experts, st));
    if ((rs = routed()) != MOE_OK) return rs;
    MOE_TRY(launch_score_topk(dst, 1, nullptr, bias, T, c.n_experts, c.top_k, c.route_scale,
                              r.topk_idx, r.topk_w, nullptr, st));
  }
  if (P > 0 && P <= kFusedMaxPairs) {
    MOE_TRY(launch_perm_fused(r.topk_idx, (int)P, c.n_experts, choose_bm(c), r.expert_offsets,
                              r.sorted_pairs, r.pair_pos, mtile_off ? mtile_off : ws.mtile_off,
                              sf, st));
    if (tiles_done) *tiles_done = mtile_off != nullptr;
    return MOE_OK;
  }
  MOE_TRY(launch_permute(r.topk_idx, P, c.n_experts, r.expert_offsets, r.sorted_pairs,
                         r.pair_pos, ws.perm_scratch, choose_bm(c), mtile_off, st));
  if (tiles_done) *tiles_done = mtile_off != nullptr;
  return MOE_OK;
}

moe_status enqueue_ffn(const moe_config& c, const uint8_t* xq, const uint8_t* xs,
                       const moe_routing& r, const moe_expert_weights& w, void* out, int out_fp32,
                       uint8_t* hq, uint8_t* hs, int32_t* mtile_off, hipStream_t st,
                       bool tiles_done = false) {
  const int64_t P = c.tokens * c.top_k;
  if (P == 0) return MOE_OK;
  const int bm = choose_bm(c);
  const int64_t mt_max64 = (P + bm - 1) / bm + std::min<int64_t>(c.n_experts, P);
  const int mt_max = (int)mt_max64;
  if (!tiles_done) MOE_TRY(launch_tile_prefix(r.expert_offsets, c.n_experts, bm, mtile_off, st));
  ExpertGemmArgs a{};
  a.expert_offsets = r.expert_offsets;
  a.sorted_pairs = r.sorted_pairs;
  a.mtile_off = mtile_off;
  a.E = c.n_experts;
  a.top_k = c.top_k;
  a.P = P;
  a.limit = c.swiglu_limit;
  // GEMM1: x (FP8) x [w1 | w3] -> clamped SwiGLU -> hq, hs
  a.a = xq;
  a.a_scale = xs;
  a.w = w.w1;
  a.w_scale = w.w1_scale;
  a.w3 = w.w3;
  a.w3_scale = w.w3_scale;
  a.K = c.hidden;
  a.N = c.inter;
  a.fp8w = c.expert_format == MOE_EXPERTS_FP8;
  a.hq = hq;
  a.hs = hs;
  const int fmt = c.expert_format;
  MOE_TRY(fmt == MOE_EXPERTS_NVFP4    ? launch_expert_gemm1_nv(a, bm, mt_max, st)
          : fmt == MOE_EXPERTS_W4AFP8 ? launch_expert_gemm1_w4(a, bm, mt_max, st)
                                      : launch_expert_gemm1(a, bm, mt_max, st));
  // GEMM2: hq (FP8) x w2 -> out
  ExpertGemmArgs b = a;
  b.a = hq;
  b.a_scale = hs;
  b.w = w.w2;
  b.w_scale = w.w2_scale;
  b.w3 = nullptr;
  b.w3_scale = nullptr;
  b.K = c.inter;
  b.N = c.hidden;
  b.out = out;
  b.out_fp32 = out_fp32;
  MOE_TRY(fmt == MOE_EXPERTS_NVFP4    ? launch_expert_gemm2_nv(b, bm, mt_max, st)
          : fmt == MOE_EXPERTS_W4AFP8 ? launch_expert_gemm2_w4(b, bm, mt_max, st)
                                      : launch_expert_gemm2(b, bm, mt_max, st));
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_NULL_ARG: return "MOE_ERR_NULL_ARG: a required pointer is NULL";
    case MOE_ERR_BAD_SHAPE: return "MOE_ERR_BAD_SHAPE: a size is outside the supported range";
    case MOE_ERR_MISALIGNED: return "MOE_ERR_MISALIGNED: a pointer is not 16-byte aligned";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL: workspace below moe_workspace_size()";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: combination not implemented";
    case MOE_ERR_ARCH: return "MOE_ERR_ARCH: the current device is not gfx950 (MI355X)";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP call or kernel launch failed";
    case MOE_ERR_SCRATCH_TOO_SMALL:
      return "MOE_ERR_SCRATCH_TOO_SMALL: the call needs more workspace than the static scratch "
             "of moe_layer_noalloc holds (MOE_NOALLOC_SCRATCH_BYTES); use moe_layer";
  }
  return "MOE_ERR_UNKNOWN";
}

size_t moe_workspace_size(const moe_config* cfg, moe_op op) {
  if (check_cfg(cfg) != MOE_OK) return 0;
  Carver cv(nullptr);
  switch (op) {
    case MOE_OP_ROUTE: carve_route(cv, *cfg); break;
    case MOE_OP_EXPERT_FFN: carve_ffn(cv, *cfg); break;
    case MOE_OP_LAYER: carve_layer(cv, *cfg); break;
    default: return 0;
  }
  return cv.off;
}

moe_status moe_quant_act(const uint16_t* x, int64_t rows, int32_t cols, uint8_t* q,
                         uint8_t* scale, void* stream) {
  if (rows < 0 || cols < 128 || cols % 128 || cols > (1 << 20)) return MOE_ERR_BAD_SHAPE;
  if (rows > 0 && (!x || !q || !scale)) return MOE_ERR_NULL_ARG;
  if (rows > 0 && (!aligned16(x) || (reinterpret_cast<uintptr_t>(q) & 7u)))
    return MOE_ERR_MISALIGNED;
  if (rows == 0) return MOE_OK;
  moe_status s = check_device();
  if (s != MOE_OK) return s;
  return hip_status(launch_quant_act(x, rows, cols, q, scale, static_cast<hipStream_t>(stream)));
}

moe_status moe_route(const moe_config* cfg, const uint16_t* x, const uint16_t* w_gate,
                     const float* bias, const int64_t* token_ids, const float* logits_in,
                     float* logits_out, const moe_routing* out, void* ws, size_t ws_bytes,
                     void* stream) {
  moe_status s = check_cfg(cfg);
  if (s != MOE_OK) return s;
  const moe_config& c = *cfg;
  if (!out) return MOE_ERR_NULL_ARG;
  if ((s = check_routing_ptrs(out)) != MOE_OK) return s;
  if (c.route_mode == MOE_ROUTE_HASH) {
    if (c.tokens > 0 && !token_ids) return MOE_ERR_NULL_ARG;
  } else if (!logits_in && c.tokens > 0) {
    if (!x || !w_gate) return MOE_ERR_NULL_ARG;
    if (!aligned16(x) || !aligned16(w_gate)) return MOE_ERR_MISALIGNED;
  }
  if (logits_out && !aligned16(logits_out)) return MOE_ERR_MISALIGNED;
  if (logits_in && !aligned16(logits_in)) return MOE_ERR_MISALIGNED;
  const size_t need = moe_workspace_size(cfg, MOE_OP_ROUTE);
  if (ws_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (need && !ws) return MOE_ERR_NULL_ARG;
  if (!aligned16(ws)) return MOE_ERR_MISALIGNED;
  if ((s = check_device()) != MOE_OK) return s;
  Carver cv(ws);
  RouteWs rws = carve_route(cv, c);
  hipStream_t st = static_cast<hipStream_t>(stream);
  return enqueue_route(c, x, w_gate, bias, token_ids, logits_in, logits_out, *out, rws, st);
}

moe_status moe_expert_ffn(const moe_config* cfg, const uint8_t* xq, const uint8_t* xs,
                          const moe_routing* r, const moe_expert_weights* w, void* out_pairs,
                          uint8_t* hq_out, uint8_t* hs_out, void* ws, size_t ws_bytes,
                          void* stream) {
  moe_status s = check_cfg(cfg);
  if (s != MOE_OK) return s;
  const moe_config& c = *cfg;
  if (!r || !w) return MOE_ERR_NULL_ARG;
  if ((s = check_weights(w)) != MOE_OK) return s;
  if (!r->expert_offsets || !r->sorted_pairs) return MOE_ERR_NULL_ARG;
  if (!aligned16(r->expert_offsets) || !aligned16(r->sorted_pairs)) return MOE_ERR_MISALIGNED;
  if ((hq_out == nullptr) != (hs_out == nullptr)) return MOE_ERR_NULL_ARG;
  if (c.tokens > 0) {
    if (!xq || !xs || !out_pairs) return MOE_ERR_NULL_ARG;
    if (!aligned16(xq) || !aligned16(xs) || !aligned16(out_pairs)) return MOE_ERR_MISALIGNED;
    if (hq_out && (!aligned16(hq_out) || !aligned16(hs_out))) return MOE_ERR_MISALIGNED;
  }
  const size_t need = moe_workspace_size(cfg, MOE_OP_EXPERT_FFN);
  if (ws_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (need && !ws) return MOE_ERR_NULL_ARG;
  if (!aligned16(ws)) return MOE_ERR_MISALIGNED;
  if ((s = check_device()) != MOE_OK) return s;
  Carver cv(ws);
  FfnWs f = carve_ffn(cv, c);
  uint8_t* hq = hq_out ? hq_out : f.hq;
  uint8_t* hs = hs_out ? hs_out : f.hs;
  return enqueue_ffn(c, xq, xs, *r, *w, out_pairs, c.out_fp32, hq, hs, f.mtile_off,
                     static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

// Argument checks of moe_layer, its graph capture and its no-allocation
// variant (everything but the workspace), host-side only.
moe_status layer_args_check(const moe_config* cfg, const uint16_t* x, const uint16_t* w_gate,
                            const float* bias, const int64_t* token_ids,
                            const moe_expert_weights* w, const moe_shared_weights* shared,
                            const uint16_t* y, const moe_routing* routing_out) {
  moe_status s = check_cfg(cfg);
  if (s != MOE_OK) return s;
  const moe_config& c = *cfg;
  if ((s = check_weights(w)) != MOE_OK) return s;
  if (c.tokens > 0) {
    if (!x || !y) return MOE_ERR_NULL_ARG;
    if (!aligned16(x) || !aligned16(y)) return MOE_ERR_MISALIGNED;
    if (c.route_mode == MOE_ROUTE_HASH) {
      if (!token_ids) return MOE_ERR_NULL_ARG;
    } else {
      if (!w_gate) return MOE_ERR_NULL_ARG;
      if (!aligned16(w_gate) || (bias && !aligned16(bias))) return MOE_ERR_MISALIGNED;
    }
  }
  if (shared) {
    if (!shared->w1 || !shared->w3 || !shared->w2) return MOE_ERR_NULL_ARG;
    if (!aligned16(shared->w1) || !aligned16(shared->w3) || !aligned16(shared->w2))
      return MOE_ERR_MISALIGNED;
  }
  if (routing_out && (s = check_routing_ptrs(routing_out)) != MOE_OK) return s;
  return MOE_OK;
}

moe_status layer_check(const moe_config* cfg, const uint16_t* x, const uint16_t* w_gate,
                       const float* bias, const int64_t* token_ids, const moe_expert_weights* w,
                       const moe_shared_weights* shared, const uint16_t* y,
                       const moe_routing* routing_out, const void* ws, size_t ws_bytes) {
  moe_status s = layer_args_check(cfg, x, w_gate, bias, token_ids, w, shared, y, routing_out);
  if (s != MOE_OK) return s;
  const size_t need = moe_workspace_size(cfg, MOE_OP_LAYER);
  if (ws_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (need && !ws) return MOE_ERR_NULL_ARG;
  if (!aligned16(ws)) return MOE_ERR_MISALIGNED;
  return MOE_OK;
}

// Where moe_layer runs a shared expert that does not ride in the routing
// launches: kProcessSide forks it onto the process's per-device side stream
// (under its mutex), kPrivateSide onto a side stream and events the caller
// owns (graph capture: a capture-private pair, so that no other call can
// enqueue onto a stream that joined the capture), kInline on the caller's
// stream after routing (no stream or event is created).
enum class SharedPlacement { kProcessSide, kPrivateSide, kInline };

// The launch sequence of moe_layer (arguments already checked, device
// checked, `ws` large enough).
moe_status layer_enqueue(const moe_config& c, const uint16_t* x, const uint16_t* w_gate,
                         const float* bias, const int64_t* token_ids,
                         const moe_expert_weights* w, const moe_shared_weights* shared,
                         uint16_t* y, const moe_routing* routing_out, void* ws,
                         hipStream_t st, SharedPlacement placement, SideStream* private_side);

}  // namespace

extern "C" {

moe_status moe_layer(const moe_config* cfg, const uint16_t* x, const uint16_t* w_gate,
                     const float* bias, const int64_t* token_ids, const moe_expert_weights* w,
                     const moe_shared_weights* shared, uint16_t* y,
                     const moe_routing* routing_out, void* ws, size_t ws_bytes, void* stream) {
  moe_status s = layer_check(cfg, x, w_gate, bias, token_ids, w, shared, y, routing_out, ws,
                             ws_bytes);
  if (s != MOE_OK) return s;
  if ((s = check_device()) != MOE_OK) return s;
  return layer_enqueue(*cfg, x, w_gate, bias, token_ids, w, shared, y, routing_out, ws,
                       static_cast<hipStream_t>(stream), SharedPlacement::kProcessSide, nullptr);
}

}  // extern "C"

namespace {

moe_status layer_enqueue(const moe_config& c, const uint16_t* x, const uint16_t* w_gate,
                         const float* bias, const int64_t* token_ids,
                         const moe_expert_weights* w, const moe_shared_weights* shared,
                         uint16_t* y, const moe_routing* routing_out, void* ws,
                         hipStream_t st, SharedPlacement placement, SideStream* private_side) {
  moe_status s = MOE_OK;
  Carver cv(ws);
  LayerWs l = carve_layer(cv, c);
  const moe_routing& r = routing_out ? *routing_out : l.routing;
  if (c.tokens == 0)
    return enqueue_route(c, x, w_gate, bias, token_ids, nullptr, nullptr, r, l.route, st);

  // Caller's stream: quantize x, route, routed experts, combine.  Decode-sized
  // batches with score routing carry the shared expert inside the routing
  // launches (split-K up projection beside the router, SwiGLU beside the
  // top-k, split-K down projection beside the permutation; the combine adds
  // the down slices): one stream, no fork and join, whose two cross-stream
  // waits cost ~5 us each at T = 64.  Otherwise the shared expert (which
  // needs only x) runs on the side stream and joins before the combine.
  // Small batches fork it once routing is enqueued, so that it overlaps the
  // bandwidth-bound expert GEMMs rather than the latency-bound routing
  // kernels (forking first cost 2% at T = 64); batches of at least
  // kEarlyForkTokens fork it early, where its GEMMs are long enough to fill
  // the GPU the routing kernels leave idle: hash routing before the
  // quantization (1.6% less layer time at T = 32768 than forking after
  // routing), score routing right after the router GEMM is enqueued -- forked
  // before it, the shared up projection's workgroups took the GPU first and
  // the router GEMM, on the critical path, waited for slots (184 us at
  // T = 4096; the layer 1.5% slower).
  const bool quant_in_router =
      c.route_mode == MOE_ROUTE_SQRTSOFTPLUS && router_splits(c.tokens, c.hidden) > 1;
  const bool fused_shared = shared && quant_in_router &&
                            router_tile_splits(c.tokens, c.hidden, c.n_experts) == 1 &&
                            shared_split_ok(c.tokens, c.hidden, c.inter) &&
                            c.tokens * c.top_k <= kFusedMaxPairs;
  SharedFused sf{};
  if (fused_shared)
    sf = SharedFused{shared->w1, shared->w3, shared->w2, l.hsh, l.shpart, (int)c.tokens,
                     c.hidden, c.inter, c.swiglu_limit};
  const float* ysh = nullptr;
  int ysh_parts = 1;
  std::unique_lock<std::mutex> lock;
  SideStream* side = nullptr;
  auto fork_shared = [&]() -> moe_status {
    if (placement == SharedPlacement::kInline) {
      // no side stream: the shared expert's GEMMs run here, in stream order
      MOE_TRY(launch_shared_up(x, shared->w1, shared->w3, l.hsh, l.shpart, c.tokens, c.hidden,
                               c.inter, c.swiglu_limit, st));
      MOE_TRY(launch_shared_down(l.hsh, shared->w2, l.ysh, l.shpart, c.tokens, c.hidden,
                                 c.inter, st));
      ysh = l.ysh;
      return MOE_OK;
    }
    if (placement == SharedPlacement::kPrivateSide) {
      side = private_side;
    } else {
      if ((s = side_stream(side)) != MOE_OK) return s;
      lock = std::unique_lock<std::mutex>(side->mu);
      if ((s = side_init_locked(*side)) != MOE_OK) return s;
    }
    hipStream_t ss = side->stream;
    MOE_TRY(hipEventRecord(side->fork, st));
    MOE_TRY(hipStreamWaitEvent(ss, side->fork, 0));
    MOE_TRY(launch_shared_up(x, shared->w1, shared->w3, l.hsh, l.shpart, c.tokens, c.hidden,
                             c.inter, c.swiglu_limit, ss));
    MOE_TRY(launch_shared_down(l.hsh, shared->w2, l.ysh, l.shpart, c.tokens, c.hidden, c.inter,
                               ss));
    MOE_TRY(hipEventRecord(side->join, ss));
    ysh = l.ysh;
    return MOE_OK;
  };
  const bool side_shared = shared && !fused_shared;
  const bool early_fork = side_shared && c.tokens >= kEarlyForkTokens &&
                          placement != SharedPlacement::kInline;
  // score routing forks right after the router GEMM is enqueued, hash routing
  // before the quantization
  const bool fork_after_router = early_fork && c.route_mode == MOE_ROUTE_SQRTSOFTPLUS;
  if (early_fork && !fork_after_router && (s = fork_shared()) != MOE_OK) return s;
  const std::function<moe_status()> fork_fn = fork_shared;
  // small score-routed batches quantize x inside the split-K router launch
  if (!quant_in_router) MOE_TRY(launch_quant_act(x, c.tokens, c.hidden, l.xq, l.xs, st));
  bool tiles_done = false;
  if ((s = enqueue_route(c, x, w_gate, bias, token_ids, nullptr, nullptr, r, l.route, st,
                         l.ffn.mtile_off, &tiles_done, quant_in_router ? l.xq : nullptr,
                         quant_in_router ? l.xs : nullptr, fused_shared ? &sf : nullptr,
                         fork_after_router ? &fork_fn : nullptr)) != MOE_OK)
    return s;
  if (side_shared && !early_fork && (s = fork_shared()) != MOE_OK) return s;
  if ((s = enqueue_ffn(c, l.xq, l.xs, r, *w, l.o, 1, l.ffn.hq, l.ffn.hs, l.ffn.mtile_off, st,
                       tiles_done)) != MOE_OK)
    return s;
  if (side_shared && placement != SharedPlacement::kInline)
    MOE_TRY(hipStreamWaitEvent(st, side->join, 0));
  if (fused_shared) {
    ysh = l.shpart;
    ysh_parts = c.inter / kSharedSplitK;
  }
  MOE_TRY(launch_combine(l.o, r.topk_w, r.pair_pos, ysh, ysh_parts, y, c.tokens, c.hidden,
                         c.top_k, st));
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_expert_cast_fp8(const moe_config* cfg, const moe_expert_weights* src,
                               const moe_expert_weights* dst, void* stream) {
  moe_status s = check_cfg(cfg);
  if (s != MOE_OK) return s;
  if ((s = check_weights(src)) != MOE_OK || (s = check_weights(dst)) != MOE_OK) return s;
  if ((s = check_device()) != MOE_OK) return s;
  const moe_config& c = *cfg;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t E = c.n_experts;
  MOE_TRY(launch_cast_fp8(src->w1, src->w1_scale, const_cast<uint8_t*>(dst->w1),
                          const_cast<uint8_t*>(dst->w1_scale), E * c.inter, c.hidden, st));
  MOE_TRY(launch_cast_fp8(src->w3, src->w3_scale, const_cast<uint8_t*>(dst->w3),
                          const_cast<uint8_t*>(dst->w3_scale), E * c.inter, c.hidden, st));
  MOE_TRY(launch_cast_fp8(src->w2, src->w2_scale, const_cast<uint8_t*>(dst->w2),
                          const_cast<uint8_t*>(dst->w2_scale), E * c.hidden, c.inter, st));
  return MOE_OK;
}

struct moe_graph {
  hipGraphExec_t exec;
};

moe_status moe_layer_graph_create(const moe_config* cfg, const uint16_t* x,
                                  const uint16_t* w_gate, const float* bias,
                                  const int64_t* token_ids, const moe_expert_weights* w,
                                  const moe_shared_weights* shared, uint16_t* y,
                                  const moe_routing* routing_out, void* ws, size_t ws_bytes,
                                  moe_graph** graph_out) {
  if (!graph_out) return MOE_ERR_NULL_ARG;
  *graph_out = nullptr;
  moe_status s = layer_check(cfg, x, w_gate, bias, token_ids, w, shared, y, routing_out, ws,
                             ws_bytes);
  if (s != MOE_OK) return s;
  if ((s = check_device()) != MOE_OK) return s;
  // the capture stream and, for a shared expert on a side stream, a side
  // stream and two events of this capture's own: a stream that joined the
  // capture stays in it until hipStreamEndCapture, so no other call may
  // enqueue onto it meanwhile
  hipStream_t cs = nullptr;
  SideStream priv;
  auto release = [&]() {
    if (priv.join) (void)hipEventDestroy(priv.join);
    if (priv.fork) (void)hipEventDestroy(priv.fork);
    if (priv.stream) (void)hipStreamDestroy(priv.stream);
    if (cs) (void)hipStreamDestroy(cs);
  };
  if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess ||
      (shared && side_init_locked(priv) != MOE_OK) ||
      hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess) {
    release();
    return MOE_ERR_HIP;
  }
  s = layer_enqueue(*cfg, x, w_gate, bias, token_ids, w, shared, y, routing_out, ws, cs,
                    SharedPlacement::kPrivateSide, &priv);
  hipGraph_t g = nullptr;
  const hipError_t ec = hipStreamEndCapture(cs, &g);
  if (s == MOE_OK && (ec != hipSuccess || !g)) s = MOE_ERR_HIP;
  hipGraphExec_t ge = nullptr;
  if (s == MOE_OK && hipGraphInstantiate(&ge, g, nullptr, nullptr, 0) != hipSuccess) s = MOE_ERR_HIP;
  if (g) (void)hipGraphDestroy(g);
  release();
  if (s != MOE_OK) return s;
  moe_graph* h = new (std::nothrow) moe_graph{ge};
  if (!h) {
    (void)hipGraphExecDestroy(ge);
    return MOE_ERR_HIP;
  }
  *graph_out = h;
  return MOE_OK;
}

moe_status moe_graph_launch(const moe_graph* graph, void* stream) {
  if (!graph) return MOE_ERR_NULL_ARG;
  return hip_status(hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream)));
}

moe_status moe_graph_destroy(moe_graph* graph) {
  if (!graph) return MOE_OK;
  const hipError_t e = hipGraphExecDestroy(graph->exec);
  delete graph;
  return hip_status(e);
}

}  // extern "C"

// Workspace of moe_layer_noalloc: a device array of MOE_NOALLOC_SCRATCH_BYTES
// in this library's code object, one copy per device, alive until the process
// ends.  Host code never passes `scratch` itself to a kernel (on the host the
// name is only a registration handle); it takes the device address from
// hipGetSymbolAddress once per device and uses that.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

struct ScratchAddr {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchAddr g_scratch[64];

// Device address of `scratch` on the current device (looked up on the first
// call per device, with that device current).
moe_status scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_ERR_HIP;
  ScratchAddr& a = g_scratch[dev];
  std::call_once(a.once, [&a]() {
    a.err = hipGetSymbolAddress(&a.ptr, HIP_SYMBOL(scratch));
  });
  if (a.err != hipSuccess || !a.ptr) return MOE_ERR_HIP;
  *out = a.ptr;
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_layer_noalloc(const moe_config* cfg, const uint16_t* x, const uint16_t* w_gate,
                             const float* bias, const int64_t* token_ids,
                             const moe_expert_weights* w, const moe_shared_weights* shared,
                             uint16_t* y, const moe_routing* routing_out, void* stream) {
  moe_status s = layer_args_check(cfg, x, w_gate, bias, token_ids, w, shared, y, routing_out);
  if (s != MOE_OK) return s;
  if (moe_workspace_size(cfg, MOE_OP_LAYER) > MOE_NOALLOC_SCRATCH_BYTES)
    return MOE_ERR_SCRATCH_TOO_SMALL;
  if ((s = check_device()) != MOE_OK) return s;
  void* ws = nullptr;
  if ((s = scratch_address(&ws)) != MOE_OK) return s;
  return layer_enqueue(*cfg, x, w_gate, bias, token_ids, w, shared, y, routing_out, ws,
                       static_cast<hipStream_t>(stream), SharedPlacement::kInline, nullptr);
}

}  // extern "C"
