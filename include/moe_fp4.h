/*
 * moe_fp4.h - C ABI of a routed mixture-of-experts FFN layer with block-scaled
 * FP4 experts and sqrtsoftplus routing, for AMD Instinct MI355X (gfx950).
 *
 * What the layer computes (sources are the pages this library follows):
 *
 *  "DeepSeek-V4-Flash-SI" model card, section 架构特性 (Mixture of Experts):
 *    each layer has 256 routed experts and 1 shared expert; every token picks
 *    its top-6 routed experts through the gate network, scored with
 *    sqrtsoftplus (the first three layers use hash routing, a deterministic
 *    choice from the token id instead); routing scale 1.5; SwiGLU with its
 *    activation clamped to +-10.
 *  same card, section 架构特性 (低精度计算): expert weights are FP4 E2M1 with
 *    one F8_E8M0 block scale per 32 elements; activations are quantized online
 *    to FP8 E4M3 in groups of 128 elements with a power-of-two scale;
 *    non-expert weights (gate, shared expert) stay bf16.
 *  same card, 模型训练 table: dynamic FP8 E4M3 activation quant, ue8m0 scale.
 *  "DeepSeek-V4-Flash-0731-W4AFP8-mt" card, sections 量化方式 / 权重约定:
 *    expert tensors are w1, w2, w3, stored [N, K/2] with two 4-bit values
 *    per byte (the example w1 is [2048, 2048] bytes for K = 4096).
 *  "如何自己复现DeepSeek-V4.1-Flash-Quark-PTPC-FP8" article, 排除清单: the gate
 *    (*ffn.gate*) is never quantized.
 *
 * Readings taken where the pages are silent (the oracle follows the same):
 *  - E2M1: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit; E8M0 byte b is
 *    2^(b-127); E4M3 is the OCP "fn" variant (max 448, no infinities),
 *    rounded to nearest even.
 *  - Inside a weight byte the even K element is the low nibble.
 *  - Activation scale per 128 elements: 2^e with e the smallest integer such
 *    that max|v| <= 448 * 2^e (an all-zero block takes e = -127), stored as
 *    the E8M0 byte e + 127.
 *  - Router: z = x W_gate^T in fp32; s = sqrt(ln(1 + e^z)) evaluated in
 *    double and rounded to fp32; key = s + bias (bias optional, selection
 *    only); the k largest keys win, equal keys go to the lower expert id;
 *    weights w_j = (s_j / sum_selected s) * route_scale in fp32, the sum taken
 *    in rank order.
 *  - Hash routing: SplitMix64 seeded with (hash_seed << 32) ^ token_id; each
 *    output r gives r mod E, r >= 2^64 - (2^64 mod E) is rejected, repeated
 *    experts are skipped; the first k distinct experts in draw order, each
 *    weighted route_scale / k.
 *  - Expert FFN: w1 is the gate, w3 the up projection; both SwiGLU inputs are
 *    clamped to [-limit, limit]; h = silu(g) * u is requantized to FP8 per 128
 *    before w2; the routing weight is applied after w2.
 *  - Shared expert: the same clamped SwiGLU in bf16, h rounded to bf16 before
 *    its down projection, added with weight 1.
 *  - Combine: y[t] = sum_j w[t,j] * o[t,j] + shared[t] (fp32), rounded to bf16.
 *  - No capacity limit: every (token, expert) pair is computed.
 *
 * Conventions of every entry point:
 *  - All tensor pointers are DEVICE pointers to caller-owned, contiguous,
 *    row-major memory, 16-byte aligned. The library allocates no device
 *    memory for a call (scratch comes from the caller's workspace), keeps no
 *    data between calls and never copies data to the host.
 *  - Process-level resources the library keeps (created on first use, held
 *    until the process ends, never freed by a call): per device, a cached
 *    architecture check and the CU count; for moe_layer calls that run the
 *    shared expert on a second stream (see moe_layer), one side stream
 *    (default priority, non-blocking), two events (timing disabled) and a
 *    mutex that keeps concurrent calls' fork/join pairs from interleaving;
 *    for moe_layer_noalloc, its static device scratch.
 *    moe_layer_graph_create makes a capture stream and, with a shared
 *    expert, a side stream and two events of its own, and destroys them
 *    before it returns; the graph it returns holds its instantiated graph
 *    until moe_graph_destroy.
 *  - `stream` is a hipStream_t (NULL = the default stream). Every call
 *    validates its arguments on the host, enqueues its kernels on `stream`
 *    and returns; nothing is synchronised. Results are ready when the stream
 *    reaches the call.
 *  - Argument errors are reported before anything is enqueued (no GPU call
 *    is made for them). Calls on distinct streams with distinct workspaces
 *    may run concurrently.
 *  - Inputs must be finite; NaN/Inf inputs give unspecified results.
 *  - bf16 tensors are passed as uint16_t bit patterns.
 */
#ifndef MOE_FP4_H
#define MOE_FP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_NULL_ARG = 1,            /* a required pointer is NULL              */
  MOE_ERR_BAD_SHAPE = 2,           /* a size is out of the supported range    */
  MOE_ERR_MISALIGNED = 3,          /* a pointer is not 16-byte aligned        */
  MOE_ERR_WORKSPACE_TOO_SMALL = 4, /* ws_bytes < moe_workspace_size(...)      */
  MOE_ERR_UNSUPPORTED = 5,         /* a valid but unimplemented combination   */
  MOE_ERR_ARCH = 6,                /* the current device is not gfx950        */
  MOE_ERR_HIP = 7,                 /* a HIP launch reported an error          */
  MOE_ERR_SCRATCH_TOO_SMALL = 8    /* moe_layer_noalloc: the call needs more
                                      than MOE_NOALLOC_SCRATCH_BYTES        */
} moe_status;

typedef enum moe_route_mode {
  MOE_ROUTE_SQRTSOFTPLUS = 0, /* gate logits -> sqrtsoftplus -> top-k       */
  MOE_ROUTE_HASH = 1          /* SplitMix64 over the token id -> k experts  */
} moe_route_mode;

/* Routed expert weight format ("DeepSeek-V4-Pro-0813-nvfp4-DSpark" article,
 * 阶段一: the MXFP4 checkpoint, or its lossless per-128 cast to FP8 experts). */
typedef enum moe_expert_format {
  MOE_EXPERTS_MXFP4 = 0,      /* E2M1 nibbles + E8M0 per 32 (the checkpoint) */
  MOE_EXPERTS_FP8 = 1,        /* E4M3 bytes + E8M0 per 128                   */
  MOE_EXPERTS_NVFP4 = 2,      /* E2M1 nibbles + E4M3 per 16 (阶段三导出);
                                 needs hidden % 512 == 0 and inter % 512 == 0,
                                 else MOE_ERR_UNSUPPORTED                   */
  MOE_EXPERTS_W4AFP8 = 3      /* signed INT4 + float32 per 128
                                 ("DeepSeek-V4-Flash-0731-W4AFP8-mt" card,
                                 量化方式 / 权重约定); same size limits as NVFP4 */
} moe_expert_format;

typedef enum moe_op {
  MOE_OP_ROUTE = 0,
  MOE_OP_EXPERT_FFN = 1,
  MOE_OP_LAYER = 2
} moe_op;

/* Supported ranges (checked; MOE_ERR_BAD_SHAPE otherwise):
 *   0 <= tokens, tokens * top_k < 2^31;
 *   hidden, inter: multiples of 128 in [128, 16384];
 *   1 <= n_experts <= 512;  1 <= top_k <= min(8, n_experts);
 *   route_scale finite; swiglu_limit > 0 (+inf disables the clamp). */
typedef struct moe_config {
  int64_t tokens;      /* T: rows of x                                     */
  int32_t hidden;      /* H: model width (K of w1/w3, N of w2)             */
  int32_t inter;       /* I: expert intermediate width                     */
  int32_t n_experts;   /* E: routed experts                                */
  int32_t top_k;       /* k: experts per token                             */
  float route_scale;   /* 1.5 on the pages                                 */
  float swiglu_limit;  /* 10.0 on the pages                                */
  int32_t route_mode;  /* moe_route_mode                                   */
  int32_t out_fp32;    /* moe_expert_ffn: 1 -> out_pairs fp32, 0 -> bf16   */
  uint64_t hash_seed;  /* MOE_ROUTE_HASH only                              */
  int32_t expert_format; /* moe_expert_format of the routed expert weights  */
  int32_t reserved;      /* set to 0                                       */
} moe_config;

/* Routed expert weights, stacked over experts, checkpoint layout:
 *   w1, w3:             [E, I, H/2] bytes, E2M1 nibbles along H (K)
 *   w1_scale, w3_scale: [E, I, H/32] E8M0 bytes
 *   w2:                 [E, H, I/2] bytes, E2M1 nibbles along I (K)
 *   w2_scale:           [E, H, I/32] E8M0 bytes
 * With expert_format MOE_EXPERTS_FP8: w1, w3 [E, I, H] and w2 [E, H, I]
 * E4M3 bytes, scales [E, I, H/128] and [E, H, I/128] E8M0 bytes
 * (moe_expert_cast_fp8 writes them).  With MOE_EXPERTS_NVFP4: the nibble
 * arrays as for MXFP4, scales [E, I, H/16] and [E, H, I/16] E4M3 bytes
 * (one per 16 elements of K, no per-tensor scale).  With
 * MOE_EXPERTS_W4AFP8: the same byte arrays hold two's complement INT4
 * pairs (even element of K in the low nibble) and the scale pointers point
 * to float32 arrays [E, I, H/128] and [E, H, I/128], 16-byte aligned, that
 * multiply the integers (the checkpoint's weight_scale_inv).            */
typedef struct moe_expert_weights {
  const uint8_t* w1;
  const uint8_t* w1_scale;
  const uint8_t* w3;
  const uint8_t* w3_scale;
  const uint8_t* w2;
  const uint8_t* w2_scale;
} moe_expert_weights;

/* Shared expert, bf16: w1, w3 [I, H]; w2 [H, I]. */
typedef struct moe_shared_weights {
  const uint16_t* w1;
  const uint16_t* w3;
  const uint16_t* w2;
} moe_shared_weights;

/* Routing of T tokens, P = T * k pairs, pair p = t * k + j (j = rank):
 *   topk_idx       [T, k] int32, experts in rank order
 *   topk_w         [T, k] fp32, routing weights
 *   expert_offsets [E + 1] int32, exclusive prefix of pairs per expert
 *   sorted_pairs   [P] int32, pair ids grouped by expert, ascending p
 *                  within an expert (a stable counting sort)
 *   pair_pos       [P] int32, inverse: sorted_pairs[pair_pos[p]] == p     */
typedef struct moe_routing {
  int32_t* topk_idx;
  float* topk_w;
  int32_t* expert_offsets;
  int32_t* sorted_pairs;
  int32_t* pair_pos;
} moe_routing;

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_str(moe_status s);

/* Bytes of device workspace `op` needs for `cfg` (0 if cfg is invalid or
 * NULL). Pure host function. The layer's workspace holds the FP8 copies of x
 * and h, the per-pair expert outputs (P x H fp32), the shared expert's h and
 * output, and the routing scratch. */
size_t moe_workspace_size(const moe_config* cfg, moe_op op);

/* Online FP8 activation quantization ("DeepSeek-V4-Flash-SI" card,
 * 低精度计算; 模型训练 table): rows of `cols` bf16 values, cols % 128 == 0.
 *   x      [rows, cols] bf16
 *   q      [rows, cols] E4M3 bytes (out)
 *   scale  [rows, cols/128] E8M0 bytes (out)
 * rows == 0 is a no-op. x, q, scale need 16, 8 and 1-byte alignment. */
moe_status moe_quant_act(const uint16_t* x, int64_t rows, int32_t cols,
                         uint8_t* q, uint8_t* scale, void* stream);

/* Routing ("DeepSeek-V4-Flash-SI" card, 架构特性 MoE paragraph).
 * Score mode: logits z = x W_gate^T (x [T, H] bf16, w_gate [E, H] bf16) unless
 *   logits_in [T, E] fp32 is given (then x and w_gate may be NULL); bias [E]
 *   fp32 or NULL; logits_out [T, E] fp32 or NULL receives z.
 * Hash mode: token_ids [T] int64 required; x, w_gate, bias, logits ignored.
 * Writes every array of `out` (all required). `ws` needs
 * moe_workspace_size(cfg, MOE_OP_ROUTE) bytes. */
moe_status moe_route(const moe_config* cfg, const uint16_t* x, const uint16_t* w_gate,
                     const float* bias, const int64_t* token_ids, const float* logits_in,
                     float* logits_out, const moe_routing* out, void* ws, size_t ws_bytes,
                     void* stream);

/* Routed experts on pre-quantized activations (w1|w3 -> clamped SwiGLU ->
 * FP8 requant -> w2), in sorted-pair order ("DeepSeek-V4-Flash-SI" card,
 * 架构特性: the MoE paragraph's SwiGLU with its activation clamped to
 * +-limit for every selected expert; the 低精度计算 paragraph's FP4 E2M1
 * weights with an E8M0 scale per 32 and online FP8 E4M3 activations with a
 * power-of-two scale per 128 -- here both expert inputs, x and h).
 *   xq [T, H] E4M3, xs [T, H/128] E8M0 (from moe_quant_act)
 *   r: expert_offsets and sorted_pairs are read (topk_* and pair_pos unused)
 *   out_pairs [P, H]: fp32 if cfg->out_fp32 else bf16; row i belongs to
 *     pair r->sorted_pairs[i]; unweighted expert output
 *   hq_out [P, I] E4M3 and hs_out [P, I/128] E8M0: NULL, or both given to
 *     receive the requantized SwiGLU activations
 * `ws` needs moe_workspace_size(cfg, MOE_OP_EXPERT_FFN) bytes. */
moe_status moe_expert_ffn(const moe_config* cfg, const uint8_t* xq, const uint8_t* xs,
                          const moe_routing* r, const moe_expert_weights* w, void* out_pairs,
                          uint8_t* hq_out, uint8_t* hs_out, void* ws, size_t ws_bytes,
                          void* stream);

/* The whole layer ("DeepSeek-V4-Flash-SI" card, 架构特性: the MoE
 * paragraph's per-token top-k routed experts -- sqrtsoftplus scores, or hash
 * routing from the token id -- with routing scale 1.5, plus one shared
 * expert, every expert a SwiGLU clamped to +-limit; the 低精度计算
 * paragraph's FP4 expert weights, online FP8 activations and bf16 gate and
 * shared expert): route, quantize x, routed experts, shared expert (if
 * `shared` is non-NULL), weighted combine.  A shared expert that does not
 * ride in the decode-sized routing launches runs on this library's side
 * stream for the device, forked from `stream` and joined back before the
 * combine (see the conventions above).
 *   x [T, H] bf16; w_gate [E, H] bf16 (score mode); bias [E] fp32 or NULL;
 *   token_ids [T] int64 (hash mode); y [T, H] bf16 (out).
 *   routing_out: NULL, or arrays that receive the routing (all required).
 * `ws` needs moe_workspace_size(cfg, MOE_OP_LAYER) bytes. */
moe_status moe_layer(const moe_config* cfg, const uint16_t* x, const uint16_t* w_gate,
                     const float* bias, const int64_t* token_ids, const moe_expert_weights* w,
                     const moe_shared_weights* shared, uint16_t* y,
                     const moe_routing* routing_out, void* ws, size_t ws_bytes, void* stream);

/* MXFP4 -> FP8 expert weights ("DeepSeek-V4-Pro-0813-nvfp4-DSpark" article,
 * 阶段一, 关于 MXFP4 的无损种子): per row and 128 elements of K the new E8M0
 * exponent is the largest of the four per-32 exponents, and each element is
 * the E4M3 code (round to nearest even, sign kept) of its E2M1 value times
 * 2^(its exponent - the new one).  Lossless when the four exponents of every
 * block span at most 8.  src: MXFP4 layout, dst: FP8 layout (see
 * moe_expert_weights), both for cfg's E, H, I (cfg->expert_format ignored);
 * caller-owned device buffers, 16-byte aligned, not overlapping. */
moe_status moe_expert_cast_fp8(const moe_config* cfg, const moe_expert_weights* src,
                               const moe_expert_weights* dst, void* stream);

/* Graph replay of the layer ("DeepSeek-V4-Flash-SI" card, 模型推理 /
 * 推理模式: the MoE GEMM path captured into a graph to cut kernel-launch
 * overhead; 模型效果 / 质量标准: graph output identical to eager).
 * moe_layer_graph_create records one moe_layer call (same arguments, no
 * stream) into a HIP graph on a private stream and instantiates it; every
 * pointer, the config and the shared/routing structs' contents are baked in.
 * moe_graph_launch replays it on `stream`: the caller updates x (and any
 * inputs) in place between replays and keeps every buffer, the weights and
 * `ws` alive until moe_graph_destroy.  Replays of one graph must not overlap
 * each other or an eager call on the same workspace.  The graph contains no
 * memset nodes.  Errors: those of moe_layer (nothing is created), or
 * MOE_ERR_HIP if capture or instantiation fails; *graph_out is NULL then. */
typedef struct moe_graph moe_graph;
moe_status moe_layer_graph_create(const moe_config* cfg, const uint16_t* x,
                                  const uint16_t* w_gate, const float* bias,
                                  const int64_t* token_ids, const moe_expert_weights* w,
                                  const moe_shared_weights* shared, uint16_t* y,
                                  const moe_routing* routing_out, void* ws, size_t ws_bytes,
                                  moe_graph** graph_out);
moe_status moe_graph_launch(const moe_graph* graph, void* stream);
moe_status moe_graph_destroy(moe_graph* graph);   /* NULL is a no-op */

/* moe_layer without a workspace argument, for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses
 * that forbid allocation).  It runs the same kernels as moe_layer on a
 * static device scratch array of MOE_NOALLOC_SCRATCH_BYTES that the library
 * holds on every device it runs on until the process ends; it calls no
 * allocation routine and creates no stream or event (a shared expert that
 * moe_layer would fork onto its side stream runs on `stream` in order).
 * Arguments and results are those of moe_layer.
 * Errors: those of moe_layer's argument checks, reported before any GPU
 * call; MOE_ERR_SCRATCH_TOO_SMALL when moe_workspace_size(cfg,
 * MOE_OP_LAYER) exceeds the scratch (then nothing is enqueued; moe_layer
 * with a caller workspace handles the call).  64 MiB hold, e.g., the layer
 * at hidden 4096, inter 2048, 256 experts, top-6 up to 256 tokens.
 * Every call on a device shares that device's scratch and leaves its
 * contents behind (no kernel needs it cleared): calls that may overlap on
 * one device -- on different streams, or from different threads without
 * ordering -- race on it and must not be issued. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_layer_noalloc(const moe_config* cfg, const uint16_t* x, const uint16_t* w_gate,
                             const float* bias, const int64_t* token_ids,
                             const moe_expert_weights* w, const moe_shared_weights* shared,
                             uint16_t* y, const moe_routing* routing_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FP4_H */
