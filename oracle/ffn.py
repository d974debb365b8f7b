"""Expert FFN, shared expert, combine and the whole layer (oracle; test
infrastructure only).

"DeepSeek-V4-Flash-SI" card, 架构特性: each token runs its 6 selected routed
experts plus one shared expert; SwiGLU activation with a +-10 clamp; expert
weights FP4 E2M1 + E8M0/32, activations FP8 E4M3 per 128 with a power-of-two
scale, non-expert weights bf16.  Expert tensors are named w1, w2, w3 (the
W4AFP8-mt card, 量化方式); w2 is the down projection (the QLoRA card maps
shared_experts.w2 to down_proj).

Readings where the pages are silent (listed with the others in the design
notes):
* w1 is the gate projection (inside silu), w3 the up projection;
* the clamp bounds both SwiGLU inputs: h = silu(clip(g)) * clip(u);
* both routed GEMM inputs (x and h) are FP8-quantized per 128; h is rounded
  to fp32 (the GEMM accumulator precision) before its quantization;
* the routing weight is applied after w2, in the combine;
* the shared expert runs in bf16 with the same clamped SwiGLU; its h is
  rounded to bf16 before its down projection; it is added with weight 1;
* the combine sums the k weighted expert outputs in rank order, then adds the
  shared expert; the layer output is that sum rounded to bf16.

All GEMMs here are float64 sums of exactly dequantized operands (dequantized
FP4 x FP8 products have at most 7 significant bits, so these sums are exact
or within a few float64 ulps).
"""

from concurrent.futures import ThreadPoolExecutor

import numpy as np
from threadpoolctl import threadpool_limits

from . import formats, quant, route as route_mod


def silu(v):
    v = np.asarray(v, dtype=np.float64)
    return v / (1.0 + np.exp(-v))


def clamped_swiglu(g, u, limit):
    gc = np.clip(g, -limit, limit)
    uc = np.clip(u, -limit, limit)
    return silu(gc) * uc


def expert_ffn(xq, xs, routing, w, top_k, limit=10.0, experts=None, weight_format="mxfp4",
               out=None):
    """Routed experts on quantized activations.

    xq u8 [T, H], xs u8 [T, H/128]; routing from route.route; w dict with
    w1, w1_scale, w3, w3_scale ([E, I, H/2], [E, I, H/32]) and w2, w2_scale
    ([E, H, I/2], [E, H, I/32]); with weight_format "fp8" the FP8 expert
    layout instead: [E, N, K] E4M3 bytes with [E, N, K/128] scales; with
    "nvfp4" the same nibbles with [E, N, K/16] E4M3 scales; with "w4afp8"
    the nibbles are signed INT4 with [E, N, K/128] float32 scales.
    Returns dict: hq u8 [P, I], hs u8 [P, I/128], h fp32 [P, I] (before its
    quantization) and o float64 [P, H], all rows in sorted-pair order.
    `experts` (a list of expert ids) computes only those experts' rows, the
    others are left zero; `out` (a dict of such arrays) receives the rows in
    place of new arrays.  Experts are independent, so callers may run
    disjoint expert lists at once into one `out`.
    """
    off = routing["expert_offsets"]
    sp = routing["sorted_pairs"]
    P = sp.size
    E = off.size - 1
    I = w["w1"].shape[1]
    H = w["w2"].shape[1]
    deq = {"mxfp4": quant.mxfp4_dequant, "fp8": quant.fp8_dequant,
           "nvfp4": quant.nvfp4_dequant, "w4afp8": quant.int4_dequant}[weight_format]
    if out is None:
        out = {"hq": np.zeros((P, I), np.uint8), "hs": np.zeros((P, I // 128), np.uint8),
               "h": np.zeros((P, I), np.float32), "o": np.zeros((P, H), np.float64)}
    hq, hs, hf, o = out["hq"], out["hs"], out["h"], out["o"]
    for e in (range(E) if experts is None else experts):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        tok = sp[lo:hi] // top_k
        xd = quant.act_dequant(xq[tok], xs[tok])
        W1 = deq(w["w1"][e], w["w1_scale"][e])
        W3 = deq(w["w3"][e], w["w3_scale"][e])
        W2 = deq(w["w2"][e], w["w2_scale"][e])
        g = xd @ W1.T
        u = xd @ W3.T
        h = clamped_swiglu(g, u, limit).astype(np.float32)
        q, s = quant.act_quant(h.astype(np.float64))
        hq[lo:hi], hs[lo:hi], hf[lo:hi] = q, s, h
        o[lo:hi] = quant.act_dequant(q, s) @ W2.T
    return out


def shared_expert(x_u16, w1_u16, w3_u16, w2_u16, limit=10.0):
    """bf16 shared expert: ysh = bf16(clamped_swiglu(x W1^T, x W3^T)) W2^T."""
    x = formats.bf16_decode(x_u16)
    g = x @ formats.bf16_decode(w1_u16).T
    u = x @ formats.bf16_decode(w3_u16).T
    h = formats.bf16_round(clamped_swiglu(g, u, limit))
    return h @ formats.bf16_decode(w2_u16).T


def combine(o, routing, ysh=None):
    """y[t] = sum_j w[t, j] * o[pair_pos[t*k + j]] (+ ysh[t]), j in rank order."""
    w = routing["topk_w"].astype(np.float64)
    T, k = w.shape
    pp = routing["pair_pos"].reshape(T, k)
    y = np.zeros((T, o.shape[1]), np.float64)
    for j in range(k):
        y += w[:, j:j + 1] * o[pp[:, j]]
    if ysh is not None:
        y += ysh
    return y


def layer(inp, top_k, route_scale=1.5, limit=10.0, mode="score", hash_seed=0,
          weight_format="mxfp4", workers=1):
    """The whole MoE FFN layer on the inputs of synth.make_inputs; with
    weight_format "fp8" the routed experts run on the FP8 cast of the MXFP4
    weights (quant.fp8_experts_from_mxfp4); with "nvfp4" inp's w*_scale are
    the NVFP4 per-16 E4M3 scales of the same nibbles; with "w4afp8" the
    nibbles are INT4 codes and inp's w*_scale their float32 per-128 scales.

    `workers` > 1 runs the experts on that many threads, each on its own
    experts (the results do not depend on it).

    Returns dict with the routing, xq/xs, hq/hs, o, ysh (or None), y (float64)
    and y_bf16 (uint16 bit patterns)."""
    x = inp["x"]
    xq, xs = quant.act_quant(formats.bf16_decode(x))
    if mode == "hash":
        r = route_mod.route(k=top_k, route_scale=route_scale, mode="hash",
                            token_ids=inp["token_ids"], seed=hash_seed,
                            n_experts=inp["w1"].shape[0])
    else:
        r = route_mod.route(x, inp["w_gate"], k=top_k, bias=inp.get("bias"),
                            route_scale=route_scale)
    w = quant.fp8_experts_from_mxfp4(inp) if weight_format == "fp8" else inp
    if workers <= 1:
        f = expert_ffn(xq, xs, r, w, top_k, limit, weight_format=weight_format)
    else:
        P, I, H = r["sorted_pairs"].size, w["w1"].shape[1], w["w2"].shape[1]
        f = {"hq": np.zeros((P, I), np.uint8), "hs": np.zeros((P, I // 128), np.uint8),
             "h": np.zeros((P, I), np.float32), "o": np.zeros((P, H), np.float64)}
        used = [e for e in range(r["expert_offsets"].size - 1)
                if r["expert_offsets"][e + 1] > r["expert_offsets"][e]]
        # one BLAS thread per worker: the workers already fill the cores
        with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
            list(ex.map(lambda es: expert_ffn(xq, xs, r, w, top_k, limit, experts=es,
                                              weight_format=weight_format, out=f),
                        [used[i::workers] for i in range(workers)]))
    ysh = None
    if inp.get("shared_w1") is not None:
        ysh = shared_expert(x, inp["shared_w1"], inp["shared_w3"], inp["shared_w2"], limit)
    y = combine(f["o"], r, ysh)
    out = dict(r)
    out.update(f)
    out.update({"xq": xq, "xs": xs, "ysh": ysh, "y": y, "y_bf16": formats.bf16_encode(y)})
    return out
