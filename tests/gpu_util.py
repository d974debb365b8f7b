"""Helpers of the GPU parity tests: move seeded inputs to the device, build
configs, and compare the HIP results with the oracle's."""

import numpy as np
import torch

import synth


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(u16):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).cuda().view(torch.bfloat16)


def host(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def config(moe, wl, tokens=None, **kw):
    c = moe.Config(tokens=wl.tokens if tokens is None else tokens, hidden=wl.hidden, inter=wl.inter,
                   n_experts=wl.n_experts, top_k=wl.top_k, route_scale=wl.route_scale,
                   swiglu_limit=wl.swiglu_limit,
                   route_mode=moe.ROUTE_HASH if wl.mode == "hash" else moe.ROUTE_SQRTSOFTPLUS,
                   hash_seed=wl.seed)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def device_inputs(inp):
    d = {"x": dev_bf16(inp["x"]), "w_gate": dev_bf16(inp["w_gate"]),
         "bias": dev(inp["bias"]) if inp.get("bias") is not None else None,
         "token_ids": dev(inp["token_ids"])}
    d["weights"] = {n: dev(inp[n]) for n in ("w1", "w1_scale", "w3", "w3_scale", "w2", "w2_scale")}
    d["shared"] = None
    if inp.get("shared_w1") is not None:
        d["shared"] = {"w1": dev_bf16(inp["shared_w1"]), "w3": dev_bf16(inp["shared_w3"]),
                       "w2": dev_bf16(inp["shared_w2"])}
    return d


def norm_err(got, ref):
    """max |got - ref| / RMS(ref)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    return float(np.max(np.abs(got - ref)) / rms) if ref.size else 0.0


def near_tie_tokens(scores, bias, k, rel=1e-5):
    """Tokens whose k-th and (k+1)-th selection keys (oracle, fp32) differ by
    less than rel * (|key| + 1): either choice is a correct routing when the
    logits come from fp32 GEMMs with different summation orders."""
    key = scores.astype(np.float32) if bias is None else (scores + bias[None, :]).astype(np.float32)
    srt = -np.sort(-key.astype(np.float64), axis=1)
    if key.shape[1] <= k:
        return np.zeros(key.shape[0], bool)
    gap = srt[:, k - 1] - srt[:, k]
    return gap < rel * (np.abs(srt[:, k - 1]) + 1.0)


def oracle_continue_from_h(inp, ref, hq, hs, workers=1, weight_format="mxfp4"):
    """The oracle's layer output continued from given FP8 h codes instead of
    its own: o = deq(hq) w2^T per expert, then the oracle's combine with its
    routing weights and shared expert.  hq, hs are in the oracle's sorted-pair
    order (ref's routing).  Used where several h byte patterns are correct
    (each a rounding of h within the GEMM's accumulation error): given the
    GPU's choice, the rest of the layer has one result."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    from oracle import ffn, quant

    deq = {"mxfp4": quant.mxfp4_dequant, "fp8": quant.fp8_dequant,
           "nvfp4": quant.nvfp4_dequant, "w4afp8": quant.int4_dequant}[weight_format]
    off = ref["expert_offsets"]
    o = np.zeros(ref["o"].shape, np.float64)
    used = [e for e in range(len(off) - 1) if off[e + 1] > off[e]]

    def run(es):
        for e in es:
            lo, hi = int(off[e]), int(off[e + 1])
            W2 = deq(inp["w2"][e], inp["w2_scale"][e])
            o[lo:hi] = quant.act_dequant(hq[lo:hi], hs[lo:hi]) @ W2.T

    with threadpool_limits(1), ThreadPoolExecutor(max(1, workers)) as ex:
        list(ex.map(run, [used[i::max(1, workers)] for i in range(max(1, workers))]))
    return ffn.combine(o, ref, ref["ysh"])


def check_flipped_h_codes(inp, ref, hq, hs, top_k, limit, tau, weight_format="mxfp4"):
    """Every h code (in a block whose scale agrees) that differs from the
    oracle's must be a rounding of a value within the GEMM's accumulation
    error of the oracle's h: g and u of those elements are recomputed exactly
    (one dot product each) with their bound tau * sum |x w|, carried through
    the clamp and silu, and the code's value must lie within one E4M3 step
    (at the code's binade) plus that bound of the oracle's h.  Block scales
    may differ only where the oracle's amax lies within the bound of a
    scale boundary (checked on the block's largest element).  Returns the
    number of differing codes checked."""
    from oracle import ffn, formats, quant

    deq = {"mxfp4": quant.mxfp4_dequant, "fp8": quant.fp8_dequant,
           "nvfp4": quant.nvfp4_dequant, "w4afp8": quant.int4_dequant}[weight_format]
    off, sp = ref["expert_offsets"], ref["sorted_pairs"]
    blk = hq.shape[1] // hs.shape[1]

    def dh_of(rows, cols):
        """Accumulation bound on h at (rows, cols) of the oracle's order."""
        e_of = np.searchsorted(off, rows, side="right") - 1
        tok = sp[rows] // top_k
        xd = quant.act_dequant(ref["xq"][tok], ref["xs"][tok])
        g = np.zeros(len(rows)); u = np.zeros(len(rows))
        bg = np.zeros(len(rows)); bu = np.zeros(len(rows))
        for e in np.unique(e_of):
            m = e_of == e
            c = cols[m]
            W1 = deq(inp["w1"][e][c], inp["w1_scale"][e][c])
            W3 = deq(inp["w3"][e][c], inp["w3_scale"][e][c])
            g[m] = np.sum(xd[m] * W1, axis=1)
            u[m] = np.sum(xd[m] * W3, axis=1)
            bg[m] = tau * np.sum(np.abs(xd[m]) * np.abs(W1), axis=1)
            bu[m] = tau * np.sum(np.abs(xd[m]) * np.abs(W3), axis=1)
        gc, uc = np.clip(g, -limit, limit), np.clip(u, -limit, limit)
        sg = ffn.silu(gc)
        return 1.1 * np.abs(uc) * bg + np.abs(sg) * bu + 2.0 ** -18 * np.abs(sg * uc)

    h = ref["h"].astype(np.float64)
    # block scales: only at a boundary, within the bound of the block's amax
    sr, sc = np.nonzero(hs != ref["hs"])
    if len(sr):
        hb = np.abs(h[sr].reshape(len(sr), -1, blk)[np.arange(len(sr)), sc])
        j = np.argmax(hb, axis=1)
        amax = hb[np.arange(len(sr)), j]
        d = dh_of(sr, sc * blk + j)
        e = ref["hs"][sr, sc].astype(np.int64) - 127
        near = (np.abs(amax - np.ldexp(448.0, e)) <= d) | (np.abs(amax - np.ldexp(448.0, e - 1)) <= d)
        assert np.all(near), "block scale differs away from a boundary"
    same_scale = np.repeat(hs == ref["hs"], blk, axis=1)
    rows, cols = np.nonzero((hq != ref["hq"]) & same_scale)
    if len(rows) == 0:
        return 0
    d = dh_of(rows, cols)
    scale = np.ldexp(1.0, ref["hs"][rows, cols // blk].astype(np.int64) - 127)
    v = h[rows, cols]
    dq = formats.e4m3_decode(hq[rows, cols]).astype(np.float64) * scale
    a = np.abs(v) / scale + d / scale
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    step = np.ldexp(1.0, np.maximum(ex - 1, -6) - 3) * scale
    bad = np.abs(dq - v) > step + d
    assert not bad.any(), f"{bad.sum()} of {len(rows)} differing h codes outside the accumulation bound"
    return len(rows)