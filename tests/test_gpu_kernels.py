"""Per-step parity of the HIP library (through the C ABI) against the oracle
on the same seeded inputs: activation quant and routing bit-exact, the
router GEMM and the expert GEMMs within tolerances derived from their
arithmetic (see the design notes)."""

import numpy as np
import pytest
import torch

import splitmix_construct
import synth
from oracle import formats, quant, route as oroute, ffn
from gpu_util import config, dev, dev_bf16, device_inputs, host, near_tie_tokens, norm_err

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("block_scaled_fp4_sqrtsoftplus_amd")


def _adversarial_rows(H):
    rows = []
    z = np.zeros(H)
    rows.append(z.copy())                               # all zero
    r = z.copy(); r[1::2] = -0.0; rows.append(r)        # signed zeros
    r = np.full(H, 448.0 * 2.0 ** -3); rows.append(r)   # amax exactly on a boundary
    fin = formats.e4m3_decode(np.arange(1, 126))
    mids = (fin[1:] + fin[:-1]) / 2                     # E4M3 rounding midpoints (bf16-exact)
    r = np.resize(np.concatenate([mids, -mids]), H); r[0] = 448.0; rows.append(r * 2.0 ** -5)
    r = np.resize(2.0 ** -np.arange(120, 134.0), H); rows.append(r)   # bf16 subnormals
    r = np.full(H, 3.3895313892515355e38); r[::3] *= -1; rows.append(r)  # bf16 max
    return formats.bf16_encode(np.stack(rows))


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill"])
def test_quant_act_bit_exact(name):
    wl = synth.WORKLOADS[name]
    x = synth.make_inputs(wl.replace(n_experts=1), tokens=min(wl.tokens, 512))["x"]
    x = np.concatenate([x, _adversarial_rows(wl.hidden)])
    q, s = moe.quant_act(dev_bf16(x))
    torch.cuda.synchronize()
    rq, rs = quant.act_quant(formats.bf16_decode(x))
    assert np.array_equal(host(s), rs)
    assert np.array_equal(host(q), rq)


def test_quant_act_ragged_and_empty():
    x = formats.bf16_encode(np.random.default_rng(1).standard_normal((3, 384)))
    q, s = moe.quant_act(dev_bf16(x))
    rq, rs = quant.act_quant(formats.bf16_decode(x))
    assert np.array_equal(host(q), rq) and np.array_equal(host(s), rs)
    q0, s0 = moe.quant_act(torch.empty((0, 256), dtype=torch.bfloat16, device="cuda"))
    assert q0.shape == (0, 256)


def _routing_case(name, tokens=None, experts=None):
    wl = synth.WORKLOADS[name]
    if experts is not None:
        wl = wl.replace(n_experts=experts)
    inp = synth.make_inputs(wl, tokens=tokens, experts_only=[])
    return wl, inp


def _check_routing(g, ref):
    for n in ("topk_idx", "topk_w", "expert_offsets", "sorted_pairs", "pair_pos"):
        got = host(g[n]).reshape(np.asarray(ref[n]).shape)
        assert np.array_equal(got, ref[n]), n


@pytest.mark.parametrize("name,tokens", [("tiny", None), ("decode", None), ("prefill", None),
                                         ("skewed", None)])
def test_route_given_logits_bit_exact(name, tokens):
    wl, inp = _routing_case(name, tokens)
    z = oroute.router_logits(inp["x"], inp["w_gate"])
    ref = oroute.route(logits=z, k=wl.top_k, bias=inp["bias"], route_scale=wl.route_scale)
    cfg = config(moe, wl, tokens=z.shape[0])
    g = moe.route(cfg, logits_in=dev(z), bias=dev(inp["bias"]) if inp["bias"] is not None else None)
    torch.cuda.synchronize()
    _check_routing(g, ref)
    if name == "skewed":
        load = np.bincount(ref["topk_idx"].ravel(), minlength=wl.n_experts)
        print(f"skewed load: max/mean {load.max() / load.mean():.1f}, top5 {np.sort(load)[-5:]}")


@pytest.mark.parametrize("E,k", [(8, 2), (40, 6), (64, 8), (256, 1), (512, 6), (3, 3)])
def test_route_ties_and_shapes(E, k):
    # integer logits force many equal keys: the lower expert id must win
    rng = np.random.default_rng(E * 10 + k)
    T = 333
    z = rng.integers(-2, 3, (T, E)).astype(np.float32)
    ref = oroute.route(logits=z, k=k)
    cfg = moe.Config(tokens=T, hidden=128, inter=128, n_experts=E, top_k=k)
    g = moe.route(cfg, logits_in=dev(z))
    torch.cuda.synchronize()
    _check_routing(g, ref)


def test_route_empty():
    cfg = moe.Config(tokens=0, hidden=128, inter=128, n_experts=16, top_k=4)
    g = moe.route(cfg, logits_in=torch.empty((0, 16), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    assert np.all(host(g["expert_offsets"]) == 0)


@pytest.mark.parametrize("name,E", [("tiny", 24), ("tiny", 384), ("hash", None)])
def test_hash_route_bit_exact(name, E):
    wl = synth.WORKLOADS[name]
    if E is not None:
        wl = wl.replace(mode="hash", n_experts=E, top_k=6)   # not powers of two
    ids = synth.make_inputs(wl.replace(n_experts=1), experts_only=[])["token_ids"]
    if E is not None:
        # tokens whose streams put a draw exactly at, and just below, the
        # rejection limit 2**64 - (2**64 mod E), and one at the top mid-stream
        cases = splitmix_construct.rejection_tokens(wl.seed, E, 6)
        ids = np.concatenate([ids, np.array([c[0] for c in cases], np.int64)])
    ref = oroute.route(k=wl.top_k, route_scale=wl.route_scale, mode="hash", token_ids=ids,
                       seed=wl.seed, n_experts=wl.n_experts)
    if E is not None:
        assert ref["topk_idx"][-len(cases):].tolist() == [c[1] for c in cases]
    cfg = config(moe, wl, route_mode=moe.ROUTE_HASH, tokens=len(ids))
    g = moe.route(cfg, token_ids=dev(ids))
    torch.cuda.synchronize()
    _check_routing(g, ref)


@pytest.mark.parametrize("name", ["tiny", "decode", "skewed"])
def test_router_logits_within_fp32_bound(name):
    wl, inp = _routing_case(name, tokens=min(synth.WORKLOADS[name].tokens, 1024))
    cfg = config(moe, wl, tokens=inp["x"].shape[0])
    g = moe.route(cfg, x=dev_bf16(inp["x"]), w_gate=dev_bf16(inp["w_gate"]), want_logits=True,
                  bias=dev(inp["bias"]) if inp["bias"] is not None else None)
    torch.cuda.synchronize()
    z = host(g["logits"]).astype(np.float64)
    xa = np.abs(formats.bf16_decode(inp["x"]))
    wa = np.abs(formats.bf16_decode(inp["w_gate"]))
    exact = formats.bf16_decode(inp["x"]) @ formats.bf16_decode(inp["w_gate"]).T
    bound = wl.hidden * 2.0 ** -24 * (xa @ wa.T) + 2.0 ** -24 * np.abs(exact)
    assert np.all(np.abs(z - exact) <= bound)
    # end-to-end routing: identical to the oracle's except at near ties
    ref = oroute.route(inp["x"], inp["w_gate"], k=wl.top_k, bias=inp["bias"], route_scale=wl.route_scale)
    tie = near_tie_tokens(oroute.sqrtsoftplus(ref["logits"]), inp["bias"], wl.top_k)
    gi = host(g["topk_idx"])
    same = np.all(gi == ref["topk_idx"], axis=1)
    assert np.all(same | tie), f"{np.sum(~same & ~tie)} tokens routed differently without a near tie"
    assert tie.sum() <= max(2, 0.002 * len(tie))


def _ffn_case(wl, tokens, seed_tokens=None):
    inp = synth.make_inputs(wl, tokens=tokens)
    x = inp["x"]
    xq, xs = quant.act_quant(formats.bf16_decode(x))
    r = oroute.route(x, inp["w_gate"], k=wl.top_k, route_scale=wl.route_scale)
    ref = ffn.expert_ffn(xq, xs, r, inp, wl.top_k, wl.swiglu_limit)
    return inp, xq, xs, r, ref


# Accuracy of v_mfma_scale_f32_16x16x128_f8f6f4 as measured on gfx950: its
# result differs from the exact dot product by up to ~2**-14 of sum|a*b|
# (random FP4 x FP8 operands and scales); TAU allows twice that.
TAU = 2.0 ** -13
# Share of h codes that may differ from the oracle's (each one still has to be
# a rounding of a value within the accumulation bound): the GEMMs' own
# rounding differences flip 1e-4 to 4e-4 of the codes on the workloads here.
MAX_FLIP_FRAC = 2e-3


def _bounds(inp, xq, xs, r, ref, wl, deq=quant.mxfp4_dequant, tau=None, experts=None):
    """Per element of h and o: how far the GPU may sit from the oracle given
    tau (default TAU) accumulation error in each GEMM (and h's fp32
    rounding); deq dequantizes the expert weights; `experts` limits the
    bounds to those experts' rows."""
    tau = TAU if tau is None else tau
    off, sp = r["expert_offsets"], r["sorted_pairs"]
    P, I = ref["hq"].shape
    dh = np.zeros((P, I))
    absw2 = {}
    lim = wl.swiglu_limit
    for e in (range(len(off) - 1) if experts is None else experts):
        lo, hi = int(off[e]), int(off[e + 1])
        if lo == hi:
            continue
        tok = sp[lo:hi] // wl.top_k
        xd = quant.act_dequant(xq[tok], xs[tok])
        W1 = deq(inp["w1"][e], inp["w1_scale"][e])
        W3 = deq(inp["w3"][e], inp["w3_scale"][e])
        g, u = xd @ W1.T, xd @ W3.T
        bg, bu = tau * (np.abs(xd) @ np.abs(W1).T), tau * (np.abs(xd) @ np.abs(W3).T)
        gc, uc = np.clip(g, -lim, lim), np.clip(u, -lim, lim)
        dsilu = 1.1                                   # |d silu / dg| <= 1.0999
        # h in fp32: silu with the hardware exponential and reciprocal (a few
        # ulp, below 2^-19 relative for |g| <= 10) times u, one more rounding
        dh[lo:hi] = dsilu * np.abs(uc) * bg + np.abs(ffn.silu(gc)) * bu + 2.0 ** -18 * np.abs(ffn.silu(gc) * uc)
        absw2[e] = np.abs(deq(inp["w2"][e], inp["w2_scale"][e]))
    return dh, absw2


def _check_hq(hq, hs, ref, dh, max_flip_frac):
    """FP8 bytes of h.  Several byte patterns are correct: the GPU's h differs
    from the oracle's by at most dh (accumulation error), so a block scale may
    differ only where the oracle's amax is within dh of a scale boundary, and
    a code may differ only if the GPU code is a rounding of some value within
    dh of the oracle's h (one E4M3 step plus dh, in scaled units)."""
    rs, rq, h = ref["hs"], ref["hq"], ref["h"].astype(np.float64)
    P, I = rq.shape
    hb = np.abs(h).reshape(P, I // 128, 128)
    amax = hb.max(axis=2)
    damax = dh.reshape(P, I // 128, 128).max(axis=2)
    e = rs.astype(np.int64) - 127
    b_hi, b_lo = np.ldexp(448.0, e), np.ldexp(448.0, e - 1)
    near = (np.abs(amax - b_hi) <= damax) | (np.abs(amax - b_lo) <= damax)
    assert np.all((hs == rs) | near), "block scale differs away from a boundary"
    same_scale = np.repeat(hs == rs, 128, axis=1)
    scale = np.repeat(np.ldexp(1.0, e), 128, axis=1)
    dq = formats.e4m3_decode(hq).astype(np.float64) * scale
    v = h
    a = np.abs(v) / scale + dh / scale
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    step = np.ldexp(1.0, np.maximum(ex - 1, -6) - 3) * scale
    diff = (hq != rq) & same_scale
    ok = np.abs(dq - v) <= step + dh
    assert np.all(ok[diff]), f"{np.sum(~ok & diff)} codes outside the accumulation bound"
    frac = diff.sum() / diff.size
    print(f"hq code differences: {diff.sum()} of {diff.size} ({frac:.2e}); scale differences {np.sum(hs != rs)}")
    assert frac <= max_flip_frac
    return diff


def _check_o(o, hq, hs, ref, r, absw2, tau=None):
    """o = deq(hq) w2^T: the GPU may differ from the oracle by its own codes'
    difference propagated through |w2| plus TAU accumulation error."""
    tau = TAU if tau is None else tau
    off = r["expert_offsets"]
    dq = quant.act_dequant(hq, hs)
    dr = quant.act_dequant(ref["hq"], ref["hs"])
    bound = np.zeros_like(o)
    for e, aw in absw2.items():
        lo, hi = int(off[e]), int(off[e + 1])
        bound[lo:hi] = np.abs(dq[lo:hi] - dr[lo:hi]) @ aw.T + tau * (np.abs(dq[lo:hi]) @ aw.T)
    bad = np.abs(o - ref["o"]) > bound + 1e-30
    assert not bad.any(), f"{bad.sum()} outputs outside the bound"
    print(f"o: normalised max error {norm_err(o, ref['o']):.2e}")


@pytest.mark.parametrize("shape", [
    # name, tokens, overrides: several n-tiles, ragged m-tails, both m-tile sizes
    ("tiny", None, {}),
    ("tiny", 37, dict(hidden=512, inter=384, n_experts=12, top_k=3)),
    ("tiny", 200, dict(hidden=256, inter=256, n_experts=8, top_k=2)),      # 50 pairs/expert: 64-token tiles
    ("decode", 8, dict(n_experts=16)),                                      # full H, I
    ("decode", 10, dict(hidden=1024, inter=1024, n_experts=8)),             # K = 1024 streaming path
    ("decode", 6, dict(hidden=2048, inter=4096, n_experts=6, top_k=2)),     # K = 2048 / 4096 swapped
    ("tiny", 19, dict(hidden=768, inter=640, n_experts=5, top_k=5, exp_lo=-9, exp_hi=-7)),
    # > 32 pairs per expert with K in {1024, 2048, 4096}: 128-token tiles
    ("decode", 600, dict(hidden=1024, inter=1024, n_experts=8, top_k=2)),
    ("decode", 300, dict(hidden=2048, inter=4096, n_experts=4, top_k=2)),
    ("decode", 400, dict(n_experts=8, top_k=2)),
    # largest K on each GEMM (hidden / inter 16384), and a V4-Pro-sized layer
    # (H = 7168, I = 3072: K outside the streaming kernels' set)
    ("decode", 4, dict(hidden=16384, inter=512, n_experts=3, top_k=2)),
    ("decode", 4, dict(hidden=512, inter=16384, n_experts=3, top_k=2)),
    ("decode", 6, dict(hidden=7168, inter=3072, n_experts=16, top_k=6)),
])
def test_expert_ffn_parity(shape):
    name, tokens, over = shape
    wl = synth.WORKLOADS[name].replace(**over)
    inp, xq, xs, r, ref = _ffn_case(wl, tokens)
    T = inp["x"].shape[0]
    cfg = config(moe, wl, tokens=T)
    routing = {n: dev(r[n]) for n in ("topk_idx", "topk_w", "expert_offsets", "sorted_pairs", "pair_pos")}
    w = {n: dev(inp[n]) for n in ("w1", "w1_scale", "w3", "w3_scale", "w2", "w2_scale")}
    g = moe.expert_ffn(cfg, dev(xq), dev(xs), routing, w, want_h=True)
    torch.cuda.synchronize()
    dh, absw2 = _bounds(inp, xq, xs, r, ref, wl)
    hq, hs = host(g["hq"]), host(g["hs"])
    _check_hq(hq, hs, ref, dh, max_flip_frac=MAX_FLIP_FRAC)
    _check_o(host(g["out"]).astype(np.float64), hq, hs, ref, r, absw2)


def test_expert_ffn_bf16_out_matches_fp32():
    wl = synth.WORKLOADS["tiny"].replace(hidden=512, inter=256, n_experts=6, top_k=3)
    inp, xq, xs, r, ref = _ffn_case(wl, 23)
    routing = {n: dev(r[n]) for n in ("topk_idx", "topk_w", "expert_offsets", "sorted_pairs", "pair_pos")}
    w = {n: dev(inp[n]) for n in ("w1", "w1_scale", "w3", "w3_scale", "w2", "w2_scale")}
    c32 = config(moe, wl, tokens=23)
    c16 = config(moe, wl, tokens=23, out_fp32=0)
    o32 = moe.expert_ffn(c32, dev(xq), dev(xs), routing, w)["out"]
    o16 = moe.expert_ffn(c16, dev(xq), dev(xs), routing, w)["out"]
    torch.cuda.synchronize()
    assert torch.equal(o32.to(torch.bfloat16), o16)


def test_expert_ffn_unclamped_limit():
    wl = synth.WORKLOADS["tiny"].replace(swiglu_limit=float("inf"))
    inp, xq, xs, r, ref = _ffn_case(wl, None)
    assert np.abs(ref["h"]).max() > 100.0        # beyond the clamped range
    routing = {n: dev(r[n]) for n in ("topk_idx", "topk_w", "expert_offsets", "sorted_pairs", "pair_pos")}
    w = {n: dev(inp[n]) for n in ("w1", "w1_scale", "w3", "w3_scale", "w2", "w2_scale")}
    g = moe.expert_ffn(config(moe, wl), dev(xq), dev(xs), routing, w, want_h=True)
    torch.cuda.synchronize()
    dh, absw2 = _bounds(inp, xq, xs, r, ref, wl)
    hq, hs = host(g["hq"]), host(g["hs"])
    _check_hq(hq, hs, ref, dh, max_flip_frac=MAX_FLIP_FRAC)
    _check_o(host(g["out"]).astype(np.float64), hq, hs, ref, r, absw2)


def test_expert_ffn_skewed_hot_expert():
    # The skewed workload at full size (16384 tokens, 384 experts, Zipf(1.1)
    # popularity): the GPU runs every expert of the oracle's routing, and
    # every pair of the most-loaded expert (~16k pairs: ~128 m-tiles in a row
    # through the persistent tile kernel) and of the least-loaded one is
    # checked element by element.
    wl = synth.WORKLOADS["skewed"]
    print("[skewed hot expert] generating inputs", flush=True)
    inp = synth.make_inputs(wl)
    x = inp["x"]
    xq, xs = quant.act_quant(formats.bf16_decode(x))
    r = oroute.route(x, inp["w_gate"], k=wl.top_k, bias=inp["bias"], route_scale=wl.route_scale)
    load = np.diff(r["expert_offsets"])
    hot, cold = int(np.argmax(load)), int(np.argmin(np.where(load > 0, load, 1 << 30)))
    print(f"[skewed hot expert] expert {hot}: {load[hot]} pairs, expert {cold}: {load[cold]} pairs",
          flush=True)
    cfg = config(moe, wl)
    routing = {n: dev(r[n]) for n in ("topk_idx", "topk_w", "expert_offsets", "sorted_pairs", "pair_pos")}
    w = {n: dev(inp[n]) for n in ("w1", "w1_scale", "w3", "w3_scale", "w2", "w2_scale")}
    g = moe.expert_ffn(cfg, dev(xq), dev(xs), routing, w, want_h=True)
    torch.cuda.synchronize()
    ref = ffn.expert_ffn(xq, xs, r, inp, wl.top_k, wl.swiglu_limit, experts=[hot, cold])
    dh, absw2 = _bounds(inp, xq, xs, r, ref, wl, experts=[hot, cold])
    rows = np.concatenate([np.arange(r["expert_offsets"][e], r["expert_offsets"][e + 1]) for e in (hot, cold)])
    sub = {k: ref[k][rows] for k in ("hq", "hs", "h", "o")}
    rows_d = dev(rows)
    hq, hs = host(g["hq"][rows_d]), host(g["hs"][rows_d])
    _check_hq(hq, hs, sub, dh[rows], max_flip_frac=MAX_FLIP_FRAC)
    # rows renumbered from 0: hot expert first, then the cold one
    rs = {"expert_offsets": np.array([0, load[hot], load[hot] + load[cold]])}
    _check_o(host(g["out"][rows_d]).astype(np.float64), hq, hs, sub, rs, {0: absw2[hot], 1: absw2[cold]})


@pytest.mark.parametrize("T,E,H", [(1, 40, 1024), (17, 256, 4096), (37, 33, 2048), (64, 384, 4096),
                                   (5, 64, 8192), (64, 256, 6144)])
def test_router_logits_small_batches(T, E, H):
    # the decode-sized router GEMM (K split over 8 waves, LDS tree reduction)
    wl = synth.WORKLOADS["decode"].replace(n_experts=E, hidden=H)
    inp = synth.make_inputs(wl, tokens=T, experts_only=[])
    cfg = config(moe, wl, tokens=T)
    g = moe.route(cfg, x=dev_bf16(inp["x"]), w_gate=dev_bf16(inp["w_gate"]), want_logits=True)
    torch.cuda.synchronize()
    z = host(g["logits"]).astype(np.float64)
    xa = np.abs(formats.bf16_decode(inp["x"]))
    wa = np.abs(formats.bf16_decode(inp["w_gate"]))
    exact = formats.bf16_decode(inp["x"]) @ formats.bf16_decode(inp["w_gate"]).T
    bound = H * 2.0 ** -24 * (xa @ wa.T) + 2.0 ** -24 * np.abs(exact)
    assert np.all(np.abs(z - exact) <= bound)
