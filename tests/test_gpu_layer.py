"""Whole-layer parity of moe_layer (through the C ABI) against the oracle:
small shapes compared on every token, the full-size workloads on a seeded
sample of tokens (each token's output depends only on that token: no
capacity limit), plus determinism and edge cases."""

import os

import numpy as np
import pytest
import torch

import synth
from oracle import formats, ffn, route as oroute
from gpu_util import (check_flipped_h_codes, config, dev, dev_bf16, device_inputs, host,
                      near_tie_tokens, norm_err, oracle_continue_from_h)
from test_gpu_kernels import MAX_FLIP_FRAC, TAU

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("block_scaled_fp4_sqrtsoftplus_amd")

TOL = 2e-2   # max |y_gpu - y_ref| / RMS(y_ref), y_ref the float64 oracle output


def run_layer(wl, inp, d=None, tokens=None):
    d = d or device_inputs(inp)
    T = inp["x"].shape[0] if tokens is None else tokens
    cfg = config(moe, wl, tokens=T)
    y, r = moe.layer(cfg, d["x"], d["weights"], w_gate=d["w_gate"], bias=d["bias"],
                     token_ids=d["token_ids"], shared=d["shared"], want_routing=True)
    torch.cuda.synchronize()
    return host(y), {k: host(v) for k, v in r.items()}


# threads for the oracle's experts (each expert's weights are dequantized
# once per call; the machine's CPU share is 16)
ORACLE_WORKERS = min(16, len(os.sched_getaffinity(0)))


def oracle_layer(wl, inp):
    return ffn.layer(inp, wl.top_k, wl.route_scale, wl.swiglu_limit, wl.mode, wl.seed,
                     workers=ORACLE_WORKERS)


def check_routing_valid(r, T, k, E):
    idx = r["topk_idx"].reshape(T, k)
    off, sp, pp = r["expert_offsets"], r["sorted_pairs"], r["pair_pos"]
    assert off[0] == 0 and off[-1] == T * k
    assert np.array_equal(np.diff(off), np.bincount(idx.ravel(), minlength=E))
    assert np.array_equal(sp, np.argsort(idx.ravel(), kind="stable"))
    assert np.array_equal(sp[pp], np.arange(T * k))
    assert all(len(set(row)) == k for row in idx.tolist())


@pytest.mark.parametrize("shape", [
    ("tiny", None, {}),
    ("tiny", 45, dict(hidden=512, inter=384, n_experts=12, top_k=3, shared=True, exp_lo=-9, exp_hi=-7)),
    ("tiny", 150, dict(hidden=256, inter=256, n_experts=4, top_k=2, shared=True)),
    ("tiny", 33, dict(mode="hash", n_experts=20, top_k=6, hidden=384, inter=256, shared=True)),
    ("tiny", 1, dict(n_experts=8, top_k=8)),
    ("tiny", 20, dict(n_experts=512, top_k=8, hidden=256, inter=128)),   # largest E and k
    ("decode", 5, dict(n_experts=12)),
    ("decode", 300, dict(hidden=1024, inter=1024, n_experts=4, top_k=2, shared=True)),
    # a larger shared expert through the 128 x 128 bf16 tiles: ragged T (1100 =
    # 8 x 128 + 76), four up and eight down workgroup columns
    ("decode", 1100, dict(hidden=1024, inter=256, n_experts=4, top_k=2, shared=True)),
    # decode-sized shared expert through the split-K kernels (T <= 64, H and I
    # multiples of 512) on the side stream: ragged T, a full 64-token batch,
    # a single token
    ("decode", 37, dict(hidden=1024, inter=512, n_experts=8, top_k=2, shared=True)),
    ("decode", 64, dict(hidden=1536, inter=1024, n_experts=8, top_k=2, shared=True)),
    ("decode", 1, dict(hidden=512, inter=512, n_experts=4, top_k=2, shared=True)),
    # ... and inside the routing launches (split-K router: H in {2048, 4096,
    # 8192}): three, one and four down slices, ragged / full / single batches
    ("decode", 37, dict(hidden=2048, inter=1536, n_experts=16, top_k=4, shared=True)),
    ("decode", 64, dict(hidden=2048, inter=512, n_experts=8, top_k=2, shared=True)),
    ("decode", 1, dict(hidden=2048, inter=2048, n_experts=8, top_k=8, shared=True)),
])
def test_layer_parity_small(shape):
    name, tokens, over = shape
    wl = synth.WORKLOADS[name].replace(**over)
    inp = synth.make_inputs(wl, tokens=tokens)
    y, r = run_layer(wl, inp)
    ref = oracle_layer(wl, inp)
    T = inp["x"].shape[0]
    check_routing_valid(r, T, wl.top_k, wl.n_experts)
    if wl.mode == "hash":
        assert np.array_equal(r["topk_idx"], ref["topk_idx"])
        assert np.array_equal(r["topk_w"], ref["topk_w"])
    else:
        tie = near_tie_tokens(oroute.sqrtsoftplus(ref["logits"]), inp.get("bias"), wl.top_k)
        same = np.all(r["topk_idx"].reshape(T, -1) == ref["topk_idx"], axis=1)
        assert np.all(same | tie)
    err = norm_err(formats.bf16_decode(y), ref["y"])
    print(f"{name}{over}: layer error {err:.2e}")
    assert err <= TOL


def test_layer_deterministic():
    wl = synth.WORKLOADS["tiny"].replace(hidden=512, inter=256, n_experts=10, top_k=4, shared=True)
    inp = synth.make_inputs(wl, tokens=77)
    d = device_inputs(inp)
    y1, r1 = run_layer(wl, inp, d)
    y2, r2 = run_layer(wl, inp, d)
    assert np.array_equal(y1, y2)
    for k in r1:
        assert np.array_equal(r1[k], r2[k])


def test_layer_empty_batch():
    wl = synth.WORKLOADS["tiny"]
    inp = synth.make_inputs(wl, tokens=1)
    d = device_inputs(inp)
    cfg = config(moe, wl, tokens=0)
    x0 = torch.empty((0, wl.hidden), dtype=torch.bfloat16, device="cuda")
    y, r = moe.layer(cfg, x0, d["weights"], w_gate=d["w_gate"], want_routing=True)
    torch.cuda.synchronize()
    assert y.shape == (0, wl.hidden) and np.all(host(r["expert_offsets"]) == 0)


def test_layer_token_permutation_equivariant():
    wl = synth.WORKLOADS["tiny"].replace(hidden=256, inter=128, n_experts=8, top_k=2)
    inp = synth.make_inputs(wl, tokens=40)
    y, _ = run_layer(wl, inp)
    perm = np.random.default_rng(9).permutation(40)
    inp2 = dict(inp)
    inp2["x"] = inp["x"][perm]
    y2, _ = run_layer(wl, inp2)
    assert np.array_equal(y2, y[perm])


# tokens checked against the oracle at full size (every token's output depends
# on that token alone, so a sample is an exact check of those tokens); the
# routing and permutation are checked on every token
SAMPLE = {"decode": 64, "prefill": 1024, "skewed": 1024, "hash": 1024, "e512": 1024}


@pytest.mark.parametrize("name", ["decode", "prefill", "skewed", "hash", "e512"])
def test_layer_full_size_sampled(name):
    if name == "e512":
        # the largest expert count through the 128-pair tile kernel: 20480
        # pairs over 512 experts (40 per expert), K = 1024
        wl = synth.WORKLOADS["decode"].replace(name="e512", tokens=2560, hidden=1024, inter=1024,
                                               n_experts=512, top_k=8)
    else:
        wl = synth.WORKLOADS[name]
    print(f"[{name}] generating inputs T={wl.tokens} E={wl.n_experts}", flush=True)
    inp = synth.make_inputs(wl)
    d = device_inputs(inp)
    y, r = run_layer(wl, inp, d)
    T = wl.tokens
    check_routing_valid(r, T, wl.top_k, wl.n_experts)
    load = np.diff(r["expert_offsets"])
    print(f"[{name}] expert load max/mean {load.max() / load.mean():.1f}, experts used {np.sum(load > 0)}")
    rng = np.random.default_rng(4242)
    S = np.sort(rng.choice(T, min(T, SAMPLE[name]), replace=False))
    print(f"[{name}] oracle on {len(S)} tokens", flush=True)
    sub = dict(inp)
    sub["x"] = inp["x"][S]
    sub["token_ids"] = inp["token_ids"][S]
    ref = oracle_layer(wl, sub)
    gidx = r["topk_idx"].reshape(T, -1)[S]
    if wl.mode == "hash":
        assert np.array_equal(gidx, ref["topk_idx"])
        keep = np.ones(len(S), bool)
    else:
        tie = near_tie_tokens(oroute.sqrtsoftplus(ref["logits"]), inp.get("bias"), wl.top_k)
        same = np.all(gidx == ref["topk_idx"], axis=1)
        assert np.all(same | tie)
        keep = same
    assert keep.sum() >= len(S) - 1

    # The GPU's FP8 h codes of the sampled pairs: moe_expert_ffn on the layer's
    # own routing and quantized x runs the kernels moe_layer ran.  Several h
    # byte patterns are correct (a code may sit one step away where h is within
    # the GEMM's accumulation error of a rounding midpoint; the expert FFN tests
    # check each such code against that bound element by element), and one
    # flipped code moves an output by up to several percent of RMS(y), so the
    # layer output is compared with the oracle continued from the GPU's codes
    # (a unique result), and the codes are checked to be rare roundings
    # within the accumulation bound.
    k = wl.top_k
    xq_d, xs_d = moe.quant_act(d["x"])
    rd = {n: dev(r[n]) for n in ("topk_idx", "topk_w", "expert_offsets", "sorted_pairs", "pair_pos")}
    g = moe.expert_ffn(config(moe, wl), xq_d, xs_d, rd, d["weights"], want_h=True)
    torch.cuda.synchronize()
    ks = np.flatnonzero(keep)
    p_gpu = (S[ks][:, None] * k + np.arange(k)[None, :]).ravel()
    p_ref = (ks[:, None] * k + np.arange(k)[None, :]).ravel()
    rows_gpu = dev(r["pair_pos"][p_gpu].astype(np.int64))
    rows_ref = ref["pair_pos"][p_ref]
    hq, hs = ref["hq"].copy(), ref["hs"].copy()
    hq[rows_ref] = host(g["hq"][rows_gpu])
    hs[rows_ref] = host(g["hs"][rows_gpu])
    del g
    flips = hq != ref["hq"]
    scale_flips = hs != ref["hs"]
    print(f"[{name}] h codes differing from the oracle's: {flips.mean():.2e}, "
          f"block scales: {scale_flips.sum()} of {scale_flips.size}")
    assert flips.mean() <= MAX_FLIP_FRAC
    assert scale_flips.mean() <= 1e-4
    check_flipped_h_codes(sub, ref, hq, hs, wl.top_k, wl.swiglu_limit, TAU)

    y_cont = oracle_continue_from_h(sub, ref, hq, hs, workers=ORACLE_WORKERS)
    yg = formats.bf16_decode(y[S])
    err = norm_err(yg[keep], y_cont[keep])
    direct = norm_err(yg[keep], ref["y"][keep])
    moved = norm_err(y_cont[keep], ref["y"][keep])
    print(f"[{name}] sampled layer error {err:.2e} over {keep.sum()} tokens (vs the oracle continued "
          f"from the GPU's h codes); vs the oracle's own codes {direct:.2e}, of which the codes' "
          f"choice moves the exact result by {moved:.2e}")
    assert err <= TOL
    # the direct difference is the bar plus what the code choice itself moves
    rms = np.sqrt(np.mean(ref["y"][keep] ** 2))
    assert np.all(np.abs(yg[keep] - ref["y"][keep])
                  <= TOL * rms + np.abs(y_cont[keep] - ref["y"][keep]) + 1e-12)
