"""NVFP4 expert weights (E2M1 nibbles, one E4M3 scale per 16 elements, the
"DeepSeek-V4-Pro-0813-nvfp4-DSpark" article's 阶段三导出 format) through the
routed experts and the whole layer, against the oracle's NVFP4 dequant.  The
synthetic per-16 scales all carry mantissa bits, so the path cannot lean on
power-of-two scales."""

import numpy as np
import pytest
import torch

import synth
from gpu_util import config, dev, device_inputs, host, norm_err
from oracle import ffn, formats, quant, route as oroute
from test_gpu_kernels import _bounds, _check_hq, MAX_FLIP_FRAC, _check_o

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("block_scaled_fp4_sqrtsoftplus_amd")


def _nv_inputs(wl, tokens):
    inp = synth.make_inputs(wl, tokens=tokens)
    inp.update(synth.nvfp4_scales(wl))
    return inp


@pytest.mark.parametrize("shape", [
    ("decode", 8, dict(n_experts=16)),                                    # K = 4096 / 2048
    ("decode", 10, dict(hidden=1024, inter=1024, n_experts=8)),           # K = 1024
    ("tiny", 37, dict(hidden=512, inter=512, n_experts=12, top_k=3)),     # K = 512: one group of steps
    ("tiny", 200, dict(hidden=512, inter=1024, n_experts=6, top_k=2)),    # many 16-pair tiles per expert
    ("decode", 6, dict(hidden=4608, inter=5120, n_experts=4, top_k=2)),   # K > 4096: scales loaded per group
])
def test_nvfp4_expert_ffn_parity(shape):
    name, tokens, over = shape
    wl = synth.WORKLOADS[name].replace(**over)
    inp = _nv_inputs(wl, tokens)
    xq, xs = quant.act_quant(formats.bf16_decode(inp["x"]))
    r = oroute.route(inp["x"], inp["w_gate"], k=wl.top_k, route_scale=wl.route_scale)
    ref = ffn.expert_ffn(xq, xs, r, inp, wl.top_k, wl.swiglu_limit, weight_format="nvfp4")
    T = inp["x"].shape[0]
    cfg = config(moe, wl, tokens=T, expert_format=moe.EXPERTS_NVFP4)
    routing = {n: dev(r[n]) for n in ("topk_idx", "topk_w", "expert_offsets", "sorted_pairs", "pair_pos")}
    w = {n: dev(inp[n]) for n in ("w1", "w1_scale", "w3", "w3_scale", "w2", "w2_scale")}
    g = moe.expert_ffn(cfg, dev(xq), dev(xs), routing, w, want_h=True)
    torch.cuda.synchronize()
    dh, absw2 = _bounds(inp, xq, xs, r, ref, wl, deq=quant.nvfp4_dequant)
    hq, hs = host(g["hq"]), host(g["hs"])
    _check_hq(hq, hs, ref, dh, max_flip_frac=MAX_FLIP_FRAC)
    _check_o(host(g["out"]).astype(np.float64), hq, hs, ref, r, absw2)


def _scale_bf16(x16, k):
    """bf16 bits times 2^k (exact: only the exponent field moves)."""
    x32 = (x16.astype(np.uint32) << 16).view(np.float32) * np.float32(2.0 ** k)
    out = (x32.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((out.astype(np.uint32) << 16).view(np.float32), x32)
    return out


@pytest.mark.parametrize("k", [-24, 16])
def test_nvfp4_expert_ffn_activation_scale_range(k):
    """The 64-pair kernel stages activations with their power-of-two scale
    applied in fp16 only while every scale of the tile is 2^e, -15 <= e <= 7;
    activations far outside (here x times 2^-24: GEMM1 and, through the tiny
    h, GEMM2; x times 2^16: GEMM1) take the unscaled staging instead."""
    wl = synth.WORKLOADS["tiny"].replace(hidden=512, inter=1024, n_experts=6, top_k=2)
    inp = _nv_inputs(wl, 200)
    inp["x"] = _scale_bf16(inp["x"], k)
    xq, xs = quant.act_quant(formats.bf16_decode(inp["x"]))
    e = xs.astype(np.int64) - 127
    assert (e < -15).any() if k < 0 else (e > 7).any()
    r = oroute.route(inp["x"], inp["w_gate"], k=wl.top_k, route_scale=wl.route_scale)
    ref = ffn.expert_ffn(xq, xs, r, inp, wl.top_k, wl.swiglu_limit, weight_format="nvfp4")
    T = inp["x"].shape[0]
    cfg = config(moe, wl, tokens=T, expert_format=moe.EXPERTS_NVFP4)
    routing = {n: dev(r[n]) for n in ("topk_idx", "topk_w", "expert_offsets", "sorted_pairs", "pair_pos")}
    w = {n: dev(inp[n]) for n in ("w1", "w1_scale", "w3", "w3_scale", "w2", "w2_scale")}
    g = moe.expert_ffn(cfg, dev(xq), dev(xs), routing, w, want_h=True)
    torch.cuda.synchronize()
    dh, absw2 = _bounds(inp, xq, xs, r, ref, wl, deq=quant.nvfp4_dequant)
    hq, hs = host(g["hq"]), host(g["hs"])
    _check_hq(hq, hs, ref, dh, max_flip_frac=MAX_FLIP_FRAC)
    _check_o(host(g["out"]).astype(np.float64), hq, hs, ref, r, absw2)


@pytest.mark.parametrize("shape", [
    ("tiny", 45, dict(hidden=512, inter=512, n_experts=12, top_k=3, shared=True)),
    ("decode", 5, dict(n_experts=12)),
])
def test_nvfp4_layer_parity(shape):
    name, tokens, over = shape
    wl = synth.WORKLOADS[name].replace(**over)
    inp = _nv_inputs(wl, tokens)
    d = device_inputs(inp)
    T = inp["x"].shape[0]
    cfg = config(moe, wl, tokens=T, expert_format=moe.EXPERTS_NVFP4)
    y = moe.layer(cfg, d["x"], d["weights"], w_gate=d["w_gate"], bias=d["bias"], shared=d["shared"])
    torch.cuda.synchronize()
    ref = ffn.layer(inp, wl.top_k, wl.route_scale, wl.swiglu_limit, weight_format="nvfp4")
    err = norm_err(formats.bf16_decode(host(y)), ref["y"])
    print(f"nvfp4 experts {name}{over}: layer error {err:.2e}")
    assert err <= 2e-2
