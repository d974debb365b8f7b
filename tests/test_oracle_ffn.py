"""Pins of the oracle's expert FFN, shared expert, combine and whole layer:
an independent implementation through library routines (torch float64
matmuls, torch's float8_e4m3fn and bfloat16 casts, torch.frexp), exact
integer arithmetic, the clamp bound, and special cases of the layer (one
expert, all experts, token permutation, duplicate tokens)."""

import numpy as np
import pytest
import torch

import synth
from oracle import ffn, formats, quant, route

SILU10 = 10.0 / (1.0 + np.exp(-10.0))


def _e2m1_as_e4m3(c):
    c = torch.as_tensor(np.asarray(c, np.int64))
    s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
    mag = torch.where(e > 0, ((e + 6) << 3) | (m << 2), torch.where(m == 1, torch.full_like(e, 48), torch.zeros_like(e)))
    return ((s << 7) | mag).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)


def t_fp4(packed, scales):
    p = torch.as_tensor(packed)
    n, kh = p.shape
    codes = torch.stack([p & 0xF, p >> 4], dim=2).reshape(n, 2 * kh)
    v = _e2m1_as_e4m3(codes.numpy()).reshape(n, -1, 32)
    sc = torch.ldexp(torch.ones(1, dtype=torch.float64), torch.as_tensor(scales.astype(np.int64) - 127).to(torch.float64))
    return (v * sc[:, :, None]).reshape(n, 2 * kh)


def t_quant(v):
    t = torch.as_tensor(v, dtype=torch.float64).reshape(v.shape[0], -1, 128)
    amax = t.abs().amax(dim=2)
    m, x = torch.frexp(amax)
    e = torch.where(m <= 0.875, x - 9, x - 8)
    e = torch.where(amax == 0, torch.full_like(e, -127), e).clamp(-127, 127)
    q = torch.ldexp(t, -e[:, :, None].double()).float().to(torch.float8_e4m3fn)
    deq = q.to(torch.float64) * torch.ldexp(torch.ones(1, dtype=torch.float64), e.double())[:, :, None]
    return q.view(torch.uint8).reshape(v.shape), deq.reshape(v.shape)


def t_bf16(u16):
    return torch.as_tensor(u16.view(np.int16)).view(torch.bfloat16).to(torch.float64)


def t_expert(xrow_deq, inp, e, limit):
    W1 = t_fp4(inp["w1"][e], inp["w1_scale"][e])
    W3 = t_fp4(inp["w3"][e], inp["w3_scale"][e])
    W2 = t_fp4(inp["w2"][e], inp["w2_scale"][e])
    g = xrow_deq @ W1.T
    u = xrow_deq @ W3.T
    g, u = g.clamp(-limit, limit), u.clamp(-limit, limit)
    h = (torch.nn.functional.silu(g) * u).float().double()
    hq, hd = t_quant(h.numpy())
    return hq, hd @ W2.T


def t_layer(inp, r, limit=10.0):
    x = t_bf16(inp["x"])
    _, xd = t_quant(x.numpy())
    T, k = r["topk_idx"].shape
    y = torch.zeros(T, x.shape[1], dtype=torch.float64)
    for t in range(T):
        for j in range(k):
            _, o = t_expert(xd[t:t + 1], inp, int(r["topk_idx"][t, j]), limit)
            y[t] += float(r["topk_w"][t, j]) * o[0]
    if inp.get("shared_w1") is not None:
        g = x @ t_bf16(inp["shared_w1"]).T
        u = x @ t_bf16(inp["shared_w3"]).T
        h = (torch.nn.functional.silu(g.clamp(-limit, limit)) * u.clamp(-limit, limit)).to(torch.bfloat16).double()
        y += h @ t_bf16(inp["shared_w2"]).T
    return y.numpy()


def _small(name="tiny", **kw):
    wl = synth.WORKLOADS[name].replace(**kw)
    return wl, synth.make_inputs(wl)


def test_layer_vs_library_route_tiny():
    wl, inp = _small()
    out = ffn.layer(inp, wl.top_k)
    ref = t_layer(inp, out)
    assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-9 * np.abs(ref).max())
    # the quantized x must agree bit for bit
    xq, _ = t_quant(t_bf16(inp["x"]).numpy())
    assert np.array_equal(out["xq"], xq.numpy())


def test_layer_vs_library_route_shared_expert():
    wl, inp = _small("decode", tokens=3, hidden=256, inter=256, n_experts=6, top_k=3)
    out = ffn.layer(inp, wl.top_k)
    ref = t_layer(inp, out)
    assert np.allclose(out["y"], ref, rtol=1e-9, atol=1e-9 * np.abs(ref).max())


def test_hq_bytes_vs_library_route():
    wl, inp = _small()
    out = ffn.layer(inp, wl.top_k)
    _, xd = t_quant(t_bf16(inp["x"]).numpy())
    for r, p in enumerate(out["sorted_pairs"]):
        t, j = divmod(int(p), wl.top_k)
        hq, _ = t_expert(xd[t:t + 1], inp, int(out["topk_idx"][t, j]), 10.0)
        assert np.array_equal(out["hq"][r], hq.numpy()[0])


def test_gemm_exact_integer_case():
    # all weight scales 2**0 and integer activations: every product is a
    # multiple of 0.5 and every sum is exact, so g, u are integer sums / 2
    rng = np.random.default_rng(31)
    T, H, I, E = 8, 256, 128, 1
    inp = {
        "w1": rng.integers(0, 256, (E, I, H // 2), dtype=np.uint8),
        "w3": rng.integers(0, 256, (E, I, H // 2), dtype=np.uint8),
        "w2": rng.integers(0, 256, (E, H, I // 2), dtype=np.uint8),
    }
    for n in ("w1", "w3", "w2"):
        inp[n + "_scale"] = np.full(inp[n].shape[:2] + (inp[n].shape[2] // 16,), 127, np.uint8)
    xi = rng.integers(-7, 8, (T, H))
    xi[:, 0] = 7                                         # amax 7 in every block -> codes exact
    xi[:, 128] = 7
    xq, xs = quant.act_quant(xi.astype(np.float64))
    assert np.array_equal(quant.act_dequant(xq, xs), xi)
    r = route.route(logits=np.zeros((T, E), np.float32), k=1)
    out = ffn.expert_ffn(xq, xs, r, inp, 1, limit=np.inf)
    # integer reference: twice the E2M1 values are integers
    twice = np.array([0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12], np.int64)
    c1 = quant.unpack_nibbles(inp["w1"][0]).astype(np.int64)
    c3 = quant.unpack_nibbles(inp["w3"][0]).astype(np.int64)
    g2 = xi @ twice[c1].T                               # int64, exact: = 2 g
    u2 = xi @ twice[c3].T
    g, u = g2 / 2.0, u2 / 2.0
    h = (g / (1 + np.exp(-g)) * u).astype(np.float32)
    assert np.array_equal(out["h"][np.argsort(r["sorted_pairs"])], h)


def test_clamp_bound_and_unclamped_limit():
    wl, inp = _small()
    out = ffn.layer(inp, wl.top_k)
    h = out["h"].astype(np.float64)
    assert np.abs(h).max() <= SILU10 * 10.0 + 1e-4
    assert np.abs(h).max() > 90.0                        # the tiny layer saturates
    big = ffn.layer(inp, wl.top_k, limit=np.inf)
    ref = t_layer(inp, big, limit=np.inf)
    assert np.allclose(big["y"], ref, rtol=1e-12, atol=1e-9 * np.abs(ref).max())
    assert np.abs(big["h"]).max() > SILU10 * 10.0


def test_single_expert_layer_is_scaled_ffn():
    # E = k = 1: every token goes to expert 0 with weight 1.5 * s/s = 1.5
    wl, inp = _small(n_experts=1, top_k=1)
    out = ffn.layer(inp, 1)
    assert np.all(out["topk_w"] == np.float32(1.5))
    _, xd = t_quant(t_bf16(inp["x"]).numpy())
    _, o = t_expert(xd, inp, 0, 10.0)
    assert np.allclose(out["y"], 1.5 * o.numpy(), rtol=1e-12, atol=1e-9)


def test_all_experts_layer_is_weighted_sum():
    wl, inp = _small(top_k=8)                             # k = E = 8
    out = ffn.layer(inp, 8)
    assert np.array_equal(np.sort(out["topk_idx"], 1), np.tile(np.arange(8), (wl.tokens, 1)))
    _, xd = t_quant(t_bf16(inp["x"]).numpy())
    z = route.router_logits(inp["x"], inp["w_gate"])
    s = route.sqrtsoftplus(z).astype(np.float64)
    y = np.zeros_like(out["y"])
    for e in range(8):
        _, o = t_expert(xd, inp, e, 10.0)
        y += 1.5 * s[:, e:e + 1] / s.sum(1, keepdims=True) * o.numpy()
    assert np.allclose(out["y"], y, rtol=1e-6, atol=1e-6 * np.abs(y).max())


def test_token_permutation_equivariance_and_duplicates():
    wl, inp = _small()
    out = ffn.layer(inp, wl.top_k)
    perm = np.random.default_rng(5).permutation(wl.tokens)
    inp2 = dict(inp)
    inp2["x"] = inp["x"][perm]
    out2 = ffn.layer(inp2, wl.top_k)
    assert np.array_equal(out2["y"], out["y"][perm])
    inp3 = dict(inp)
    inp3["x"] = np.concatenate([inp["x"][:4], inp["x"][:4]])
    out3 = ffn.layer(inp3, wl.top_k)
    assert np.array_equal(out3["y"][:4], out3["y"][4:])
    assert np.array_equal(out3["y"][:4], out["y"][:4])


def test_hash_layer_uses_hash_routing():
    wl, inp = _small(mode="hash", n_experts=16, top_k=6)
    out = ffn.layer(inp, 6, mode="hash", hash_seed=wl.seed)
    idx, w = route.hash_route(inp["token_ids"], wl.seed, 16, 6)
    assert np.array_equal(out["topk_idx"], idx) and np.all(out["topk_w"] == np.float32(0.25))
    ref = t_layer(inp, out)
    assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-9 * np.abs(ref).max())
