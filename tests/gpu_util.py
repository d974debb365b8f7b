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
