"""Seeded synthetic inputs for the routed-MoE layer.

Shared by the tests, the oracle's callers and bench.py.  This module draws
random inputs of the workloads' shapes and distributions only; it holds none
of the layer's arithmetic (no decoding, quantization, routing or GEMM).

Workloads (shapes of a DeepSeek-V4-Flash-class MoE layer: hidden 4096, 256
routed experts + 1 shared, top-6, as the "DeepSeek-V4-Flash-SI" card's
模型概述 / 架构特性 sections give them; 384 experts for the V4.1-Flash /
V4-Pro variants; expert intermediate 2048 as the W4AFP8-mt card's w1 example
[2048, 2048 bytes] for K = 4096 implies):

  tiny     T=16,    H=256,  E=8,   k=2, I=128,  no shared, exponents -6..0
  decode   T=64,    H=4096, E=256, k=6, I=2048, bf16 shared expert
  prefill  T=4096,  the decode layer
  skewed   T=16384, H=4096, E=384, k=6, I=2048, no shared, Zipf gate bias
  hash     T=32768, H=4096, E=256, k=6, I=2048, bf16 shared, hash routing

Recipe (numpy PCG64 streams keyed by (seed, tensor[, expert]), seed = 1000 +
workload number, so that each tensor -- and each expert -- is drawn
independently of the others and of the token count):
  x        N(0, 1) fp32 -> bf16 (round to nearest even)        [T, H]
  w_gate   N(0, 0.02) -> bf16                                   [E, H]
  bias     skewed only: frozen Zipf(1.1) calibration (zipf_bias) [E] fp32
  w1, w3   uniform bytes (both nibbles uniform over 16 codes)   [E, I, H/2]
  w2       uniform bytes                                        [E, H, I/2]
  scales   E8M0 bytes 127 + uniform{exp_lo..exp_hi}             [E, N, K/32]
  shared   N(0, 0.02) -> bf16: w1, w3 [I, H], w2 [H, I]
  token_ids  uniform on [0, 129280) (vocabulary size 129,280)   [T] int64
The E8M0 exponent range -9..-7 of the full-size workloads makes the
pre-activation standard deviation about 0.97, so the +-10 clamp is only
touched in the tails; the tiny workload's -6..0 saturates most of them.
"""

import os
from dataclasses import dataclass, field

import numpy as np
import torch

VOCAB = 129280


@dataclass(frozen=True)
class Workload:
    name: str
    tokens: int
    hidden: int
    inter: int
    n_experts: int
    top_k: int
    shared: bool
    mode: str = "score"          # "score" (sqrtsoftplus) or "hash"
    zipf_bias: bool = False
    exp_lo: int = -9
    exp_hi: int = -7
    seed: int = 0
    route_scale: float = 1.5
    swiglu_limit: float = 10.0

    def replace(self, **kw):
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    "tiny": Workload("tiny", 16, 256, 128, 8, 2, False, exp_lo=-6, exp_hi=0, seed=1001),
    "decode": Workload("decode", 64, 4096, 2048, 256, 6, True, seed=1002),
    "prefill": Workload("prefill", 4096, 4096, 2048, 256, 6, True, seed=1003),
    "skewed": Workload("skewed", 16384, 4096, 2048, 384, 6, False, zipf_bias=True, seed=1004),
    "hash": Workload("hash", 32768, 4096, 2048, 256, 6, True, mode="hash", seed=1005),
}


def _bf16_bits(a32):
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def zipf_ranks(wl: Workload):
    """Popularity ranks 1..E of the experts (a seeded permutation) for the
    skewed workload's Zipf target."""
    rng = np.random.Generator(np.random.PCG64([wl.seed, 3]))
    return rng.permutation(wl.n_experts) + 1


ZIPF_BIAS_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "zipf_bias_skewed.txt")


def zipf_bias(wl: Workload):
    """The skewed workload's gate bias [E] fp32, frozen in zipf_bias_skewed.txt
    (calibrated once so that expert popularity follows Zipf(1.1) over the
    ranks of zipf_ranks; the file's header names the script and recipe)."""
    vals = [int(l, 16) for l in open(ZIPF_BIAS_FILE) if l.strip() and not l.startswith("#")]
    b = np.array(vals, np.uint32).view(np.float32)
    if len(b) != wl.n_experts:
        raise ValueError(f"frozen Zipf bias holds {len(b)} experts, workload has {wl.n_experts}")
    return b


def make_inputs(wl: Workload, tokens=None, experts_only=None):
    """Draw the inputs of workload `wl` (optionally with a different token
    count).  Returns a dict of numpy arrays; bf16 tensors are uint16 bit
    patterns.  `experts_only` (a list of expert ids) leaves the other experts'
    weight bytes zero-filled to save memory in samples; the drawn values of
    the listed experts are unchanged."""
    T = wl.tokens if tokens is None else tokens
    H, I, E = wl.hidden, wl.inter, wl.n_experts

    def rng(*key):
        return np.random.Generator(np.random.PCG64([wl.seed, *key]))

    out = {}
    out["x"] = _bf16_bits(rng(1).standard_normal((T, H), dtype=np.float32))
    out["w_gate"] = _bf16_bits(rng(2).standard_normal((E, H), dtype=np.float32) * np.float32(0.02))
    out["bias"] = zipf_bias(wl) if wl.zipf_bias else None
    nexp = wl.exp_hi - wl.exp_lo + 1

    def draw_expert(r, n, k):
        nib = r.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
        sc = (127 + wl.exp_lo + r.integers(0, nexp, size=(n, k // 32))).astype(np.uint8)
        return nib, sc

    w1 = np.zeros((E, I, H // 2), np.uint8)
    w1s = np.zeros((E, I, H // 32), np.uint8)
    w3 = np.zeros((E, I, H // 2), np.uint8)
    w3s = np.zeros((E, I, H // 32), np.uint8)
    w2 = np.zeros((E, H, I // 2), np.uint8)
    w2s = np.zeros((E, H, I // 32), np.uint8)
    keep = None if experts_only is None else set(int(e) for e in experts_only)
    for e in range(E):
        if keep is not None and e not in keep:
            continue
        r = rng(4, e)
        w1[e], w1s[e] = draw_expert(r, I, H)
        w3[e], w3s[e] = draw_expert(r, I, H)
        w2[e], w2s[e] = draw_expert(r, H, I)
    out.update(w1=w1, w1_scale=w1s, w3=w3, w3_scale=w3s, w2=w2, w2_scale=w2s)
    if wl.shared:
        r = rng(5)
        out["shared_w1"] = _bf16_bits(r.standard_normal((I, H), dtype=np.float32) * np.float32(0.02))
        out["shared_w3"] = _bf16_bits(r.standard_normal((I, H), dtype=np.float32) * np.float32(0.02))
        out["shared_w2"] = _bf16_bits(r.standard_normal((H, I), dtype=np.float32) * np.float32(0.02))
    else:
        out["shared_w1"] = out["shared_w3"] = out["shared_w2"] = None
    out["token_ids"] = rng(6).integers(0, VOCAB, size=T, dtype=np.int64)
    return out


def nvfp4_scales(wl: Workload, experts_only=None):
    """Per-16 E4M3 scale bytes for NVFP4 expert weights of workload `wl`
    (the nibble arrays of make_inputs are reused): positive E4M3 codes with
    exponent field 1 and a uniform mantissa, i.e. values (1 + m/8) * 2**-6,
    so every scale carries mantissa bits.  Returns w1_scale, w3_scale
    [E, I, H/16] and w2_scale [E, H, I/16] uint8."""
    H, I, E = wl.hidden, wl.inter, wl.n_experts
    keep = None if experts_only is None else set(int(e) for e in experts_only)
    out = {"w1_scale": np.zeros((E, I, H // 16), np.uint8), "w3_scale": np.zeros((E, I, H // 16), np.uint8),
           "w2_scale": np.zeros((E, H, I // 16), np.uint8)}
    for e in range(E):
        if keep is not None and e not in keep:
            continue
        r = np.random.Generator(np.random.PCG64([wl.seed, 7, e]))
        for n, shape in (("w1_scale", (I, H // 16)), ("w3_scale", (I, H // 16)), ("w2_scale", (H, I // 16))):
            out[n][e] = (0x08 | r.integers(0, 8, size=shape)).astype(np.uint8)
    return out


def w4afp8_scales(wl: Workload, experts_only=None, pow2=False):
    """Per-128 float32 scales for W4AFP8 expert weights of workload `wl` (the
    nibble arrays of make_inputs are reused as INT4 codes, uniform over all
    16): 2**e * U(0.5, 0.75) with e uniform on the workload's exponent range,
    which puts the weights' second moment near that of the MXFP4 draw; with
    pow2 the factor U is left out (exact powers of two).  Returns w1_scale,
    w3_scale [E, I, H/128] and w2_scale [E, H, I/128] float32."""
    H, I, E = wl.hidden, wl.inter, wl.n_experts
    keep = None if experts_only is None else set(int(e) for e in experts_only)
    nexp = wl.exp_hi - wl.exp_lo + 1
    out = {"w1_scale": np.zeros((E, I, H // 128), np.float32), "w3_scale": np.zeros((E, I, H // 128), np.float32),
           "w2_scale": np.zeros((E, H, I // 128), np.float32)}
    for e in range(E):
        if keep is not None and e not in keep:
            continue
        r = np.random.Generator(np.random.PCG64([wl.seed, 8, e]))
        for n, shape in (("w1_scale", (I, H // 128)), ("w3_scale", (I, H // 128)), ("w2_scale", (H, I // 128))):
            ex = wl.exp_lo + r.integers(0, nexp, size=shape)
            f = np.ones(shape) if pow2 else r.uniform(0.5, 0.75, size=shape)
            out[n][e] = np.ldexp(f, ex).astype(np.float32)
    return out
