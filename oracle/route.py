"""Routing steps of the layer (oracle; test infrastructure only).

"DeepSeek-V4-Flash-SI" card, 架构特性, MoE paragraph: every token picks its
top-6 routed experts through the gate network; most layers score experts with
sqrtsoftplus and take the top-k, the first three layers pick experts
deterministically from the token id (hash routing); the routing scale is 1.5.
The PTPC-FP8 article (排除清单) keeps the gate (*ffn.gate*) unquantized: the
router reads bf16 activations and bf16 gate weights.

Readings where the pages are silent (listed with the others in the design
notes):
* router logits are the exact dot products of the bf16 values, rounded once
  to fp32 (here: float64 accumulation, then one rounding);
* s = sqrt(softplus(z)) = sqrt(ln(1 + e**z)), evaluated in float64 and
  rounded to fp32;
* an optional per-expert gate bias shifts the selection key only
  (key = fp32(s + b)); the weights use the unbiased s;
* experts are ranked by key, larger first, equal keys by lower expert index;
  the k selected are reported in rank order;
* weights: w_j = fp32(fp32(s_j / S) * 1.5) with S the fp32 sum of the k
  selected s taken in rank order;
* hash routing: SplitMix64 (Steele, Lea and Flood, "Fast splittable
  pseudorandom number generators", OOPSLA 2014) seeded with
  (seed << 32) xor token_id; each output r is reduced to r mod E, values of r
  at or above 2**64 - (2**64 mod E) are rejected, repeats are skipped, the
  first k distinct experts are kept in draw order, each weighted
  fp32(1.5 / k);
* the token -> expert permutation is a stable counting sort of the pair ids
  p = t*k + j by expert; no capacity limit, no dropped pairs.
"""

import numpy as np

from . import formats

MASK64 = (1 << 64) - 1
SPLITMIX_GAMMA = 0x9E3779B97F4A7C15
SPLITMIX_M1 = 0xBF58476D1CE4E5B9
SPLITMIX_M2 = 0x94D049BB133111EB


def router_logits(x_u16, wg_u16):
    """z[t, e] = sum_h x[t, h] * Wg[e, h]: bf16 inputs, float64 sums (bf16
    products are exact in float64), one rounding to fp32."""
    x = formats.bf16_decode(x_u16)
    w = formats.bf16_decode(wg_u16)
    return (x @ w.T).astype(np.float32)


def sqrtsoftplus(z):
    """s = sqrt(ln(1 + exp(z))) in float64, rounded to fp32."""
    z = np.asarray(z, dtype=np.float64)
    return np.sqrt(np.log1p(np.exp(z))).astype(np.float32)


def topk_select(scores, k, bias=None, route_scale=1.5):
    """Top-k of fp32 scores [T, E] (plus an optional selection bias [E]).
    Returns (idx int32 [T, k] in rank order, w fp32 [T, k])."""
    s = np.asarray(scores, dtype=np.float32)
    T, E = s.shape
    key = s if bias is None else (s + np.asarray(bias, dtype=np.float32)[None, :])
    key = key.astype(np.float32)
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    scale = np.float32(route_scale)
    for t in range(T):
        # rank: larger key first; equal keys keep ascending expert order
        order = sorted(range(E), key=lambda e: (-float(key[t, e]), e))
        sel = order[:k]
        total = np.float32(0.0)
        for e in sel:
            total = np.float32(total + s[t, e])
        for j, e in enumerate(sel):
            idx[t, j] = e
            w[t, j] = np.float32(np.float32(s[t, e] / total) * scale)
    return idx, w


def splitmix64_stream(state, n):
    """The first n outputs of SplitMix64 from the given 64-bit state (Python
    integers, arbitrary precision, masked to 64 bits)."""
    out = []
    for _ in range(n):
        state = (state + SPLITMIX_GAMMA) & MASK64
        z = state
        z = ((z ^ (z >> 30)) * SPLITMIX_M1) & MASK64
        z = ((z ^ (z >> 27)) * SPLITMIX_M2) & MASK64
        out.append(z ^ (z >> 31))
    return out, state


def hash_route_token(token_id, seed, n_experts, k):
    """Hash routing of one token: k distinct experts in draw order."""
    state = (((seed & MASK64) << 32) ^ (token_id & MASK64)) & MASK64
    limit = (1 << 64) - ((1 << 64) % n_experts)
    chosen = []
    while len(chosen) < k:
        (r,), state = splitmix64_stream(state, 1)
        if r >= limit:
            continue
        e = r % n_experts
        if e not in chosen:
            chosen.append(e)
    return chosen


def hash_route(token_ids, seed, n_experts, k, route_scale=1.5):
    ids = np.asarray(token_ids, dtype=np.int64)
    idx = np.array([hash_route_token(int(t) & MASK64, seed, n_experts, k) for t in ids],
                   dtype=np.int32).reshape(len(ids), k)
    w = np.full((len(ids), k), np.float32(np.float32(route_scale) / np.float32(k)),
                dtype=np.float32)
    return idx, w


def permutation(topk_idx, n_experts):
    """Stable counting sort of the pairs p = t*k + j by expert.

    Returns (expert_offsets int32 [E+1], sorted_pairs int32 [P],
    pair_pos int32 [P]) with sorted_pairs[pair_pos[p]] == p."""
    flat = np.asarray(topk_idx).reshape(-1)
    P = flat.size
    counts = [0] * n_experts
    for e in flat.tolist():
        counts[e] += 1
    offsets = [0] * (n_experts + 1)
    for e in range(n_experts):
        offsets[e + 1] = offsets[e] + counts[e]
    fill = list(offsets[:n_experts])
    sorted_pairs = np.empty(P, dtype=np.int32)
    pair_pos = np.empty(P, dtype=np.int32)
    for p, e in enumerate(flat.tolist()):
        pos = fill[e]
        fill[e] += 1
        sorted_pairs[pos] = p
        pair_pos[p] = pos
    return np.asarray(offsets, dtype=np.int32), sorted_pairs, pair_pos


def route(x_u16=None, wg_u16=None, k=6, bias=None, route_scale=1.5, logits=None,
          mode="score", token_ids=None, seed=0, n_experts=None):
    """Whole routing step. Returns dict with logits (score mode), topk_idx,
    topk_w, expert_offsets, sorted_pairs, pair_pos."""
    out = {}
    if mode == "hash":
        idx, w = hash_route(token_ids, seed, n_experts, k, route_scale)
    else:
        z = router_logits(x_u16, wg_u16) if logits is None else np.asarray(logits, np.float32)
        out["logits"] = z
        n_experts = z.shape[1]
        idx, w = topk_select(sqrtsoftplus(z), k, bias, route_scale)
    out["topk_idx"], out["topk_w"] = idx, w
    off, sp, pp = permutation(idx, n_experts)
    out["expert_offsets"], out["sorted_pairs"], out["pair_pos"] = off, sp, pp
    return out
