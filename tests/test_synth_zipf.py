"""The skewed workload's expert popularity follows Zipf(1.1).

The frozen gate bias (synth/zipf_bias_skewed.txt) was calibrated on tokens
drawn from a separate seed; here the oracle routes the workload's own 16384
tokens with it (held-out check).  Zipf(1.1) over 384 experts gives rank r a
share r**-1.1 / sum; with top-6 that is ~75x the mean load for rank 1, above
the cap of 64x (an expert takes each token at most once), then 35, 23, 16.5,
13, 10.6 ... x the mean (a few percent more once rank 1's excess is spread)."""

import numpy as np

import synth
from oracle import route


def test_skewed_popularity_is_zipf():
    wl = synth.WORKLOADS["skewed"]
    T, E, k = wl.tokens, wl.n_experts, wl.top_k
    inp = synth.make_inputs(wl, experts_only=[])
    r = route.route(inp["x"], inp["w_gate"], k=k, bias=inp["bias"])
    load = np.bincount(r["topk_idx"].ravel(), minlength=E)
    mean = T * k / E
    ranks = synth.zipf_ranks(wl)
    by_rank = load[np.argsort(ranks)] / mean
    assert np.count_nonzero(load) == E                      # every expert used
    assert 56 <= by_rank[0] <= 64                           # rank 1 near the per-token cap
    assert np.all(by_rank[:5] >= 12)                        # ranks 1-5 >= 12x the mean
    p = np.arange(1, E + 1, dtype=np.float64) ** -1.1
    zipf = p / p.sum() * E                                  # uncapped Zipf, x mean
    rel = by_rank[1:20] / zipf[1:20]
    assert np.all((rel > 0.9) & (rel < 1.2)), np.round(by_rank[:20], 1)
    # the tail follows the same law: ranks 100-384 hold about their Zipf share
    tail = load[np.argsort(ranks)][99:].sum() / (T * k)
    assert abs(tail - p[99:].sum() / p.sum()) < 0.05


def test_zipf_bias_is_selection_only():
    # the bias moves the top-k key only: with it the weights are still the
    # normalised unbiased scores times 1.5
    wl = synth.WORKLOADS["skewed"]
    inp = synth.make_inputs(wl, tokens=64, experts_only=[])
    r = route.route(inp["x"], inp["w_gate"], k=wl.top_k, bias=inp["bias"])
    s = route.sqrtsoftplus(r["logits"])
    for t in range(64):
        sel = s[t, r["topk_idx"][t]]
        assert np.allclose(r["topk_w"][t], 1.5 * sel / sel.sum(), rtol=1e-6)
