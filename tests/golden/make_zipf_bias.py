"""Write the skewed workload's frozen gate bias (synth/zipf_bias_skewed.txt).

The skewed workload is a 16384-token batch over 384 routed experts (the
V4.1-Flash / V4-Pro expert count) whose gate carries a per-expert bias so
that expert popularity follows Zipf(s = 1.1) over a seeded rank order.  The
bias only moves the selection key (key = s + b); the routing weights use the
unbiased score.

Calibration (routing by the oracle only; inputs from synth's generators):
  * ranks r_e: synth.zipf_ranks (a seeded permutation of 1..E);
  * target loads: L_e = P * r_e**-1.1 / sum_r r**-1.1 with P = T * k pairs,
    capped at T (an expert takes a token at most once) and the excess spread
    over the uncapped experts in proportion to their targets until none
    exceeds the cap;
  * calibration tokens: the workload's activations drawn from a separate
    seed (the gate weights are the workload's own);
  * b = 0, then 100 iterations of b_e += 0.05 * (ln L_e - ln max(load_e, 0.5)),
    load_e the number of calibration tokens the oracle routes to expert e
    under the current bias;
  * b is rounded to fp32 and frozen.

Run from the repository root: python tests/golden/make_zipf_bias.py
(about a minute on 8 cores).
"""

import os
import sys
from concurrent.futures import ProcessPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth                                   # noqa: E402
from oracle import route                       # noqa: E402

ZIPF_S = 1.1
ITERS = 100
STEP = 0.05
CAL_SEED = 2004                                # separate from the workload's 1004
OUT = os.path.join(ROOT, "synth", "zipf_bias_skewed.txt")


def target_loads(ranks, T, k):
    p = ranks.astype(np.float64) ** -ZIPF_S
    p /= p.sum()
    L = p * T * k
    capped = np.zeros(len(L), bool)
    while np.any(L > T + 1e-9):
        capped |= L > T
        excess = (L[capped] - T).sum()
        L[capped] = T
        free = ~capped
        L[free] += excess * L[free] / L[free].sum()
    return L


_S = None


def _init(scores):
    global _S
    _S = scores


def _select(args):
    lo, hi, bias, k = args
    idx, _ = route.topk_select(_S[lo:hi], k, bias)
    return idx


def main():
    wl = synth.WORKLOADS["skewed"]
    T, E, k = wl.tokens, wl.n_experts, wl.top_k
    ranks = synth.zipf_ranks(wl)
    L = target_loads(ranks, T, k)
    cal = synth.make_inputs(wl.replace(seed=CAL_SEED, zipf_bias=False), experts_only=[])
    gate = synth.make_inputs(wl.replace(zipf_bias=False), tokens=1, experts_only=[])["w_gate"]
    s = route.sqrtsoftplus(route.router_logits(cal["x"], gate))
    b = np.zeros(E, np.float64)
    chunks = [(i, min(i + 1024, T)) for i in range(0, T, 1024)]
    with ProcessPoolExecutor(8, initializer=_init, initargs=(s,)) as ex:
        for it in range(ITERS):
            b32 = b.astype(np.float32)
            idx = np.concatenate(list(ex.map(_select, [(lo, hi, b32, k) for lo, hi in chunks])))
            load = np.bincount(idx.ravel(), minlength=E).astype(np.float64)
            b += STEP * (np.log(L) - np.log(np.maximum(load, 0.5)))
            if it % 10 == 9 or it == 0:
                order = np.argsort(ranks)
                print(f"iter {it + 1}: used {np.count_nonzero(load)}/{E}, top ranks x mean "
                      f"{np.round(load[order[:6]] / (T * k / E), 1).tolist()}", flush=True)
    b32 = b.astype(np.float32)
    with open(OUT, "w") as f:
        f.write("# Gate bias of the skewed workload (T = 16384, E = 384, top-6): expert\n"
                "# popularity calibrated to Zipf(1.1) over the rank order of\n"
                "# synth.zipf_ranks, written by tests/golden/make_zipf_bias.py (oracle\n"
                "# routing of calibration tokens drawn from seed 2004; 100 steps of\n"
                "# b += 0.05 * (ln target - ln max(load, 0.5))).  One fp32 bit pattern per\n"
                "# expert, in expert order.\n")
        for v in b32:
            f.write(f"0x{int(np.float32(v).view(np.uint32)):08x}\n")
    print("wrote", OUT)


if __name__ == "__main__":
    main()
