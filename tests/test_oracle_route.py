"""Pins of the oracle's routing: sqrtsoftplus against high-precision values
(mpmath) and its closed-form limits, top-k against brute force with forced
ties, the weights' normalisation, SplitMix64 against its published outputs,
hash routing properties and its rejection rule on tokens constructed to reach
it, the router logits against exact integer arithmetic, exact rational dot
products and torch's float64 matmul, and the permutation against a library
stable sort."""

import itertools
import os
from fractions import Fraction

import mpmath
import numpy as np
import pytest
import torch

import splitmix_construct
from oracle import formats, route

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_sqrtsoftplus_high_precision():
    mpmath.mp.dps = 50
    rng = np.random.default_rng(21)
    z = np.concatenate([rng.standard_normal(3000) * 3, rng.uniform(-80, 80, 500),
                        [0.0, -0.0, 1e-7, -30.0, 30.0, 88.0]]).astype(np.float32)
    ours = route.sqrtsoftplus(z)
    ref = np.array([float(mpmath.sqrt(mpmath.log(1 + mpmath.exp(mpmath.mpf(float(v))))))
                    for v in z]).astype(np.float32)
    assert np.array_equal(ours, ref)


def test_sqrtsoftplus_closed_forms():
    assert route.sqrtsoftplus(np.float32(0.0)) == np.float32(np.sqrt(np.log(2.0)))
    big = np.array([40.0, 60.0, 80.0], np.float32)          # ln(1+e^z) = z + e^-z
    assert np.array_equal(route.sqrtsoftplus(big), np.sqrt(big.astype(np.float64)).astype(np.float32))
    small = np.array([-40.0, -60.0, -80.0], np.float32)     # sqrt(ln(1+e^z)) -> e^(z/2)
    assert np.allclose(route.sqrtsoftplus(small), np.exp(small.astype(np.float64) / 2), rtol=1e-6)
    zz = np.linspace(-10, 10, 1001).astype(np.float32)
    s = route.sqrtsoftplus(zz)
    assert np.all(np.diff(s) >= 0) and np.all(s > 0)        # monotone, positive


def _brute_topk(key, k):
    """Among all k-subsets take the one whose keys, sorted descending, are
    lexicographically largest, ties broken by the smaller sorted index list;
    report it in rank order (key descending, index ascending)."""
    E = len(key)
    best = None
    for sub in itertools.combinations(range(E), k):
        ks = sorted((key[e] for e in sub), reverse=True)
        cand = (tuple(ks), tuple(-e for e in sub))
        if best is None or cand > best[0]:
            best = (cand, sub)
    sub = best[1]
    return sorted(sub, key=lambda e: (-key[e], e))


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(22)
    for E, k in [(4, 1), (6, 2), (8, 3), (10, 4), (12, 6), (7, 7)]:
        z = rng.integers(-3, 4, size=(40, E)).astype(np.float32)   # many equal logits
        s = route.sqrtsoftplus(z)
        idx, _ = route.topk_select(s, k)
        for t in range(z.shape[0]):
            assert list(idx[t]) == _brute_topk([float(v) for v in s[t]], k)


def test_topk_bias_selects_but_does_not_weight():
    s = np.array([[1.0, 0.9, 0.8, 0.7]], np.float32)
    bias = np.array([0.0, 0.0, 0.0, 1.0], np.float32)
    idx, w = route.topk_select(s, 2, bias)
    assert list(idx[0]) == [3, 0]
    assert w[0, 0] == np.float32(np.float32(np.float32(0.7) / np.float32(1.7)) * np.float32(1.5))


def test_weights_normalised_times_scale():
    rng = np.random.default_rng(23)
    s = route.sqrtsoftplus(rng.standard_normal((500, 64)).astype(np.float32) * 1.3)
    _, w = route.topk_select(s, 6)
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.5) <= 6 * 2.0 ** -22)
    eq = np.ones((3, 16), np.float32)
    idx, w = route.topk_select(eq, 6)
    assert np.all(idx == np.arange(6)) and np.all(w == np.float32(0.25))


def test_splitmix64_published_outputs():
    ref = [int(l, 16) for l in open(os.path.join(GOLDEN, "splitmix64_seed0.txt"))
           if l.strip() and not l.startswith("#")]
    out, _ = route.splitmix64_stream(0, len(ref))
    assert out == ref


def _splitmix_np(state, n):
    """Vectorised uint64 SplitMix64 (wrapping numpy arithmetic)."""
    s = np.asarray(state, np.uint64).copy()
    outs = []
    with np.errstate(over="ignore"):
        for _ in range(n):
            s = s + np.uint64(route.SPLITMIX_GAMMA)
            z = s.copy()
            z = (z ^ (z >> np.uint64(30))) * np.uint64(route.SPLITMIX_M1)
            z = (z ^ (z >> np.uint64(27))) * np.uint64(route.SPLITMIX_M2)
            outs.append(z ^ (z >> np.uint64(31)))
    return np.stack(outs, 1)


def test_hash_route_properties():
    rng = np.random.default_rng(24)
    ids = rng.integers(0, 129280, 20000)
    seed, E, k = 1005, 256, 6
    idx, w = route.hash_route(ids, seed, E, k)
    assert np.all(w == np.float32(0.25))
    assert all(len(set(r)) == k for r in idx.tolist())
    assert np.array_equal(route.hash_route(ids[:50], seed, E, k)[0], idx[:50])  # deterministic
    # for E = 256 (a power of two) nothing is rejected by the range test, so the
    # first draws are r mod 256 of the plain stream, duplicates skipped
    st = (np.uint64(seed) << np.uint64(32)) ^ ids.astype(np.uint64)
    draws = (_splitmix_np(st[:200], 24) % np.uint64(E)).astype(np.int64)
    for t in range(200):
        seen = []
        for e in draws[t]:
            if e not in seen:
                seen.append(int(e))
        assert seen[:k] == list(idx[t])
    # uniform use of the experts (chi-square, 255 dof; p ~ 1e-6 bound)
    counts = np.bincount(idx.ravel(), minlength=E)
    exp = idx.size / E
    chi2 = ((counts - exp) ** 2 / exp).sum()
    assert chi2 < 255 + 5 * np.sqrt(2 * 255)


@pytest.mark.parametrize("E,seed", [(384, 1004), (384, 1005), (24, 1001), (200, 7)])
def test_hash_rejection_constructed(E, seed):
    # tokens whose streams hold a draw at the limit 2**64 - (2**64 mod E), one
    # below it, and one at 2**64 - 1 mid-stream (built by inverting SplitMix64,
    # tests/splitmix_construct.py): the oracle must drop the first and the
    # third and keep the second; a > for >= or a limit off by one fails
    for tid, expect, what in splitmix_construct.rejection_tokens(seed, E, 6):
        got = route.hash_route_token(tid & route.MASK64, seed, E, 6)
        assert got == expect, what
    # the same tokens through the vectorised route
    cases = splitmix_construct.rejection_tokens(seed, E, 6)
    idx, w = route.hash_route(np.array([c[0] for c in cases], np.int64), seed, E, 6)
    assert idx.tolist() == [c[1] for c in cases]
    assert np.all(w == np.float32(0.25))


def test_hash_construction_round_trip():
    # the inverse used above agrees with the published outputs' generator
    rng = np.random.default_rng(26)
    for _ in range(200):
        v = int(rng.integers(0, 1 << 63)) * 2 + int(rng.integers(0, 2))
        seed = int(rng.integers(0, 1 << 32))
        i = int(rng.integers(0, 5))
        tid = splitmix_construct.token_with_draw(seed, i, v)
        out, _ = route.splitmix64_stream(splitmix_construct.start_state(seed, tid), i + 1)
        assert out[i] == v


def _bf16_bits_exact(u):
    """bf16 bit pattern -> (integer significand, power of two), decoded from
    the bits by hand (sign, 8-bit exponent with bias 127, 7-bit fraction)."""
    u = int(u)
    sign = -1 if u & 0x8000 else 1
    ex = (u >> 7) & 0xFF
    fr = u & 0x7F
    assert ex != 0xFF
    if ex == 0:
        return sign * fr, -133
    return sign * (128 + fr), ex - 134


def _exact_dot(xr, wr):
    """Exact dot product of two bf16 rows as a Fraction."""
    terms = [(_bf16_bits_exact(a), _bf16_bits_exact(b)) for a, b in zip(xr, wr)]
    lo = min(ea + eb for (_, ea), (_, eb) in terms)
    total = sum(ma * mb << (ea + eb - lo) for (ma, ea), (mb, eb) in terms)
    return Fraction(total) * Fraction(2) ** lo


def test_router_logits_exact_integers():
    # bf16 integers with dot products below 2**24: every logit is exact, and
    # must equal the int64 product with the gate's rows (z = x Wg^T; T, E and H
    # distinct so that a transposed operand cannot pass)
    rng = np.random.default_rng(27)
    T, E, H = 7, 11, 1536
    xi = rng.integers(-9, 10, (T, H))
    wi = rng.integers(-9, 10, (E, H))
    z = route.router_logits(formats.bf16_encode(xi.astype(np.float64)),
                            formats.bf16_encode(wi.astype(np.float64)))
    assert z.dtype == np.float32 and z.shape == (T, E)
    assert np.array_equal(z.astype(np.int64), xi @ wi.T)
    assert np.all(np.abs(xi @ wi.T) < 2 ** 24)


def test_router_logits_correctly_rounded():
    # N(0,1) activations against N(0,0.02) gate rows at the full hidden size:
    # each logit is the exact dot product rounded once to fp32, up to the
    # float64 accumulation's own error (H * 2**-53 of sum |x w|); fp32
    # accumulation, a truncating rounding or a dropped term exceeds this
    rng = np.random.default_rng(28)
    T, E, H = 4, 6, 4096
    xu = formats.bf16_encode(rng.standard_normal((T, H)))
    wu = formats.bf16_encode(rng.standard_normal((E, H)) * 0.02)
    z = route.router_logits(xu, wu)
    absdot = np.abs(formats.bf16_decode(xu)) @ np.abs(formats.bf16_decode(wu)).T
    for t in range(T):
        for e in range(E):
            ex = _exact_dot(xu[t], wu[e])
            half_ulp = Fraction(float(np.spacing(np.abs(z[t, e])))) / 2
            slack = Fraction(H * 2.0 ** -53 * float(absdot[t, e]))
            assert abs(Fraction(float(z[t, e])) - ex) <= half_ulp + slack, (t, e)


def test_router_logits_library_route():
    # torch float64 matmul of the same bf16 tensors (torch's own bf16 decode),
    # rounded to fp32: equal except where the two float64 summation orders
    # straddle an fp32 rounding boundary (at most 1 ulp, rarely)
    rng = np.random.default_rng(29)
    T, E, H = 64, 256, 4096
    xu = formats.bf16_encode(rng.standard_normal((T, H)))
    wu = formats.bf16_encode(rng.standard_normal((E, H)) * 0.02)
    z = route.router_logits(xu, wu)
    xt = torch.from_numpy(xu.view(np.int16)).view(torch.bfloat16).double()
    wt = torch.from_numpy(wu.view(np.int16)).view(torch.bfloat16).double()
    ref = (xt @ wt.T).float().numpy()
    diff = np.abs(z.astype(np.float64) - ref)
    assert np.all(diff <= np.spacing(np.abs(ref)))
    assert np.mean(diff == 0) > 0.999


def test_permutation_vs_stable_sort():
    rng = np.random.default_rng(25)
    for T, k, E in [(1, 1, 1), (5, 2, 8), (333, 6, 256), (1000, 6, 384)]:
        idx = rng.integers(0, E, (T, k)).astype(np.int32)
        off, sp, pp = route.permutation(idx, E)
        ref = np.argsort(idx.ravel(), kind="stable")
        assert np.array_equal(sp, ref)
        assert off[0] == 0 and off[-1] == T * k
        assert np.array_equal(np.diff(off), np.bincount(idx.ravel(), minlength=E))
        assert np.array_equal(sp[pp], np.arange(T * k))
