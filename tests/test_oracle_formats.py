"""Pins of the oracle's element codecs against closed forms, brute force and
library routines (torch's float8_e4m3fn and bfloat16 conversions)."""

import numpy as np
import pytest
import torch

from oracle import formats


# E2M1 (1 sign, 2 exponent bits with bias 1, 1 mantissa bit) has the
# magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}: the OCP Microscaling Formats (MX)
# v1.0 specification's FP4 E2M1 element.  Checked here through properties a
# wrong table would break, and against torch's E4M3 values (the
# "DeepSeek-V4-Pro-0813-nvfp4-DSpark" article states E2M1 -> E4M3 is a
# lossless cast, so every E2M1 value must be an E4M3 value).
def test_e2m1_grid_properties():
    t = formats.e2m1_table()
    pos = t[:8]
    assert pos[0] == 0.0 and np.all(np.diff(pos) > 0)
    assert np.array_equal(t[8:], -pos) and np.signbit(t[8])   # sign bit only
    assert pos[1] == 0.5 and pos[7] == 6.0                     # min subnormal, max normal
    # one mantissa bit: each binade [2^e, 2^(e+1)) holds exactly two values
    for lo in (1.0, 2.0, 4.0):
        inside = pos[(pos >= lo) & (pos < 2 * lo)]
        assert np.array_equal(inside, [lo, 1.5 * lo])
    e4 = torch.tensor(t, dtype=torch.float32).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(e4, t)


def test_e8m0_decode():
    b = np.arange(255)
    v = formats.e8m0_decode(b)
    assert np.array_equal(v, 2.0 ** (b - 127.0))
    assert v[127] == 1.0 and v[0] == 2.0 ** -127
    assert np.isnan(formats.e8m0_decode(255))


def _torch_e4m3(codes):
    return torch.tensor(codes, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_decode_all_codes_vs_torch():
    codes = np.arange(256)
    ours = formats.e4m3_decode(codes)
    ref = _torch_e4m3(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(codes[nan]) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))
    assert np.nanmax(ours) == 448.0 and np.nanmin(np.abs(ours[ours != 0])) == 2.0 ** -9


def _brute_e4m3(v):
    """Nearest finite E4M3 value by exhaustive search, ties to the even code,
    beyond +-448 saturate; sign kept."""
    codes = np.array([c for c in range(128) if c != 0x7F])
    vals = formats.e4m3_decode(codes)          # decode is pinned against torch above
    out = np.empty(v.shape, np.uint8)
    for i, x in enumerate(v.ravel()):
        a = min(abs(x), 448.0)
        d = np.abs(vals - a)
        best = np.flatnonzero(d == d.min())
        c = codes[best[0]] if len(best) == 1 else [c for c in codes[best] if c % 2 == 0][0]
        out.ravel()[i] = c | (0x80 if np.signbit(x) else 0)
    return out


def test_e4m3_encode_brute_force():
    rng = np.random.default_rng(7)
    fin = formats.e4m3_decode(np.arange(127))
    fin = fin[~np.isnan(fin)]
    mids = (fin[1:] + fin[:-1]) / 2                           # exact ties
    v = np.concatenate([
        fin, -fin, mids, -mids,
        np.nextafter(mids, 0), np.nextafter(mids, 1e9),
        rng.uniform(-500, 500, 3000), rng.standard_normal(3000) * 2.0 ** rng.integers(-12, 8, 3000),
        [0.0, -0.0, 448.0, 449.0, 464.0, 480.0, 1e6, -1e6, 2.0 ** -10, 2.0 ** -11, -2.0 ** -10],
    ])
    assert np.array_equal(formats.e4m3_encode(v), _brute_e4m3(v))


def test_e4m3_encode_vs_torch_every_bf16():
    # every finite bf16 bit pattern with |v| <= 448: torch's fp32 -> e4m3fn cast
    # rounds to nearest even, and agrees with ours in that range
    u = np.arange(0, 1 << 16, dtype=np.uint32)
    f = (u << np.uint32(16)).view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) <= 448.0)]
    ours = formats.e4m3_encode(f.astype(np.float64))
    ref = torch.from_numpy(f).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_saturates_and_keeps_sign():
    assert formats.e4m3_encode(np.array([448.0, 464.0, 1e30]))[0] == 0x7E
    assert np.all(formats.e4m3_encode(np.array([464.0, 1e30])) == 0x7E)
    assert np.all(formats.e4m3_encode(np.array([-464.0, -1e30])) == 0xFE)
    assert formats.e4m3_encode(np.array([-0.0]))[0] == 0x80
    assert formats.e4m3_encode(np.array([-1e-30]))[0] == 0x80


def test_bf16_round_vs_torch():
    rng = np.random.default_rng(3)
    f = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(2.0) ** rng.integers(-30, 30, 20000).astype(np.float32),
        (rng.integers(0, 1 << 16, 5000, dtype=np.uint32) << np.uint32(16) | np.uint32(0x8000)).view(np.float32),
    ]).astype(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 3e38) & (np.abs(f) > 1.2e-38)]
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(formats.bf16_encode(f.astype(np.float64)), ref)
    back = formats.bf16_decode(ref)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy())
