"""Pins of the oracle's block quantization: error bounds and code ranges, an
independent implementation through library routines (torch.frexp and torch's
float8_e4m3fn cast), the two lossless casts the "DeepSeek-V4-Pro-0813-nvfp4-
DSpark" article states (MXFP4 -> NVFP4 in 阶段三导出; E2M1 -> E4M3 with a
per-128 scale in "关于 MXFP4 的无损种子"), and the weight shapes the W4AFP8-mt
card prints."""

import os

import numpy as np
import torch

import synth
from oracle import ffn, formats, quant, route

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(rng, r, c):
    v = rng.standard_normal((r, c)) * 2.0 ** rng.integers(-20, 20, (r, 1))
    return formats.bf16_round(v)


def _torch_act_quant(v):
    """Independent per-128 quantization with torch: the exponent from
    torch.frexp (amax = m * 2**x, m in [0.5, 1)): the smallest e with
    amax <= 448 * 2**e, with 448 = 0.875 * 2**9, is x - 9 when m <= 0.875
    and x - 8 otherwise; the codes from torch's round-to-nearest-even fp8
    cast."""
    t = torch.from_numpy(v).reshape(v.shape[0], -1, 128)
    amax = t.abs().amax(dim=2)
    m, x = torch.frexp(amax)
    e = torch.where(m <= 0.875, x - 9, x - 8)
    e = torch.where(amax == 0, torch.full_like(e, -127), e).clamp(-127, 127)
    scaled = torch.ldexp(t, -e[:, :, None].to(torch.float64))
    codes = scaled.to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.reshape(v.shape).numpy(), (e + 127).to(torch.uint8).numpy()


def test_act_quant_matches_library_route():
    rng = np.random.default_rng(11)
    v = _rows(rng, 64, 1024)
    v[3, :128] = 0.0
    v[4, 128:256] = -0.0
    v[5, 256:384] = 448.0 * 2.0 ** -3          # amax exactly on a boundary
    q, s = quant.act_quant(v)
    tq, ts = _torch_act_quant(v)
    assert np.array_equal(s, ts)
    assert np.array_equal(q, tq)


def test_act_quant_bounds():
    rng = np.random.default_rng(12)
    v = _rows(rng, 200, 512)
    q, s = quant.act_quant(v)
    e = s.astype(np.int64) - 127
    d = quant.act_dequant(q, s)
    vb = v.reshape(200, 4, 128)
    scaled = np.abs(vb) * np.ldexp(1.0, -e)[:, :, None]
    assert scaled.max() <= 448.0                                  # never saturates
    mx = np.abs(formats.e4m3_decode(q)).reshape(200, 4, 128).max(axis=2)
    assert mx.min() >= 224.0 and mx.max() <= 448.0               # scale is tight
    # rounding error at most half an E4M3 step of the element's binade
    a = np.abs(scaled)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    half = np.ldexp(1.0, np.maximum(ex - 1, -6) - 4) * np.ldexp(1.0, e)[:, :, None]
    assert np.all(np.abs(d.reshape(vb.shape) - vb) <= half)


def test_act_quant_exact_rows_and_edges():
    # a row that is already E4M3 values times 2**e comes back unchanged
    codes = np.arange(0, 0x7F)
    vals = formats.e4m3_decode(codes)
    row = np.concatenate([vals, [448.0]])[None, :] * 2.0 ** -5
    q, s = quant.act_quant(row)
    assert s[0, 0] == 127 - 5 and np.array_equal(quant.act_dequant(q, s), row)
    # zero block: scale byte 0 (2**-127), codes 0 and 0x80 for -0
    z = np.zeros((1, 128))
    z[0, 1::2] = -0.0
    q, s = quant.act_quant(z)
    assert s[0, 0] == 0 and np.all(q[0, 0::2] == 0) and np.all(q[0, 1::2] == 0x80)
    # exponent boundaries: amax = 448 * 2**e exactly -> e; one ulp above -> e + 1
    for e in (-20, -3, 0, 5):
        b = np.zeros((2, 128))
        b[0, 7] = 448.0 * 2.0 ** e
        b[1, 7] = np.nextafter(448.0 * 2.0 ** e, np.inf)
        _, s = quant.act_quant(b)
        assert s[0, 0] == e + 127 and s[1, 0] == e + 128
    # tiny amax clamps the exponent at -127
    t = np.zeros((1, 128))
    t[0, 0] = 2.0 ** -133
    q, s = quant.act_quant(t)
    assert s[0, 0] == 0 and formats.e4m3_decode(q[0, 0]) == 2.0 ** -6


def _e2m1_as_e4m3_byte(c):
    """Bit-level E2M1 -> E4M3 re-encoding (no arithmetic): sign moves to bit 7;
    a normal E2M1 (exponent field e in 1..3, bias 1) becomes exponent field
    e + 6 (bias 7) with its mantissa bit as the top E4M3 mantissa bit; the
    E2M1 subnormal 0.5 is 2**-1, exponent field 6; zero stays zero."""
    c = np.asarray(c, np.int64)
    s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
    mag = np.where(e > 0, ((e + 6) << 3) | (m << 2), np.where(m == 1, 6 << 3, 0))
    return ((s << 7) | mag).astype(np.uint8)


def test_mxfp4_dequant_vs_library_route():
    rng = np.random.default_rng(13)
    n, k = 48, 256
    packed = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    scales = rng.integers(110, 140, (n, k // 32)).astype(np.uint8)
    ours = quant.mxfp4_dequant(packed, scales)
    lo, hi = packed & 0xF, packed >> 4
    codes = np.stack([lo, hi], axis=2).reshape(n, k)          # element 2j low nibble
    vals = torch.tensor(_e2m1_as_e4m3_byte(codes)).view(torch.float8_e4m3fn).to(torch.float64)
    sc = torch.ldexp(torch.ones(n, k // 32, dtype=torch.float64),
                     torch.tensor(scales.astype(np.int64) - 127, dtype=torch.float64))
    ref = (vals.reshape(n, k // 32, 32) * sc[:, :, None]).reshape(n, k).numpy()
    assert np.array_equal(ours, ref)


def test_nvfp4_dequant_vs_library_route():
    # per-16 E4M3 scales with mantissa bits, decoded through torch's fp8 type
    rng = np.random.default_rng(17)
    n, k = 24, 256
    packed = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    s16 = (rng.integers(1, 15, (n, k // 16)) << 3 | rng.integers(0, 8, (n, k // 16))).astype(np.uint8)
    ours = quant.nvfp4_dequant(packed, s16)
    lo, hi = packed & 0xF, packed >> 4
    codes = np.stack([lo, hi], axis=2).reshape(n, k)
    vals = torch.tensor(_e2m1_as_e4m3_byte(codes)).view(torch.float8_e4m3fn).to(torch.float64)
    sc = torch.tensor(s16).view(torch.float8_e4m3fn).to(torch.float64)
    ref = (vals.reshape(n, k // 16, 16) * sc[:, :, None]).reshape(n, k).numpy()
    assert np.array_equal(ours, ref)


def test_nvfp4_experts_equal_mxfp4_experts_when_lossless():
    # MXFP4 re-expressed as NVFP4 (power-of-two per-16 scales): the oracle's
    # NVFP4 expert FFN must reproduce the MXFP4 one bit for bit
    wl = synth.WORKLOADS["tiny"].replace(hidden=512, inter=256, n_experts=5, top_k=2)
    inp = synth.make_inputs(wl, tokens=20)
    nv = {}
    for nme in ("w1", "w3", "w2"):
        q, sc = zip(*(quant.nvfp4_from_mxfp4(inp[nme][e], inp[nme + "_scale"][e]) for e in range(5)))
        nv[nme], nv[nme + "_scale"] = np.stack(q), np.stack(sc)
    xq, xs = quant.act_quant(formats.bf16_decode(inp["x"]))
    r = route.route(inp["x"], inp["w_gate"], k=2)
    a = ffn.expert_ffn(xq, xs, r, inp, 2)
    b = ffn.expert_ffn(xq, xs, r, nv, 2, weight_format="nvfp4")
    for key in ("hq", "hs", "h", "o"):
        assert np.array_equal(a[key], b[key]), key


def test_mxfp4_to_nvfp4_lossless():
    # same nibbles, per-16 E4M3 scales: identical values whenever 2**(b-127)
    # is an E4M3 value, b in [118, 135]
    rng = np.random.default_rng(14)
    n, k = 64, 512
    packed = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    scales = rng.integers(118, 136, (n, k // 32)).astype(np.uint8)
    p2, s16 = quant.nvfp4_from_mxfp4(packed, scales)
    assert np.array_equal(p2, packed) and s16.shape == (n, k // 16)
    assert np.array_equal(quant.nvfp4_dequant(p2, s16), quant.mxfp4_dequant(packed, scales))
    # NVFP4 scale bytes double, weight bytes unchanged (the article's table)
    assert s16.nbytes == 2 * scales.nbytes and p2.nbytes == packed.nbytes
    # outside that range the cast is not lossless
    bad = scales.copy()
    bad[0, 0] = 136
    assert not np.array_equal(quant.nvfp4_dequant(*quant.nvfp4_from_mxfp4(packed, bad)),
                              quant.mxfp4_dequant(packed, bad))


def test_e2m1_to_e4m3_per128_cast():
    rng = np.random.default_rng(15)
    n, k = 32, 1024
    packed = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    base = rng.integers(100, 140, (n, k // 128, 1))
    spread = rng.integers(0, 9, (n, k // 128, 4))                # span <= 8: lossless
    scales = (base + spread).reshape(n, k // 32).astype(np.uint8)
    q, s = quant.e4m3_from_mxfp4(packed, scales)
    # decode through torch's E4M3 (library), not the oracle's decoder
    vals = torch.tensor(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    deq = (vals.reshape(n, k // 128, 128) * np.ldexp(1.0, s.astype(np.int64) - 127)[:, :, None]).reshape(n, k)
    assert np.array_equal(deq, quant.mxfp4_dequant(packed, scales))
    # a span of 9 loses the 0.5 * 2**-9 values: detected as lossy
    scales2 = scales.copy().reshape(n, k // 128, 4)
    scales2[:, :, 0] = scales2[:, :, 1:].max(axis=2) - 9
    scales2 = scales2.reshape(n, k // 32)
    packed2 = packed.copy()
    packed2[:, :16] = 0x11                                       # code 1 = 0.5 in block 0
    q2, s2 = quant.e4m3_from_mxfp4(packed2, scales2)
    v2 = torch.tensor(q2).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    d2 = (v2.reshape(n, k // 128, 128) * np.ldexp(1.0, s2.astype(np.int64) - 127)[:, :, None]).reshape(n, k)
    assert not np.array_equal(d2, quant.mxfp4_dequant(packed2, scales2))


def test_fp8_dequant_vs_library_route():
    rng = np.random.default_rng(16)
    n, k = 8, 512
    codes = rng.integers(0, 256, (n, k), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0                            # no NaN codes
    scales = rng.integers(110, 140, (n, k // 128), dtype=np.uint8)
    vals = torch.tensor(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    want = vals * np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 128, axis=1)
    assert np.array_equal(quant.fp8_dequant(codes, scales), want)


def test_fp8_experts_equal_mxfp4_experts_when_lossless():
    # the synthetic exponents span 3 values: the cast is lossless, so the FP8
    # expert path must give bit-identical h bytes and outputs
    wl = synth.WORKLOADS["tiny"].replace(hidden=512, inter=256, n_experts=6, top_k=2)
    inp = synth.make_inputs(wl, tokens=24)
    f8 = quant.fp8_experts_from_mxfp4(inp)
    assert f8["w1"].shape == (6, 256, 512) and f8["w1_scale"].shape == (6, 256, 4)
    assert f8["w2"].shape == (6, 512, 256) and f8["w2_scale"].shape == (6, 512, 2)
    for e in range(6):
        for nme in ("w1", "w3", "w2"):
            assert np.array_equal(quant.fp8_dequant(f8[nme][e], f8[nme + "_scale"][e]),
                                  quant.mxfp4_dequant(inp[nme][e], inp[nme + "_scale"][e]))
    xq, xs = quant.act_quant(formats.bf16_decode(inp["x"]))
    r = route.route(inp["x"], inp["w_gate"], k=2)
    a = ffn.expert_ffn(xq, xs, r, inp, 2)
    b = ffn.expert_ffn(xq, xs, r, f8, 2, weight_format="fp8")
    for key in ("hq", "hs", "h", "o"):
        assert np.array_equal(a[key], b[key]), key


def test_expert_layout_matches_printed_shapes():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "w4afp8_w1_shapes.txt"))
            if l.strip() and not l.startswith("#")]
    shapes = {r[0]: (int(r[1]), int(r[2])) for r in rows}
    hidden, inter = 4096, 2048
    # our w1 of one expert: [I, H/2] bytes; the printed int4 tensor has the same
    # byte shape (two 4-bit values per byte along K)
    assert shapes["w1.weight"] == (inter, hidden // 2)
    # the printed group-128 scale is [N, K/128]; ours is per 32: [N, K/32]
    assert shapes["w1.weight_scale_inv"] == (inter, hidden // 128)
    import synth
    wl = synth.WORKLOADS["decode"]
    inp = synth.make_inputs(wl.replace(n_experts=2), tokens=1)
    assert inp["w1"].shape[1:] == shapes["w1.weight"]
    assert inp["w1_scale"].shape[1:] == (inter, hidden // 32)


def test_int4_dequant_hand_values():
    # two's complement nibbles, even element of K in the low nibble:
    # 0x7F -> (-1, 7), 0x80 -> (0, -8), 0x19 -> (-7, 1), 0xF8 -> (-8, -1)
    packed = np.zeros((1, 64), np.uint8)
    packed[0, :4] = [0x7F, 0x80, 0x19, 0xF8]
    scales = np.array([[0.375]], np.float32)
    w = quant.int4_dequant(packed, scales)
    assert w.shape == (1, 128)
    assert w[0, :8].tolist() == [-0.375, 2.625, 0.0, -3.0, -2.625, 0.375, -3.0, -0.375]
    assert not w[0, 8:].any()


def test_int4_dequant_vs_library_route():
    # numpy's int8 arithmetic shift sign-extends each nibble; scales repeat
    # over their 128-element group
    rng = np.random.default_rng(21)
    n, k = 24, 640
    packed = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    scales = rng.uniform(-3.0, 3.0, (n, k // 128)).astype(np.float32)
    lo = (packed << 4).astype(np.uint8).view(np.int8) >> 4
    hi = packed.view(np.int8) >> 4
    q = np.stack([lo, hi], axis=2).reshape(n, k).astype(np.float64)
    want = q * np.repeat(scales.astype(np.float64), 128, axis=1)
    assert np.array_equal(quant.int4_dequant(packed, scales), want)
    assert set(np.unique(q)) == set(range(-8, 8))


def test_w4afp8_experts_equal_fp8_experts_for_pow2_scales():
    # INT4 codes times power-of-two group scales are E4M3 values times an
    # E8M0 scale per 128: the oracle's W4AFP8 expert FFN must reproduce the
    # FP8-expert one bit for bit on those weights
    wl = synth.WORKLOADS["tiny"].replace(hidden=512, inter=256, n_experts=5, top_k=2)
    inp = synth.make_inputs(wl, tokens=20)
    inp.update(synth.w4afp8_scales(wl, pow2=True))
    f8 = {}
    for nme in ("w1", "w3", "w2"):
        codes = quant.unpack_nibbles(inp[nme].reshape(-1, inp[nme].shape[-1]))
        q = np.where(codes >= 8, codes.astype(np.int64) - 16, codes).astype(np.float64)
        f8[nme] = formats.e4m3_encode(q).reshape(inp[nme].shape[0], inp[nme].shape[1], -1)
        e = np.log2(inp[nme + "_scale"].astype(np.float64))
        assert np.array_equal(e, np.round(e))
        f8[nme + "_scale"] = (e + 127).astype(np.uint8)
    xq, xs = quant.act_quant(formats.bf16_decode(inp["x"]))
    r = route.route(inp["x"], inp["w_gate"], k=2)
    a = ffn.expert_ffn(xq, xs, r, f8, 2, weight_format="fp8")
    b = ffn.expert_ffn(xq, xs, r, inp, 2, weight_format="w4afp8")
    for key in ("hq", "hs", "h", "o"):
        assert np.array_equal(a[key], b[key]), key
    assert np.abs(a["o"]).max() > 0


def test_w4afp8_scales_draw():
    wl = synth.WORKLOADS["decode"].replace(n_experts=2)
    s = synth.w4afp8_scales(wl)
    assert s["w1_scale"].shape == (2, wl.inter, wl.hidden // 128) and s["w1_scale"].dtype == np.float32
    assert s["w2_scale"].shape == (2, wl.hidden, wl.inter // 128)
    v = s["w1_scale"].astype(np.float64)
    m, e = np.frexp(v)          # v = m * 2**e, m in [0.5, 1)
    assert (m >= 0.5).all() and (m < 0.75).all()
    assert e.min() >= wl.exp_lo and e.max() <= wl.exp_hi
