"""Block quantization steps of the layer (oracle; test infrastructure only).

* act_quant      - online FP8 E4M3 activation quantization, one power-of-two
                   (ue8m0) scale per 128 consecutive elements of a row.
                   "DeepSeek-V4-Flash-SI" card, 架构特性 / 低精度计算 and the
                   模型训练 table (dynamic FP8 E4M3, ue8m0 scale).
* mxfp4_dequant  - expert weights: E2M1 nibbles, two per byte along K, with
                   one E8M0 scale per 32 elements of K.  Same card,
                   低精度计算; layout [N, K/2] bytes + [N, K/32] scales as the
                   "DeepSeek-V4-Flash-0731-W4AFP8-mt" card's 权重约定 section
                   shows for the expert tensors.
* nvfp4_from_mxfp4 / nvfp4_dequant - the lossless re-expression of an MXFP4
                   block as NVFP4 (same nibbles, one E4M3 scale per 16
                   elements): "DeepSeek-V4-Pro-0813-nvfp4-DSpark", 阶段三导出.
* e4m3_from_mxfp4 - the lossless E2M1 -> E4M3 cast with the scale rewritten
                   per 128-block: same article, 阶段一 ("关于 MXFP4 的无损种子"),
                   which also names the FP8-expert checkpoint option.
* fp8_dequant    - FP8 expert weights as that cast leaves them: E4M3 bytes
                   [N, K] with one E8M0 scale per 128 elements of K.
* int4_dequant   - W4AFP8 expert weights: signed INT4, two per byte along K,
                   one float32 scale per 128 elements of K
                   ("DeepSeek-V4-Flash-0731-W4AFP8-mt" card, 量化方式 and
                   权重约定: symmetric INT4 with group size 128,
                   weight_scale_inv float32 [N, K/128]).

Readings where the pages are silent (listed with the others in the design
notes):
* the power-of-two activation scale is 2**e with e the smallest integer such
  that amax <= 448 * 2**e (so no element saturates); an all-zero block takes
  e = -127; e is clamped to [-127, 127] and stored as the byte e + 127;
* within a byte the even element of K sits in the low nibble;
* the per-128 scale of the E4M3 cast is the largest of its four per-32
  exponents;
* an INT4 nibble is two's complement (-8..7) and the float32
  weight_scale_inv multiplies it (w = q * scale_inv).
"""

import numpy as np

from . import formats

ACT_BLOCK = 128
W_BLOCK = 32


def pow2_scale_exponent(amax):
    """Smallest integer e with amax <= 448 * 2**e, computed exactly; amax == 0
    gives -127; the result is clamped to [-127, 127]."""
    amax = np.asarray(amax, dtype=np.float64)
    pos = amax > 0
    safe = np.where(pos, amax, 1.0)
    e = np.ceil(np.log2(safe / formats.E4M3_MAX)).astype(np.int64)
    # exact fix-up: 448 * 2**e is exact in float64, so these comparisons are exact
    for _ in range(2):
        too_small = safe > np.ldexp(formats.E4M3_MAX, e)
        e = np.where(too_small, e + 1, e)
        too_big = safe <= np.ldexp(formats.E4M3_MAX, e - 1)
        e = np.where(too_big, e - 1, e)
    e = np.where(pos, e, -127)
    return np.clip(e, -127, 127)


def act_quant(v, block=ACT_BLOCK):
    """Quantize rows of float64 values to E4M3 codes with one E8M0 scale per
    `block` consecutive elements.  Returns (codes u8 [rows, cols],
    scales u8 [rows, cols/block])."""
    v = np.asarray(v, dtype=np.float64)
    rows, cols = v.shape
    assert cols % block == 0
    vb = v.reshape(rows, cols // block, block)
    amax = np.max(np.abs(vb), axis=2)
    e = pow2_scale_exponent(amax)
    scaled = vb * np.ldexp(1.0, -e)[:, :, None]     # exact: power-of-two scale
    codes = formats.e4m3_encode(scaled).reshape(rows, cols)
    return codes, (e + 127).astype(np.uint8)


_E4M3_TABLE = formats.e4m3_decode(np.arange(256))
_E2M1_TABLE = formats.e2m1_table()


def act_dequant(codes, scales, block=ACT_BLOCK):
    codes = np.asarray(codes)
    rows, cols = codes.shape
    val = _E4M3_TABLE[codes].reshape(rows, cols // block, block)
    sc = formats.e8m0_decode(scales)[:, :, None]
    return (val * sc).reshape(rows, cols)


def unpack_nibbles(packed):
    """[N, K/2] bytes -> [N, K] codes; element 2j is the low nibble of byte j."""
    p = np.asarray(packed, dtype=np.uint8)
    n, kh = p.shape
    out = np.empty((n, 2 * kh), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def mxfp4_dequant(packed, scales, block=W_BLOCK):
    """Dequantize one [N, K] MXFP4 matrix to float64."""
    codes = unpack_nibbles(packed)
    n, k = codes.shape
    assert scales.shape == (n, k // block)
    val = _E2M1_TABLE[codes].reshape(n, k // block, block)
    return (val * formats.e8m0_decode(scales)[:, :, None]).reshape(n, k)


def nvfp4_from_mxfp4(packed, scales):
    """Re-express an MXFP4 matrix as NVFP4: the same nibble bytes and one E4M3
    scale per 16 elements, each the E4M3 code of its parent per-32 scale.
    Exact only when every 2**(b-127) is an E4M3 value, i.e. b in [118, 135]."""
    s = formats.e8m0_decode(scales)
    s16 = np.repeat(s, 2, axis=1)
    return np.asarray(packed, dtype=np.uint8).copy(), formats.e4m3_encode(s16)


def nvfp4_dequant(packed, scales16):
    codes = unpack_nibbles(packed)
    n, k = codes.shape
    val = formats.e2m1_decode(codes).reshape(n, k // 16, 16)
    return (val * formats.e4m3_decode(scales16)[:, :, None]).reshape(n, k)


def e4m3_from_mxfp4(packed, scales):
    """Cast an MXFP4 matrix to E4M3 elements with one E8M0 scale per 128: the
    nibbles are split and decoded through the FP4 table, the new block
    exponent is the largest of the four per-32 exponents, and each element is
    re-encoded relative to it.  Lossless iff within every 128-block the four
    per-32 exponents span at most 8 (the E4M3 subnormal floor 2**-9 against
    the smallest E2M1 magnitude 0.5)."""
    codes = unpack_nibbles(packed)
    n, k = codes.shape
    e32 = np.asarray(scales).astype(np.int64) - 127               # [n, k/32]
    e128 = e32.reshape(n, k // 128, 4).max(axis=2)                # [n, k/128]
    rel = np.repeat(e32 - np.repeat(e128, 4, axis=1), 32, axis=1)  # [n, k], <= 0
    vals = formats.e2m1_decode(codes) * np.ldexp(1.0, rel)
    return formats.e4m3_encode(vals), (e128 + 127).astype(np.uint8)


def fp8_dequant(codes, scales, block=ACT_BLOCK):
    """Dequantize one [N, K] FP8 expert matrix (E4M3 bytes, one E8M0 scale
    per 128 elements of K) to float64."""
    codes = np.asarray(codes, dtype=np.uint8)
    n, k = codes.shape
    assert scales.shape == (n, k // block)
    val = formats.e4m3_decode(codes).astype(np.float64).reshape(n, k // block, block)
    return (val * formats.e8m0_decode(scales)[:, :, None]).reshape(n, k)


def fp8_experts_from_mxfp4(w):
    """All routed expert matrices of a weight dict (w1, w3, w2 and their
    scales, stacked over experts) cast to FP8 with e4m3_from_mxfp4."""
    out = {}
    for n in ("w1", "w3", "w2"):
        q, sc = zip(*(e4m3_from_mxfp4(w[n][e], w[n + "_scale"][e]) for e in range(w[n].shape[0])))
        out[n], out[n + "_scale"] = np.stack(q), np.stack(sc)
    return out


def int4_dequant(packed, scales, block=ACT_BLOCK):
    """Dequantize one [N, K] W4AFP8 matrix to float64: the nibbles of
    [N, K/2] bytes read as two's complement integers -8..7 (even element of K
    in the low nibble), times the float32 scale of their 128-element group
    of K, scales [N, K/128]."""
    codes = unpack_nibbles(packed).astype(np.int64)
    q = np.where(codes >= 8, codes - 16, codes)
    n, k = q.shape
    sc = np.asarray(scales, dtype=np.float32).astype(np.float64)
    assert sc.shape == (n, k // block)
    return (q.astype(np.float64).reshape(n, k // block, block) * sc[:, :, None]).reshape(n, k)
