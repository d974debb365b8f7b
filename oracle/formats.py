"""Element codecs of the layer (oracle; test infrastructure only).

E2M1 ("FP4", the expert-weight element), E8M0 (the per-32 weight scale and
the per-128 activation scale), OCP E4M3FN ("FP8", the activation element) and
bfloat16 (router, shared expert and the layer output).

Sources: "DeepSeek-V4-Flash-SI" card, 架构特性 / 低精度计算 (FP4 E2M1 +
F8_E8M0 per 32; FP8 E4M3 activations with power-of-two scales);
"DeepSeek-V4-Pro-0813-nvfp4-DSpark" article, 阶段三导出 table (E8M0 is a pure
power of two) and the e2m1fn -> e4m3fn cast (the 'fn' variants: finite, no
infinities).  Rounding of the FP8 encoder is round-half-to-even with
saturation to the largest finite value, the "half_even" rounding named in the
PTPC-FP8 article's 量化脚本参数逐行拆解 section; the pages leave the FP8
encoder's rounding otherwise open.
"""

import numpy as np

# --------------------------------------------------------------------------
# E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit, no inf/NaN.
# exponent field 0 is subnormal: 0.5 * m; otherwise 2**(e-1) * (1 + m/2).
# --------------------------------------------------------------------------


def e2m1_decode(codes):
    """Decode 4-bit E2M1 codes (0..15, any int array) to float64."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = c & 0x1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return sign * mag


def e2m1_table():
    """The 16-entry FP4 table indexed by code."""
    return e2m1_decode(np.arange(16))


# --------------------------------------------------------------------------
# E8M0: an unsigned 8-bit biased exponent, value 2**(b - 127); 255 is NaN.
# --------------------------------------------------------------------------


def e8m0_decode(b):
    b = np.asarray(b).astype(np.int64)
    out = np.ldexp(1.0, b - 127)
    return np.where(b == 255, np.nan, out)


# --------------------------------------------------------------------------
# OCP E4M3FN: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits.  Exponent
# field 0 is subnormal (m * 2**-9).  S.1111.111 is NaN; no infinities, so the
# largest finite magnitude is 1.75 * 2**8 = 448.
# --------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_decode(b):
    b = np.asarray(b).astype(np.int64) & 0xFF
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 0x7
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((b & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e4m3_encode(v):
    """Round float64 values to E4M3FN codes: nearest, ties to even mantissa,
    magnitudes beyond 448 saturate to 448, the sign of zero is kept.

    The step between neighbouring E4M3 values in the binade [2**E, 2**(E+1))
    is 2**(E-3); below 2**-6 (the subnormal range) the step is 2**-9.  The
    magnitude is divided by its step (exact: a power of two), rounded half to
    even, and multiplied back; the code is then read off the rounded value.
    """
    v = np.asarray(v, dtype=np.float64)
    neg = np.signbit(v)
    a = np.abs(v)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))   # a = f * 2**ex, f in [0.5, 1)
    binade = np.maximum(ex - 1, -6)             # floor(log2 a), floored at -6
    step = np.ldexp(1.0, binade - 3)
    q = np.rint(a / step) * step                # np.rint: half to even
    q = np.where(a > 0, q, 0.0)
    q = np.minimum(q, E4M3_MAX)
    # read the code off q (q is an exact E4M3 magnitude now)
    _, qx = np.frexp(np.where(q > 0, q, 1.0))
    qb = qx - 1
    sub = q < 2.0 ** -6
    e_field = np.where(sub, 0, qb + 7)
    m_field = np.where(sub, np.rint(q / 2.0 ** -9),
                       np.rint((q / np.ldexp(1.0, qb) - 1.0) * 8.0))
    code = (e_field.astype(np.int64) << 3) | m_field.astype(np.int64)
    code = np.where(q == 0, 0, code)
    code = code | np.where(neg, 0x80, 0)
    return code.astype(np.uint8)


# --------------------------------------------------------------------------
# bfloat16: the upper 16 bits of an IEEE binary32.
# --------------------------------------------------------------------------


def bf16_decode(u16):
    u = np.asarray(u16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def bf16_round(v):
    """Round float64 values to bfloat16 (nearest, ties to even) and return the
    rounded values as float64.  Done on the exact float64 value: bf16 has an
    8-bit significand, so the rounding is on multiples of 2**(E-7)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    binade = np.maximum(ex - 1, -126)           # bf16 shares fp32's exponent range
    step = np.ldexp(1.0, binade - 7)
    q = np.rint(a / step) * step
    return np.copysign(np.where(a > 0, q, 0.0), v)


def bf16_encode(v):
    """float64 -> bf16 bit patterns (uint16), nearest-even, via bf16_round."""
    r = bf16_round(v).astype(np.float32)        # exact: r has <= 8 significant bits
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
