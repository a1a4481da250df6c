"""Bit-pattern codecs of the oracle: IEEE binary16, bfloat16 and OCP FP8 E4M3.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages fix no storage format beyond "FP16" for the cache and "FP8" for its
quantised form ("LLM推理引擎深度实战：从PagedAttention到分布式推理部署", §5.3).  The
readings taken here:

* float16: IEEE 754 binary16 (1 sign, 5 exponent bits with bias 15, 10 fraction
  bits, subnormals, Inf and NaN).
* bfloat16: the upper 16 bits of an IEEE binary32.
* FP8: OCP 8-bit floating point, E4M3 "fn" variant (1 sign, 4 exponent bits
  with bias 7, 3 fraction bits, subnormals, no infinities, NaN only at
  S.1111.111, largest finite magnitude 448).  This is the FP8 format gfx950
  implements natively.

All decoders return float64 and are written from the bit-field definitions,
not through a library conversion.  The encoder rounds to the nearest
representable E4M3 value with ties to even and saturates magnitudes above 448
to 448 ("satfinite").
"""

import numpy as np

E4M3_MAX = 448.0


def _f16_fields(bits):
    """IEEE binary16 bit patterns -> float64, from the sign, exponent and fraction fields."""
    b = np.asarray(bits).astype(np.uint32)
    sign = np.where((b >> 15) & 1, -1.0, 1.0)
    exp = ((b >> 10) & 0x1F).astype(np.int64)
    frac = (b & 0x3FF).astype(np.float64)
    normal = sign * np.ldexp(1.0 + frac / 1024.0, exp - 15)
    subnormal = sign * np.ldexp(frac, -24)  # frac * 2^-10 * 2^-14
    special = np.where(frac == 0, sign * np.inf, np.nan)
    return np.where(exp == 0, subnormal, np.where(exp == 31, special, normal))


# All 65536 binary16 values, evaluated once from the field definition above.
_F16_TABLE = _f16_fields(np.arange(1 << 16, dtype=np.uint32))


def decode_f16(bits):
    """IEEE binary16 bit patterns (uint16 array) -> float64 (table of the field definition)."""
    return _F16_TABLE[np.asarray(bits).astype(np.uint16)]


def decode_bf16(bits):
    """bfloat16 bit patterns (uint16 array) -> float64: the top half of a binary32."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def _e4m3_value(code):
    """Value of one OCP E4M3 (fn) code, from its bit fields."""
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    frac = code & 0x7
    if exp == 0xF and frac == 0x7:
        return float("nan")
    if exp == 0:
        return sign * frac * 2.0 ** -9  # subnormal: 2^(1-7) * frac/8
    return sign * (1.0 + frac / 8.0) * 2.0 ** (exp - 7)


_E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_table():
    """float64 values of all 256 E4M3 codes (NaN at 0x7F and 0xFF)."""
    return _E4M3_TABLE.copy()


def decode_e4m3(codes):
    """E4M3 codes (uint8 array) -> float64."""
    return _E4M3_TABLE[np.asarray(codes).astype(np.uint8)]


# The 127 finite non-negative E4M3 values, in code order 0x00..0x7E, which is
# also ascending value order.
_E4M3_POS = _E4M3_TABLE[:0x7F]


def encode_e4m3(x):
    """float32 values -> E4M3 codes: round to nearest, ties to even, satfinite.

    For each |x| the two neighbouring representable magnitudes are found and
    the nearer one is taken; on an exact tie the one with the even code (even
    last fraction bit) wins.  Magnitudes of 448 and above become 448 (0x7E).
    The sign bit of x is kept, so -0.0 and negative values that round to zero
    encode as 0x80.  NaN encodes as 0x7F / 0xFF.
    """
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x).astype(np.float64)
    neg = np.signbit(x)
    nan = np.isnan(x)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    lo = np.searchsorted(_E4M3_POS, a, side="right") - 1  # largest value <= a
    lo = np.clip(lo, 0, 0x7E)
    hi = np.minimum(lo + 1, 0x7E)
    d_lo = a - _E4M3_POS[lo]  # exact in float64
    d_hi = _E4M3_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi != lo) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = mag | np.where(neg, 0x80, 0x00).astype(np.uint8)
    return np.where(nan, np.uint8(0x7F) | np.where(neg, 0x80, 0).astype(np.uint8), code).astype(np.uint8)


def decode_bits(bits, dtype):
    """Decode a bit-pattern array of the named storage dtype to float64.

    dtype: "f16" (uint16 patterns), "bf16" (uint16 patterns) or "fp8_e4m3"
    (uint8 codes).
    """
    if dtype == "f16":
        return decode_f16(bits)
    if dtype == "bf16":
        return decode_bf16(bits)
    if dtype == "fp8_e4m3":
        return decode_e4m3(bits)
    raise ValueError(f"unknown dtype {dtype!r}")
