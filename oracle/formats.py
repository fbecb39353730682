"""Bit-level number formats used by the block-scaled FP8 path (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages fix the formats by name only: the FP8 operands are
``torch.float8_e4m3fn`` ("DeepInside DeepGEMM", section 4, the dense
example), the scale factors are FP32 or "packed UE8M0, four values in a
single torch.int" (same page, section 2), and the BF16 masked GEMM takes
bfloat16 operands ("DeepGEMM CUDA Graph Compatibility for Masked Grouped
GEMMs", capture example).  The bit layouts below are the published
definitions of those formats (OCP 8-bit floating point E4M3, IEEE-754
binary32 and its upper-half bfloat16, OCP MX E8M0), written out from their
fields.

Pins (tests/test_oracle_formats.py): spec values of named codes
(tests/golden/e4m3_spec_values.txt), agreement with torch's own float8_e4m3fn
and bfloat16 conversions on every code / on random values, encode(decode(c))
== c on every finite code, and ties-to-even on every midpoint; bf16_round
against torch's float32 -> bfloat16 conversion on random and midpoint values
and on hand-picked ties.
"""

import numpy as np

E4M3_MAX = 448.0  # largest finite E4M3 magnitude: exponent field 15, mantissa 6


def _build_e4m3_table():
    """Value of every E4M3 byte, from its fields.

    sign = bit 7, exponent = bits 6..3 (bias 7), mantissa = bits 2..0.
    Exponent 0 is subnormal: (m/8) * 2^(1-7).  Exponent 15 with mantissa 7
    is NaN (both signs); there is no infinity.
    """
    table = np.empty(256, dtype=np.float64)
    for byte in range(256):
        sign = -1.0 if (byte >> 7) & 1 else 1.0
        exp = (byte >> 3) & 0xF
        man = byte & 0x7
        if exp == 15 and man == 7:
            table[byte] = np.nan
        elif exp == 0:
            table[byte] = sign * (man / 8.0) * 2.0 ** (1 - 7)
        else:
            table[byte] = sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return table


_E4M3_TABLE = _build_e4m3_table()
# The 127 non-negative finite codes 0x00..0x7E in increasing value order
# (the byte order of non-negative codes is the value order).
_E4M3_POS = _E4M3_TABLE[:127].copy()


def e4m3_decode(codes):
    """Decode E4M3 bytes (uint8 array) to float64 values."""
    codes = np.asarray(codes, dtype=np.uint8)
    return _E4M3_TABLE[codes]


def e4m3_encode(t):
    """Encode float values to E4M3 bytes: saturate, then round to nearest even.

    t is clamped to [-448, 448] (so the NaN codes are never produced), then
    the nearest representable magnitude is found by bisection over the 127
    sorted non-negative codes; an exact tie goes to the code whose mantissa
    LSB is 0 (the even byte).  The sign bit is the sign of t, so a negative
    value that rounds to zero encodes as 0x80.
    """
    t = np.asarray(t, dtype=np.float64)
    neg = np.signbit(t)
    mag = np.minimum(np.abs(t), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, mag, side="left")  # first code with value >= mag
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - mag
    exact = d_hi == 0.0
    pick = np.where(d_lo < d_hi, lo, hi)
    tie = (d_lo == d_hi) & ~exact
    pick = np.where(tie, np.where(hi % 2 == 0, hi, lo), pick)
    pick = np.where(exact, hi, pick)
    return (pick.astype(np.uint8) | (neg.astype(np.uint8) << 7)).astype(np.uint8)


def bf16_decode(bits):
    """Decode bfloat16 bit patterns (uint16) to float64: they are the upper
    16 bits of an IEEE binary32."""
    bits = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return bits.view(np.float32).astype(np.float64)


def bf16_round(x):
    """Round float64 values to the nearest bfloat16 value, ties to even,
    returned as float64 (one rounding, from the format: 8 significant bits
    for normal values, a fixed step of 2^-133 below 2^-126; values beyond
    the largest bfloat16 become infinite)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)  # x = m * 2^e, 0.5 <= |m| < 1
    normal = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)  # np.rint rounds half to even
    sub = np.ldexp(np.rint(np.ldexp(x, 133)), -133)
    out = np.where(np.abs(x) < 2.0 ** -126, sub, normal)
    big = np.abs(out) >= 2.0 ** 128
    with np.errstate(over="ignore"):
        out = np.where(big, np.copysign(np.inf, x), out)
    return np.where(np.isnan(x), np.nan, out)


def ue8m0_decode(e):
    """Decode unsigned E8M0 exponent bytes: value 2^(e-127); byte 255 is NaN."""
    e = np.asarray(e).astype(np.int64)
    out = np.ldexp(1.0, e - 127)
    return np.where(e == 255, np.nan, out)


def f32_bits(x):
    """IEEE binary32 bit patterns of float32 values, as uint32."""
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)
