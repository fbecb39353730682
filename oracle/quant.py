"""FP8 quantizers and UE8M0 packing (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What is computed:
  * Per-token cast: every row of x is cut into 1x128 blocks along K (the
    activation scale granularity of the dense example in "DeepInside
    DeepGEMM", section 4: one scale per row per 128-wide K-block).  Each
    block gets one FP32 scale s = amax / 448 (448 is the largest finite
    E4M3 magnitude, so the block maximum maps onto it) and its elements are
    stored as e4m3(x / s).
  * Per-block cast: the same over 128x128 blocks (the weight granularity:
    one scale per 128 rows of B per 128-wide K-block).
  * use_ue8m0: the scale is rounded up to a power of two, so it can be
    stored as an unsigned E8M0 exponent ("packed UE8M0 format", same page,
    section 2).
  * pack_ue8m0_to_int: the exponent byte of each FP32 scale, four
    consecutive K-blocks per little-endian int32 ("[GH-ISSUE #414]
    pack_ue8m0_to_int is not CUDA Graph capture safe", section "Expected
    behavior": shift the int32 view right by 23 and keep the low byte).

Readings where the pages are silent:
  * amax is floored at AMAX_FLOOR = 1e-4 so an all-zero block has a finite
    scale and encodes to zeros.
  * s is the correctly rounded FP32 quotient amax/448, and the quantized
    value is e4m3(fp32(x / s)) with a correctly rounded FP32 division.
  * UE8M0 rounds the FP32 scale up: the smallest power of two >= s.
  * A partial last block (K % 128 != 0 or rows % 128 != 0) uses the
    elements that exist.

Pins: tests/test_oracle_quant.py (including an exact pin of the scale and
quotient rule: every scale equals RN32(max(amax, 1e-4) / 448) and every
code e4m3(RN32(x / s)), both quotients computed with integer arithmetic on
the binary32 inputs, on 10^4+ blocks of FP32 and BF16-valued sources) and
tests/test_oracle_pack.py.
"""

import numpy as np

from .formats import E4M3_MAX, e4m3_encode, f32_bits

AMAX_FLOOR = np.float32(1e-4)
BLOCK = 128


def _scale_from_amax(amax, use_ue8m0):
    """FP32 scale for a block maximum (float32 array)."""
    amax = np.maximum(np.asarray(amax, dtype=np.float32), AMAX_FLOOR)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)  # IEEE binary32 division
    if use_ue8m0:
        # smallest power of two >= s: frexp gives s = f * 2^e with f in [0.5, 1);
        # s is already a power of two exactly when f == 0.5.
        f, e = np.frexp(s.astype(np.float64))
        s = np.where(f == 0.5, s.astype(np.float64), np.ldexp(1.0, e)).astype(np.float32)
    return s


def per_token_cast_to_fp8(x, use_ue8m0=False):
    """Quantize x [..., K] (float32) with one scale per 1x128 block of each row.

    Returns (q uint8 [..., K] E4M3 codes, sf float32 [..., ceil(K/128)]).
    """
    x = np.asarray(x, dtype=np.float32)
    K = x.shape[-1]
    nkb = -(-K // BLOCK)
    q = np.empty(x.shape, dtype=np.uint8)
    sf = np.empty(x.shape[:-1] + (nkb,), dtype=np.float32)
    for kb in range(nkb):
        blk = x[..., kb * BLOCK:(kb + 1) * BLOCK]
        amax = np.abs(blk).max(axis=-1)
        s = _scale_from_amax(amax, use_ue8m0)
        sf[..., kb] = s
        q[..., kb * BLOCK:(kb + 1) * BLOCK] = e4m3_encode((blk / s[..., None]).astype(np.float32))
    return q, sf


def per_block_cast_to_fp8(x, use_ue8m0=False):
    """Quantize x [(G,) N, K] (float32) with one scale per 128x128 block.

    Returns (q uint8 same shape, sf float32 [(G,) ceil(N/128), ceil(K/128)]).
    """
    x = np.asarray(x, dtype=np.float32)
    N, K = x.shape[-2], x.shape[-1]
    nnb, nkb = -(-N // BLOCK), -(-K // BLOCK)
    q = np.empty(x.shape, dtype=np.uint8)
    sf = np.empty(x.shape[:-2] + (nnb, nkb), dtype=np.float32)
    for nb in range(nnb):
        rows = slice(nb * BLOCK, (nb + 1) * BLOCK)
        for kb in range(nkb):
            cols = slice(kb * BLOCK, (kb + 1) * BLOCK)
            blk = x[..., rows, cols]
            amax = np.abs(blk).max(axis=(-2, -1))
            s = _scale_from_amax(amax, use_ue8m0)
            sf[..., nb, kb] = s
            q[..., rows, cols] = e4m3_encode((blk / s[..., None, None]).astype(np.float32))
    return q, sf


def pack_ue8m0_to_int(x):
    """Pack FP32 power-of-two scales x [..., n] into int32 [..., ceil(n/4)].

    Byte j of the result holds the binary32 exponent field (bits 30..23) of
    x[..., 4i + j]; the sign bit and the mantissa are dropped, which is what
    an arithmetic right shift by 23 followed by a cast to uint8 keeps.
    Missing tail elements (n % 4 != 0) contribute zero bytes.

    Returns (packed int32 array, number of inputs that are not valid UE8M0,
    i.e. negative or with a non-zero mantissa -- the validity predicate of
    the issue's Summary section).
    """
    bits = f32_bits(x)
    n = bits.shape[-1]
    nw = -(-n // 4)
    exp_byte = ((bits >> np.uint32(23)) & np.uint32(0xFF)).astype(np.uint64)
    out = np.zeros(bits.shape[:-1] + (nw,), dtype=np.uint64)
    for j in range(n):
        out[..., j // 4] += exp_byte[..., j] << np.uint64(8 * (j % 4))
    invalid = int(np.count_nonzero(((bits >> np.uint32(31)) != 0) | ((bits & np.uint32(0x7FFFFF)) != 0)))
    return out.astype(np.uint32).view(np.int32), invalid
