"""Shared helpers of the parity tests: device transfers, the BF16 output
comparison at the stated tolerance, and sentinel handling."""

import sys

import numpy as np

import oracle

# Tolerance of a BF16 GEMM output against the float64 oracle:
#   normalised difference 1 - 2 sum(xy) / (sum(x^2) + sum(y^2)) <= 1e-3, and
#   per element |x - y| <= 1e-2 * rms(y) + 2^-8 * |y|
# (2^-8 is the bf16 rounding bound; 1e-2 rms covers FP32 accumulation).
DIFF_TOL = 1e-3
ABS_RMS_TOL = 1e-2
REL_TOL = 2.0 ** -8

SENTINEL_BF16 = 0x7FA5  # a NaN pattern: any write over it is visible


def say(msg):
    """Print a progress line naming the case before a GPU step."""
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(arr, dtype=None):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(arr))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def to_host(t):
    import torch

    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_bits_to_f64(bits):
    return oracle.bf16_decode(bits)


def norm_diff(x, y):
    x = np.asarray(x, dtype=np.float64).ravel()
    y = np.asarray(y, dtype=np.float64).ravel()
    den = float((x * x).sum() + (y * y).sum())
    if den == 0.0:
        return 0.0
    return 1.0 - 2.0 * float((x * y).sum()) / den


def assert_bf16_close(got_bits, ref, what=""):
    """got_bits: uint16 bf16 patterns; ref: float64 oracle values (same shape)."""
    got = bf16_bits_to_f64(got_bits)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    d = norm_diff(got, ref)
    assert d <= DIFF_TOL, f"{what}: normalised diff {d:.3e} > {DIFF_TOL}"
    if ref.size == 0:
        return
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = np.abs(got - ref)
    bound = ABS_RMS_TOL * rms + REL_TOL * np.abs(ref)
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[:5]
        details = ", ".join(f"{tuple(i)}: got {got[tuple(i)]:.6g} ref {ref[tuple(i)]:.6g}" for i in idx)
        raise AssertionError(f"{what}: {int(bad.sum())} elements outside tolerance (rms {rms:.4g}); {details}")


# ---------------------------------------------------------------------------
# Exact binary32 rounding (host-side pins; no numpy float32 arithmetic)
# ---------------------------------------------------------------------------

def rn32(v):
    """Round a rational (fractions.Fraction) to the nearest binary32 value,
    ties to even, with binary32's subnormal range; returns a Fraction."""
    from fractions import Fraction as F

    if v == 0:
        return F(0)
    sgn = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if F(2) ** e > a:
        e -= 1
    while F(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    unit = F(2) ** (e - 23)
    m = a / unit
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > F(1, 2) or (rem == F(1, 2) and fl % 2 == 1):
        fl += 1
    return sgn * fl * unit


def _mant_exp(v):
    """|v| = m * 2^e with m a non-negative integer (v a finite Python float)."""
    import math

    f, e = math.frexp(abs(v))
    return int(f * (1 << 53)), e - 53


def rn32_quot(x, y):
    """The correctly rounded binary32 quotient RN(x / y) of two finite
    binary32 values (y != 0), ties to even, computed with integer arithmetic
    only; returned as a Python float (which holds every binary32 exactly).
    The sign of a zero result is the sign of the exact quotient."""
    import math

    neg = (math.copysign(1.0, x) < 0) != (y < 0)
    if x == 0:
        return -0.0 if neg else 0.0
    mx, ex = _mant_exp(x)
    my, ey = _mant_exp(y)
    P = 64
    q, r = divmod(mx << P, my)  # |x / y| = (q + r / my) * 2^(ex - ey - P), q >= 2^63
    base = ex - ey - P
    e_top = q.bit_length() - 1 + base  # floor(log2 |x / y|)
    e_eff = max(e_top, -126)
    drop = (e_eff - 23) - base  # bits of q below the binary32 unit in the last place (> 0)
    kept = q >> drop
    rem = q - (kept << drop)
    half = 1 << (drop - 1)
    if rem > half or (rem == half and (r != 0 or kept & 1)):
        kept += 1
    val = math.ldexp(kept, e_eff - 23)
    return -val if neg else val
