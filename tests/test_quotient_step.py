"""The quantizers' division step, emulated exactly on the host.

The GPU casts compute x / s as y = RN(x r), e = x - y s (exact with an FMA),
q = RN(y + r e) with r = RN(1 / s) computed once per block.  These tests
check, with exact rational arithmetic, that q is the correctly rounded
binary32 quotient RN(x / s) that the oracle's division gives, for random
operands of the quantizers' range and for quotients placed at and next to
the midpoints between adjacent E4M3 values (where a one-ulp error would flip
the FP8 byte).  Host logic only: nothing here touches the GPU path."""

from fractions import Fraction as F

import numpy as np

import oracle
from helpers import rn32


def step(x, s):
    r = rn32(1 / s)
    y = rn32(x * r)
    e = x - y * s  # exact: the FMA residual of a faithful quotient is representable
    return rn32(y + r * e)


def _cases(seed, n):
    rng = np.random.default_rng(seed)
    pos = oracle.e4m3_decode(np.arange(127, dtype=np.uint8)).astype(np.float64)
    mids = (pos[:-1] + pos[1:]) / 2
    for i in range(n):
        amax = F(float(np.float32(abs(rng.standard_normal()) * 10.0 ** int(rng.integers(-4, 4)) + 1e-4)))
        s = rn32(amax / 448)
        if i % 2 == 0:
            x = F(float(np.float32(rng.standard_normal() * float(amax))))
        else:
            m = F(float(mids[rng.integers(mids.size)])) * (1 if rng.random() < 0.5 else -1)
            x = rn32(rn32(m * s) + int(rng.integers(-2, 3)) * F(2) ** -149)
        yield x, s


def test_correction_step_is_the_correctly_rounded_quotient():
    n = 0
    for x, s in _cases(7, 3000):
        ref = rn32(x / s)
        if x == 0 or abs(ref) < F(2) ** -126:
            continue
        assert step(x, s) == ref, (float(x), float(s))
        n += 1
    assert n > 2500


def test_power_of_two_scales_are_exact():
    # UE8M0 scales: r is exact, so y is the exact quotient and the correction adds zero
    rng = np.random.default_rng(8)
    for _ in range(500):
        s = F(2) ** int(rng.integers(-20, 20))
        x = F(float(np.float32(rng.standard_normal() * 100)))
        assert step(x, s) == rn32(x / s)
