"""Pins of the oracle's number formats (E4M3, bfloat16, UE8M0) against the
format definitions, torch's own conversions and exhaustive checks."""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import formats

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load_spec():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_spec_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, val = line.split()
            rows.append((int(code, 16), val))
    return rows


def test_e4m3_spec_values():
    for code, val in _load_spec():
        got = oracle.e4m3_decode(np.array([code], dtype=np.uint8))[0]
        if val == "nan":
            assert math.isnan(got), hex(code)
        elif val == "-0":
            assert got == 0.0 and math.copysign(1.0, got) < 0, hex(code)
        else:
            assert got == float(val), (hex(code), got, val)


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))
    # exactly two NaN codes, no infinities
    assert nan.sum() == 2 and not np.isinf(ours).any()


def test_e4m3_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_decode(codes)), codes)


def test_e4m3_midpoints_round_to_even_code():
    pos = oracle.e4m3_decode(np.arange(127, dtype=np.uint8))
    for c in range(126):
        mid = (pos[c] + pos[c + 1]) / 2.0
        even = c if c % 2 == 0 else c + 1
        for sign, sbit in ((1.0, 0), (-1.0, 0x80)):
            assert oracle.e4m3_encode(np.array([sign * mid]))[0] == (even | sbit), (c, mid)
            # one float64 ulp either side of the midpoint breaks the tie
            below = np.nextafter(mid, 0.0)
            above = np.nextafter(mid, np.inf)
            assert oracle.e4m3_encode(np.array([sign * below]))[0] == (c | sbit)
            assert oracle.e4m3_encode(np.array([sign * above]))[0] == ((c + 1) | sbit)


def test_e4m3_encode_matches_torch_random():
    rng = np.random.default_rng(7)
    # log-uniform magnitudes across the subnormal, normal and top range
    mag = np.exp2(rng.uniform(-14.0, math.log2(448.0), size=200_000)).astype(np.float32)
    sign = np.where(rng.uniform(size=mag.size) < 0.5, -1.0, 1.0).astype(np.float32)
    x = np.concatenate([mag * sign, np.float32([0.0, -0.0, 448.0, -448.0, 2.0**-10, -(2.0**-10)])])
    x = np.clip(x, -448.0, 448.0).astype(np.float32)
    ours = oracle.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_saturates_and_keeps_sign_of_zero():
    x = np.array([500.0, 1e9, -464.0, -1e30, -0.0, -1e-9, 1e-9, 2.0**-10, -(2.0**-10)], dtype=np.float64)
    got = oracle.e4m3_encode(x)
    assert list(got) == [0x7E, 0x7E, 0xFE, 0xFE, 0x80, 0x80, 0x00, 0x00, 0x80]
    # 2^-10 is exactly half the smallest subnormal: ties to the even code 0
    assert oracle.e4m3_encode(np.array([3 * 2.0**-10]))[0] == 0x02  # 1.5 * 2^-9 -> even 2 * 2^-9


def test_bf16_decode_matches_torch():
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    ours = oracle.bf16_decode(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_ue8m0_decode_closed_form():
    e = np.arange(255)
    assert np.array_equal(oracle.ue8m0_decode(e), np.array([math.ldexp(1.0, int(v) - 127) for v in e]))
    assert math.isnan(oracle.ue8m0_decode(np.array([255]))[0])
    assert oracle.ue8m0_decode(np.array([127]))[0] == 1.0


def test_bf16_round_matches_torch_on_float32():
    # torch's float32 -> bfloat16 conversion rounds to nearest even: on
    # float32 inputs the oracle's one rounding from float64 must agree
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(20000) * np.exp2(rng.integers(-30, 30, 20000))).astype(np.float32)
    # exact midpoints between neighbouring bfloat16 values (bit 15 set, bits 0..14 clear)
    mid = ((rng.integers(0x00800000, 0x7f000000, 5000, dtype=np.int64) & ~0xffff) | 0x8000).astype(np.uint32)
    x = np.concatenate([x, mid.view(np.float32), -mid.view(np.float32), np.float32([0.0, -0.0, 1.0, 3.0e38])])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = formats.bf16_round(x.astype(np.float64))
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))


def test_bf16_round_hand_picked_ties():
    u = 2.0 ** -7  # bfloat16 spacing in [1, 2)
    assert formats.bf16_round(1 + u / 2) == 1.0  # tie: to the even neighbour 1
    assert formats.bf16_round(1 + 3 * u / 2) == 1 + 2 * u  # tie: to the even neighbour 1 + 2u
    assert formats.bf16_round(-(1 + 3 * u / 2)) == -(1 + 2 * u)
    # one rounding from float64: just above a tie rounds up (rounding through
    # float32 first would land on the tie and go to the even value 1)
    assert formats.bf16_round(1 + u / 2 + 2.0 ** -40) == 1 + u
    # below 2^-126 the step is 2^-133
    assert formats.bf16_round(2.0 ** -133 * 2.5) == 2.0 ** -133 * 2
    assert formats.bf16_round(2.0 ** -133 * 3.5) == 2.0 ** -133 * 4
    assert np.isinf(formats.bf16_round(2.0 ** 128))
