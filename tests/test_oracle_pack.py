"""Pins of the oracle's UE8M0 packing: hand-derived examples of the page's
expression, an exhaustive closed form over every exponent byte, and the
validity count."""

import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load():
    rows = []
    with open(os.path.join(GOLDEN, "ue8m0_pack_examples.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lhs, packed, invalid = [p.strip() for p in line.split("|")]
            bits = np.array([int(t, 16) for t in lhs.split()], dtype=np.uint32)
            rows.append((bits.view(np.float32), int(packed), int(invalid)))
    return rows


def test_pack_golden_examples():
    for x, packed, invalid in _load():
        out, bad = oracle.pack_ue8m0_to_int(x[None, :])
        assert out.shape == (1, 1) and out.dtype == np.int32
        assert int(out[0, 0]) == packed
        assert bad == invalid


def test_pack_exhaustive_exponents_closed_form():
    # 2^(e-127) has exponent field e (e = 0 is the subnormal/zero band: use 2^-127 and 0.0)
    e = np.arange(256)
    with np.errstate(over="ignore"):
        vals = np.ldexp(1.0, e - 127).astype(np.float32)
    vals[0] = np.float32(0.0)
    vals[255] = np.float32(np.inf)  # exponent field 255
    for lane in range(4):
        x = np.full((256, 4), np.float32(1.0))
        x[:, lane] = vals
        out, bad = oracle.pack_ue8m0_to_int(x)
        want = np.full(256, 0x7F7F7F7F, dtype=np.int64)
        want = (want & ~(0xFF << (8 * lane))) | (e.astype(np.int64) << (8 * lane))
        want = np.where(want >= 2**31, want - 2**32, want)
        assert np.array_equal(out[:, 0].astype(np.int64), want)
        # only the subnormal-band zero (exponent 0, mantissa 0) is still "valid"; inf is valid too
        assert bad == 0


def test_pack_tail_and_shape():
    x = np.ldexp(1.0, np.arange(10).reshape(2, 5) - 3).astype(np.float32)
    out, _ = oracle.pack_ue8m0_to_int(x)
    assert out.shape == (2, 2)
    w = out.view(np.uint32)
    # element 4 of each row sits alone in the low byte of word 1
    assert w[0, 1] == 127 + 4 - 3 and w[1, 1] == 127 + 9 - 3


def test_pack_roundtrip_with_unpack():
    rng = np.random.default_rng(3)
    e = rng.integers(1, 255, size=(3, 5, 16))
    x = np.ldexp(1.0, e - 127).astype(np.float32)
    out, bad = oracle.pack_ue8m0_to_int(x)
    assert bad == 0 and out.shape == (3, 5, 4)
    assert np.array_equal(oracle.scales_from_packed_ue8m0(out, 16), x.astype(np.float64))
