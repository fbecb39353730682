"""Pins of the oracle's FP8 quantizers: invariants that hold for the
correct scale and indexing, error bounds of round-to-nearest, exact
closed-form cases, and the UE8M0 power-of-two rounding."""

import numpy as np
import pytest

import oracle
from moe_grouped_gemm_x128_amd import synth

F32_EPS = 2.0 ** -23


def _blocks_1x128(x):
    """Yield (index tuple, block values) for every 1x128 block of x [R, K]."""
    R, K = x.shape
    for r in range(R):
        for kb in range(-(-K // 128)):
            yield (r, kb), x[r, kb * 128:(kb + 1) * 128]


def _check_fp32_scaled(x, q, s):
    """Invariants of s = fp32(amax/448) and q = e4m3(fp32(x/s)) for one block."""
    amax = float(np.abs(x).max())
    dq = oracle.e4m3_decode(q)
    if amax >= 1e-4:
        # amax / fl(amax/448) is within an ulp of 448, so the maximum encodes to 448
        assert np.abs(dq).max() == 448.0
        assert abs(s * 448.0 - amax) <= amax * F32_EPS
    else:
        assert s == np.float32(np.float32(1e-4) / np.float32(448.0))
    # round-to-nearest error bound: half an e4m3 ulp relative (2^-4) for normals,
    # half the subnormal step 2^-10 (in units of s) below 2^-6, plus the fp32 division
    t = x.astype(np.float64) / float(s)
    err = np.abs(dq - t)
    bound = np.where(np.abs(t) >= 2.0 ** -6, 2.0 ** -4 * np.abs(t), 2.0 ** -10) + np.abs(t) * 2 * F32_EPS
    assert np.all(err <= bound)


def test_per_token_invariants_random():
    x = synth.normal_f32(11, (7, 640)) * np.float32(3.0)
    x[2, :128] = 0.0  # an all-zero block
    x[3, 128:256] *= np.float32(1e-3)
    q, sf = oracle.per_token_cast_to_fp8(x)
    assert q.shape == x.shape and sf.shape == (7, 5) and q.dtype == np.uint8 and sf.dtype == np.float32
    for (r, kb), blk in _blocks_1x128(x):
        _check_fp32_scaled(blk, q[r, kb * 128:(kb + 1) * 128], sf[r, kb])
    assert np.all(q[2, :128] == 0)


def test_per_token_partial_last_block():
    x = synth.normal_f32(12, (3, 300))
    q, sf = oracle.per_token_cast_to_fp8(x)
    assert sf.shape == (3, 3)
    for (r, kb), blk in _blocks_1x128(x):
        _check_fp32_scaled(blk, q[r, kb * 128:(kb + 1) * 128], sf[r, kb])


def test_per_token_exact_closed_form():
    # values that are e4m3-exact multiples of 2^k with a block maximum of
    # 448 * 2^k: the scale is exactly 2^k and the codes come back unchanged
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 0x7E, size=(4, 256)).astype(np.uint8) | (rng.integers(0, 2, size=(4, 256)).astype(np.uint8) << 7)
    codes[:, 0] = 0x7E
    codes[:, 128] = 0xFE
    ks = np.array([[-3, 2], [0, 5], [-10, -1], [7, 0]])
    x = oracle.e4m3_decode(codes).reshape(4, 2, 128) * np.exp2(ks)[:, :, None]
    x = x.reshape(4, 256).astype(np.float32)
    q, sf = oracle.per_token_cast_to_fp8(x)
    assert np.array_equal(sf, np.exp2(ks).astype(np.float32))
    # -0 codes decode to -0.0 and re-encode to 0x80, so the bytes are identical
    assert np.array_equal(q, codes)


def test_per_token_blocks_are_independent():
    # changing one block changes only that block's codes and scale
    x = synth.normal_f32(13, (2, 512))
    q0, s0 = oracle.per_token_cast_to_fp8(x)
    x2 = x.copy()
    x2[1, 256:384] *= np.float32(50.0)
    q1, s1 = oracle.per_token_cast_to_fp8(x2)
    mask = np.ones_like(s0, dtype=bool)
    mask[1, 2] = False
    assert np.array_equal(s0[mask], s1[mask]) and s0[1, 2] != s1[1, 2]
    qm = np.ones_like(q0, dtype=bool)
    qm[1, 256:384] = False
    assert np.array_equal(q0[qm], q1[qm])


@pytest.mark.parametrize("shape", [(256, 384), (200, 256), (2, 130, 260)])
def test_per_block_invariants(shape):
    x = synth.normal_f32(14, shape)
    q, sf = oracle.per_block_cast_to_fp8(x)
    N, K = shape[-2], shape[-1]
    assert sf.shape == shape[:-2] + (-(-N // 128), -(-K // 128))
    xs = x.reshape((-1, N, K))
    qs = q.reshape((-1, N, K))
    ss = sf.reshape((-1,) + sf.shape[-2:])
    for g in range(xs.shape[0]):
        for nb in range(ss.shape[1]):
            for kb in range(ss.shape[2]):
                r = slice(nb * 128, (nb + 1) * 128)
                c = slice(kb * 128, (kb + 1) * 128)
                _check_fp32_scaled(xs[g, r, c].ravel(), qs[g, r, c].ravel(), ss[g, nb, kb])


def test_per_block_transposed_scale_would_fail():
    # the 2x3 block grid is not square: a swapped (kb, nb) index cannot satisfy the invariants
    x = synth.normal_f32(15, (256, 384))
    x[:128, 128:256] *= np.float32(100.0)
    q, sf = oracle.per_block_cast_to_fp8(x)
    assert sf[0, 1] > 10 * sf[1, 0]


@pytest.mark.parametrize("per_block", [False, True])
def test_ue8m0_scales(per_block):
    x = synth.normal_f32(16, (256, 512)) * np.float32(0.37)
    f = oracle.per_block_cast_to_fp8 if per_block else oracle.per_token_cast_to_fp8
    q, sf = f(x, use_ue8m0=True)
    _, sf32 = f(x, use_ue8m0=False)
    m, e = np.frexp(sf.astype(np.float64))
    assert np.all(m == 0.5)  # powers of two
    # the smallest power of two not below the FP32 scale
    assert np.all(sf >= sf32) and np.all(sf.astype(np.float64) / 2 < sf32)
    dq = np.abs(oracle.e4m3_decode(q))
    if per_block:
        bmax = dq.reshape(2, 128, 4, 128).max(axis=(1, 3))
    else:
        bmax = dq.reshape(256, 4, 128).max(axis=2)
    assert np.all((bmax >= 224.0) & (bmax <= 448.0))
    # a power-of-two scale divides exactly: every code is the RNE of x / s
    s_full = np.repeat(np.repeat(sf, 128, axis=-1), 128, axis=0) if per_block else np.repeat(sf, 128, axis=-1)
    t = x.astype(np.float64) / s_full.astype(np.float64)
    assert np.array_equal(q, oracle.e4m3_encode(t))


def test_ue8m0_scale_of_exact_power_of_two_is_kept():
    # amax = 448 * 2^-3 gives s = 2^-3 exactly, which is already a power of two
    x = np.zeros((1, 128), dtype=np.float32)
    x[0, 5] = 448.0 / 8
    x[0, 6] = 1.0
    _, sf = oracle.per_token_cast_to_fp8(x, use_ue8m0=True)
    assert sf[0, 0] == np.float32(0.125)
    x[0, 5] = np.nextafter(np.float32(56.0), np.float32(100.0))
    _, sf = oracle.per_token_cast_to_fp8(x, use_ue8m0=True)
    assert sf[0, 0] == np.float32(0.25)


# ---------------------------------------------------------------------------
# Exact pin of the scale and quotient rule (reading of "FP32 amax/448 scales",
# "DeepInside DeepGEMM", section 4: FP32 scale factors per 128-wide K-block):
#   s = RN32(max(amax, 1e-4) / 448), q = e4m3(RN32(x / s)),
# each quotient the correctly rounded binary32 one.  The expected values come
# from integer arithmetic on the binary32 inputs (helpers.rn32_quot), never
# from numpy's float32 division, so a scale taken as amax * RN(1/448) or a
# quotient taken as x * RN(1/s) fails here.
# ---------------------------------------------------------------------------

from helpers import rn32_quot  # noqa: E402

FLOOR = float(np.float32(1e-4))


def _exact_scale(amax, ue8m0):
    import math

    s = rn32_quot(max(float(amax), FLOOR), 448.0)
    if ue8m0:
        f, e = math.frexp(s)
        s = s if f == 0.5 else math.ldexp(1.0, e)
    return s


def _exact_codes(vals, s):
    t = np.array([rn32_quot(float(v), s) for v in vals], dtype=np.float64)
    return oracle.e4m3_encode(t)


def _varied_rows(seed, rows, K, bf16):
    """N(0,1) rows whose 1x128 blocks span many binades (some below the
    amax floor, some all zero), optionally rounded to bfloat16 values."""
    rng = np.random.default_rng(seed)
    x = synth.normal_f32(seed, (rows, K))
    mag = np.exp2(rng.integers(-30, 12, size=(rows, K // 128))).astype(np.float32)
    x = (x.reshape(rows, K // 128, 128) * mag[..., None]).reshape(rows, K)
    x[0, :128] = 0.0
    x[1, 128:256] = 0.0
    x[1, 200] = -3.0  # amax 3: RN(3/448) differs from 3 * RN(1/448)
    if bf16:
        x = (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    return x


def _per_token_mismatches(x, q, sf, ue8m0, code_rows=None):
    R, K = x.shape
    bad_s = bad_q = 0
    for r in range(R):
        for kb in range(K // 128):
            blk = x[r, kb * 128:(kb + 1) * 128]
            s = _exact_scale(np.abs(blk).max(), ue8m0)
            bad_s += int(float(sf[r, kb]) != s)
            if code_rows is None or r in code_rows:
                bad_q += int(np.count_nonzero(_exact_codes(blk, s) != q[r, kb * 128:(kb + 1) * 128]))
    return bad_s, bad_q


@pytest.mark.parametrize("bf16", [False, True])
def test_per_token_scale_and_codes_exact(bf16):
    # 5120 blocks per source; every code of every block
    x = _varied_rows(21 + bf16, 40, 128 * 128, bf16)
    q, sf = oracle.per_token_cast_to_fp8(x)
    assert (np.abs(x).reshape(40, 128, 128).max(axis=-1) < FLOOR).any()  # the floor is exercised
    assert _per_token_mismatches(x, q, sf, False) == (0, 0)


@pytest.mark.parametrize("bf16", [False, True])
def test_per_token_ue8m0_scale_exact(bf16):
    x = _varied_rows(23 + bf16, 16, 128 * 64, bf16)
    q, sf = oracle.per_token_cast_to_fp8(x, use_ue8m0=True)
    assert _per_token_mismatches(x, q, sf, True, code_rows={0, 1, 2, 3}) == (0, 0)


@pytest.mark.parametrize("bf16", [False, True])
def test_per_block_scale_and_codes_exact(bf16):
    rng = np.random.default_rng(25 + bf16)
    G, N, K = 3, 384, 2048
    x = synth.normal_f32(25 + bf16, (G, N, K))
    mag = np.exp2(rng.integers(-30, 12, size=(G, N // 128, K // 128))).astype(np.float32)
    x = (x.reshape(G, N // 128, 128, K // 128, 128) * mag[:, :, None, :, None]).reshape(G, N, K)
    x[1, :128, :128] = 0.0
    if bf16:
        x = (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    q, sf = oracle.per_block_cast_to_fp8(x)
    for g in range(G):
        for nb in range(N // 128):
            for kb in range(K // 128):
                blk = x[g, nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128].ravel()
                qb = q[g, nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128].ravel()
                s = _exact_scale(np.abs(blk).max(), False)
                assert float(sf[g, nb, kb]) == s, (g, nb, kb)
                idx = np.unique(np.concatenate([rng.choice(blk.size, 1024, replace=False),
                                                [int(np.argmax(np.abs(blk)))]]))
                assert np.array_equal(_exact_codes(blk[idx], s), qb[idx]), (g, nb, kb)


def test_scale_of_amax_3_is_the_correctly_rounded_quotient():
    # 3/448 = (0.011011...)_2 * 2^-6 = 1.1011011..._2 * 2^-8; the 23 fraction
    # bits 10110110110110110110110 are followed by 1101..., so the correctly
    # rounded binary32 is fraction 0x5B6DB7 with biased exponent 119:
    # 0x3BDB6DB7.  3 * RN(1/448) rounds to 0x3BDB6DB8 instead.
    x = np.zeros((1, 128), dtype=np.float32)
    x[0, 7] = 3.0
    x[0, 8] = -1.0
    _, sf = oracle.per_token_cast_to_fp8(x)
    assert int(sf.view(np.uint32)[0, 0]) == 0x3BDB6DB7
    assert rn32_quot(3.0, 448.0) == float(np.array([0x3BDB6DB7], dtype=np.uint32).view(np.float32)[0])
    recip = np.float32(np.float32(3.0) * (np.float32(1.0) / np.float32(448.0)))
    assert int(recip.view(np.uint32)) == 0x3BDB6DB8


def test_exact_pin_rejects_a_reciprocal_multiply_scale(monkeypatch):
    # a planted mistake in the oracle: s = amax * RN(1/448)
    import oracle.quant as oq

    def wrong_scale(amax, use_ue8m0):
        amax = np.maximum(np.asarray(amax, dtype=np.float32), oq.AMAX_FLOOR)
        return (amax * (np.float32(1.0) / np.float32(448.0))).astype(np.float32)

    monkeypatch.setattr(oq, "_scale_from_amax", wrong_scale)
    x = _varied_rows(27, 8, 128 * 32, False)
    q, sf = oracle.per_token_cast_to_fp8(x)
    bad_s, _ = _per_token_mismatches(x, q, sf, False, code_rows=set())
    assert bad_s > 0


def test_exact_pin_rejects_a_reciprocal_multiply_quotient():
    # a planted mistake, q = e4m3(RN(x * RN(1/s))): a one-ulp quotient error
    # flips a code only next to a midpoint between E4M3 values, so the block
    # holds values placed there (x = RN(m s) + j ulp for midpoints m)
    rng = np.random.default_rng(28)
    pos = oracle.e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    x = np.zeros((64, 128), dtype=np.float32)
    for r in range(64):
        amax = np.float32(abs(rng.standard_normal()) * 3.0 + 0.1)
        s = np.float32(amax / np.float32(448.0))
        x[r, 0] = amax
        m = mids[rng.integers(mids.size, size=127)].astype(np.float32)
        v = (m * s).astype(np.float32)
        j = rng.integers(-3, 4, size=127)
        x[r, 1:] = (v.view(np.int32) + j.astype(np.int32)).view(np.float32)
    q, sf = oracle.per_token_cast_to_fp8(x)
    assert _per_token_mismatches(x, q, sf, False) == (0, 0)
    s_full = np.repeat(sf, 128, axis=-1)
    q_bad = oracle.e4m3_encode((x * (np.float32(1.0) / s_full).astype(np.float32)).astype(np.float32))
    assert not np.array_equal(q_bad, q)
    _, bad_q = _per_token_mismatches(x, q_bad, sf, False)
    assert bad_q > 0
