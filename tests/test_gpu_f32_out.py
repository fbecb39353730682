"""GPU parity of the dense GEMMs with an FP32 output D (fp8_gemm_nt and
bf16_gemm_nt with an F32 d): the FP32 accumulator, C added, stored without
rounding ("DeepInside DeepGEMM", section 4: the call takes the output dtype).

Tolerance: every output is a sum of K exact products (E4M3 or BF16
significands) times scales, plus C; S is the sum of the absolute values of
all those terms (C included), the oracle's own GEMM over the absolute
values of codes and scales, exact in float64; u = 2^-24.
  BF16: a sum formed by FP32 additions that round to nearest, in any order
  and grouping, is within (K + 2) u S of the exact sum (first order in u).
  FP8: the FP32 steps outside the matrix core (scale products, the promote
  FMA per K-block, the C addition) contribute at most (KB + 2) u S for KB
  blocks, but the matrix core's own sum of a 128-term block is not an IEEE
  FP32 sum -- its limited precision is why the partial is promoted per
  block ("DeepGEMM tested by Novita AI", "Technological Innovations") -- so
  each block sum may also be off by a fraction E of the block's absolute
  sum: E = 2^-15 (the largest deviation measured on gfx950 is 2^-16.3 of S;
  a BF16 rounding of D would be about 2^-9 of |D| and fails).  Bound:
  (E + (KB + 2) u) S.  The test also checks, bit for
bit, that the F32 output rounded to BF16 (torch's round-to-nearest-even
conversion) equals the BF16-output GEMM: both store the same accumulator."""

import numpy as np
import pytest

import oracle
from moe_grouped_gemm_x128_amd import synth

from helpers import say, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

U = 2.0 ** -24
E_BLOCK = 2.0 ** -15  # block-sum error of the matrix core, relative to the block's absolute sum


def _mg():
    import moe_grouped_gemm_x128_amd as mg

    return mg


def _dev_bf16(bits):
    return to_dev(bits.view(np.int16)).view(torch.bfloat16)


def q_tok(xt, ue8m0=False):
    mg = _mg()
    K = xt.shape[-1]
    q = torch.empty(xt.shape, dtype=torch.uint8, device="cuda")
    sf = torch.empty((K // 128, xt.shape[0]), dtype=torch.float32, device="cuda").t()
    mg.per_token_cast_to_fp8(xt, q, sf, ue8m0)
    return q, sf


def q_blk(xt, ue8m0=False):
    mg = _mg()
    N, K = xt.shape
    q = torch.empty(xt.shape, dtype=torch.uint8, device="cuda")
    sf = torch.empty((-(-N // 128), K // 128), dtype=torch.float32, device="cuda")
    mg.per_block_cast_to_fp8(xt, q, sf, ue8m0)
    return q, sf


def nan_f32(M, N, pad=0):
    buf = torch.full((M, N + pad), float("nan"), dtype=torch.float32, device="cuda")
    return buf, buf[:, :N]


def assert_f32_close(got, ref, S, nround, what, e_block=E_BLOCK):
    """got float32 from the device, ref float64 exact, S the sum of absolute
    terms (C included); bound (e_block + (nround + 2) u) S."""
    assert got.shape == ref.shape, what
    assert np.all(np.isfinite(got)), f"{what}: non-finite (unwritten) output"
    bound = (e_block + (nround + 2) * U) * S * (1 + 1e-6) + np.finfo(np.float32).tiny
    err = np.abs(got.astype(np.float64) - ref)
    say(f"  {what}: largest error / S = 2^{np.log2(max(float((err / np.maximum(S, 1e-300)).max()), 2.0 ** -60)):.1f}")
    bad = err > bound
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} outside the bound; first {i}: got {got[i]!r} ref {ref[i]!r} "
                             f"bound {bound[i]:.3g}")


def _abs_fp8(codes):
    return np.asarray(codes, dtype=np.uint8) & np.uint8(0x7F)


# dense FP8 plans: 128-row tiles (N <= 128 and above), the 256 x 192 tile
# (one launch below a round of tiles) and a whole round of 256 x 256 tiles
FP8_SHAPES = [(128, 256, 512), (64, 100, 256), (1, 130, 128), (200, 300, 384), (257, 64, 256), (64, 2112, 1024),
              (4000, 4000, 256)]


@pytest.mark.parametrize("M,N,K", FP8_SHAPES)
def test_fp8_dense_f32_out(M, N, K):
    say(f"fp8_gemm_nt F32 d M={M} N={N} K={K}")
    mg = _mg()
    xa = synth.normal_f32(701, (M, K))
    xb = synth.normal_f32(702, (N, K))
    a, sfa = q_tok(to_dev(xa))
    b, sfb = q_blk(to_dev(xb))
    buf, d = nan_f32(M, N, pad=3)
    mg.fp8_gemm_nt(a, b, sfa, sfb, None, d)
    d16 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    mg.fp8_gemm_nt(a, b, sfa, sfb, None, d16)
    torch.cuda.synchronize()
    # the same accumulator: F32 rounded to BF16 equals the BF16 output
    assert torch.equal(d.to(torch.bfloat16).view(torch.int16), d16.view(torch.int16))
    assert torch.isnan(buf[:, N:]).all(), "row padding written"
    ra, rsfa = oracle.per_token_cast_to_fp8(xa)
    rb, rsfb = oracle.per_block_cast_to_fp8(xb)
    assert np.array_equal(to_host(a), ra) and np.array_equal(to_host(b), rb)
    ref = oracle.fp8_gemm_nt(ra, rb, rsfa, rsfb)
    S = oracle.fp8_gemm_nt(_abs_fp8(ra), _abs_fp8(rb), np.abs(rsfa), np.abs(rsfb))
    assert_f32_close(to_host(d), ref, S, K // 128, f"fp8 F32 d {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(192, 384, 1024), (4000, 4000, 512)])
def test_fp8_dense_f32_out_packed_ue8m0(M, N, K):
    say(f"fp8_gemm_nt F32 d, packed UE8M0 scales M={M} N={N} K={K}")
    mg = _mg()
    xa = synth.normal_f32(711, (M, K))
    xb = synth.normal_f32(712, (N, K))
    a, sfa = q_tok(to_dev(xa), True)
    b, sfb = q_blk(to_dev(xb), True)
    pa = torch.empty((M, K // 512), dtype=torch.int32, device="cuda")
    pb = torch.empty((-(-N // 128), K // 512), dtype=torch.int32, device="cuda")
    mg.pack_ue8m0_to_int(sfa.contiguous(), pa)
    mg.pack_ue8m0_to_int(sfb, pb)
    _, d = nan_f32(M, N)
    mg.fp8_gemm_nt(a, b, pa, pb, None, d)
    d16 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    mg.fp8_gemm_nt(a, b, pa, pb, None, d16)
    torch.cuda.synchronize()
    assert torch.equal(d.to(torch.bfloat16).view(torch.int16), d16.view(torch.int16))
    ra, rsfa = oracle.per_token_cast_to_fp8(xa, True)
    rb, rsfb = oracle.per_block_cast_to_fp8(xb, True)
    ref = oracle.fp8_gemm_nt(ra, rb, rsfa, rsfb)
    S = oracle.fp8_gemm_nt(_abs_fp8(ra), _abs_fp8(rb), rsfa, rsfb)
    assert_f32_close(to_host(d), ref, S, K // 128, f"fp8 F32 d UE8M0 {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(200, 300, 384), (64, 2112, 512), (4000, 4000, 256)])
def test_fp8_dense_f32_accumulate_in_place(M, N, K):
    """d = C first, then d += A . B^T twice with c = d (the in-place
    accumulation of an FP32 output): d = C + 2 A . B^T."""
    say(f"fp8_gemm_nt F32 in-place accumulate M={M} N={N} K={K}")
    mg = _mg()
    xa = synth.normal_f32(721, (M, K))
    xb = synth.normal_f32(722, (N, K))
    xc = synth.normal_f32(723, (M, N)) * np.float32(8.0)
    a, sfa = q_tok(to_dev(xa))
    b, sfb = q_blk(to_dev(xb))
    d = to_dev(xc)
    mg.fp8_gemm_nt(a, b, sfa, sfb, d, d)
    torch.cuda.synchronize()
    d1 = to_host(d).copy()
    mg.fp8_gemm_nt(a, b, sfa, sfb, d, d)
    torch.cuda.synchronize()
    ra, rsfa = oracle.per_token_cast_to_fp8(xa)
    rb, rsfb = oracle.per_block_cast_to_fp8(xb)
    P = oracle.fp8_gemm_nt(ra, rb, rsfa, rsfb)
    S = oracle.fp8_gemm_nt(_abs_fp8(ra), _abs_fp8(rb), np.abs(rsfa), np.abs(rsfb))
    c = xc.astype(np.float64)
    assert_f32_close(d1, c + P, S + np.abs(c), K // 128, f"fp8 F32 d = C + AB^T {M}x{N}x{K}")
    # second call: its C is the first result as stored (float32)
    assert_f32_close(to_host(d), d1.astype(np.float64) + P, S + np.abs(d1), K // 128, f"fp8 F32 d += AB^T {M}x{N}x{K}")


def test_fp8_dense_f32_out_bf16_c():
    M, N, K = 300, 520, 512
    say(f"fp8_gemm_nt F32 d with BF16 c M={M} N={N} K={K}")
    mg = _mg()
    xa = synth.normal_f32(731, (M, K))
    xb = synth.normal_f32(732, (N, K))
    cbits = synth.bf16_bits_from_f32(synth.normal_f32(733, (M, N)) * np.float32(8.0))
    a, sfa = q_tok(to_dev(xa))
    b, sfb = q_blk(to_dev(xb))
    _, d = nan_f32(M, N)
    mg.fp8_gemm_nt(a, b, sfa, sfb, _dev_bf16(cbits), d)
    torch.cuda.synchronize()
    ra, rsfa = oracle.per_token_cast_to_fp8(xa)
    rb, rsfb = oracle.per_block_cast_to_fp8(xb)
    c = oracle.bf16_decode(cbits)
    S = oracle.fp8_gemm_nt(_abs_fp8(ra), _abs_fp8(rb), np.abs(rsfa), np.abs(rsfb)) + np.abs(c)
    assert_f32_close(to_host(d), oracle.fp8_gemm_nt(ra, rb, rsfa, rsfb, c), S, K // 128, "fp8 F32 d, BF16 c")


# dense BF16 plans: 128-row tiles, the 256 x 192 tile, a round of 256 x 256
# tiles, and the two-launch split (256 x 256 on [0, 4096), 256 x 192 after)
@pytest.mark.parametrize("M,N,K", [(128, 256, 512), (1, 130, 64), (200, 300, 384), (64, 2112, 1024),
                                   (4000, 4000, 128), (4000, 7100, 4096)])
def test_bf16_dense_f32_out(M, N, K):
    say(f"bf16_gemm_nt F32 d M={M} N={N} K={K}")
    mg = _mg()
    ab = synth.bf16_bits_from_f32(synth.normal_f32(741, (M, K)))
    bb = synth.bf16_bits_from_f32(synth.normal_f32(742, (N, K)))
    a, b = _dev_bf16(ab), _dev_bf16(bb)
    _, d = nan_f32(M, N)
    mg.bf16_gemm_nt(a, b, None, d)
    d16 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    mg.bf16_gemm_nt(a, b, None, d16)
    torch.cuda.synchronize()
    assert torch.equal(d.to(torch.bfloat16).view(torch.int16), d16.view(torch.int16))
    dh = to_host(d)
    rows = slice(None)
    if M * N * K > 1e10:  # the oracle on sampled rows (every column)
        rows = np.unique(np.concatenate([np.random.default_rng(743).choice(M, 24, replace=False), [0, M - 1]]))
    ref = oracle.bf16_gemm_nt(ab[rows], bb)
    S = oracle.bf16_gemm_nt(ab[rows] & np.uint16(0x7FFF), bb & np.uint16(0x7FFF))
    assert_f32_close(dh[rows], ref, S, K, f"bf16 F32 d {M}x{N}x{K}", e_block=0.0)


def test_bf16_dense_f32_accumulate_in_place():
    M, N, K = 260, 700, 512
    say(f"bf16_gemm_nt F32 in-place accumulate M={M} N={N} K={K}")
    mg = _mg()
    ab = synth.bf16_bits_from_f32(synth.normal_f32(751, (M, K)))
    bb = synth.bf16_bits_from_f32(synth.normal_f32(752, (N, K)))
    xc = synth.normal_f32(753, (M, N)) * np.float32(8.0)
    d = to_dev(xc)
    mg.bf16_gemm_nt(_dev_bf16(ab), _dev_bf16(bb), d, d)
    torch.cuda.synchronize()
    c = xc.astype(np.float64)
    S = oracle.bf16_gemm_nt(ab & np.uint16(0x7FFF), bb & np.uint16(0x7FFF)) + np.abs(c)
    assert_f32_close(to_host(d), oracle.bf16_gemm_nt(ab, bb, c), S, K, "bf16 F32 d = C + AB^T", e_block=0.0)
