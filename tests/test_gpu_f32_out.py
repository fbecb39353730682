"""GPU parity of the dense GEMMs with an FP32 output D (fp8_gemm_nt and
bf16_gemm_nt with an F32 d): the FP32 accumulator, C added, stored without
rounding ("DeepInside DeepGEMM", section 4: the call takes the output dtype).

Tolerance (tests/helpers.py states the derivation): every output is a sum
of K exact products (E4M3 or BF16 significands) times scales, plus C; S is
the sum of the absolute values of all those terms (C included), the
oracle's own GEMM over the absolute values of codes and scales, exact in
float64; u = 2^-24.
  BF16: a sum formed by FP32 additions that round to nearest, in any order
  and grouping, is within (K + 2) u S of the exact sum (first order in u).
  FP8: the matrix core truncates each product inside groups of 8 K values
  to 14 bits below the group's largest exponent, so each group may be off
  by 7 * 2^-13 of the product of its operands' largest magnitudes -- its
  limited precision is why the partial is promoted per block ("DeepGEMM
  tested by Novita AI", "Technological Innovations"); with the FP32
  roundings, the bound is 7 * 2^-13 G + (18 KB + 2) u S, G the oracle's
  GEMM of the per-group maxima.  Most outputs must carry bits below BF16
  precision (an F32 output rounded to BF16 fails).
The test also checks, bit for bit, that the F32 output rounded to BF16
(torch's round-to-nearest-even conversion) equals the BF16-output GEMM:
both store the same accumulator."""

import numpy as np
import pytest

import oracle
from moe_grouped_gemm_x128_amd import synth

from helpers import assert_f32_close, fp8_bound_terms, fp8_rounding_count, say, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


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


# dense FP8 plans: 128-row tiles (N <= 128 and above), 192 x 192 tiles (one
# round of them), one round of 256 x 192 tiles (4096 x 2880) and a whole
# round of 256 x 256 tiles (4000 x 4000); _expect_tiles checks each
FP8_SHAPES = [(128, 256, 512), (64, 100, 256), (1, 130, 128), (200, 300, 384), (257, 64, 256), (64, 2112, 1024),
              (4096, 2880, 256), (4000, 4000, 256)]


def _expect_tiles(M, N, K):
    from moe_grouped_gemm_x128_amd import binding

    c = binding.query_config(binding.DG_KIND_DENSE, 1, M, N, K)
    want = {(4096, 2880): (256, 192), (4000, 4000): (256, 256)}.get((M, N), (192, 192) if M > 128 else None)
    if want is not None:
        assert (c["block_m"], c["block_n"], c["block_n2"]) == want + (0,), c


@pytest.mark.parametrize("M,N,K", FP8_SHAPES)
def test_fp8_dense_f32_out(M, N, K):
    say(f"fp8_gemm_nt F32 d M={M} N={N} K={K}")
    mg = _mg()
    _expect_tiles(M, N, K)
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
    S, Gt = fp8_bound_terms(oracle.fp8_gemm_nt, ra, rb, rsfa, rsfb)
    assert_f32_close(to_host(d), ref, S, fp8_rounding_count(K), f"fp8 F32 d {M}x{N}x{K}", G=Gt)


@pytest.mark.parametrize("M,N,K", [(192, 384, 1024), (4096, 2880, 512), (4000, 4000, 512)])
def test_fp8_dense_f32_out_packed_ue8m0(M, N, K):
    say(f"fp8_gemm_nt F32 d, packed UE8M0 scales M={M} N={N} K={K}")
    mg = _mg()
    _expect_tiles(M, N, K)
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
    S, Gt = fp8_bound_terms(oracle.fp8_gemm_nt, ra, rb, rsfa, rsfb)
    assert_f32_close(to_host(d), ref, S, fp8_rounding_count(K), f"fp8 F32 d UE8M0 {M}x{N}x{K}", G=Gt)


@pytest.mark.parametrize("M,N,K", [(200, 300, 384), (64, 2112, 512), (4096, 2880, 256), (4000, 4000, 256)])
def test_fp8_dense_f32_accumulate_in_place(M, N, K):
    """d = C first, then d += A . B^T twice with c = d (the in-place
    accumulation of an FP32 output): d = C + 2 A . B^T."""
    say(f"fp8_gemm_nt F32 in-place accumulate M={M} N={N} K={K}")
    mg = _mg()
    _expect_tiles(M, N, K)
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
    S, Gt = fp8_bound_terms(oracle.fp8_gemm_nt, ra, rb, rsfa, rsfb)
    c = xc.astype(np.float64)
    nr = fp8_rounding_count(K)
    assert_f32_close(d1, c + P, S + np.abs(c), nr, f"fp8 F32 d = C + AB^T {M}x{N}x{K}", G=Gt)
    # second call: its C is the first result as stored (float32)
    assert_f32_close(to_host(d), d1.astype(np.float64) + P, S + np.abs(d1), nr, f"fp8 F32 d += AB^T {M}x{N}x{K}", G=Gt)


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
    S, Gt = fp8_bound_terms(oracle.fp8_gemm_nt, ra, rb, rsfa, rsfb)
    assert_f32_close(to_host(d), oracle.fp8_gemm_nt(ra, rb, rsfa, rsfb, c), S + np.abs(c), fp8_rounding_count(K),
                     "fp8 F32 d, BF16 c", G=Gt)


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
    assert_f32_close(dh[rows], ref, S, K, f"bf16 F32 d {M}x{N}x{K}")


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
    assert_f32_close(to_host(d), oracle.bf16_gemm_nt(ab, bb, c), S, K, "bf16 F32 d = C + AB^T")


# ---------------------------------------------------------------------------
# grouped forms: F32 d, and the accumulate form D = C + A . B^T
# ---------------------------------------------------------------------------

def _grouped_inputs(seed, Mrows, G, N, K, per_group_a=False, ue8m0=False):
    """Codes and scales for the grouped GEMMs: A [Mrows, K] (or [G, rows, K]),
    B [G, N, K]; the oracle's and the device's quantization must agree."""
    mg = _mg()
    xa = synth.normal_f32(seed, (Mrows, K))
    xb = synth.normal_f32(seed + 1, (G, N, K))
    a = torch.empty((Mrows, K), dtype=torch.uint8, device="cuda")
    sfa = torch.empty((Mrows, K // 128), dtype=torch.float32, device="cuda")
    mg.per_token_cast_to_fp8(to_dev(xa), a, sfa, ue8m0)
    b = torch.empty((G, N, K), dtype=torch.uint8, device="cuda")
    sfb = torch.empty((G, -(-N // 128), K // 128), dtype=torch.float32, device="cuda")
    mg.per_block_cast_to_fp8(to_dev(xb), b, sfb, ue8m0)
    ra, rsfa = oracle.per_token_cast_to_fp8(xa, ue8m0)
    rb, rsfb = oracle.per_block_cast_to_fp8(xb, ue8m0)
    assert np.array_equal(to_host(a), ra) and np.array_equal(to_host(b), rb)
    return a, sfa, b, sfb, ra, rsfa, rb, rsfb


@pytest.mark.parametrize("c_kind", [None, "bf16", "f32", "inplace"])
@pytest.mark.parametrize("d_kind", ["bf16", "f32"])
def test_contiguous_f32_out_and_accumulate(c_kind, d_kind):
    """Contiguous grouped GEMM with an F32 d and/or C: mixed groups inside
    256-row tiles and skipped blocks, whose rows stay untouched."""
    say(f"contiguous d={d_kind} c={c_kind}")
    mg = _mg()
    from helpers import SENTINEL_BF16, assert_bf16_close

    G, N, K = 3, 300, 384
    layout = np.array([2, 2, -1, 0, 1, 0, 2, 7], dtype=np.int32)  # 7 >= G: skipped
    Msum = layout.size * 128
    a, sfa, b, sfb, ra, rsfa, rb, rsfb = _grouped_inputs(901, Msum, G, N, K)
    xc = synth.normal_f32(903, (Msum, N)) * np.float32(4.0)
    cref = None
    c = None
    if d_kind == "f32":
        dbuf, d = nan_f32(Msum, N, pad=4)
    else:
        d = torch.full((Msum, N), SENTINEL_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    if c_kind == "bf16":
        cbits = synth.bf16_bits_from_f32(xc)
        c, cref = _dev_bf16(cbits), oracle.bf16_decode(cbits)
    elif c_kind == "f32":
        c, cref = to_dev(xc), xc.astype(np.float64)
    elif c_kind == "inplace":
        if d_kind == "f32":
            d.copy_(to_dev(xc))
            cref = xc.astype(np.float64)
        else:
            cbits = synth.bf16_bits_from_f32(xc)
            d.copy_(_dev_bf16(cbits))
            cref = oracle.bf16_decode(cbits)
        c = d
    mg.m_grouped_fp8_gemm_nt_contiguous(a, b, sfa, sfb, d, to_dev(layout), c=c)
    torch.cuda.synchronize()
    ref_layout = np.where(layout < G, layout, -1)
    ref, written = oracle.m_grouped_fp8_gemm_nt_contiguous(ra, rb, rsfa, rsfb, ref_layout)
    if cref is not None:
        ref = ref + cref
    got = to_host(d)
    if d_kind == "f32":
        if c_kind == "inplace":
            assert np.array_equal(got[~written], xc[~written]), "skipped rows changed"
        else:
            assert np.isnan(got[~written]).all(), "skipped rows written"
        S, Gt = fp8_bound_terms(oracle.m_grouped_fp8_gemm_nt_contiguous, ra, rb, rsfa, rsfb, ref_layout)
        if cref is not None:
            S = S + np.abs(cref)
        assert_f32_close(got[written], ref[written], S[written], fp8_rounding_count(K), f"contiguous F32 d c={c_kind}",
                         G=Gt[written])
        assert torch.isnan(dbuf[:, N:]).all(), "row padding written"
        if c_kind is None:
            d16 = torch.empty((Msum, N), dtype=torch.bfloat16, device="cuda")
            mg.m_grouped_fp8_gemm_nt_contiguous(a, b, sfa, sfb, d16, to_dev(layout))
            torch.cuda.synchronize()
            rows = torch.from_numpy(written).cuda()
            assert torch.equal(d[rows].to(torch.bfloat16).view(torch.int16), d16[rows].view(torch.int16))
    else:
        if c_kind == "inplace":
            assert np.array_equal(got[~written], synth.bf16_bits_from_f32(xc)[~written]), "skipped rows changed"
        else:
            assert np.all(got[~written] == SENTINEL_BF16), "skipped rows written"
        assert_bf16_close(got[written], ref[written], f"contiguous BF16 d c={c_kind}")


@pytest.mark.parametrize("G,max_m,N,K,mm", [(3, 300, 272, 256, [300, 0, 150]), (4, 96, 200, 384, [96, 17, 0, 64])])
@pytest.mark.parametrize("c_kind", [None, "bf16", "f32", "inplace"])
@pytest.mark.parametrize("d_kind", ["bf16", "f32"])
@pytest.mark.parametrize("ue8m0", [False, True])
def test_masked_f32_out_and_accumulate(G, max_m, N, K, mm, c_kind, d_kind, ue8m0):
    """Masked grouped GEMM with an F32 d and/or C (per group, 3-D); rows past
    masked_m are neither read from c nor written."""
    say(f"masked G={G} max_m={max_m} N={N} K={K} d={d_kind} c={c_kind} ue8m0={ue8m0}")
    mg = _mg()
    from helpers import SENTINEL_BF16, assert_bf16_close

    a, sfa, b, sfb, ra, rsfa, rb, rsfb = _grouped_inputs(911, G * max_m, G, N, K, ue8m0=ue8m0)
    if ue8m0:
        pa = torch.empty((G * max_m, -(-(K // 128) // 4)), dtype=torch.int32, device="cuda")
        pb = torch.empty((G, -(-N // 128), -(-(K // 128) // 4)), dtype=torch.int32, device="cuda")
        mg.pack_ue8m0_to_int(sfa, pa)
        mg.pack_ue8m0_to_int(sfb, pb)
        sfa_d, sfb_d = pa.view(G, max_m, -1), pb
    else:
        sfa_d, sfb_d = sfa.view(G, max_m, -1), sfb
    a3 = a.view(G, max_m, K)
    xc = synth.normal_f32(913, (G, max_m, N)) * np.float32(4.0)
    if d_kind == "f32":
        d = torch.full((G, max_m, N), float("nan"), dtype=torch.float32, device="cuda")
    else:
        d = torch.full((G, max_m, N), SENTINEL_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    c, cref = None, None
    if c_kind == "bf16":
        cbits = synth.bf16_bits_from_f32(xc)
        c, cref = _dev_bf16(cbits), oracle.bf16_decode(cbits)
    elif c_kind == "f32":
        c, cref = to_dev(xc), xc.astype(np.float64)
    elif c_kind == "inplace":
        if d_kind == "f32":
            d.copy_(to_dev(xc))
            cref = xc.astype(np.float64)
        else:
            cbits = synth.bf16_bits_from_f32(xc)
            d.copy_(_dev_bf16(cbits))
            cref = oracle.bf16_decode(cbits)
        c = d
    masked_m = torch.tensor(mm, dtype=torch.int32, device="cuda")
    mg.m_grouped_fp8_gemm_nt_masked(a3, b, sfa_d, sfb_d, d, masked_m, max_m, c=c)
    torch.cuda.synchronize()
    ref, written = oracle.m_grouped_fp8_gemm_nt_masked(ra.reshape(G, max_m, K), rb, rsfa.reshape(G, max_m, -1), rsfb,
                                                       np.array(mm), max_m)
    if cref is not None:
        ref = ref + cref
    got = to_host(d)
    if c_kind == "inplace":
        keep = xc if d_kind == "f32" else synth.bf16_bits_from_f32(xc)
        assert np.array_equal(got[~written], keep[~written]), "rows past masked_m changed"
    elif d_kind == "f32":
        assert np.isnan(got[~written]).all(), "rows past masked_m written"
    else:
        assert np.all(got[~written] == SENTINEL_BF16), "rows past masked_m written"
    if d_kind == "f32":
        S, Gt = fp8_bound_terms(oracle.m_grouped_fp8_gemm_nt_masked, ra.reshape(G, max_m, K), rb,
                                rsfa.reshape(G, max_m, -1), rsfb, np.array(mm), max_m)
        if cref is not None:
            S = S + np.abs(cref)
        assert_f32_close(got[written], ref[written], S[written], fp8_rounding_count(K), f"masked F32 d c={c_kind}",
                         G=Gt[written])
    else:
        assert_bf16_close(got[written], ref[written], f"masked BF16 d c={c_kind}")


@pytest.mark.parametrize("form", ["contiguous", "masked"])
@pytest.mark.parametrize("d_kind,c_kind", [("f32", "bf16"), ("bf16", "f32"), ("f32", "inplace")])
def test_grouped_accumulate_on_256x256_tiles(form, d_kind, c_kind):
    """The grouped forms' C and F32 d on the 256 x 256 tile (its 64-column
    wave tiles store 16 consecutive columns per lane)."""
    from moe_grouped_gemm_x128_amd import binding
    from helpers import assert_bf16_close

    mg = _mg()
    N, K = 4096, 256
    if form == "contiguous":
        G, Msum = 5, 4096
        layout = np.array([(j * 7) % 6 - 1 for j in range(Msum // 128)], dtype=np.int32)  # -1 .. 4, mixed
        plan = binding.query_config(binding.DG_KIND_CONTIGUOUS, G, Msum, N, K)
        rows = Msum
    else:
        G, max_m = 16, 256
        mm = np.array([256, 0, 1, 255, 128, 129, 200, 17] * 2, dtype=np.int32)
        plan = binding.query_config(binding.DG_KIND_MASKED, G, max_m, N, K)
        rows = G * max_m
    assert (plan["block_m"], plan["block_n"]) == (256, 256), plan
    say(f"{form} on 256x256 tiles d={d_kind} c={c_kind}")
    a, sfa, b, sfb, ra, rsfa, rb, rsfb = _grouped_inputs(921, rows, G, N, K)
    xc = synth.normal_f32(923, (rows, N)) * np.float32(4.0)
    dt = torch.float32 if d_kind == "f32" else torch.bfloat16
    d = torch.zeros((rows, N), dtype=dt, device="cuda")
    if c_kind == "bf16":
        cbits = synth.bf16_bits_from_f32(xc)
        c, cref = _dev_bf16(cbits), oracle.bf16_decode(cbits)
    elif c_kind == "f32":
        c, cref = to_dev(xc), xc.astype(np.float64)
    else:
        d.copy_(to_dev(xc))
        c, cref = d, xc.astype(np.float64)
    if form == "contiguous":
        mg.m_grouped_fp8_gemm_nt_contiguous(a, b, sfa, sfb, d, to_dev(layout), c=c)
        ref, written = oracle.m_grouped_fp8_gemm_nt_contiguous(ra, rb, rsfa, rsfb, layout)
        S, Gt = fp8_bound_terms(oracle.m_grouped_fp8_gemm_nt_contiguous, ra, rb, rsfa, rsfb, layout)
    else:
        d3 = d.view(G, max_m, N)
        c3 = c.view(G, max_m, N)
        mg.m_grouped_fp8_gemm_nt_masked(a.view(G, max_m, K), b, sfa.view(G, max_m, -1), sfb, d3, to_dev(mm), max_m,
                                        c=c3)
        ref, written = oracle.m_grouped_fp8_gemm_nt_masked(ra.reshape(G, max_m, K), rb, rsfa.reshape(G, max_m, -1),
                                                           rsfb, mm, max_m)
        S, Gt = fp8_bound_terms(oracle.m_grouped_fp8_gemm_nt_masked, ra.reshape(G, max_m, K), rb,
                                rsfa.reshape(G, max_m, -1), rsfb, mm, max_m)
        ref, written, S, Gt = ref.reshape(rows, N), written.reshape(rows), S.reshape(rows, N), Gt.reshape(rows, N)
    torch.cuda.synchronize()
    ref = ref + cref
    got = to_host(d)
    if d_kind == "f32":
        assert_f32_close(got[written], ref[written], (S + np.abs(cref))[written], fp8_rounding_count(K),
                         f"{form} F32 d c={c_kind}", G=Gt[written])
    else:
        assert_bf16_close(got[written], ref[written], f"{form} BF16 d c={c_kind}")
    untouched = xc[~written] if c_kind == "inplace" else np.zeros_like(xc[~written])
    if d_kind == "f32":
        assert np.array_equal(got[~written], untouched), "rows that are not computed changed"
    else:
        assert np.all(got[~written] == 0), "rows that are not computed were written"


# one FP32 B scale (or UE8M0 exponent) per row of B with an F32 d: the
# 128-row tiles, the 192 x 192 and the 256 x 192 tile (dense), and both
# grouped forms on the 256 x 192 tile, C in place
@pytest.mark.parametrize("M,N,K", [(64, 100, 384), (100, 300, 256), (1000, 700, 512), (4096, 2880, 256)])
@pytest.mark.parametrize("ue8m0", [False, True])
def test_fp8_dense_f32_out_per_row_b_scales(M, N, K, ue8m0):
    from moe_grouped_gemm_x128_amd import binding

    say(f"fp8_gemm_nt F32 d, per-row B scales M={M} N={N} K={K} ue8m0={ue8m0}")
    mg = _mg()
    plan = binding.query_config(binding.DG_KIND_DENSE_ROWB, 1, M, N, K)
    if M > 128:
        assert (plan["block_m"], plan["block_n"]) == ((256, 192) if (M, N) == (4096, 2880) else (192, 192)), plan
    xa = synth.normal_f32(761, (M, K))
    xb = synth.normal_f32(762, (N, K))
    xc = synth.normal_f32(763, (M, N)) * np.float32(4.0)
    a, sfa = q_tok(to_dev(xa), ue8m0)
    b, sfb = q_tok(to_dev(xb), ue8m0)  # [N, K/128]: one scale per row of B
    sfb = sfb.contiguous()
    if ue8m0:
        pa = torch.empty((M, -(-K // 512)), dtype=torch.int32, device="cuda")
        pb = torch.empty((N, -(-K // 512)), dtype=torch.int32, device="cuda")
        mg.pack_ue8m0_to_int(sfa.contiguous(), pa)
        mg.pack_ue8m0_to_int(sfb, pb)
        sfa, sfb = pa, pb
    buf, d = nan_f32(M, N, pad=2)
    mg.fp8_gemm_nt(a, b, sfa, sfb, None, d)
    d16 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    mg.fp8_gemm_nt(a, b, sfa, sfb, None, d16)
    dc = to_dev(xc)
    mg.fp8_gemm_nt(a, b, sfa, sfb, dc, dc)  # in place: C + A . B^T
    torch.cuda.synchronize()
    assert torch.equal(d.to(torch.bfloat16).view(torch.int16), d16.view(torch.int16))
    assert torch.isnan(buf[:, N:]).all(), "row padding written"
    ra, rsfa = oracle.per_token_cast_to_fp8(xa, ue8m0)
    rb, rsfb = oracle.per_token_cast_to_fp8(xb, ue8m0)
    assert np.array_equal(to_host(a), ra) and np.array_equal(to_host(b), rb)
    S, Gt = fp8_bound_terms(oracle.fp8_gemm_nt, ra, rb, rsfa, rsfb)
    c = xc.astype(np.float64)
    assert_f32_close(to_host(d), oracle.fp8_gemm_nt(ra, rb, rsfa, rsfb), S, fp8_rounding_count(K),
                     f"fp8 F32 d per-row B scales {M}x{N}x{K}", G=Gt)
    assert_f32_close(to_host(dc), oracle.fp8_gemm_nt(ra, rb, rsfa, rsfb, c), S + np.abs(c), fp8_rounding_count(K),
                     f"fp8 F32 d per-row B scales, C in place {M}x{N}x{K}", G=Gt)


@pytest.mark.parametrize("form", ["contiguous", "masked"])
@pytest.mark.parametrize("ue8m0", [False, True])
def test_grouped_f32_out_per_row_b_scales(form, ue8m0):
    say(f"{form} F32 d, per-row B scales ue8m0={ue8m0}")
    mg = _mg()
    N, K = 272, 384
    if form == "contiguous":
        G = 3
        layout = np.array([2, 2, -1, 0, 1, 0, 2, 7], dtype=np.int32)
        rows = layout.size * 128
    else:
        G, max_m = 4, 160
        mm = np.array([0, 17, 160, 999], dtype=np.int32)
        rows = G * max_m
    xa = synth.normal_f32(771, (rows, K))
    xb = synth.normal_f32(772, (G, N, K))
    xc = synth.normal_f32(773, (rows, N)) * np.float32(4.0)
    a = torch.empty((rows, K), dtype=torch.uint8, device="cuda")
    sfa = torch.empty((rows, K // 128), dtype=torch.float32, device="cuda")
    mg.per_token_cast_to_fp8(to_dev(xa), a, sfa, ue8m0)
    b = torch.empty((G, N, K), dtype=torch.uint8, device="cuda")
    sfb = torch.empty((G, N, K // 128), dtype=torch.float32, device="cuda")
    mg.per_token_cast_to_fp8(to_dev(xb), b, sfb, ue8m0)
    if ue8m0:
        pa = torch.empty((rows, 1), dtype=torch.int32, device="cuda")
        pb = torch.empty((G, N, 1), dtype=torch.int32, device="cuda")
        mg.pack_ue8m0_to_int(sfa, pa)
        mg.pack_ue8m0_to_int(sfb, pb)
        sfa, sfb = pa, pb
    d = torch.full((rows, N), float("nan"), dtype=torch.float32, device="cuda")
    dc = to_dev(xc)
    ra, rsfa = oracle.per_token_cast_to_fp8(xa, ue8m0)
    rb, rsfb = oracle.per_token_cast_to_fp8(xb, ue8m0)
    if form == "contiguous":
        mg.m_grouped_fp8_gemm_nt_contiguous(a, b, sfa, sfb, d, to_dev(layout))
        mg.m_grouped_fp8_gemm_nt_contiguous(a, b, sfa, sfb, dc, to_dev(layout), c=dc)
        ref_layout = np.where(layout < G, layout, -1)
        ref, written = oracle.m_grouped_fp8_gemm_nt_contiguous(ra, rb, rsfa, rsfb, ref_layout)
        S, Gt = fp8_bound_terms(oracle.m_grouped_fp8_gemm_nt_contiguous, ra, rb, rsfa, rsfb, ref_layout)
    else:
        sfa3 = sfa.view(G, max_m, -1)
        mg.m_grouped_fp8_gemm_nt_masked(a.view(G, max_m, K), b, sfa3, sfb, d.view(G, max_m, N), to_dev(mm), max_m)
        mg.m_grouped_fp8_gemm_nt_masked(a.view(G, max_m, K), b, sfa3, sfb, dc.view(G, max_m, N), to_dev(mm), max_m,
                                        c=dc.view(G, max_m, N))
        args = (ra.reshape(G, max_m, K), rb, rsfa.reshape(G, max_m, -1), rsfb)
        ref, written = oracle.m_grouped_fp8_gemm_nt_masked(*args, mm, max_m)
        S, Gt = fp8_bound_terms(oracle.m_grouped_fp8_gemm_nt_masked, *args, mm, max_m)
        ref, written, S, Gt = ref.reshape(rows, N), written.reshape(rows), S.reshape(rows, N), Gt.reshape(rows, N)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(a), ra) and np.array_equal(to_host(b), rb)
    got, gotc = to_host(d), to_host(dc)
    assert np.isnan(got[~written]).all(), "rows outside the groups written"
    assert np.array_equal(gotc[~written], xc[~written]), "rows outside the groups changed"
    nr = fp8_rounding_count(K)
    assert_f32_close(got[written], ref[written], S[written], nr, f"{form} F32 d per-row B", G=Gt[written])
    c = xc.astype(np.float64)
    assert_f32_close(gotc[written], (ref + c)[written], (S + np.abs(c))[written], nr, f"{form} F32 d per-row B, C",
                     G=Gt[written])
