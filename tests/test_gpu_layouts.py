"""GPU parity of the casts from MN-major sources (the transpose of a
row-major [K, R] tensor) into the K-major FP8 operands of the NT GEMMs: the
NN, TN and TT forms of a GEMM whose operands are produced by these casts
("DeepInside DeepGEMM", section 2: NT, TN, NN and TT layouts on SM100;
section 5: transposition and casting fused into the producer).  Bytes and
scales must equal the oracle's cast of the same logical tensor, bit for
bit; the GEMM on them must match the oracle's GEMM of the logical
operands."""

import numpy as np
import pytest

import oracle
from moe_grouped_gemm_x128_amd import synth

from helpers import assert_bf16_close, say, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _mg():
    import moe_grouped_gemm_x128_amd as mg

    return mg


def _mn_major(x_logical, dtype):
    """Device tensor holding x_logical [.., R, K] MN-major: stored as the
    contiguous [.., K, R] and returned as its transposed view."""
    t = to_dev(np.ascontiguousarray(np.swapaxes(x_logical, -1, -2)))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.transpose(-1, -2)


def _logical(x, dtype):
    if dtype == "bf16":
        return oracle.bf16_decode(synth.bf16_bits_from_f32(x)).astype(np.float32)
    return x


@pytest.mark.parametrize("shape", [(256, 512), (100, 300), (1, 128), (64, 7168), (3, 70, 200)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ue8m0", [False, True])
def test_per_token_cast_from_mn_major(shape, dtype, ue8m0):
    say(f"per_token_cast_to_fp8 MN-major shape={shape} dtype={dtype} ue8m0={ue8m0}")
    mg = _mg()
    x = synth.normal_f32(801, shape)
    xd = _mn_major(x, dtype)
    assert xd.stride(-2) == 1 or xd.shape[-2] == 1
    q = torch.full(shape, 0x55, dtype=torch.uint8, device="cuda")
    sf = torch.full(shape[:-1] + (-(-shape[-1] // 128),), float("nan"), dtype=torch.float32, device="cuda")
    mg.per_token_cast_to_fp8(xd, q, sf, ue8m0)
    torch.cuda.synchronize()
    rq, rsf = oracle.per_token_cast_to_fp8(_logical(x, dtype), ue8m0)
    assert np.array_equal(to_host(q), rq), "codes"
    assert np.array_equal(to_host(sf).view(np.uint32), rsf.view(np.uint32)), "scales"


@pytest.mark.parametrize("shape", [(256, 512), (300, 200), (128, 7168), (2, 130, 384)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_per_block_cast_from_mn_major(shape, dtype):
    say(f"per_block_cast_to_fp8 MN-major shape={shape} dtype={dtype}")
    mg = _mg()
    x = synth.normal_f32(802, shape)
    xd = _mn_major(x, dtype)
    q = torch.full(shape, 0x55, dtype=torch.uint8, device="cuda")
    sf = torch.full(shape[:-2] + (-(-shape[-2] // 128), -(-shape[-1] // 128)), float("nan"), dtype=torch.float32,
                    device="cuda")
    mg.per_block_cast_to_fp8(xd, q, sf)
    torch.cuda.synchronize()
    rq, rsf = oracle.per_block_cast_to_fp8(_logical(x, dtype))
    assert np.array_equal(to_host(q), rq), "codes"
    assert np.array_equal(to_host(sf).view(np.uint32), rsf.view(np.uint32)), "scales"


@pytest.mark.parametrize("layout", ["TN", "NN", "TT"])
def test_gemm_layouts_through_the_casts(layout):
    """D = A . B^T where A is stored [K, M] (T: MN-major) or [M, K] (N) and B
    stored [K, N] (N: N-major, as "NN" names B untransposed) or [N, K] (T):
    the MN-major operand is cast straight into the K-major FP8 operand."""
    mg = _mg()
    M, N, K = 384, 640, 1024
    say(f"fp8 GEMM {layout} layout through the casts M={M} N={N} K={K}")
    xa = synth.normal_f32(811, (M, K))
    xb = synth.normal_f32(812, (N, K))
    a_mn, b_mn = layout[0] == "T", layout[1] == "N"
    ad = _mn_major(xa, "f32") if a_mn else to_dev(xa)
    bd = _mn_major(xb, "f32") if b_mn else to_dev(xb)
    a = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sfa = torch.empty((K // 128, M), dtype=torch.float32, device="cuda").t()
    b = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sfb = torch.empty((N // 128, K // 128), dtype=torch.float32, device="cuda")
    mg.per_token_cast_to_fp8(ad, a, sfa)
    mg.per_block_cast_to_fp8(bd, b, sfb)
    d = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    mg.fp8_gemm_nt(a, b, sfa, sfb, None, d)
    torch.cuda.synchronize()
    ra, rsfa = oracle.per_token_cast_to_fp8(xa)
    rb, rsfb = oracle.per_block_cast_to_fp8(xb)
    assert np.array_equal(to_host(a), ra) and np.array_equal(to_host(b), rb)
    assert_bf16_close(to_host(d), oracle.fp8_gemm_nt(ra, rb, rsfa, rsfb), f"{layout} GEMM")


# ---------------------------------------------------------------------------
# NN, TN and TT on operands already in FP8 and stored MN-major: the GEMM reads
# them itself (transposing LDS reads), with results equal to fp8_gemm_nt's on
# the same values bit for bit
# ---------------------------------------------------------------------------

def _stored_mn(codes_dev, pad=0):
    """The K-major codes [R, K] stored MN-major: a row-major [K, R + pad]
    buffer whose first R columns hold the transpose; returns the [K, R] view."""
    R, K = codes_dev.shape
    buf = torch.full((K, R + pad), 0x7F, dtype=torch.uint8, device="cuda")  # NaN codes in the padding
    buf[:, :R] = codes_dev.t()
    return buf[:, :R]


def _run_layout(mg, layout, a, b, a_st, b_st, sfa, sfb, c, d):
    if layout == "NN":
        mg.fp8_gemm_nn(a, b_st, sfa, sfb, c, d)
    elif layout == "TN":
        mg.fp8_gemm_tn(a_st, b_st, sfa, sfb, c, d)
    else:
        mg.fp8_gemm_tt(a_st, b, sfa, sfb, c, d)


@pytest.mark.parametrize("M,N,K", [(128, 256, 512), (272, 208, 384), (64, 96, 256), (16, 16, 128), (528, 400, 1152),
                                   (1024, 960, 2048)])
@pytest.mark.parametrize("layout", ["NN", "TN", "TT"])
def test_fp8_gemm_mn_major_operands(M, N, K, layout):
    say(f"fp8_gemm_{layout.lower()} MN-major FP8 operands M={M} N={N} K={K}")
    mg = _mg()
    from moe_grouped_gemm_x128_amd import binding

    c = binding.query_config(binding.DG_KIND_DENSE_MN, 1, M, N, K)
    assert (c["block_m"], c["block_n"], c["block_n2"]) == (256, 192, 0)
    xa = synth.normal_f32(821, (M, K))
    xb = synth.normal_f32(822, (N, K))
    a = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sfa = torch.empty((K // 128, M), dtype=torch.float32, device="cuda").t()
    b = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sfb = torch.empty((-(-N // 128), K // 128), dtype=torch.float32, device="cuda")
    mg.per_token_cast_to_fp8(to_dev(xa), a, sfa)
    mg.per_block_cast_to_fp8(to_dev(xb), b, sfb)
    a_st = _stored_mn(a, pad=16 if M % 32 else 0)
    b_st = _stored_mn(b, pad=48)
    d = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    _run_layout(mg, layout, a, b, a_st, b_st, sfa, sfb, None, d)
    dref = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    mg.fp8_gemm_nt(a, b, sfa, sfb, None, dref)
    torch.cuda.synchronize()
    assert torch.equal(d.view(torch.int16), dref.view(torch.int16)), "differs from fp8_gemm_nt on the same values"
    ra, rsfa = oracle.per_token_cast_to_fp8(xa)
    rb, rsfb = oracle.per_block_cast_to_fp8(xb)
    assert np.array_equal(to_host(a), ra) and np.array_equal(to_host(b), rb)
    assert_bf16_close(to_host(d), oracle.fp8_gemm_nt(ra, rb, rsfa, rsfb), f"{layout} FP8 {M}x{N}x{K}")


@pytest.mark.parametrize("layout", ["NN", "TN", "TT"])
def test_fp8_gemm_mn_major_ue8m0_and_accumulate(layout):
    """Packed UE8M0 scales, and D = C + A . B^T with a BF16 C, on MN-major operands."""
    M, N, K = 400, 336, 1024
    say(f"fp8_gemm_{layout.lower()} UE8M0 + accumulate M={M} N={N} K={K}")
    mg = _mg()
    xa = synth.normal_f32(831, (M, K))
    xb = synth.normal_f32(832, (N, K))
    xc = synth.normal_f32(833, (M, N)) * np.float32(4.0)
    a = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sfa = torch.empty((M, K // 128), dtype=torch.float32, device="cuda")
    b = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sfb = torch.empty((-(-N // 128), K // 128), dtype=torch.float32, device="cuda")
    mg.per_token_cast_to_fp8(to_dev(xa), a, sfa, True)
    mg.per_block_cast_to_fp8(to_dev(xb), b, sfb, True)
    pa = torch.empty((M, K // 512), dtype=torch.int32, device="cuda")
    pb = torch.empty((-(-N // 128), K // 512), dtype=torch.int32, device="cuda")
    mg.pack_ue8m0_to_int(sfa, pa)
    mg.pack_ue8m0_to_int(sfb, pb)
    cbits = synth.bf16_bits_from_f32(xc)
    c = to_dev(cbits.view(np.int16)).view(torch.bfloat16)
    a_st, b_st = _stored_mn(a), _stored_mn(b, pad=16)
    d = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    _run_layout(mg, layout, a, b, a_st, b_st, pa, pb, c, d)
    dref = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    mg.fp8_gemm_nt(a, b, pa, pb, c, dref)
    torch.cuda.synchronize()
    assert torch.equal(d.view(torch.int16), dref.view(torch.int16)), "differs from fp8_gemm_nt on the same values"
    ra, rsfa = oracle.per_token_cast_to_fp8(xa, True)
    rb, rsfb = oracle.per_block_cast_to_fp8(xb, True)
    ref = oracle.fp8_gemm_nt(ra, rb, rsfa, rsfb, c=oracle.bf16_decode(cbits))
    assert_bf16_close(to_host(d), ref, f"{layout} FP8 UE8M0 + C")


def test_fp8_gemm_nt_takes_transposed_views():
    """fp8_gemm_nt itself takes an MN-major operand given as the transposed
    view of a row-major [K, R] tensor (both operands here)."""
    M, N, K = 208, 592, 640
    say(f"fp8_gemm_nt on transposed views M={M} N={N} K={K}")
    mg = _mg()
    xa = synth.normal_f32(841, (M, K))
    xb = synth.normal_f32(842, (N, K))
    a = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sfa = torch.empty((K // 128, M), dtype=torch.float32, device="cuda").t()
    b = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sfb = torch.empty((-(-N // 128), K // 128), dtype=torch.float32, device="cuda")
    mg.per_token_cast_to_fp8(to_dev(xa), a, sfa)
    mg.per_block_cast_to_fp8(to_dev(xb), b, sfb)
    d = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    mg.fp8_gemm_nt(_stored_mn(a).t(), _stored_mn(b, pad=32).t(), sfa, sfb, None, d)
    dref = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    mg.fp8_gemm_nt(a, b, sfa, sfb, None, dref)
    torch.cuda.synchronize()
    assert torch.equal(d.view(torch.int16), dref.view(torch.int16))


@pytest.mark.parametrize("layout", ["NN", "TN", "TT"])
@pytest.mark.parametrize("M,N,K,ue8m0", [(272, 208, 384, False), (1024, 960, 2048, True)])
def test_fp8_gemm_mn_major_f32_out(layout, M, N, K, ue8m0):
    """An F32 d (the accumulator stored without rounding, C added in place)
    on MN-major operands: bit for bit the F32 output of fp8_gemm_nt on the
    same values, and within the FP32-output bound of the oracle."""
    from helpers import assert_f32_close, fp8_bound_terms, fp8_rounding_count

    say(f"fp8_gemm_{layout.lower()} F32 d M={M} N={N} K={K} ue8m0={ue8m0}")
    mg = _mg()
    xa = synth.normal_f32(851, (M, K))
    xb = synth.normal_f32(852, (N, K))
    xc = synth.normal_f32(853, (M, N)) * np.float32(4.0)
    a = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sfa = torch.empty((M, K // 128), dtype=torch.float32, device="cuda")
    b = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sfb = torch.empty((-(-N // 128), K // 128), dtype=torch.float32, device="cuda")
    mg.per_token_cast_to_fp8(to_dev(xa), a, sfa, ue8m0)
    mg.per_block_cast_to_fp8(to_dev(xb), b, sfb, ue8m0)
    if ue8m0:
        pa = torch.empty((M, -(-K // 512)), dtype=torch.int32, device="cuda")
        pb = torch.empty((-(-N // 128), -(-K // 512)), dtype=torch.int32, device="cuda")
        mg.pack_ue8m0_to_int(sfa, pa)
        mg.pack_ue8m0_to_int(sfb, pb)
        sfa, sfb = pa, pb
    a_st, b_st = _stored_mn(a, pad=16), _stored_mn(b, pad=32)
    d = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    _run_layout(mg, layout, a, b, a_st, b_st, sfa, sfb, None, d)
    dc = to_dev(xc)
    _run_layout(mg, layout, a, b, a_st, b_st, sfa, sfb, dc, dc)
    dref = torch.empty((M, N), dtype=torch.float32, device="cuda")
    mg.fp8_gemm_nt(a, b, sfa, sfb, None, dref)
    dcref = to_dev(xc)
    mg.fp8_gemm_nt(a, b, sfa, sfb, dcref, dcref)
    torch.cuda.synchronize()
    assert torch.equal(d.view(torch.int32), dref.view(torch.int32)), "differs from fp8_gemm_nt"
    assert torch.equal(dc.view(torch.int32), dcref.view(torch.int32)), "differs from fp8_gemm_nt (C in place)"
    ra, rsfa = oracle.per_token_cast_to_fp8(xa, ue8m0)
    rb, rsfb = oracle.per_block_cast_to_fp8(xb, ue8m0)
    assert np.array_equal(to_host(a), ra) and np.array_equal(to_host(b), rb)
    S, G = fp8_bound_terms(oracle.fp8_gemm_nt, ra, rb, rsfa, rsfb)
    c = xc.astype(np.float64)
    assert_f32_close(to_host(d), oracle.fp8_gemm_nt(ra, rb, rsfa, rsfb), S, fp8_rounding_count(K),
                     f"{layout} F32 d", G=G)
    assert_f32_close(to_host(dc), oracle.fp8_gemm_nt(ra, rb, rsfa, rsfb, c), S + np.abs(c), fp8_rounding_count(K),
                     f"{layout} F32 d, C in place", G=G)


@pytest.mark.parametrize("layout", ["NN", "TN", "TT"])
@pytest.mark.parametrize("ue8m0,d_kind", [(False, "bf16"), (True, "bf16"), (False, "f32"), (True, "f32")])
def test_fp8_gemm_mn_major_per_row_b_scales(layout, ue8m0, d_kind):
    """One B scale per row of B ([N, K/128], FP32 or packed UE8M0) on
    MN-major operands: bit for bit fp8_gemm_nt's result on the same values,
    and the oracle within the tolerance of the output dtype."""
    from helpers import assert_bf16_close, assert_f32_close, fp8_bound_terms, fp8_rounding_count

    M, N, K = 400, 336, 1024
    say(f"fp8_gemm_{layout.lower()} per-row B scales ue8m0={ue8m0} d={d_kind}")
    mg = _mg()
    xa = synth.normal_f32(861, (M, K))
    xb = synth.normal_f32(862, (N, K))
    a = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sfa = torch.empty((M, K // 128), dtype=torch.float32, device="cuda")
    b = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sfb = torch.empty((N, K // 128), dtype=torch.float32, device="cuda")
    mg.per_token_cast_to_fp8(to_dev(xa), a, sfa, ue8m0)
    mg.per_token_cast_to_fp8(to_dev(xb), b, sfb, ue8m0)  # one scale per row of B
    if ue8m0:
        pa = torch.empty((M, K // 512), dtype=torch.int32, device="cuda")
        pb = torch.empty((N, K // 512), dtype=torch.int32, device="cuda")
        mg.pack_ue8m0_to_int(sfa, pa)
        mg.pack_ue8m0_to_int(sfb, pb)
        sfa, sfb = pa, pb
    a_st, b_st = _stored_mn(a), _stored_mn(b, pad=16)
    dt = torch.float32 if d_kind == "f32" else torch.bfloat16
    d = torch.empty((M, N), dtype=dt, device="cuda")
    _run_layout(mg, layout, a, b, a_st, b_st, sfa, sfb, None, d)
    dref = torch.empty((M, N), dtype=dt, device="cuda")
    mg.fp8_gemm_nt(a, b, sfa, sfb, None, dref)
    torch.cuda.synchronize()
    bits = torch.int32 if d_kind == "f32" else torch.int16
    assert torch.equal(d.view(bits), dref.view(bits)), "differs from fp8_gemm_nt on the same values"
    ra, rsfa = oracle.per_token_cast_to_fp8(xa, ue8m0)
    rb, rsfb = oracle.per_token_cast_to_fp8(xb, ue8m0)
    assert np.array_equal(to_host(a), ra) and np.array_equal(to_host(b), rb)
    ref = oracle.fp8_gemm_nt(ra, rb, rsfa, rsfb)
    if d_kind == "f32":
        S, G = fp8_bound_terms(oracle.fp8_gemm_nt, ra, rb, rsfa, rsfb)
        assert_f32_close(to_host(d), ref, S, fp8_rounding_count(K), f"{layout} per-row B, F32 d", G=G)
    else:
        assert_bf16_close(to_host(d), ref, f"{layout} per-row B scales")
