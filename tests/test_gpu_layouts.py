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
