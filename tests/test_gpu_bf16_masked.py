"""GPU parity of the masked grouped BF16 GEMM against the float64 oracle."""

import numpy as np
import pytest

import oracle
from moe_grouped_gemm_x128_amd import synth

from helpers import SENTINEL_BF16, assert_bf16_close, say, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _mg():
    import moe_grouped_gemm_x128_amd as mg

    return mg


def _dev_bf16(bits):
    return to_dev(bits.view(np.int16)).view(torch.bfloat16)


@pytest.mark.parametrize("G,max_m,N,K,mm", [
    (4, 128, 300, 256, [0, 5, 128, 77]),
    (3, 200, 128, 64, [200, 199, 1000]),
    (2, 16, 1000, 512, [-4, 16]),
    (2, 256, 384, 320, [256, 130]),
    # 256 x 256 tile (one whole round: 16 experts x 4096 columns)
    (16, 256, 4096, 64, [0, 17, 256, 999, -3, 129, 128, 200, 1, 255, 64, 130, 250, 16, 0, 192]),
])
def test_bf16_masked_full_compare(G, max_m, N, K, mm):
    say(f"bf16 masked G={G} max_m={max_m} N={N} K={K} masked_m={mm}")
    mg = _mg()
    if G == 16:
        from moe_grouped_gemm_x128_amd import binding

        c = binding.query_config(binding.DG_KIND_BF16_MASKED, G, max_m, N, K)
        assert (c["block_m"], c["block_n"], c["block_n2"]) == (256, 256, 0)
    mm = np.array(mm, dtype=np.int32)
    ab = synth.bf16_bits_from_f32(synth.normal_f32(151, (G, max_m, K)))
    bb = synth.bf16_bits_from_f32(synth.normal_f32(152, (G, N, K)))
    d = torch.full((G, max_m, N), SENTINEL_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    mg.m_grouped_bf16_gemm_nt_masked(_dev_bf16(ab), _dev_bf16(bb), d, to_dev(mm), max_m)
    torch.cuda.synchronize()
    ref, written = oracle.m_grouped_bf16_gemm_nt_masked(ab, bb, mm, max_m)
    got = to_host(d)
    assert np.all(got[~written] == SENTINEL_BF16)
    assert_bf16_close(got[written], ref[written], "bf16 masked")


def test_bf16_masked_2d_operands():
    say("bf16 masked 2-D operands")
    mg = _mg()
    G, max_m, N, K = 2, 48, 96, 128
    ab = synth.bf16_bits_from_f32(synth.normal_f32(153, (G * max_m, K)))
    bb = synth.bf16_bits_from_f32(synth.normal_f32(154, (G, N, K)))
    mm = np.array([48, 31], dtype=np.int32)
    d = torch.full((G * max_m, N), SENTINEL_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    mg.m_grouped_bf16_gemm_nt_masked(_dev_bf16(ab), _dev_bf16(bb), d, to_dev(mm), max_m)
    torch.cuda.synchronize()
    ref, written = oracle.m_grouped_bf16_gemm_nt_masked(ab.reshape(G, max_m, K), bb, mm, max_m)
    got = to_host(d).reshape(G, max_m, N)
    assert np.all(got[~written] == SENTINEL_BF16)
    assert_bf16_close(got[written], ref[written], "bf16 masked 2-D")


@pytest.mark.parametrize("G,max_m,N,K,mm", [
    (4, 128, 300, 256, [0, 5, 128, 77]),
    (2, 256, 384, 320, [256, 130]),
    (16, 256, 4096, 64, [0, 17, 256, 999, -3, 129, 128, 200, 1, 255, 64, 130, 250, 16, 0, 192]),
])
def test_bf16_masked_f32_out(G, max_m, N, K, mm):
    """An F32 d: the FP32 accumulator stored without rounding (within the
    (K + 2) u S bound of FP32 summation, and rounding to the BF16 output bit
    for bit); rows past masked_m keep their NaN fill."""
    from helpers import assert_f32_close

    say(f"bf16 masked F32 d G={G} max_m={max_m} N={N} K={K}")
    mg = _mg()
    mm = np.array(mm, dtype=np.int32)
    ab = synth.bf16_bits_from_f32(synth.normal_f32(155, (G, max_m, K)))
    bb = synth.bf16_bits_from_f32(synth.normal_f32(156, (G, N, K)))
    buf = torch.full((G, max_m, N + 4), float("nan"), dtype=torch.float32, device="cuda")
    d = buf[..., :N]
    mg.m_grouped_bf16_gemm_nt_masked(_dev_bf16(ab), _dev_bf16(bb), d, to_dev(mm), max_m)
    d16 = torch.full((G, max_m, N), SENTINEL_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    mg.m_grouped_bf16_gemm_nt_masked(_dev_bf16(ab), _dev_bf16(bb), d16, to_dev(mm), max_m)
    torch.cuda.synchronize()
    ref, written = oracle.m_grouped_bf16_gemm_nt_masked(ab, bb, mm, max_m)
    S, _ = oracle.m_grouped_bf16_gemm_nt_masked(ab & np.uint16(0x7FFF), bb & np.uint16(0x7FFF), mm, max_m)
    got = to_host(d)
    assert np.isnan(got[~written]).all(), "rows past masked_m written"
    assert torch.isnan(buf[..., N:]).all(), "row padding written"
    rows = torch.from_numpy(written).cuda()
    assert torch.equal(d[rows].to(torch.bfloat16).view(torch.int16), d16[rows].view(torch.int16))
    assert_f32_close(got[written], ref[written], S[written], K, "bf16 masked F32 d")


@pytest.mark.parametrize("c_kind", ["bf16", "f32", "inplace"])
@pytest.mark.parametrize("d_kind", ["bf16", "f32"])
@pytest.mark.parametrize("G,max_m,N,K,mm", [(3, 200, 300, 192, [200, 0, 77]),
                                            (16, 256, 4096, 64, [256, 0, 1, 255, 128, 129, 200, 17] * 2)])
def test_bf16_masked_accumulate(G, max_m, N, K, mm, c_kind, d_kind):
    """D = C + A . B^T per group (m_grouped_bf16_gemm_nt_masked_acc): C BF16
    or F32 with d's shape, or d itself; rows past masked_m are neither read
    from C nor written."""
    from helpers import assert_f32_close

    say(f"bf16 masked accumulate G={G} max_m={max_m} N={N} K={K} c={c_kind} d={d_kind}")
    mg = _mg()
    mm = np.array(mm, dtype=np.int32)
    ab = synth.bf16_bits_from_f32(synth.normal_f32(157, (G, max_m, K)))
    bb = synth.bf16_bits_from_f32(synth.normal_f32(158, (G, N, K)))
    xc = synth.normal_f32(159, (G, max_m, N)) * np.float32(4.0)
    if d_kind == "f32":
        d = torch.full((G, max_m, N), float("nan"), dtype=torch.float32, device="cuda")
    else:
        d = torch.full((G, max_m, N), SENTINEL_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    cbits = synth.bf16_bits_from_f32(xc)
    if c_kind == "bf16":
        c, cref = _dev_bf16(cbits), oracle.bf16_decode(cbits)
    elif c_kind == "f32":
        c, cref = to_dev(xc), xc.astype(np.float64)
    else:
        if d_kind == "f32":
            d.copy_(to_dev(xc))
            cref = xc.astype(np.float64)
        else:
            d.copy_(_dev_bf16(cbits))
            cref = oracle.bf16_decode(cbits)
        c = d
    mg.m_grouped_bf16_gemm_nt_masked(_dev_bf16(ab), _dev_bf16(bb), d, to_dev(mm), max_m, c=c)
    torch.cuda.synchronize()
    ref, written = oracle.m_grouped_bf16_gemm_nt_masked(ab, bb, mm, max_m)
    ref = ref + cref
    got = to_host(d)
    if c_kind == "inplace":
        keep = xc if d_kind == "f32" else cbits
        assert np.array_equal(got[~written], keep[~written]), "rows past masked_m changed"
    elif d_kind == "f32":
        assert np.isnan(got[~written]).all(), "rows past masked_m written"
    else:
        assert np.all(got[~written] == SENTINEL_BF16), "rows past masked_m written"
    if d_kind == "f32":
        S, _ = oracle.m_grouped_bf16_gemm_nt_masked(ab & np.uint16(0x7FFF), bb & np.uint16(0x7FFF), mm, max_m)
        assert_f32_close(got[written], ref[written], (S + np.abs(cref))[written], K, f"bf16 masked C={c_kind}")
    else:
        assert_bf16_close(got[written], ref[written], f"bf16 masked C={c_kind}")
