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
