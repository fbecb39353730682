"""BF16 dense and contiguous-grouped GEMMs on the GPU against the oracle
(BF16 operands, FP32 accumulation, BF16 out; tolerance of tests/helpers.py).
Shapes span the 256-row tile (two stages) and the 128-row tiles (three
stages), ragged M and N, K slices 1..many, the accumulate input C, and
contiguous layouts with skipped blocks and tiles split between groups."""

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


def _sentinel(shape):
    return torch.full(shape, SENTINEL_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)


# one whole round of 256 x 256 tiles, and the split plan (256 x 256 tiles on
# columns [0, 4096), 256 x 192 on [4096, 7100), last tile 124 columns)
PLAN_L = (4000, 4000, 128)
PLAN_SPLIT = (4000, 7100, 4096)  # 64 K-slices of 64 BF16 elements


def _expect_plan(M, N, K):
    from moe_grouped_gemm_x128_amd import binding

    c = binding.query_config(binding.DG_KIND_BF16_DENSE, 1, M, N, K)
    if (M, N) == PLAN_L[:2]:
        assert (c["block_m"], c["block_n"], c["block_n2"]) == (256, 256, 0)
    elif (M, N) == PLAN_SPLIT[:2]:
        assert (c["block_n"], c["n_split"], c["block_n2"]) == (256, 4096, 192)


@pytest.mark.parametrize("M,N,K", [(128, 256, 512), (200, 300, 384), (1, 130, 64), (257, 64, 256),
                                   (64, 2112, 1024), (96, 100, 640), (300, 520, 192), PLAN_L])
def test_bf16_dense_full_compare(M, N, K):
    say(f"bf16_gemm_nt M={M} N={N} K={K}")
    mg = _mg()
    _expect_plan(M, N, K)
    ab = synth.bf16_bits_from_f32(synth.normal_f32(181, (M, K)))
    bb = synth.bf16_bits_from_f32(synth.normal_f32(182, (N, K)))
    d = _sentinel((M, N))
    mg.bf16_gemm_nt(_dev_bf16(ab), _dev_bf16(bb), None, d)
    torch.cuda.synchronize()
    assert_bf16_close(to_host(d), oracle.bf16_gemm_nt(ab, bb), f"bf16 dense {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(200, 300, 256), PLAN_L])
@pytest.mark.parametrize("c_kind", ["bf16", "f32", "inplace"])
def test_bf16_dense_accumulate_c(M, N, K, c_kind):
    say(f"bf16_gemm_nt accumulate M={M} N={N} K={K} c={c_kind}")
    _expect_plan(M, N, K)
    mg = _mg()
    ab = synth.bf16_bits_from_f32(synth.normal_f32(183, (M, K)))
    bb = synth.bf16_bits_from_f32(synth.normal_f32(184, (N, K)))
    xc = synth.normal_f32(185, (M, N)) * np.float32(4.0)
    if c_kind == "f32":
        c = to_dev(xc)
        cref = xc.astype(np.float64)
        d = _sentinel((M, N))
    else:
        cbits = synth.bf16_bits_from_f32(xc)
        cref = oracle.bf16_decode(cbits)
        c = _dev_bf16(cbits)
        d = c if c_kind == "inplace" else _sentinel((M, N))
    mg.bf16_gemm_nt(_dev_bf16(ab), _dev_bf16(bb), c, d)
    torch.cuda.synchronize()
    assert_bf16_close(to_host(d), oracle.bf16_gemm_nt(ab, bb, c=cref), f"bf16 accumulate {c_kind}")


@pytest.mark.parametrize("c_kind", [None, "bf16", "f32", "inplace"])
def test_bf16_dense_split_plan_sampled_rows(c_kind):
    """The two-launch plan (256 x 256 tiles on columns [0, 4096), 256 x 192
    on [4096, 7100), the second launch's B rows, D and C columns offset on
    the host); every column compared on sampled rows."""
    M, N, K = PLAN_SPLIT
    say(f"bf16_gemm_nt split plan {M}x{N}x{K} c={c_kind}")
    _expect_plan(M, N, K)
    mg = _mg()
    ab = synth.bf16_bits_from_f32(synth.normal_f32(191, (M, K)))
    bb = synth.bf16_bits_from_f32(synth.normal_f32(192, (N, K)))
    c, cref = None, None
    if c_kind is not None:
        xc = synth.normal_f32(193, (M, N)) * np.float32(16.0)
        if c_kind == "f32":
            c = to_dev(xc)
            cref = xc.astype(np.float64)
        else:
            cbits = synth.bf16_bits_from_f32(xc)
            cref = oracle.bf16_decode(cbits)
            c = _dev_bf16(cbits)
    d = c if c_kind == "inplace" else _sentinel((M, N))
    mg.bf16_gemm_nt(_dev_bf16(ab), _dev_bf16(bb), c, d)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.random.default_rng(194).choice(M, 32, replace=False), [0, M - 1]]))
    ref = oracle.bf16_gemm_nt(ab[rows], bb, c=None if cref is None else cref[rows])
    assert_bf16_close(to_host(d)[rows], ref, f"bf16 split plan c={c_kind}")


def test_bf16_dense_large_sampled():
    """A DeepSeek-V3-sized dense shape (4096 x 4096 x 7168), checked on
    sampled rows against the oracle."""
    M, N, K = 4096, 4096, 7168
    say(f"bf16_gemm_nt {M}x{N}x{K} sampled")
    mg = _mg()
    xa = synth.normal_f32(186, (M, K))
    xb = synth.normal_f32(187, (N, K))
    a = to_dev(xa).to(torch.bfloat16)
    b = to_dev(xb).to(torch.bfloat16)
    d = _sentinel((M, N))
    mg.bf16_gemm_nt(a, b, None, d)
    torch.cuda.synchronize()
    ab, bb = to_host(a), to_host(b)
    assert np.array_equal(ab, synth.bf16_bits_from_f32(xa)), "device bf16 cast differs from the host RNE cast"
    rows = np.unique(np.concatenate([np.random.default_rng(188).choice(M, 24, replace=False), [0, M - 1]]))
    ref = oracle.bf16_gemm_nt(ab[rows], bb)
    assert_bf16_close(to_host(d)[rows], ref, "bf16 dense large sampled")


@pytest.mark.parametrize("layout,N", [([2, -1, 0, 2, 1, -1, 5], 300), ([0, 1, 1, 0, -1, 1, 0, -1, -1, 1], 300),
                                      # 256 x 256 tile: 32 blocks x 4096 columns, one whole round
                                      ([0, 1, 1, 0, -1, 1, 0, -1, -1, 1, 2, 2, 5, 2, 0, 0] * 2, 4096)])
def test_bf16_contiguous_skips_and_mixed_tiles(layout, N):
    say(f"m_grouped_bf16_gemm_nt_contiguous N={N} layout={layout}")
    mg = _mg()
    layout = np.array(layout, dtype=np.int32)
    G, K = 3, 192 if N < 4096 else 64
    Msum = layout.size * 128
    if N == 4096:
        from moe_grouped_gemm_x128_amd import binding

        c = binding.query_config(binding.DG_KIND_BF16_CONTIGUOUS, G, Msum, N, K)
        assert (c["block_m"], c["block_n"], c["block_n2"]) == (256, 256, 0)
    ab = synth.bf16_bits_from_f32(synth.normal_f32(189, (Msum, K)))
    bb = synth.bf16_bits_from_f32(synth.normal_f32(190, (G, N, K)))
    d = _sentinel((Msum, N))
    mg.m_grouped_bf16_gemm_nt_contiguous(_dev_bf16(ab), _dev_bf16(bb), d, to_dev(layout))
    torch.cuda.synchronize()
    ref, written = oracle.m_grouped_bf16_gemm_nt_contiguous(ab, bb, np.where(layout < G, layout, -1))
    got = to_host(d)
    assert np.all(got[~written] == SENTINEL_BF16)
    assert_bf16_close(got[written], ref[written], "bf16 contiguous")


@pytest.mark.parametrize("layout,N", [([2, -1, 0, 2, 1, -1, 5], 300), ([0, 0, 1, 1, 2, 2, 0, 0] * 4, 4096)])
def test_bf16_contiguous_f32_out(layout, N):
    """An F32 d on the contiguous BF16 GEMM: the FP32 accumulator within the
    (K + 2) u S bound, rounding to the BF16 output bit for bit; skipped
    blocks keep their NaN fill."""
    from helpers import assert_f32_close

    say(f"m_grouped_bf16_gemm_nt_contiguous F32 d N={N}")
    mg = _mg()
    layout = np.array(layout, dtype=np.int32)
    G, K = 3, 192 if N < 4096 else 64
    Msum = layout.size * 128
    ab = synth.bf16_bits_from_f32(synth.normal_f32(191, (Msum, K)))
    bb = synth.bf16_bits_from_f32(synth.normal_f32(192, (G, N, K)))
    buf = torch.full((Msum, N + 2), float("nan"), dtype=torch.float32, device="cuda")
    d = buf[:, :N]
    mg.m_grouped_bf16_gemm_nt_contiguous(_dev_bf16(ab), _dev_bf16(bb), d, to_dev(layout))
    d16 = _sentinel((Msum, N))
    mg.m_grouped_bf16_gemm_nt_contiguous(_dev_bf16(ab), _dev_bf16(bb), d16, to_dev(layout))
    torch.cuda.synchronize()
    ref_layout = np.where(layout < G, layout, -1)
    ref, written = oracle.m_grouped_bf16_gemm_nt_contiguous(ab, bb, ref_layout)
    S, _ = oracle.m_grouped_bf16_gemm_nt_contiguous(ab & np.uint16(0x7FFF), bb & np.uint16(0x7FFF), ref_layout)
    got = to_host(d)
    assert np.isnan(got[~written]).all(), "skipped blocks written"
    assert torch.isnan(buf[:, N:]).all(), "row padding written"
    rows = torch.from_numpy(written).cuda()
    assert torch.equal(d[rows].to(torch.bfloat16).view(torch.int16), d16[rows].view(torch.int16))
    assert_f32_close(got[written], ref[written], S[written], K, "bf16 contiguous F32 d")


@pytest.mark.parametrize("c_kind", ["bf16", "f32", "inplace"])
@pytest.mark.parametrize("d_kind", ["bf16", "f32"])
@pytest.mark.parametrize("layout,N", [([2, -1, 0, 2, 1, -1, 5], 300), ([0, 0, 1, 1, 2, 2, 0, 0] * 4, 4096)])
def test_bf16_contiguous_accumulate(layout, N, c_kind, d_kind):
    """D = C + A . B^T (m_grouped_bf16_gemm_nt_contiguous_acc): C BF16 or
    F32 shaped like d, or d itself; skipped blocks are neither read from C
    nor written."""
    from helpers import assert_f32_close

    say(f"m_grouped_bf16_gemm_nt_contiguous accumulate N={N} c={c_kind} d={d_kind}")
    mg = _mg()
    layout = np.array(layout, dtype=np.int32)
    G, K = 3, 192 if N < 4096 else 64
    Msum = layout.size * 128
    ab = synth.bf16_bits_from_f32(synth.normal_f32(193, (Msum, K)))
    bb = synth.bf16_bits_from_f32(synth.normal_f32(194, (G, N, K)))
    xc = synth.normal_f32(195, (Msum, N)) * np.float32(4.0)
    cbits = synth.bf16_bits_from_f32(xc)
    if d_kind == "f32":
        d = torch.full((Msum, N), float("nan"), dtype=torch.float32, device="cuda")
    else:
        d = _sentinel((Msum, N))
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
    mg.m_grouped_bf16_gemm_nt_contiguous(_dev_bf16(ab), _dev_bf16(bb), d, to_dev(layout), c=c)
    torch.cuda.synchronize()
    ref_layout = np.where(layout < G, layout, -1)
    ref, written = oracle.m_grouped_bf16_gemm_nt_contiguous(ab, bb, ref_layout)
    ref = ref + cref
    got = to_host(d)
    if c_kind == "inplace":
        keep = xc if d_kind == "f32" else cbits
        assert np.array_equal(got[~written], keep[~written]), "skipped blocks changed"
    elif d_kind == "f32":
        assert np.isnan(got[~written]).all(), "skipped blocks written"
    else:
        assert np.all(got[~written] == SENTINEL_BF16), "skipped blocks written"
    if d_kind == "f32":
        S, _ = oracle.m_grouped_bf16_gemm_nt_contiguous(ab & np.uint16(0x7FFF), bb & np.uint16(0x7FFF), ref_layout)
        assert_f32_close(got[written], ref[written], (S + np.abs(cref))[written], K, f"bf16 contiguous C={c_kind}")
    else:
        assert_bf16_close(got[written], ref[written], f"bf16 contiguous C={c_kind}")
