"""GPU parity of the block-scaled FP8 GEMMs (dense, contiguous-grouped,
masked-grouped) against the float64 oracle.

Operands are quantized on the GPU by the library and independently by the
oracle (the two must agree bit for bit); the oracle GEMM consumes its own
quantized values.  Small shapes are compared in full; the full-size
DeepSeek-V3 shapes are compared on sampled rows x sampled 128-column blocks,
which the oracle computes from the corresponding slices of the inputs."""

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


def q_tok(xt, ue8m0=False):
    """Per-token quantize a device tensor [..., K]; scales M-major for 2-D."""
    mg = _mg()
    K = xt.shape[-1]
    q = torch.empty(xt.shape, dtype=torch.uint8, device="cuda")
    if xt.dim() == 2:
        sf = torch.empty((K // 128, xt.shape[0]), dtype=torch.float32, device="cuda").t()
    else:
        sf = torch.empty(xt.shape[:-1] + (K // 128,), dtype=torch.float32, device="cuda")
    mg.per_token_cast_to_fp8(xt, q, sf, ue8m0)
    return q, sf


def q_blk(xt, ue8m0=False):
    mg = _mg()
    N, K = xt.shape[-2], xt.shape[-1]
    q = torch.empty(xt.shape, dtype=torch.uint8, device="cuda")
    sf = torch.empty(xt.shape[:-2] + (-(-N // 128), K // 128), dtype=torch.float32, device="cuda")
    mg.per_block_cast_to_fp8(xt, q, sf, ue8m0)
    return q, sf


def sentinel_like(shape):
    return torch.full(shape, SENTINEL_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)


# ---------------------------------------------------------------------------
# dense
# ---------------------------------------------------------------------------

# Shapes of every launch plan of the FP8 GEMM, with ragged M and N: rows
# <= 128 (128-row tiles), one round of 192 x 192 tiles (problems below one
# round of the larger tiles), one round of 256 x 192 tiles (4096 x 2880: 240
# tiles, where 192 x 192 would take two rounds) and one whole round of
# 256 x 256 tiles (4000 x 4000).
PLAN_L = (4000, 4000, 256)
PLAN_N = (4096, 2880, 256)


def _expect_plan(kind, M, N, K):
    from moe_grouped_gemm_x128_amd import binding

    c = binding.query_config(getattr(binding, kind), 1, M, N, K)
    if (M, N) == PLAN_L[:2]:
        assert (c["block_m"], c["block_n"], c["block_n2"]) == (256, 256, 0)
    elif (M, N) == PLAN_N[:2]:
        assert (c["block_m"], c["block_n"], c["block_n2"]) == (256, 192, 0)
    elif M > 128:
        assert (c["block_m"], c["block_n"], c["block_n2"]) == (192, 192, 0)
    return c


@pytest.mark.parametrize("M,N,K", [(128, 256, 512), (200, 300, 384), (1, 130, 128), (257, 64, 256), (64, 2112, 1024),
                                   (96, 100, 640), (128, 128, 384), (1000, 700, 512), PLAN_N, PLAN_L])
def test_dense_full_compare(M, N, K):
    say(f"fp8_gemm_nt M={M} N={N} K={K}")
    mg = _mg()
    _expect_plan("DG_KIND_DENSE", M, N, K)
    xa = synth.normal_f32(101, (M, K))
    xb = synth.normal_f32(102, (N, K))
    a, sfa = q_tok(to_dev(xa))
    b, sfb = q_blk(to_dev(xb))
    d = sentinel_like((M, N))
    mg.fp8_gemm_nt(a, b, sfa, sfb, None, d)
    torch.cuda.synchronize()
    ra, rsfa = oracle.per_token_cast_to_fp8(xa)
    rb, rsfb = oracle.per_block_cast_to_fp8(xb)
    assert np.array_equal(to_host(a), ra) and np.array_equal(to_host(b), rb)
    ref = oracle.fp8_gemm_nt(ra, rb, rsfa, rsfb)
    assert_bf16_close(to_host(d), ref, f"dense {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(192, 384, 1024), (PLAN_N[0], PLAN_N[1], 512), (PLAN_L[0], PLAN_L[1], 512)])
def test_dense_ue8m0_packed_scales(M, N, K):
    say(f"fp8_gemm_nt UE8M0 packed scales M={M} N={N} K={K}")
    mg = _mg()
    _expect_plan("DG_KIND_DENSE", M, N, K)
    xa = synth.normal_f32(111, (M, K))
    xb = synth.normal_f32(112, (N, K))
    a, sfa = q_tok(to_dev(xa), ue8m0=True)
    b, sfb = q_blk(to_dev(xb), ue8m0=True)
    pa = torch.empty((M, K // 512), dtype=torch.int32, device="cuda")
    pb = torch.empty((-(-N // 128), K // 512), dtype=torch.int32, device="cuda")
    mg.pack_ue8m0_to_int(sfa.contiguous(), pa)
    mg.pack_ue8m0_to_int(sfb, pb)
    d = sentinel_like((M, N))
    mg.fp8_gemm_nt(a, b, pa, pb, None, d)
    torch.cuda.synchronize()
    ra, rsfa = oracle.per_token_cast_to_fp8(xa, True)
    rb, rsfb = oracle.per_block_cast_to_fp8(xb, True)
    rpa, _ = oracle.pack_ue8m0_to_int(rsfa)
    rpb, _ = oracle.pack_ue8m0_to_int(rsfb)
    assert np.array_equal(to_host(pa), rpa) and np.array_equal(to_host(pb), rpb)
    ref = oracle.fp8_gemm_nt(ra, rb, oracle.scales_from_packed_ue8m0(rpa, K // 128),
                             oracle.scales_from_packed_ue8m0(rpb, K // 128))
    assert_bf16_close(to_host(d), ref, "dense ue8m0")


@pytest.mark.parametrize("M,N,K", [(160, 272, 768), PLAN_L])
def test_dense_one_hot_closed_form_bit_exact(M, N, K):
    """B one-hot (column n reads K index kn[n]) and power-of-two scales: every
    output is sfa*sfb*A[m, kn[n]] exactly, representable in bf16, so the
    device result must match bit for bit; this pins the A/B/scale indexing
    and the MFMA fragment layout of each launch plan."""
    say(f"fp8_gemm_nt one-hot closed form M={M} N={N} K={K}")
    mg = _mg()
    _expect_plan("DG_KIND_DENSE", M, N, K)
    rng = np.random.default_rng(23)
    a = (rng.integers(0, 0x7E, size=(M, K)) | (rng.integers(0, 2, size=(M, K)) << 7)).astype(np.uint8)
    kn = rng.integers(0, K, size=N) if N > K else rng.permutation(K)[:N]
    b = np.zeros((N, K), dtype=np.uint8)
    b[np.arange(N), kn] = 0x38
    sfa = np.exp2(rng.integers(-6, 6, size=(M, K // 128))).astype(np.float32)
    sfb = np.exp2(rng.integers(-6, 6, size=(-(-N // 128), K // 128))).astype(np.float32)
    d = sentinel_like((M, N))
    mg.fp8_gemm_nt(to_dev(a), to_dev(b), to_dev(sfa), to_dev(sfb), None, d)
    torch.cuda.synchronize()
    ref = oracle.fp8_gemm_nt(a, b, sfa, sfb)
    ref_bits = to_host(torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16))
    assert np.array_equal(torch.from_numpy(ref_bits.view(np.int16)).view(torch.bfloat16).double().numpy(), ref)
    got = to_host(d)
    bad = np.argwhere(got != ref_bits)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}"


def _sample_rows(M, n, seed):
    rows = np.random.default_rng(seed).choice(M, size=min(n, M), replace=False)
    return np.unique(np.concatenate([rows, [0, M - 1]]))


def _sample_col_blocks(N):
    nnb = -(-N // 128)
    return sorted({0, nnb // 2, nnb - 1})


@pytest.mark.parametrize("i", range(len(synth.DENSE_V3_SHAPES)))
def test_dense_v3_shapes_sampled(i):
    N, K = synth.DENSE_V3_SHAPES[i]
    M = synth.DENSE_V3_M
    say(f"fp8_gemm_nt full size M={M} N={N} K={K}")
    mg = _mg()
    sa, sb = synth.dense_v3_seeds(i)
    xa = synth.normal_f32(sa, (M, K))
    xb = synth.normal_f32(sb, (N, K))
    a, sfa = q_tok(to_dev(xa))
    b, sfb = q_blk(to_dev(xb))
    d = sentinel_like((M, N))
    mg.fp8_gemm_nt(a, b, sfa, sfb, None, d)
    torch.cuda.synchronize()
    rows = _sample_rows(M, 40, 7 + i)
    ra, rsfa = oracle.per_token_cast_to_fp8(xa[rows])
    assert np.array_equal(to_host(a)[rows], ra)
    dh = to_host(d)
    for nb in _sample_col_blocks(N):
        cols = slice(nb * 128, min(N, nb * 128 + 128))
        rb, rsfb = oracle.per_block_cast_to_fp8(xb[cols])
        ref = oracle.fp8_gemm_nt(ra, rb, rsfa, rsfb)
        assert_bf16_close(dh[rows][:, cols], ref, f"dense {M}x{N}x{K} col block {nb}")


@pytest.mark.parametrize("M,N,K", [(200, 300, 384), (64, 2112, 1024), (130, 130, 256), PLAN_N, PLAN_L])
@pytest.mark.parametrize("c_kind", ["bf16", "f32", "inplace"])
def test_dense_accumulate_c(M, N, K, c_kind):
    """D = C + A . B^T ("DeepInside DeepGEMM", section 4): C in BF16 or FP32,
    with a padded row stride, or C being d itself; on every launch plan
    (128-row, 192 x 192, 256 x 192 and 256 x 256 tiles)."""
    say(f"fp8_gemm_nt accumulate M={M} N={N} K={K} c={c_kind}")
    mg = _mg()
    _expect_plan("DG_KIND_DENSE", M, N, K)
    xa = synth.normal_f32(171, (M, K))
    xb = synth.normal_f32(172, (N, K))
    xc = synth.normal_f32(173, (M, N)) * np.float32(8.0)
    a, sfa = q_tok(to_dev(xa))
    b, sfb = q_blk(to_dev(xb))
    if c_kind == "f32":
        cbuf = torch.zeros((M, N + 4), dtype=torch.float32, device="cuda")
        cbuf[:, :N] = to_dev(xc)
        c = cbuf[:, :N]
        cref = xc.astype(np.float64)
        d = sentinel_like((M, N))
    else:
        cbits = synth.bf16_bits_from_f32(xc)
        cref = oracle.bf16_decode(cbits)
        cbuf = torch.zeros((M, N + 8), dtype=torch.int16, device="cuda")
        cbuf[:, :N] = to_dev(cbits.view(np.int16))
        c = cbuf[:, :N].view(torch.bfloat16)
        d = c if c_kind == "inplace" else sentinel_like((M, N))
    mg.fp8_gemm_nt(a, b, sfa, sfb, c, d)
    torch.cuda.synchronize()
    ra, rsfa = oracle.per_token_cast_to_fp8(xa)
    rb, rsfb = oracle.per_block_cast_to_fp8(xb)
    ref = oracle.fp8_gemm_nt(ra, rb, rsfa, rsfb, c=cref)
    assert_bf16_close(to_host(d), ref, f"accumulate {c_kind} {M}x{N}x{K}")
    if c_kind == "inplace":
        assert np.all(to_host(cbuf)[:, N:] == 0), "the row padding of c/d was written"


def test_dense_row_stride_at_the_32bit_offset_limit():
    """A and B as row views of buffers whose row stride is the largest the
    library takes (8 MiB - 16 bytes), on the dense plan's 192 x 192 tiles;
    the next stride up is rejected.  (The 256-row tiles, which reach just
    under 2^31 bytes of 32-bit buffer offsets at this stride, are covered by
    the masked form below.)"""
    say("fp8_gemm_nt row stride 8 MiB - 16")
    mg = _mg()
    from moe_grouped_gemm_x128_amd import binding

    M, N, K = 300, 272, 256
    _expect_plan("DG_KIND_DENSE", M, N, K)
    ld = (1 << 23) - 16
    xa = synth.normal_f32(161, (M, K))
    xb = synth.normal_f32(162, (N, K))
    a_c, sfa = q_tok(to_dev(xa))
    b_c, sfb = q_blk(to_dev(xb))
    abuf = torch.zeros(M * ld, dtype=torch.uint8, device="cuda")
    bbuf = torch.zeros(N * ld, dtype=torch.uint8, device="cuda")
    a = abuf.as_strided((M, K), (ld, 1))
    b = bbuf.as_strided((N, K), (ld, 1))
    a.copy_(a_c)
    b.copy_(b_c)
    d = sentinel_like((M, N))
    mg.fp8_gemm_nt(a, b, sfa, sfb, None, d)
    torch.cuda.synchronize()
    ra, rsfa = oracle.per_token_cast_to_fp8(xa)
    rb, rsfb = oracle.per_block_cast_to_fp8(xb)
    assert np.array_equal(to_host(a_c), ra) and np.array_equal(to_host(b_c), rb)
    assert_bf16_close(to_host(d), oracle.fp8_gemm_nt(ra, rb, rsfa, rsfb), "dense row stride 8 MiB - 16")
    wide = abuf.as_strided((2, K), (ld + 16, 1))
    with pytest.raises(binding.DgmiError):
        mg.fp8_gemm_nt(wide, b, sfa[:2], sfb, None, d[:2])
    del abuf, bbuf


def test_masked_row_stride_at_the_32bit_offset_limit():
    """The masked form (one expert, 300 rows, all valid) with A and B rows
    8 MiB - 16 bytes apart: its 256-row tiles span 256 such rows, just under
    2^31 bytes of the 32-bit buffer offsets the tile loads use."""
    say("m_grouped_fp8_gemm_nt_masked row stride 8 MiB - 16, 256-row tiles")
    mg = _mg()
    from moe_grouped_gemm_x128_amd import binding

    G, max_m, N, K = 1, 300, 272, 256
    c = binding.query_config(binding.DG_KIND_MASKED, G, max_m, N, K)
    assert c["block_m"] == 256, c
    ld = (1 << 23) - 16
    xa = synth.normal_f32(163, (max_m, K))
    xb = synth.normal_f32(164, (N, K))
    a_c, sfa = q_tok(to_dev(xa))
    b_c, sfb = q_blk(to_dev(xb))
    abuf = torch.zeros(max_m * ld, dtype=torch.uint8, device="cuda")
    bbuf = torch.zeros(N * ld, dtype=torch.uint8, device="cuda")
    a = abuf.as_strided((G, max_m, K), (max_m * ld, ld, 1))
    b = bbuf.as_strided((G, N, K), (N * ld, ld, 1))
    a[0].copy_(a_c)
    b[0].copy_(b_c)
    sfa3 = sfa.contiguous().view(G, max_m, K // 128)
    sfb3 = sfb.view(G, -(-N // 128), K // 128)
    d = sentinel_like((G, max_m, N))
    mm = torch.tensor([max_m], dtype=torch.int32, device="cuda")
    mg.m_grouped_fp8_gemm_nt_masked(a, b, sfa3, sfb3, d, mm, max_m)
    torch.cuda.synchronize()
    ra, rsfa = oracle.per_token_cast_to_fp8(xa)
    rb, rsfb = oracle.per_block_cast_to_fp8(xb)
    assert np.array_equal(to_host(a_c), ra) and np.array_equal(to_host(b_c), rb)
    assert_bf16_close(to_host(d)[0], oracle.fp8_gemm_nt(ra, rb, rsfa, rsfb), "masked row stride 8 MiB - 16")
    del abuf, bbuf


# ---------------------------------------------------------------------------
# contiguous grouped
# ---------------------------------------------------------------------------

def test_contiguous_small_with_skips():
    say("contiguous small, shuffled layout with -1 blocks")
    mg = _mg()
    G, N, K = 3, 300, 256
    layout = np.array([2, -1, 0, 2, 1, -1, 5], dtype=np.int32)  # 5 >= G: skipped too
    Msum = layout.size * 128
    xa = synth.normal_f32(121, (Msum, K))
    xb = synth.normal_f32(122, (G, N, K))
    a, sfa = q_tok(to_dev(xa))
    b, sfb = q_blk(to_dev(xb))
    d = sentinel_like((Msum, N))
    mg.m_grouped_fp8_gemm_nt_contiguous(a, b, sfa, sfb, d, to_dev(layout))
    torch.cuda.synchronize()
    ra, rsfa = oracle.per_token_cast_to_fp8(xa)
    rb, rsfb = oracle.per_block_cast_to_fp8(xb)
    ref_layout = np.where(layout < G, layout, -1)
    ref, written = oracle.m_grouped_fp8_gemm_nt_contiguous(ra, rb, rsfa, rsfb, ref_layout)
    got = to_host(d)
    assert np.all(got[~written] == SENTINEL_BF16)
    assert_bf16_close(got[written], ref[written], "contiguous small")


def test_contiguous_mixed_groups_in_one_tile():
    """Adjacent 128-row blocks of different groups (and a skipped one next
    to a computed one) in every position."""
    say("contiguous alternating groups")
    mg = _mg()
    G, N, K = 2, 256, 384
    layout = np.array([0, 1, 1, 0, -1, 1, 0, -1, -1, 1], dtype=np.int32)
    Msum = layout.size * 128
    xa = synth.normal_f32(123, (Msum, K))
    xb = synth.normal_f32(124, (G, N, K))
    a, sfa = q_tok(to_dev(xa))
    b, sfb = q_blk(to_dev(xb))
    d = sentinel_like((Msum, N))
    mg.m_grouped_fp8_gemm_nt_contiguous(a, b, sfa, sfb, d, to_dev(layout))
    torch.cuda.synchronize()
    ra, rsfa = oracle.per_token_cast_to_fp8(xa)
    rb, rsfb = oracle.per_block_cast_to_fp8(xb)
    ref, written = oracle.m_grouped_fp8_gemm_nt_contiguous(ra, rb, rsfa, rsfb, layout)
    got = to_host(d)
    assert np.all(got[~written] == SENTINEL_BF16)
    assert_bf16_close(got[written], ref[written], "contiguous alternating")


def test_contiguous_mixed_groups_256x256_tile():
    """Skipped blocks, out-of-range ids and tiles split between two groups on
    the 256 x 256 tile (32 blocks x 4096 columns: one whole round of tiles),
    compared in full."""
    say("contiguous mixed groups, 256 x 256 tile")
    mg = _mg()
    from moe_grouped_gemm_x128_amd import binding

    G, N, K = 3, 4096, 128
    layout = np.array([0, 1, 1, 0, -1, 1, 0, -1, -1, 1, 2, 2, 5, 2, 0, 0] * 2, dtype=np.int32)
    Msum = layout.size * 128
    c = binding.query_config(binding.DG_KIND_CONTIGUOUS, G, Msum, N, K)
    assert (c["block_m"], c["block_n"], c["block_n2"]) == (256, 256, 0)
    xa = synth.normal_f32(125, (Msum, K))
    xb = synth.normal_f32(126, (G, N, K))
    a, sfa = q_tok(to_dev(xa))
    b, sfb = q_blk(to_dev(xb))
    d = sentinel_like((Msum, N))
    mg.m_grouped_fp8_gemm_nt_contiguous(a, b, sfa, sfb, d, to_dev(layout))
    torch.cuda.synchronize()
    ra, rsfa = oracle.per_token_cast_to_fp8(xa)
    rb, rsfb = oracle.per_block_cast_to_fp8(xb)
    ref_layout = np.where(layout < G, layout, -1)
    ref, written = oracle.m_grouped_fp8_gemm_nt_contiguous(ra, rb, rsfa, rsfb, ref_layout)
    got = to_host(d)
    assert np.all(got[~written] == SENTINEL_BF16)
    assert_bf16_close(got[written], ref[written], "contiguous 256 x 256 tile")


@pytest.mark.parametrize("layout", [[0, 1, 1], [1, 1, 0, 0, 2], [-1, 2, 2]])
def test_contiguous_odd_block_counts(layout):
    """256-row tiles on an odd number of 128-row blocks: runs end on a
    single block, one of them the layout's last."""
    say(f"contiguous odd block count {layout}")
    mg = _mg()
    from moe_grouped_gemm_x128_amd import binding

    G, N, K = 3, 200, 256
    layout = np.array(layout, dtype=np.int32)
    Msum = layout.size * 128
    c = binding.query_config(binding.DG_KIND_CONTIGUOUS, G, Msum, N, K)
    assert c["block_m"] == 256
    xa = synth.normal_f32(129, (Msum, K))
    xb = synth.normal_f32(130, (G, N, K))
    a, sfa = q_tok(to_dev(xa))
    b, sfb = q_blk(to_dev(xb))
    d = sentinel_like((Msum, N))
    mg.m_grouped_fp8_gemm_nt_contiguous(a, b, sfa, sfb, d, to_dev(layout))
    torch.cuda.synchronize()
    ra, rsfa = oracle.per_token_cast_to_fp8(xa)
    rb, rsfb = oracle.per_block_cast_to_fp8(xb)
    ref, written = oracle.m_grouped_fp8_gemm_nt_contiguous(ra, rb, rsfa, rsfb, layout)
    got = to_host(d)
    assert np.all(got[~written] == SENTINEL_BF16)
    assert_bf16_close(got[written], ref[written], "contiguous odd block count")


def test_contiguous_long_runs_at_odd_offsets():
    """Runs of one group longer than 64 blocks (longer than a wave's part of
    the run-start scan), starting at odd block offsets, with odd lengths (a
    single-block tile at the run's end), next to skipped blocks."""
    say("contiguous long runs at odd offsets")
    mg = _mg()
    from moe_grouped_gemm_x128_amd import binding

    G, N, K = 3, 320, 256
    layout = np.array([1] + [0] * 151 + [2] * 3 + [-1] + [1] * 65 + [2] * 2 + [7] + [0] * 130, dtype=np.int32)
    Msum = layout.size * 128
    c = binding.query_config(binding.DG_KIND_CONTIGUOUS, G, Msum, N, K)
    assert c["block_m"] == 256 and c["grid"] == layout.size * -(-N // c["block_n"])
    xa = synth.normal_f32(127, (Msum, K))
    xb = synth.normal_f32(128, (G, N, K))
    a, sfa = q_tok(to_dev(xa))
    b, sfb = q_blk(to_dev(xb))
    d = sentinel_like((Msum, N))
    mg.m_grouped_fp8_gemm_nt_contiguous(a, b, sfa, sfb, d, to_dev(layout))
    torch.cuda.synchronize()
    ra, rsfa = oracle.per_token_cast_to_fp8(xa)
    rb, rsfb = oracle.per_block_cast_to_fp8(xb)
    ref_layout = np.where(layout < G, layout, -1)
    ref, written = oracle.m_grouped_fp8_gemm_nt_contiguous(ra, rb, rsfa, rsfb, ref_layout)
    got = to_host(d)
    assert np.all(got[~written] == SENTINEL_BF16)
    assert_bf16_close(got[written], ref[written], "contiguous long runs")


@pytest.mark.parametrize("dtype", ["fp8", "bf16"])
def test_contiguous_layout_longer_than_a_workgroup(dtype):
    """1100 blocks: the tile-start scan takes three passes over the layout
    (512 threads a pass), with runs crossing the pass boundaries at even and
    at odd offsets, a run covering a whole pass, and skipped blocks."""
    say(f"contiguous 1100-block layout {dtype}")
    mg = _mg()
    from moe_grouped_gemm_x128_amd import binding

    rng = np.random.default_rng(1100)
    runs = [(0, 3), (1, 508), (2, 2), (0, 1), (-1, 1), (1, 600), (2, 5)]  # 1120 blocks, cut to 1100
    layout = np.concatenate([np.full(n, g, dtype=np.int32) for g, n in runs])[:1100]
    layout[rng.choice(1100, 40, replace=False)] = -1
    G, N, K = 3, 136, 128
    Msum = layout.size * 128
    kind = binding.DG_KIND_CONTIGUOUS if dtype == "fp8" else binding.DG_KIND_BF16_CONTIGUOUS
    c = binding.query_config(kind, G, Msum, N, K)
    assert c["block_m"] == 256 and c["grid"] == 1100 * -(-N // c["block_n"])
    xa = synth.normal_f32(131, (Msum, K))
    xb = synth.normal_f32(132, (G, N, K))
    d = sentinel_like((Msum, N))
    if dtype == "fp8":
        a, sfa = q_tok(to_dev(xa))
        b, sfb = q_blk(to_dev(xb))
        mg.m_grouped_fp8_gemm_nt_contiguous(a, b, sfa, sfb, d, to_dev(layout))
        ra, rsfa = oracle.per_token_cast_to_fp8(xa)
        rb, rsfb = oracle.per_block_cast_to_fp8(xb)
        ref, written = oracle.m_grouped_fp8_gemm_nt_contiguous(ra, rb, rsfa, rsfb, layout)
    else:
        ab, bb = synth.bf16_bits_from_f32(xa), synth.bf16_bits_from_f32(xb)
        mg.m_grouped_bf16_gemm_nt_contiguous(to_dev(ab.view(np.int16)).view(torch.bfloat16),
                                             to_dev(bb.view(np.int16)).view(torch.bfloat16), d, to_dev(layout))
        ref, written = oracle.m_grouped_bf16_gemm_nt_contiguous(ab, bb, layout)
    torch.cuda.synchronize()
    got = to_host(d)
    assert np.all(got[~written] == SENTINEL_BF16)
    assert_bf16_close(got[written], ref[written], f"contiguous 1100-block layout {dtype}")


@pytest.mark.parametrize("nblk,block_m,run", [(8192, 256, 40), (8192, 256, 3), (8193, 128, 40)])
def test_contiguous_largest_tile_list(nblk, block_m, run):
    """The longest layout the 256-row tiles' LDS list holds (8192 blocks,
    16 scan passes; runs of 1..40 blocks, or of 1..3 so that the list holds
    about 5500 tiles), and one block more, which takes 128-row tiles: 5
    groups with skipped (-1) and out-of-range (>= G) ids; FP8 codes and
    scales drawn directly (every finite E4M3 magnitude), the whole output
    against the oracle."""
    say(f"contiguous largest tile list: {nblk} blocks, runs of 1..{run}")
    mg = _mg()
    from moe_grouped_gemm_x128_amd import binding

    G, N, K = 5, 64, 128
    rng = np.random.default_rng(8192 + nblk + run)
    ids, lens = rng.integers(-1, G + 1, size=nblk), rng.integers(1, run + 1, size=nblk)
    layout = np.repeat(ids, lens)[:nblk].astype(np.int32)
    M = nblk * 128
    c = binding.query_config(binding.DG_KIND_CONTIGUOUS, G, M, N, K)
    assert c["block_m"] == block_m
    if block_m == 256:
        assert c["grid"] == nblk * -(-N // c["block_n"])

    def codes(shape):
        v = rng.integers(0, 0x7F, size=shape, dtype=np.uint8)
        return v | (rng.integers(0, 2, size=shape, dtype=np.uint8) << np.uint8(7))

    ra, rb = codes((M, K)), codes((G, N, K))
    rsfa = rng.uniform(2.0 ** -10, 2.0 ** -6, size=(M, K // 128)).astype(np.float32)
    rsfb = rng.uniform(2.0 ** -10, 2.0 ** -6, size=(G, 1, K // 128)).astype(np.float32)
    d = sentinel_like((M, N))
    mg.m_grouped_fp8_gemm_nt_contiguous(to_dev(ra), to_dev(rb), to_dev(rsfa), to_dev(rsfb), d, to_dev(layout))
    torch.cuda.synchronize()
    ref, written = oracle.m_grouped_fp8_gemm_nt_contiguous(ra, rb, rsfa, rsfb, np.where(layout < G, layout, -1))
    got = to_host(d)
    assert np.all(got[~written] == SENTINEL_BF16)
    assert_bf16_close(got[written], ref[written], f"contiguous {nblk} blocks")


@pytest.mark.parametrize("si", [0, 1])
def test_contiguous_prefill_full_size_sampled(si):
    N, K = synth.CONTIG["shapes"][si]
    G, per = synth.CONTIG["G"], synth.CONTIG["rows_per_group"]
    Msum = G * per
    say(f"contiguous full size G={G} Msum={Msum} N={N} K={K}")
    mg = _mg()
    xa = synth.normal_f32(synth.CONTIG["seed_a"] + 10 * si, (Msum, K))
    xb_dev = torch.empty((G, N, K), dtype=torch.float32, device="cuda")
    xb_host = []
    for g, chunk in enumerate(synth.normal_f32_chunks(synth.CONTIG["seed_b"] + 10 * si, (G, N, K))):
        xb_dev[g].copy_(torch.from_numpy(chunk))
        xb_host.append(chunk)
    layout = synth.contiguous_layout(G, per)
    a, sfa = q_tok(to_dev(xa))
    b, sfb = q_blk(xb_dev)
    del xb_dev
    d = sentinel_like((Msum, N))
    mg.m_grouped_fp8_gemm_nt_contiguous(a, b, sfa, sfb, d, to_dev(layout))
    torch.cuda.synchronize()
    dh = to_host(d)
    rows = _sample_rows(Msum, 48, 31 + si)
    ra, rsfa = oracle.per_token_cast_to_fp8(xa[rows])
    for nb in _sample_col_blocks(N):
        cols = slice(nb * 128, min(N, nb * 128 + 128))
        for g in range(G):
            sel = (rows // per) == g
            if not sel.any():
                continue
            rb, rsfb = oracle.per_block_cast_to_fp8(xb_host[g][cols])
            ref = oracle.fp8_gemm_nt(ra[sel], rb, rsfa[sel], rsfb)
            assert_bf16_close(dh[rows[sel]][:, cols], ref, f"contiguous g={g} col block {nb}")


# ---------------------------------------------------------------------------
# masked grouped
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("ue8m0", [False, True])
def test_masked_small_sentinel_and_clamp(ue8m0):
    say(f"masked small ue8m0={ue8m0}")
    mg = _mg()
    G, max_m, N, K = 6, 160, 200, 256
    mm = np.array([0, 17, 160, 999, -3, 129], dtype=np.int32)
    xa = synth.normal_f32(131, (G, max_m, K))
    xb = synth.normal_f32(132, (G, N, K))
    a, sfa = q_tok(to_dev(xa), ue8m0)
    b, sfb = q_blk(to_dev(xb), ue8m0)
    if ue8m0:
        pa = torch.empty((G, max_m, 1), dtype=torch.int32, device="cuda")
        pb = torch.empty((G, 2, 1), dtype=torch.int32, device="cuda")
        mg.pack_ue8m0_to_int(sfa, pa)
        mg.pack_ue8m0_to_int(sfb, pb)
        sfa, sfb = pa, pb
    d = sentinel_like((G, max_m, N))
    mg.m_grouped_fp8_gemm_nt_masked(a, b, sfa, sfb, d, to_dev(mm), max_m)
    torch.cuda.synchronize()
    ra, rsfa = oracle.per_token_cast_to_fp8(xa, ue8m0)
    rb, rsfb = oracle.per_block_cast_to_fp8(xb, ue8m0)
    ref, written = oracle.m_grouped_fp8_gemm_nt_masked(ra, rb, rsfa, rsfb, mm, max_m)
    got = to_host(d)
    assert np.all(got[~written] == SENTINEL_BF16)
    assert_bf16_close(got[written], ref[written], "masked small")


@pytest.mark.parametrize("ue8m0", [False, True])
def test_masked_sentinel_and_clamp_256x256_tile(ue8m0):
    """masked_m of 0, within the first 128 rows (the waves of rows 128..255
    compute nothing), exactly 128, full, beyond max_m and negative, on the
    256 x 256 tile (16 experts x 4096 columns: one whole round)."""
    say(f"masked 256 x 256 tile ue8m0={ue8m0}")
    mg = _mg()
    from moe_grouped_gemm_x128_amd import binding

    G, max_m, N, K = 16, 256, 4096, 128
    mm = np.array([0, 17, 256, 999, -3, 129, 128, 200, 1, 255, 64, 130, 250, 16, 0, 192], dtype=np.int32)
    c = binding.query_config(binding.DG_KIND_MASKED, G, max_m, N, K)
    assert (c["block_m"], c["block_n"], c["block_n2"]) == (256, 256, 0)
    xa = synth.normal_f32(133, (G, max_m, K))
    xb = synth.normal_f32(134, (G, N, K))
    a, sfa = q_tok(to_dev(xa), ue8m0)
    b, sfb = q_blk(to_dev(xb), ue8m0)
    if ue8m0:
        pa = torch.empty((G, max_m, 1), dtype=torch.int32, device="cuda")
        pb = torch.empty((G, N // 128, 1), dtype=torch.int32, device="cuda")
        mg.pack_ue8m0_to_int(sfa, pa)
        mg.pack_ue8m0_to_int(sfb, pb)
        sfa, sfb = pa, pb
    d = sentinel_like((G, max_m, N))
    mg.m_grouped_fp8_gemm_nt_masked(a, b, sfa, sfb, d, to_dev(mm), max_m)
    torch.cuda.synchronize()
    ra, rsfa = oracle.per_token_cast_to_fp8(xa, ue8m0)
    rb, rsfb = oracle.per_block_cast_to_fp8(xb, ue8m0)
    ref, written = oracle.m_grouped_fp8_gemm_nt_masked(ra, rb, rsfa, rsfb, mm, max_m)
    got = to_host(d)
    assert np.all(got[~written] == SENTINEL_BF16)
    assert_bf16_close(got[written], ref[written], "masked 256 x 256 tile")


def test_masked_2d_views_and_all_zero():
    say("masked 2-D views, masked_m all zero then all max")
    mg = _mg()
    G, max_m, N, K = 3, 64, 128, 128
    xa = synth.normal_f32(141, (G * max_m, K))
    xb = synth.normal_f32(142, (G, N, K))
    a, sfa = q_tok(to_dev(xa))
    b, sfb = q_blk(to_dev(xb))
    d = sentinel_like((G * max_m, N))
    mg.m_grouped_fp8_gemm_nt_masked(a, b, sfa.contiguous(), sfb, d, to_dev(np.zeros(G, np.int32)), max_m)
    torch.cuda.synchronize()
    assert np.all(to_host(d) == SENTINEL_BF16)
    mg.m_grouped_fp8_gemm_nt_masked(a, b, sfa.contiguous(), sfb, d, to_dev(np.full(G, max_m, np.int32)), max_m)
    torch.cuda.synchronize()
    ra, rsfa = oracle.per_token_cast_to_fp8(xa)
    rb, rsfb = oracle.per_block_cast_to_fp8(xb)
    got = to_host(d).reshape(G, max_m, N)
    for g in range(G):
        ref = oracle.fp8_gemm_nt(ra[g * max_m:(g + 1) * max_m], rb[g], rsfa[g * max_m:(g + 1) * max_m], rsfb[g])
        assert_bf16_close(got[g], ref, f"masked full group {g}")


@pytest.mark.parametrize("si", [0, 1])
def test_masked_decode_full_size_sampled(si):
    N, K = synth.MASKED["shapes"][si]
    G, max_m = synth.MASKED["G"], synth.MASKED["max_m"]
    say(f"masked full size G={G} max_m={max_m} N={N} K={K}")
    mg = _mg()
    mm = synth.masked_m_decode(synth.MASKED["seed_m"], G)
    xa = synth.normal_f32(synth.MASKED["seed_a"] + 10 * si, (G, max_m, K))
    xb_dev = torch.empty((G, N, K), dtype=torch.float32, device="cuda")
    sample_groups = [0, 7, G - 1]
    xb_keep = {}
    for g, chunk in enumerate(synth.normal_f32_chunks(synth.MASKED["seed_b"] + 10 * si, (G, N, K))):
        xb_dev[g].copy_(torch.from_numpy(chunk))
        if g in sample_groups:
            xb_keep[g] = chunk
    a, sfa = q_tok(to_dev(xa))
    b, sfb = q_blk(xb_dev)
    del xb_dev
    d = sentinel_like((G, max_m, N))
    mg.m_grouped_fp8_gemm_nt_masked(a, b, sfa, sfb, d, to_dev(mm), max_m)
    torch.cuda.synchronize()
    dh = to_host(d)
    # rows at and beyond masked_m stay untouched in every group
    for g in range(G):
        assert np.all(dh[g, mm[g]:] == SENTINEL_BF16), g
    for g in sample_groups:
        v = int(mm[g])
        rows = _sample_rows(v, 24, 50 + g)
        ra, rsfa = oracle.per_token_cast_to_fp8(xa[g, rows])
        for nb in _sample_col_blocks(N):
            cols = slice(nb * 128, min(N, nb * 128 + 128))
            rb, rsfb = oracle.per_block_cast_to_fp8(xb_keep[g][cols])
            ref = oracle.fp8_gemm_nt(ra, rb, rsfa, rsfb)
            assert_bf16_close(dh[g, rows][:, cols], ref, f"masked g={g} col block {nb}")


# ---------------------------------------------------------------------------
# one B scale per row of B (the per-row b_sf of "DeepInside DeepGEMM",
# section 4): B quantized per token like A, sfb [N, K/128]
# ---------------------------------------------------------------------------

def _rowb_plan(kind, G, M, N, K):
    from moe_grouped_gemm_x128_amd import binding

    c = binding.query_config(getattr(binding, kind), G, M, N, K)
    assert c["block_n2"] == 0
    return c


@pytest.mark.parametrize("M,N,K", [(200, 300, 384), (128, 256, 512), (96, 100, 640), (4000, 4000, 256), (1, 130, 128),
                                   (4096, 2880, 256)])
@pytest.mark.parametrize("ue8m0", [False, True])
def test_dense_per_row_b_scales_full_compare(M, N, K, ue8m0):
    say(f"fp8_gemm_nt per-row B scales M={M} N={N} K={K} ue8m0={ue8m0}")
    mg = _mg()
    c = _rowb_plan("DG_KIND_DENSE_ROWB", 1, M, N, K)
    if M > 128:  # 192 x 192 tiles where one round of them costs less; 4096 x 2880 keeps 256 x 192
        assert (c["block_m"], c["block_n"]) == ((256, 192) if (M, N) == (4096, 2880) else (192, 192))
    xa = synth.normal_f32(191, (M, K))
    xb = synth.normal_f32(192, (N, K))
    a, sfa = q_tok(to_dev(xa), ue8m0)
    b, sfb = q_tok(to_dev(xb), ue8m0)  # [N, K/128], N-major view
    if ue8m0:
        pa = torch.empty((M, -(-K // 512)), dtype=torch.int32, device="cuda")
        pb = torch.empty((N, -(-K // 512)), dtype=torch.int32, device="cuda")
        mg.pack_ue8m0_to_int(sfa.contiguous(), pa)
        mg.pack_ue8m0_to_int(sfb.contiguous(), pb)
        dsa, dsb = pa, pb
    else:
        dsa, dsb = sfa, sfb.contiguous()  # A scales M-major, B scales K-major
    d = sentinel_like((M, N))
    mg.fp8_gemm_nt(a, b, dsa, dsb, None, d)
    torch.cuda.synchronize()
    ra, rsfa = oracle.per_token_cast_to_fp8(xa, ue8m0)
    rb, rsfb = oracle.per_token_cast_to_fp8(xb, ue8m0)
    assert np.array_equal(to_host(a), ra) and np.array_equal(to_host(b), rb)
    assert rsfb.shape == (N, K // 128)
    assert_bf16_close(to_host(d), oracle.fp8_gemm_nt(ra, rb, rsfa, rsfb), f"per-row B scales {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(160, 272, 768), (100, 300, 512), (64, 100, 384)])
def test_dense_per_row_b_scales_one_hot_bit_exact(M, N, K):
    """One-hot B with power-of-two per-row scales: every output is
    sfa[m, kb] * sfb[n, kb] * A[m, kn[n]] exactly; pins the per-lane column
    scale indexing of each tile."""
    say(f"fp8_gemm_nt per-row B scales one-hot M={M} N={N} K={K}")
    mg = _mg()
    _rowb_plan("DG_KIND_DENSE_ROWB", 1, M, N, K)
    rng = np.random.default_rng(193)
    a = (rng.integers(0, 0x7E, size=(M, K)) | (rng.integers(0, 2, size=(M, K)) << 7)).astype(np.uint8)
    kn = rng.integers(0, K, size=N)
    b = np.zeros((N, K), dtype=np.uint8)
    b[np.arange(N), kn] = 0x38
    sfa = np.exp2(rng.integers(-6, 6, size=(M, K // 128))).astype(np.float32)
    sfb = np.exp2(rng.integers(-6, 6, size=(N, K // 128))).astype(np.float32)
    d = sentinel_like((M, N))
    mg.fp8_gemm_nt(to_dev(a), to_dev(b), to_dev(sfa), to_dev(sfb), None, d)
    torch.cuda.synchronize()
    ref = oracle.fp8_gemm_nt(a, b, sfa, sfb)
    ref_bits = to_host(torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16))
    got = to_host(d)
    bad = np.argwhere(got != ref_bits)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}"


def test_dense_pages_example_per_row_scales_and_c():
    """The pages' dense call as printed: M = N = K = 4096, A and B cast from
    normal values to E4M3, random-normal FP32 scales (either sign) of shape
    [m, k/128] and [n, k/128], a BF16 accumulate input C; D = C + A . B^T,
    compared on sampled rows."""
    say("fp8_gemm_nt pages example 4096^3, per-row B scales, C")
    mg = _mg()
    M = N = K = 4096
    _rowb_plan("DG_KIND_DENSE_ROWB", 1, M, N, K)
    a = torch.from_numpy(synth.normal_f32(194, (M, K))).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    b = torch.from_numpy(synth.normal_f32(195, (N, K))).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    sfa = synth.normal_f32(196, (M, K // 128))
    sfb = synth.normal_f32(197, (N, K // 128))
    cbits = synth.bf16_bits_from_f32(synth.normal_f32(198, (M, N)) * np.float32(16.0))
    c = to_dev(cbits.view(np.int16)).view(torch.bfloat16)
    d = sentinel_like((M, N))
    mg.fp8_gemm_nt(to_dev(a), to_dev(b), to_dev(sfa), to_dev(sfb), c, d)
    torch.cuda.synchronize()
    rows = _sample_rows(M, 24, 199)
    ref = oracle.fp8_gemm_nt(a[rows], b, sfa[rows], sfb, c=oracle.bf16_decode(cbits[rows]))
    assert_bf16_close(to_host(d)[rows], ref, "pages example")


@pytest.mark.parametrize("ue8m0", [False, True])
def test_grouped_per_row_b_scales(ue8m0):
    """Masked (with clamping and untouched rows) and contiguous (with skipped
    and mixed blocks) grouped GEMMs with sfb [G, N, K/128]."""
    say(f"grouped per-row B scales ue8m0={ue8m0}")
    mg = _mg()
    G, max_m, N, K = 4, 160, 200, 512
    mm = np.array([0, 17, 160, 999], dtype=np.int32)
    xa = synth.normal_f32(201, (G, max_m, K))
    xb = synth.normal_f32(202, (G, N, K))
    a, sfa = q_tok(to_dev(xa), ue8m0)
    b, sfb = q_tok(to_dev(xb), ue8m0)  # [G, N, K/128]
    if ue8m0:
        pa = torch.empty((G, max_m, 1), dtype=torch.int32, device="cuda")
        pb = torch.empty((G, N, 1), dtype=torch.int32, device="cuda")
        mg.pack_ue8m0_to_int(sfa, pa)
        mg.pack_ue8m0_to_int(sfb, pb)
        dsa, dsb = pa, pb
    else:
        dsa, dsb = sfa, sfb
    d = sentinel_like((G, max_m, N))
    mg.m_grouped_fp8_gemm_nt_masked(a, b, dsa, dsb, d, to_dev(mm), max_m)
    torch.cuda.synchronize()
    ra, rsfa = oracle.per_token_cast_to_fp8(xa, ue8m0)
    rb, rsfb = oracle.per_token_cast_to_fp8(xb, ue8m0)
    ref, written = oracle.m_grouped_fp8_gemm_nt_masked(ra, rb, rsfa, rsfb, mm, max_m)
    got = to_host(d)
    assert np.all(got[~written] == SENTINEL_BF16)
    assert_bf16_close(got[written], ref[written], "masked per-row B scales")

    layout = np.array([2, -1, 0, 3, 1, 3], dtype=np.int32)
    Msum = layout.size * 128
    xg = synth.normal_f32(203, (Msum, K))
    ag, sfg = q_tok(to_dev(xg), ue8m0)
    if ue8m0:
        pg = torch.empty((Msum, 1), dtype=torch.int32, device="cuda")
        mg.pack_ue8m0_to_int(sfg.contiguous(), pg)
        dsg = pg
    else:
        dsg = sfg
    dg = sentinel_like((Msum, N))
    mg.m_grouped_fp8_gemm_nt_contiguous(ag, b, dsg, dsb, dg, to_dev(layout))
    torch.cuda.synchronize()
    rg, rsfg = oracle.per_token_cast_to_fp8(xg, ue8m0)
    refc, wc = oracle.m_grouped_fp8_gemm_nt_contiguous(rg, rb, rsfg, rsfb, layout)
    gotc = to_host(dg)
    assert np.all(gotc[~wc] == SENTINEL_BF16)
    assert_bf16_close(gotc[wc], refc[wc], "contiguous per-row B scales")


@pytest.mark.gpu
def test_masked_scales_m_major_per_expert():
    """A's scales stored M-major per expert ([G, K/128, max_m] seen through a
    transposed view, the layout of the masked decode benchmark), written by
    the per-token cast: the same codes and scales as the K-major layout, and
    the masked GEMM's output bit-identical to the K-major run and within the
    oracle's tolerance; rows past masked_m untouched."""
    say("masked, A scales M-major per expert")
    mg = _mg()
    G, max_m, N, K = 4, 256, 512, 512
    KB = K // 128
    mm = np.array([200, 256, 1, 129], dtype=np.int32)
    xa = synth.normal_f32(811, (G, max_m, K))
    xb = synth.normal_f32(812, (G, N, K))
    xa_d = to_dev(xa)
    a1 = torch.empty((G, max_m, K), dtype=torch.uint8, device="cuda")
    s1 = torch.empty((G, max_m, KB), dtype=torch.float32, device="cuda")
    a2 = torch.empty_like(a1)
    s2 = torch.empty((G, KB, max_m), dtype=torch.float32, device="cuda").transpose(1, 2)
    assert s2.stride() == (KB * max_m, 1, max_m)
    mg.per_token_cast_to_fp8(xa_d, a1, s1)
    mg.per_token_cast_to_fp8(xa_d, a2, s2)
    b, sfb = q_blk(to_dev(xb), False)
    d1 = sentinel_like((G, max_m, N))
    d2 = sentinel_like((G, max_m, N))
    mmd = to_dev(mm)
    mg.m_grouped_fp8_gemm_nt_masked(a1, b, s1, sfb, d1, mmd, max_m)
    mg.m_grouped_fp8_gemm_nt_masked(a2, b, s2, sfb, d2, mmd, max_m)
    torch.cuda.synchronize()
    assert torch.equal(a1, a2) and torch.equal(s1, s2)
    assert torch.equal(d1.view(torch.int16), d2.view(torch.int16))  # bit patterns (the sentinel is a NaN)
    ra, rsfa = oracle.per_token_cast_to_fp8(xa)
    rb, rsfb = oracle.per_block_cast_to_fp8(xb)
    ref, written = oracle.m_grouped_fp8_gemm_nt_masked(ra, rb, rsfa, rsfb, mm, max_m)
    got = to_host(d2)
    assert np.all(got[~written] == SENTINEL_BF16)
    assert_bf16_close(got[written], ref[written], "masked, M-major A scales")
