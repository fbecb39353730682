"""GPU parity of the dense FP8 GEMM with FP8 output (fp8_gemm_nt_fp8_out):
the GEMM and the per-token FP8 cast of its BF16 result in one kernel.

Two checks per case:
  * bit for bit against the library's own two-step path, fp8_gemm_nt into a
    BF16 tensor followed by per_token_cast_to_fp8 of that tensor (q and the
    scales must be the same bytes);
  * against the float64 oracle (oracle.fp8_gemm_nt_fp8_out) within the
    tolerance derived below: the dequantized output q * s must lie within
    the E4M3 rounding of the GEMM's own tolerance band around the oracle's
    exact D, and every block scale must be the oracle's block maximum / 448
    up to that band (UE8M0: the same power of two, or its neighbour where
    the block maximum lies within the band of a power of two).

Tolerance: the BF16 D of the device lies within g = 1e-2 rms(D) + 2^-8 |D|
of the exact D (the tolerance of every BF16 GEMM output here); the E4M3
code of x / s is within half a step of it: 2^-4 |x| for normal codes, 2^-10
s below 2^-6 s.  Hence |q s - D| <= 2^-4 (|D| + g) + 2^-10 s + g."""

import numpy as np
import pytest

import oracle
from moe_grouped_gemm_x128_amd import synth

from helpers import ABS_RMS_TOL, REL_TOL, say, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _mg():
    import moe_grouped_gemm_x128_amd as mg

    return mg


def _e4m3(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


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


def two_step(a, b, sfa, sfb, c, ue8m0):
    """fp8_gemm_nt into BF16, then per_token_cast_to_fp8 of that tensor."""
    mg = _mg()
    M, N = a.shape[0], b.shape[0]
    # row stride padded to 16 bytes, as the quantizer reads its input rows
    d = torch.empty((M, -(-N // 8) * 8), dtype=torch.bfloat16, device="cuda")[:, :N]
    mg.fp8_gemm_nt(a, b, sfa, sfb, c, d)
    q = torch.empty((M, -(-N // 16) * 16), dtype=torch.uint8, device="cuda")[:, :N]  # 4-byte aligned rows
    sf = torch.empty((M, -(-N // 128)), dtype=torch.float32, device="cuda")
    mg.per_token_cast_to_fp8(d, q, sf, ue8m0)
    return q, sf


def out_buffers(M, N, q_pad=0, sf_m_major=False):
    """q [M, N] (row stride N rounded up to 4 bytes, plus q_pad) filled with
    0x55 and sfq [M, ceil(N/128)] filled with NaN, so any element left
    unwritten shows."""
    nnb = -(-N // 128)
    qbuf = torch.full((M, -(-N // 4) * 4 + q_pad), 0x55, dtype=torch.uint8, device="cuda")
    q = qbuf[:, :N]
    if sf_m_major:
        sfq = torch.full((nnb, M), float("nan"), dtype=torch.float32, device="cuda").t()
    else:
        sfq = torch.full((M, nnb), float("nan"), dtype=torch.float32, device="cuda")
    return qbuf, q, sfq


def assert_fp8_out_close(q, sf, D, ue8m0, what):
    """q uint8 [M, N] and sf float32 [M, nnb] from the device; D float64, the
    oracle's exact D (C included)."""
    M, N = D.shape
    assert q.shape == (M, N) and sf.shape == (M, -(-N // 128)), what
    assert np.all(np.isfinite(sf)) and np.all(sf > 0), f"{what}: scale not written or not positive"
    s = np.repeat(sf.astype(np.float64), 128, axis=1)[:, :N]
    deq = _e4m3(q) * s
    assert np.all(np.isfinite(deq)), f"{what}: NaN code"
    rms = float(np.sqrt(np.mean(D * D))) if D.size else 0.0
    g = ABS_RMS_TOL * rms + REL_TOL * np.abs(D)
    bound = 2.0 ** -4 * (np.abs(D) + g) + 2.0 ** -10 * s + g
    bad = np.abs(deq - D) > bound
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} values outside tolerance; first {i}: "
                             f"q*s {deq[i]:.6g} D {D[i]:.6g} s {s[i]:.4g}")
    for kb in range(sf.shape[1]):
        blk = D[:, kb * 128:(kb + 1) * 128]
        amax = np.maximum(np.abs(blk).max(axis=1), 1e-4)
        band = ABS_RMS_TOL * rms + 2 * REL_TOL * amax
        if not ue8m0:
            assert np.all(np.abs(sf[:, kb] * 448.0 - amax) <= band), f"{what}: block {kb} scale"
        else:
            lo, hi = (amax - band) / 448.0, (amax + band) / 448.0
            p = sf[:, kb].astype(np.float64)
            assert np.all(np.frexp(p)[0] == 0.5), f"{what}: block {kb} scale not a power of two"
            # the smallest power of two >= some value in [lo, hi]
            assert np.all((p >= lo) & (p / 2 < hi)), f"{what}: block {kb} UE8M0 scale"


def run_case(M, N, K, c_kind=None, ue8m0=False, in_ue8m0=False, q_pad=0, sf_m_major=False, seed=0, rowb=False):
    """rowb: one B scale per row of B ([N, K/128]) instead of 128 x 128 blocks."""
    mg = _mg()
    xa = synth.normal_f32(900 + seed, (M, K))
    xb = synth.normal_f32(901 + seed, (N, K))
    a, sfa = q_tok(to_dev(xa), in_ue8m0)
    if rowb:
        b, sfb = q_tok(to_dev(xb), in_ue8m0)
        sfb = sfb.contiguous()
    else:
        b, sfb = q_blk(to_dev(xb), in_ue8m0)
    c, cref = None, None
    if c_kind is not None:
        xc = synth.normal_f32(902 + seed, (M, N)) * np.float32(4.0)
        if c_kind == "f32":
            cbuf = torch.zeros((M, N + 4), dtype=torch.float32, device="cuda")
            cbuf[:, :N] = to_dev(xc)
            c = cbuf[:, :N]
            cref = xc.astype(np.float64)
        else:
            c = to_dev(xc).to(torch.bfloat16)
            cref = c.float().cpu().numpy().astype(np.float64)
    qbuf, q, sfq = out_buffers(M, N, q_pad, sf_m_major)
    mg.fp8_gemm_nt_fp8_out(a, b, sfa, sfb, c, q, sfq, ue8m0)
    q2, sf2 = two_step(a, b, sfa, sfb, c, ue8m0)
    torch.cuda.synchronize()
    qh, sfh = to_host(q), to_host(sfq)
    # bit for bit against the two-step path
    diff = np.argwhere(qh != to_host(q2))
    assert diff.size == 0, f"{diff.shape[0]} codes differ from GEMM -> cast, first {diff[:4].tolist()}"
    assert np.array_equal(sfh.view(np.uint32), to_host(sf2).view(np.uint32)), "scales differ from GEMM -> cast"
    if qbuf.shape[1] > N:
        assert np.all(to_host(qbuf[:, N:]) == 0x55), "row padding of q written"
    # the oracle, on its own quantized operands
    ra, rsfa = oracle.per_token_cast_to_fp8(xa, in_ue8m0)
    rb, rsfb = (oracle.per_token_cast_to_fp8 if rowb else oracle.per_block_cast_to_fp8)(xb, in_ue8m0)
    assert np.array_equal(to_host(a), ra) and np.array_equal(to_host(b), rb)
    D = oracle.fp8_gemm_nt(ra, rb, rsfa, rsfb, cref)
    assert_fp8_out_close(qh, sfh, D, ue8m0, f"fp8 out {M}x{N}x{K} c={c_kind} ue8m0={ue8m0}")
    return qh, sfh


# (M, N, K): 128 x 128 tile (N <= 128), 128 x 256 tile (rows <= 128), 256 x
# 256 tile (rows > 128); ragged N ending inside a 16-column lane group (word
# stores) and inside a word (byte stores); waves whose rows all lie past M
# (M = 50 on the 128-row tiles, M = 300 on the 256-row tile).
SHAPES = [(64, 100, 256), (50, 128, 384), (1, 130, 128), (50, 2112, 512), (128, 256, 384), (96, 1000, 640),
          (200, 300, 384), (300, 70, 256), (257, 2050, 256), (4000, 4000, 256)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_fp8_out_shapes(M, N, K):
    say(f"fp8_gemm_nt_fp8_out M={M} N={N} K={K}")
    run_case(M, N, K, seed=M % 7)


@pytest.mark.parametrize("M,N,K", [(64, 100, 256), (96, 1000, 640), (200, 300, 384), (4000, 4000, 256)])
@pytest.mark.parametrize("c_kind", ["bf16", "f32"])
def test_fp8_out_accumulate_c(M, N, K, c_kind):
    say(f"fp8_gemm_nt_fp8_out accumulate M={M} N={N} K={K} c={c_kind}")
    run_case(M, N, K, c_kind=c_kind, seed=3)


@pytest.mark.parametrize("M,N,K", [(64, 100, 256), (96, 1000, 640), (300, 2050, 512)])
@pytest.mark.parametrize("in_ue8m0", [False, True])
def test_fp8_out_ue8m0_output_scales(M, N, K, in_ue8m0):
    say(f"fp8_gemm_nt_fp8_out UE8M0 output scales M={M} N={N} K={K} UE8M0 inputs={in_ue8m0}")
    run_case(M, N, K, ue8m0=True, in_ue8m0=in_ue8m0, seed=5)


@pytest.mark.parametrize("q_pad,sf_m_major", [(16, False), (4, True), (12, False)])
def test_fp8_out_strided_outputs(q_pad, sf_m_major):
    """q with a padded row stride (N + 16: 16-byte aligned rows, 16-byte
    stores; N + 4 and N + 12: 4-byte aligned rows, word stores) and M-major
    scales; the padding stays untouched."""
    for M, N, K in ((64, 208, 256), (260, 528, 256)):
        say(f"fp8_gemm_nt_fp8_out strided q_pad={q_pad} sf_m_major={sf_m_major} M={M} N={N} K={K}")
        run_case(M, N, K, q_pad=q_pad, sf_m_major=sf_m_major, seed=9)


def test_fp8_out_packed_ue8m0_input_scales():
    """Input scales packed four to an int32, as fp8_gemm_nt takes them."""
    mg = _mg()
    M, N, K = 300, 520, 1024
    say(f"fp8_gemm_nt_fp8_out packed UE8M0 inputs M={M} N={N} K={K}")
    xa = synth.normal_f32(921, (M, K))
    xb = synth.normal_f32(922, (N, K))
    a, sfa = q_tok(to_dev(xa), True)
    b, sfb = q_blk(to_dev(xb), True)
    pa = torch.empty((M, K // 512), dtype=torch.int32, device="cuda")
    pb = torch.empty((-(-N // 128), K // 512), dtype=torch.int32, device="cuda")
    mg.pack_ue8m0_to_int(sfa.contiguous(), pa)
    mg.pack_ue8m0_to_int(sfb, pb)
    _, q, sfq = out_buffers(M, N)
    mg.fp8_gemm_nt_fp8_out(a, b, pa, pb, None, q, sfq, False)
    q2, sf2 = two_step(a, b, pa, pb, None, False)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(q), to_host(q2)) and np.array_equal(to_host(sfq), to_host(sf2))
    ra, rsfa = oracle.per_token_cast_to_fp8(xa, True)
    rb, rsfb = oracle.per_block_cast_to_fp8(xb, True)
    D = oracle.fp8_gemm_nt(ra, rb, rsfa, rsfb)
    assert_fp8_out_close(to_host(q), to_host(sfq), D, False, "fp8 out, packed UE8M0 inputs")


@pytest.mark.parametrize("i", [0, 3])
def test_fp8_out_full_size_sampled(i):
    """A DeepSeek-V3 dense shape at M = 4096: the whole output bit for bit
    against GEMM -> cast, and sampled rows (every column) against the
    oracle."""
    N, K = synth.DENSE_V3_SHAPES[i]
    M = synth.DENSE_V3_M
    say(f"fp8_gemm_nt_fp8_out full size M={M} N={N} K={K}")
    mg = _mg()
    sa, sb = synth.dense_v3_seeds(i)
    xa = synth.normal_f32(sa, (M, K))
    xb = synth.normal_f32(sb, (N, K))
    a, sfa = q_tok(to_dev(xa))
    b, sfb = q_blk(to_dev(xb))
    _, q, sfq = out_buffers(M, N)
    mg.fp8_gemm_nt_fp8_out(a, b, sfa, sfb, None, q, sfq, False)
    q2, sf2 = two_step(a, b, sfa, sfb, None, False)
    torch.cuda.synchronize()
    qh, sfh = to_host(q), to_host(sfq)
    assert np.array_equal(qh, to_host(q2)) and np.array_equal(sfh, to_host(sf2))
    rows = np.unique(np.concatenate([np.random.default_rng(60 + i).choice(M, 16, replace=False), [0, M - 1]]))
    ra, rsfa = oracle.per_token_cast_to_fp8(xa[rows])
    assert np.array_equal(to_host(a)[rows], ra)
    rb, rsfb = oracle.per_block_cast_to_fp8(xb)
    D = oracle.fp8_gemm_nt(ra, rb, rsfa, rsfb)
    assert_fp8_out_close(qh[rows], sfh[rows], D, False, f"fp8 out full size {M}x{N}x{K}")


def test_fp8_out_graph_replay():
    """Captured once and replayed three times with the inputs rewritten in
    between; every replay equals an eager call on the same inputs."""
    mg = _mg()
    M, N, K = 512, 2048, 1024
    say(f"fp8_gemm_nt_fp8_out graph replay M={M} N={N} K={K}")
    xb = to_dev(synth.normal_f32(931, (N, K)))
    b, sfb = q_blk(xb)
    a = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sfa = torch.empty((K // 128, M), dtype=torch.float32, device="cuda").t()
    _, q, sfq = out_buffers(M, N)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            mg.fp8_gemm_nt_fp8_out(a, b, sfa, sfb, None, q, sfq, True, stream=stream)
    torch.cuda.current_stream().wait_stream(stream)
    for r in range(3):
        xa = to_dev(synth.normal_f32(940 + r, (M, K)))
        a2, sfa2 = q_tok(xa)
        a.copy_(a2)
        sfa.copy_(sfa2)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _, qe, sfe = out_buffers(M, N)
        mg.fp8_gemm_nt_fp8_out(a, b, sfa, sfb, None, qe, sfe, True)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(q), to_host(qe)) and np.array_equal(to_host(sfq), to_host(sfe)), f"replay {r}"


# one B scale per row of B: the 256 x 128 tile above 128 rows, the 128-row
# tiles below; FP32 and UE8M0 input scales, C, both output scale formats
@pytest.mark.parametrize("M,N,K", [(300, 520, 512), (4096, 2048, 256), (200, 130, 384), (64, 300, 384),
                                   (100, 100, 256)])
@pytest.mark.parametrize("in_ue8m0,ue8m0,c_kind", [(False, False, None), (True, True, "bf16"), (False, True, "f32")])
def test_fp8_out_per_row_b_scales(M, N, K, in_ue8m0, ue8m0, c_kind):
    from moe_grouped_gemm_x128_amd import binding

    say(f"fp8_gemm_nt_fp8_out per-row B scales M={M} N={N} K={K} in_ue8m0={in_ue8m0} ue8m0={ue8m0} c={c_kind}")
    plan = binding.query_config(binding.DG_KIND_DENSE_FP8_OUT_ROWB, 1, M, N, K)
    if M > 128:
        assert (plan["block_m"], plan["block_n"]) == (256, 128), plan
    run_case(M, N, K, c_kind=c_kind, ue8m0=ue8m0, in_ue8m0=in_ue8m0, seed=40, rowb=True)
