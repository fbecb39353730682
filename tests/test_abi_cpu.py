"""The C-ABI library loads, exports every entry point include/dgmi.h
declares, and rejects malformed descriptors on the host before any launch.
No compute call is made here (no GPU needed): every call below fails
validation, which returns before touching the device."""

import ctypes
import os
import re
import subprocess

import pytest
import torch

from moe_grouped_gemm_x128_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dgmi.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libdgmi.so is not built (python -m moe_grouped_gemm_x128_amd.build)")
    return binding.load_library()


def test_header_declares_expected_entry_points():
    assert _declared() == sorted(binding.ENTRY_POINTS)


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in _declared():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_bf16_gemm_validation_errors(lib):
    D = binding.describe
    M, N, K = 128, 64, 128
    a, b, d = _t((M, K), torch.bfloat16), _t((N, K), torch.bfloat16), _t((M, N), torch.bfloat16)

    def dense(a, b, c, d):
        return lib.bf16_gemm_nt(ctypes.byref(D(a)), ctypes.byref(D(b)), ctypes.byref(D(c)) if c is not None else None,
                                ctypes.byref(D(d)), None)

    assert dense(a.float(), b, None, d) == binding.DG_INVALID_ARG          # dtype
    assert dense(a, _t((N, K + 64), torch.bfloat16), None, d) == binding.DG_INVALID_ARG  # K mismatch
    assert dense(a, b, None, _t((M, N + 1), torch.bfloat16)) == binding.DG_INVALID_ARG  # d shape
    assert dense(_t((M, 96), torch.bfloat16), _t((N, 96), torch.bfloat16), None, d) == binding.DG_UNSUPPORTED  # K % 64
    assert dense(a, b, _t((M, N), torch.int32), d) == binding.DG_INVALID_ARG  # c dtype
    assert dense(a, b, None, _t((M, N), torch.int32)) == binding.DG_INVALID_ARG  # d dtype (BF16 or F32)
    dmis = D(_t((M, N), torch.float32))
    dmis.data += 2  # F32 d not 4-byte aligned
    assert lib.bf16_gemm_nt(ctypes.byref(D(a)), ctypes.byref(D(b)), None, ctypes.byref(dmis), None) \
        == binding.DG_INVALID_ARG
    assert "aligned" in binding.last_error()
    lay = _t((2,), torch.int32)
    bg = _t((3, N, K), torch.bfloat16)
    dg = _t((256, N), torch.bfloat16)

    def contig(a, b, d, layout):
        return lib.m_grouped_bf16_gemm_nt_contiguous(ctypes.byref(D(a)), ctypes.byref(D(b)), ctypes.byref(D(d)),
                                                     ctypes.byref(D(layout)) if layout is not None else None, None)

    assert contig(_t((256, K), torch.bfloat16), bg, dg, None) == binding.DG_INVALID_ARG  # no layout
    assert contig(_t((200, K), torch.bfloat16), bg, _t((200, N), torch.bfloat16), lay) == binding.DG_INVALID_ARG  # Msum % 128
    assert contig(_t((256, K), torch.bfloat16), bg, dg, _t((3,), torch.int32)) == binding.DG_INVALID_ARG  # layout length
    assert contig(_t((256, K), torch.bfloat16), _t((N, K), torch.bfloat16), dg, lay) == binding.DG_INVALID_ARG  # b rank
    # an F32 d is taken (past validation the CPU build's launch fails: no GPU here)
    assert contig(_t((256, K), torch.bfloat16), bg, _t((256, N), torch.float32), lay) not in (binding.DG_UNSUPPORTED,
                                                                                           binding.DG_INVALID_ARG)
    # accumulate forms: c with d's shape (masked: per group), BF16 or F32, not overlapping d partly
    ag = _t((256, K), torch.bfloat16)

    def contig_acc(c, d=dg):
        return lib.m_grouped_bf16_gemm_nt_contiguous_acc(ctypes.byref(D(ag)), ctypes.byref(D(bg)), ctypes.byref(D(c)),
                                                         ctypes.byref(D(d)), ctypes.byref(D(lay)), None)

    assert contig_acc(_t((256, N + 1), torch.bfloat16)) == binding.DG_INVALID_ARG  # c shape
    assert contig_acc(_t((256, N), torch.int32)) == binding.DG_INVALID_ARG  # c dtype
    big = _t((257, N), torch.bfloat16)
    assert contig_acc(big[1:], d=big[:256]) == binding.DG_INVALID_ARG  # partial overlap of c and d
    assert "overlaps" in binding.last_error()
    assert contig_acc(dg) not in (binding.DG_UNSUPPORTED, binding.DG_INVALID_ARG)  # in place: taken
    max_m = 64
    am, dm, mm = _t((3, max_m, K), torch.bfloat16), _t((3, max_m, N), torch.float32), _t((3,), torch.int32)

    def masked_acc(c):
        return lib.m_grouped_bf16_gemm_nt_masked_acc(ctypes.byref(D(am)), ctypes.byref(D(bg)), ctypes.byref(D(c)),
                                                     ctypes.byref(D(dm)), ctypes.byref(D(mm)), max_m, None)

    assert masked_acc(_t((2, max_m, N), torch.float32)) == binding.DG_INVALID_ARG  # groups
    assert masked_acc(_t((3, max_m, N + 8), torch.float32)[..., :N]) not in (binding.DG_UNSUPPORTED,
                                                                           binding.DG_INVALID_ARG)  # own strides
    assert lib.m_grouped_bf16_gemm_nt_masked_acc(ctypes.byref(D(am)), ctypes.byref(D(bg)), ctypes.byref(D(dm)),
                                                 ctypes.byref(D(dm)), None, max_m, None) == binding.DG_INVALID_ARG


def test_query_config_is_a_pure_function_of_shapes(lib):
    c = binding.query_config(binding.DG_KIND_DENSE, 1, 4096, 2112, 7168)
    assert c == binding.query_config(binding.DG_KIND_DENSE, 1, 4096, 2112, 7168)
    assert c["grid"] == -(-4096 // c["block_m"]) * -(-c["n_split"] // c["block_n"])
    m = binding.query_config(binding.DG_KIND_MASKED, 32, 256, 4096, 7168)
    assert m["grid"] == 32 * -(-256 // m["block_m"]) * -(-m["n_split"] // m["block_n"])
    b = binding.query_config(binding.DG_KIND_BF16_MASKED, 64, 128, 7168, 2048)
    assert b["grid"] == 64 * -(-128 // b["block_m"]) * -(-b["n_split"] // b["block_n"])
    bd = binding.query_config(binding.DG_KIND_BF16_DENSE, 1, 4096, 7168, 2048)
    assert bd["grid"] == -(-4096 // bd["block_m"]) * -(-bd["n_split"] // bd["block_n"])
    assert bd["grid2"] == (-(-4096 // bd["block_m"]) * -(-(7168 - bd["n_split"]) // bd["block_n2"]) if bd["block_n2"] else 0)
    c = binding.query_config(binding.DG_KIND_CONTIGUOUS, 4, 32768, 4096, 7168)
    bc = binding.query_config(binding.DG_KIND_BF16_CONTIGUOUS, 4, 32768, 4096, 7168)
    tiles = -(-32768 // c["block_m"]) * -(-4096 // c["block_n"])
    # 256-row contiguous tiles: one workgroup per 128-row block and column
    # tile (at most one tile starts at each block)
    assert c["grid"] == ((32768 // 128) * 16 if c["block_m"] == 256 else tiles) and bc["grid"] == c["grid"]
    c = binding.query_config(binding.DG_KIND_CONTIGUOUS, 4, 33152, 4096, 7168)  # 259 blocks
    assert c["block_m"] == 256 and c["grid"] == 259 * 16
    # past 8192 blocks the tile list would not fit: 128-row tiles
    for kind in (binding.DG_KIND_CONTIGUOUS, binding.DG_KIND_BF16_CONTIGUOUS):
        assert binding.query_config(kind, 4, 8192 * 128, 4096, 7168)["block_m"] == 256
        big = binding.query_config(kind, 4, 8193 * 128, 4096, 7168)
        assert big["block_m"] == 128 and big["grid"] == 8193 * -(-4096 // big["block_n"])
    with pytest.raises(binding.DgmiError):
        binding.query_config(12, 1, 1, 1, 1)  # no such kind


@pytest.mark.parametrize("M,N,tile", [
    (4096, 7168, (256, 256, 512)),  # above 128 rows: 256 x 256, whatever fills the last round
    (4096, 2112, (256, 256, 512)),
    (129, 4096, (256, 256, 512)),
    (128, 4096, (128, 256, 512)),  # up to 128 rows: the 128-row tiles
    (64, 128, (128, 128, 256)),
    (1, 100, (128, 128, 256)),
])
def test_fp8_out_plan(lib, M, N, tile):
    # the FP8-output GEMM uses only the tiles whose waves cover 64 columns, one launch
    c = binding.query_config(binding.DG_KIND_DENSE_FP8_OUT, 1, M, N, 7168)
    assert (c["block_m"], c["block_n"], c["threads"]) == tile
    assert c["n_split"] == N and c["block_n2"] == 0 and c["grid2"] == 0
    assert c["grid"] == -(-M // tile[0]) * -(-N // tile[1])
    # one B scale per row: the 256 x 128 tile above 128 rows (the 256 x 256
    # tile has no registers for the per-lane column scales)
    r = binding.query_config(binding.DG_KIND_DENSE_FP8_OUT_ROWB, 1, M, N, 7168)
    want = (256, 128, 512) if M > 128 else tile
    assert (r["block_m"], r["block_n"], r["threads"]) == want
    assert r["grid"] == -(-M // want[0]) * -(-N // want[1])


@pytest.mark.parametrize("N,K,fp8_plan,bf16_plan", [
    # 144 tiles of 256 x 256 fill 56% of one round: FP8 242 of 192 x 192,
    # BF16 176 of 256 x 192
    (2112, 7168, (192, 192, 2112, 0), (192, 192, 2112, 0)),
    (24576, 1536, (256, 256, 24576, 0), (256, 256, 24576, 0)),    # 6 whole rounds
    # 1.75 rounds: BF16 splits into 256 tiles of 256 x 256, then 256 of
    # 256 x 192; the FP8 kernel gains nothing from it (power-limited clock)
    (7168, 16384, (256, 256, 7168, 0), (256, 256, 4096, 192)),
    (4096, 7168, (256, 256, 4096, 0), (256, 256, 4096, 0)),        # one whole round
    (7168, 2048, (256, 256, 7168, 0), (256, 256, 7168, 0)),        # too few K-slices to pay for a second launch
    (2880, 256, (256, 192, 2880, 0), (256, 192, 2880, 0)),         # 240 tiles of 256 x 192: one round
])
def test_launch_plan_of_the_dense_v3_shapes(lib, N, K, fp8_plan, bf16_plan):
    """The launch plan fills whole rounds of one workgroup per compute unit
    (256): one launch of the 256 x 256, 256 x 192 or (dense FP8) 192 x 192
    tile, or (BF16) columns [0, n_split) on the first and [n_split, N) on the
    second."""
    for kind, plan in ((binding.DG_KIND_DENSE, fp8_plan), (binding.DG_KIND_BF16_DENSE, bf16_plan)):
        block_m, block_n, n_split, block_n2 = plan
        c = binding.query_config(kind, 1, 4096, N, K)
        assert (c["block_m"], c["block_n"], c["n_split"], c["block_n2"]) == (block_m, block_n, n_split, block_n2)
        assert c["grid"] == -(-4096 // block_m) * -(-n_split // block_n)
        assert c["grid2"] == (16 * -(-(N - n_split) // block_n2) if block_n2 else 0)
        assert c["lds_bytes"] <= 160 * 1024 and c["lds_bytes2"] <= 160 * 1024


def test_launch_plan_of_the_grouped_shapes(lib):
    # masked decode, 32 experts x 256 rows: whole rounds of 256 x 256 at
    # N = 4096; at N = 7168 (3.5 rounds, 16 K-slices) a split does not pay
    m = binding.query_config(binding.DG_KIND_MASKED, 32, 256, 4096, 7168)
    assert (m["block_n"], m["n_split"], m["block_n2"], m["grid"]) == (256, 4096, 0, 512)
    m = binding.query_config(binding.DG_KIND_MASKED, 32, 256, 7168, 2048)
    assert (m["block_n"], m["n_split"], m["block_n2"], m["grid"], m["grid2"]) == (256, 7168, 0, 896, 0)
    # contiguous prefill: whole rounds of 256 x 256 (a workgroup per 128-row
    # block and column tile, those past the listed tiles exit)
    for N in (4096, 7168):
        c = binding.query_config(binding.DG_KIND_CONTIGUOUS, 4, 32768, N, 7168)
        assert (c["block_n"], c["n_split"], c["block_n2"], c["grid"]) == (256, N, 0, 256 * N // 256)
    # rows <= 128: one launch of a 128-row tile
    s = binding.query_config(binding.DG_KIND_MASKED, 64, 128, 7168, 2048)
    assert (s["block_m"], s["n_split"], s["block_n2"], s["grid2"]) == (128, 7168, 0, 0)


def _t(shape, dtype, stride=None):
    t = torch.empty(shape, dtype=dtype)
    if stride is not None:
        t = torch.empty_strided(shape, stride, dtype=dtype)
    return t


def _call_dense(lib, a, b, sfa, sfb, d, c=None):
    D = binding.describe
    return lib.fp8_gemm_nt(ctypes.byref(D(a)), ctypes.byref(D(b)), ctypes.byref(D(sfa)), ctypes.byref(D(sfb)),
                           ctypes.byref(D(c)) if c is not None else None, ctypes.byref(D(d)), None)


def test_dense_validation_errors(lib):
    M, N, K = 128, 256, 512
    a = _t((M, K), torch.uint8)
    b = _t((N, K), torch.uint8)
    sfa = _t((M, K // 128), torch.float32)
    sfb = _t((N // 128, K // 128), torch.float32)
    d = _t((M, N), torch.bfloat16)
    # wrong dtype of d (BF16 or F32 only)
    assert _call_dense(lib, a, b, sfa, sfb, _t((M, N), torch.int32)) == binding.DG_INVALID_ARG
    assert "dtype" in binding.last_error()
    # F32 d: 4-byte aligned
    D = binding.describe
    f32buf = torch.empty((M, N + 1), dtype=torch.float32)
    dmis = D(f32buf[:, :N])
    dmis.data += 2
    assert lib.fp8_gemm_nt(ctypes.byref(D(a)), ctypes.byref(D(b)), ctypes.byref(D(sfa)), ctypes.byref(D(sfb)), None,
                           ctypes.byref(dmis), None) == binding.DG_INVALID_ARG
    assert "aligned" in binding.last_error()
    # K mismatch
    assert _call_dense(lib, a, _t((N, K + 128), torch.uint8), sfa, sfb, d) == binding.DG_INVALID_ARG
    # wrong scale shape (neither one per 128x128 block nor one per row)
    assert _call_dense(lib, a, b, sfa, _t((N // 128 + 1, K // 128), torch.float32), d) == binding.DG_INVALID_ARG
    # mixed scale formats
    assert _call_dense(lib, a, b, sfa, _t((2, 1), torch.int32), d) == binding.DG_INVALID_ARG
    # one B scale per row: N rows (any other count is rejected), same format as sfa
    assert _call_dense(lib, a, b, sfa, _t((N + 1, K // 128), torch.float32), d) == binding.DG_INVALID_ARG
    assert _call_dense(lib, a, b, sfa, _t((N - 1, K // 128), torch.float32), d) == binding.DG_INVALID_ARG
    assert _call_dense(lib, a, b, sfa, _t((N, K // 128 + 1), torch.float32), d) == binding.DG_INVALID_ARG
    assert _call_dense(lib, a, b, _t((M, 1), torch.int32), _t((N, 2), torch.int32), d) == binding.DG_INVALID_ARG
    # non-unit inner stride
    assert _call_dense(lib, a.t(), b, sfa, sfb, d) == binding.DG_INVALID_ARG
    # K not a multiple of 128 -> unsupported
    a2, b2 = _t((M, 200), torch.uint8), _t((N, 200), torch.uint8)
    assert _call_dense(lib, a2, b2, _t((M, 2), torch.float32), _t((2, 2), torch.float32), d) == binding.DG_UNSUPPORTED
    # accumulate input: wrong shape, wrong dtype, partial overlap with d
    assert _call_dense(lib, a, b, sfa, sfb, d, c=_t((M, N + 1), torch.bfloat16)) == binding.DG_INVALID_ARG
    assert _call_dense(lib, a, b, sfa, sfb, d, c=_t((M, N), torch.int32)) == binding.DG_INVALID_ARG
    big = _t((M + 1, N), torch.bfloat16)
    assert _call_dense(lib, a, b, sfa, sfb, big[1:], c=big[:-1]) == binding.DG_INVALID_ARG
    # output aliasing an input
    alias = torch.empty(M * K, dtype=torch.uint8)
    a3 = alias.view(M, K)
    d3 = alias.view(torch.bfloat16)[: M * N].view(M, N) if M * K * 1 >= M * N * 2 else None
    if d3 is not None:
        assert _call_dense(lib, a3, b, sfa, sfb, d3) == binding.DG_INVALID_ARG
    # misaligned operand rows
    ab = _t((M, K + 8), torch.uint8)[:, :K]
    assert _call_dense(lib, ab, b, sfa, sfb, d) == binding.DG_INVALID_ARG
    assert "aligned" in binding.last_error()
    # a row stride whose 256-row tile would overflow the kernels' 32-bit offsets
    wide = _t((2, K), torch.uint8, stride=(1 << 23, 1))
    assert _call_dense(lib, wide, b, _t((2, K // 128), torch.float32), sfb, _t((2, N), torch.bfloat16)) == binding.DG_UNSUPPORTED
    assert "row strides" in binding.last_error()


def test_mn_major_validation_errors(lib):
    """fp8_gemm_nn / _tn / _tt: stored operands row-major; an MN-major operand
    needs rows % 16 == 0, a K-row stride of at least its rows that is a
    multiple of 16 with K x stride below 2^31, block scales and a BF16 d."""
    D = binding.describe
    M, N, K = 128, 256, 512
    a, a_st = _t((M, K), torch.uint8), _t((K, M), torch.uint8)
    b, b_st = _t((N, K), torch.uint8), _t((K, N), torch.uint8)
    sfa = _t((M, K // 128), torch.float32)
    sfb = _t((N // 128, K // 128), torch.float32)
    d = _t((M, N), torch.bfloat16)

    def call(name, a, b, sfb=sfb, d=d, sfa=sfa):
        return getattr(lib, name)(ctypes.byref(D(a)), ctypes.byref(D(b)), ctypes.byref(D(sfa)), ctypes.byref(D(sfb)),
                                  None, ctypes.byref(D(d)), None)

    # stored operands that are not row-major
    assert call("fp8_gemm_nn", a, b_st.t()) == binding.DG_INVALID_ARG
    assert call("fp8_gemm_tt", a_st.t(), b) == binding.DG_INVALID_ARG
    # rows not a multiple of 16
    a20 = _t((K, 120), torch.uint8)
    assert call("fp8_gemm_tn", a20, b_st, sfa=_t((120, K // 128), torch.float32),
                d=_t((120, N), torch.bfloat16)) == binding.DG_UNSUPPORTED
    assert "multiple of 16" in binding.last_error()
    # one B scale per row and an F32 d are taken (past validation the CPU
    # build's launch fails: no GPU here)
    assert call("fp8_gemm_nn", a, b_st, sfb=_t((N, K // 128), torch.float32)) not in (binding.DG_UNSUPPORTED,
                                                                                   binding.DG_INVALID_ARG)
    assert call("fp8_gemm_nn", a, b_st, d=_t((M, N), torch.float32)) not in (binding.DG_UNSUPPORTED,
                                                                          binding.DG_INVALID_ARG)
    # K-row stride below the row count, and not a multiple of 16
    short = _t((K, N), torch.uint8, stride=(N - 16, 1))
    assert call("fp8_gemm_nn", a, short) == binding.DG_UNSUPPORTED
    # an operand spanning 2^31 bytes or more (descriptor only: K = 8192 K-rows 2^18 bytes apart)
    Kb = 8192
    big = D(b_st)
    big.shape[0], big.stride[0] = Kb, 1 << 18
    ab = _t((M, Kb), torch.uint8)
    rc = lib.fp8_gemm_nn(ctypes.byref(D(ab)), ctypes.byref(big), ctypes.byref(D(_t((M, Kb // 128), torch.float32))),
                         ctypes.byref(D(_t((N // 128, Kb // 128), torch.float32))), None, ctypes.byref(D(d)), None)
    assert rc == binding.DG_UNSUPPORTED and "2^31" in binding.last_error()
    odd = _t((K, N + 8), torch.uint8)[:, :N]
    assert call("fp8_gemm_nn", a, odd) == binding.DG_INVALID_ARG
    assert "aligned" in binding.last_error()
    # shape mismatches
    assert call("fp8_gemm_tn", a_st, _t((K + 128, N), torch.uint8)) == binding.DG_INVALID_ARG
    assert call("fp8_gemm_tt", _t((K, M + 16), torch.uint8), b) == binding.DG_INVALID_ARG


def test_masked_validation_errors(lib):
    G, max_m, N, K = 4, 64, 256, 256
    D = binding.describe
    a = _t((G, max_m, K), torch.uint8)
    b = _t((G, N, K), torch.uint8)
    sfa = _t((G, max_m, K // 128), torch.float32)
    sfb = _t((G, N // 128, K // 128), torch.float32)
    d = _t((G, max_m, N), torch.bfloat16)
    mm = _t((G,), torch.int32)

    def call(a=a, b=b, sfa=sfa, sfb=sfb, d=d, mm=mm, max_m=max_m):
        return lib.m_grouped_fp8_gemm_nt_masked(ctypes.byref(D(a)), ctypes.byref(D(b)), ctypes.byref(D(sfa)),
                                                ctypes.byref(D(sfb)), ctypes.byref(D(d)),
                                                ctypes.byref(D(mm)) if mm is not None else None, max_m, None)

    assert call(mm=None) == binding.DG_INVALID_ARG
    assert call(mm=_t((G + 1,), torch.int32)) == binding.DG_INVALID_ARG
    assert call(mm=_t((G,), torch.float32)) == binding.DG_INVALID_ARG
    assert call(max_m=max_m + 1) == binding.DG_INVALID_ARG
    assert call(d=_t((G, max_m, N + 8), torch.bfloat16)) == binding.DG_INVALID_ARG
    # accumulate form: c with d's shape, BF16 or F32, not overlapping d partly
    def acc(c, d=d):
        return lib.m_grouped_fp8_gemm_nt_masked_acc(ctypes.byref(D(a)), ctypes.byref(D(b)), ctypes.byref(D(sfa)),
                                                    ctypes.byref(D(sfb)), ctypes.byref(D(c)), ctypes.byref(D(d)),
                                                    ctypes.byref(D(mm)), max_m, None)

    assert acc(_t((G, max_m, N + 1), torch.bfloat16)) == binding.DG_INVALID_ARG
    assert acc(_t((G, max_m, N), torch.int32)) == binding.DG_INVALID_ARG
    assert acc(_t((G + 1, max_m, N), torch.bfloat16)) == binding.DG_INVALID_ARG
    big = _t((G, max_m + 1, N), torch.bfloat16)
    assert acc(big[:, 1:], d=big[:, :-1]) == binding.DG_INVALID_ARG
    assert call(max_m=-1) == binding.DG_INVALID_ARG


def test_contiguous_validation_errors(lib):
    G, Msum, N, K = 2, 384, 256, 256
    D = binding.describe
    a = _t((Msum, K), torch.uint8)
    b = _t((G, N, K), torch.uint8)
    sfa = _t((Msum, 2), torch.float32)
    sfb = _t((G, 2, 2), torch.float32)
    d = _t((Msum, N), torch.bfloat16)

    def call(layout, a=a, sfa=sfa, d=d):
        return lib.m_grouped_fp8_gemm_nt_contiguous(ctypes.byref(D(a)), ctypes.byref(D(b)), ctypes.byref(D(sfa)),
                                                    ctypes.byref(D(sfb)), ctypes.byref(D(d)),
                                                    ctypes.byref(D(layout)) if layout is not None else None, None)

    assert call(None) == binding.DG_INVALID_ARG
    assert call(_t((Msum // 128 + 1,), torch.int32)) == binding.DG_INVALID_ARG
    a2, sfa2, d2 = _t((200, K), torch.uint8), _t((200, 2), torch.float32), _t((200, N), torch.bfloat16)
    assert call(_t((1,), torch.int32), a=a2, sfa=sfa2, d=d2) == binding.DG_INVALID_ARG


def test_quantizer_and_pack_validation_errors(lib):
    D = binding.describe
    x = _t((4, 256), torch.float32)
    q = _t((4, 256), torch.uint8)
    sf = _t((4, 2), torch.float32)
    assert lib.per_token_cast_to_fp8(ctypes.byref(D(x)), ctypes.byref(D(q)), ctypes.byref(D(_t((4, 3), torch.float32))), 0, None) == binding.DG_INVALID_ARG
    assert lib.per_token_cast_to_fp8(ctypes.byref(D(x)), ctypes.byref(D(_t((4, 255), torch.uint8))), ctypes.byref(D(sf)), 0, None) == binding.DG_INVALID_ARG
    assert lib.per_block_cast_to_fp8(ctypes.byref(D(x)), ctypes.byref(D(q)), ctypes.byref(D(sf)), 0, None) == binding.DG_INVALID_ARG
    assert lib.per_token_cast_to_fp8(ctypes.byref(D(x.to(torch.int32))), ctypes.byref(D(q)), ctypes.byref(D(sf)), 0, None) == binding.DG_INVALID_ARG
    s = _t((3, 10), torch.float32)
    assert lib.pack_ue8m0_to_int(ctypes.byref(D(s)), ctypes.byref(D(_t((3, 2), torch.int32))), None, None) == binding.DG_INVALID_ARG
    assert lib.pack_ue8m0_to_int(ctypes.byref(D(s)), ctypes.byref(D(_t((3, 3), torch.float32))), None, None) == binding.DG_INVALID_ARG
    assert lib.pack_ue8m0_to_int(None, ctypes.byref(D(_t((3, 3), torch.int32))), None, None) == binding.DG_INVALID_ARG


def test_launch_plan_with_per_row_b_scales(lib):
    # above 128 rows the 256 x 192 tile, one launch, in every form; 128-row
    # tiles below
    for kind, G in ((binding.DG_KIND_DENSE_ROWB, 1), (binding.DG_KIND_CONTIGUOUS_ROWB, 4), (binding.DG_KIND_MASKED_ROWB, 4)):
        c = binding.query_config(kind, G, 4096, 7168, 7168)
        assert (c["block_m"], c["block_n"], c["block_n2"], c["n_split"]) == (256, 192, 0, 7168)
    s = binding.query_config(binding.DG_KIND_DENSE_ROWB, 1, 64, 4096, 7168)
    assert (s["block_m"], s["block_n2"]) == (128, 0)


def test_empty_problems_return_ok_without_a_launch(lib):
    """Zero rows, columns or groups are legal and launch nothing (here, with
    no GPU, any launch would fail and return LAUNCH_FAILED)."""
    D = binding.describe
    K = 256
    f32, u8, bf, i32 = torch.float32, torch.uint8, torch.bfloat16, torch.int32
    # dense FP8: M = 0, then N = 0
    assert _call_dense(lib, _t((0, K), u8), _t((64, K), u8), _t((0, 2), f32), _t((1, 2), f32), _t((0, 64), bf)) == 0
    assert _call_dense(lib, _t((8, K), u8), _t((0, K), u8), _t((8, 2), f32), _t((0, 2), f32), _t((8, 0), bf)) == 0
    # masked FP8 and BF16 with no groups, and with max_m = 0
    for G, max_m in ((0, 64), (3, 0)):
        assert lib.m_grouped_fp8_gemm_nt_masked(
            ctypes.byref(D(_t((G, max_m, K), u8))), ctypes.byref(D(_t((G, 128, K), u8))),
            ctypes.byref(D(_t((G, max_m, 2), f32))), ctypes.byref(D(_t((G, 1, 2), f32))),
            ctypes.byref(D(_t((G, max_m, 128), bf))), ctypes.byref(D(_t((G,), i32))), max_m, None) == 0
        assert lib.m_grouped_bf16_gemm_nt_masked(
            ctypes.byref(D(_t((G, max_m, K), bf))), ctypes.byref(D(_t((G, 128, K), bf))),
            ctypes.byref(D(_t((G, max_m, 128), bf))), ctypes.byref(D(_t((G,), i32))), max_m, None) == 0
    # contiguous FP8 and BF16 with no rows
    assert lib.m_grouped_fp8_gemm_nt_contiguous(
        ctypes.byref(D(_t((0, K), u8))), ctypes.byref(D(_t((2, 128, K), u8))), ctypes.byref(D(_t((0, 2), f32))),
        ctypes.byref(D(_t((2, 1, 2), f32))), ctypes.byref(D(_t((0, 128), bf))), ctypes.byref(D(_t((0,), i32))),
        None) == 0
    assert lib.m_grouped_bf16_gemm_nt_contiguous(
        ctypes.byref(D(_t((0, K), bf))), ctypes.byref(D(_t((2, 128, K), bf))), ctypes.byref(D(_t((0, 128), bf))),
        ctypes.byref(D(_t((0,), i32))), None) == 0
    # dense BF16 with M = 0
    assert lib.bf16_gemm_nt(ctypes.byref(D(_t((0, K), bf))), ctypes.byref(D(_t((64, K), bf))), None,
                            ctypes.byref(D(_t((0, 64), bf))), None) == 0
    # quantizers with no rows, pack with no scales
    assert lib.per_token_cast_to_fp8(ctypes.byref(D(_t((0, K), f32))), ctypes.byref(D(_t((0, K), u8))),
                                     ctypes.byref(D(_t((0, 2), f32))), 0, None) == 0
    assert lib.per_block_cast_to_fp8(ctypes.byref(D(_t((0, K), f32))), ctypes.byref(D(_t((0, K), u8))),
                                     ctypes.byref(D(_t((0, 2), f32))), 1, None) == 0
    assert lib.pack_ue8m0_to_int(ctypes.byref(D(_t((3, 0), f32))), ctypes.byref(D(_t((3, 0), i32))), None, None) == 0
    assert lib.pack_ue8m0_to_int(ctypes.byref(D(_t((0, 8), f32))), ctypes.byref(D(_t((0, 2), i32))), None, None) == 0


def _call_fp8_out(lib, a, b, sfa, sfb, q, sfq, c=None, ue8m0=0):
    D = binding.describe
    r = lambda t: ctypes.byref(D(t)) if t is not None else None  # noqa: E731
    return lib.fp8_gemm_nt_fp8_out(r(a), r(b), r(sfa), r(sfb), r(c), r(q), r(sfq), ue8m0, None)


def test_fp8_out_validation_errors(lib):
    M, N, K = 128, 256, 512
    f32, u8, bf = torch.float32, torch.uint8, torch.bfloat16
    a, b = _t((M, K), u8), _t((N, K), u8)
    sfa, sfb = _t((M, K // 128), f32), _t((N // 128, K // 128), f32)
    q, sfq = _t((M, N), u8), _t((M, N // 128), f32)
    # missing outputs
    assert _call_fp8_out(lib, a, b, sfa, sfb, None, sfq) == binding.DG_INVALID_ARG
    assert _call_fp8_out(lib, a, b, sfa, sfb, q, None) == binding.DG_INVALID_ARG
    # q must be E4M3 [M, N]
    assert _call_fp8_out(lib, a, b, sfa, sfb, _t((M, N), bf), sfq) == binding.DG_INVALID_ARG
    assert _call_fp8_out(lib, a, b, sfa, sfb, _t((M, N + 1), u8), sfq) == binding.DG_INVALID_ARG
    # q rows 4-byte aligned
    assert _call_fp8_out(lib, a, b, sfa, sfb, _t((M, N + 2), u8)[:, :N], sfq) == binding.DG_INVALID_ARG
    assert "4-byte" in binding.last_error()
    # sfq F32 [M, ceil(N/128)]
    assert _call_fp8_out(lib, a, b, sfa, sfb, q, _t((M, N // 128 + 1), f32)) == binding.DG_INVALID_ARG
    assert _call_fp8_out(lib, a, b, sfa, sfb, q, _t((M, N // 128), bf)) == binding.DG_INVALID_ARG
    assert _call_fp8_out(lib, a, b, sfa, sfb, q, _t((M + 1, N // 128), f32)) == binding.DG_INVALID_ARG
    # one B scale per row is taken (past validation the CPU build's launch fails: no GPU here)
    assert _call_fp8_out(lib, a, b, sfa, _t((N, K // 128), f32), q, sfq) not in (binding.DG_UNSUPPORTED,
                                                                              binding.DG_INVALID_ARG)
    # sfq overlapping q, c overlapping q
    buf = torch.empty(M * N + 64, dtype=u8)
    q2 = buf[: M * N].view(M, N)
    sfq2 = buf[:8].view(f32)[: M * (N // 128)].view(M, N // 128) if M * N // 128 * 4 <= 8 else None
    alias = torch.empty(M * N, dtype=u8)
    assert _call_fp8_out(lib, a, b, sfa, sfb, alias.view(M, N), alias[: M * (N // 128) * 4].view(f32).view(M, N // 128)) \
        == binding.DG_INVALID_ARG
    assert "overlaps" in binding.last_error()
    cbuf = torch.empty(M * N, dtype=bf)
    assert _call_fp8_out(lib, a, b, sfa, sfb, cbuf.view(u8)[: M * N].view(M, N), sfq, c=cbuf.view(M, N)) \
        == binding.DG_INVALID_ARG
    del q2, sfq2
    # c of the wrong shape
    assert _call_fp8_out(lib, a, b, sfa, sfb, q, sfq, c=_t((M, N - 1), bf)) == binding.DG_INVALID_ARG
    # K not a multiple of 128
    assert _call_fp8_out(lib, _t((M, 200), u8), _t((N, 200), u8), _t((M, 2), f32), _t((2, 2), f32), q, sfq) \
        == binding.DG_UNSUPPORTED
    # empty problems launch nothing
    assert _call_fp8_out(lib, _t((0, K), u8), b, _t((0, 4), f32), sfb, _t((0, N), u8), _t((0, 2), f32)) == 0
    assert _call_fp8_out(lib, a, _t((0, K), u8), sfa, _t((0, 4), f32), _t((M, 0), u8), _t((M, 0), f32)) == 0


def test_moe_dispatch_and_combine_validation_errors(lib):
    D = binding.describe
    f32, bf, u8, i32 = torch.float32, torch.bfloat16, torch.uint8, torch.int32
    T, K, k, G, max_m, N = 16, 256, 4, 8, 32, 128

    def dispatch(x=None, topk=None, a=None, sfa=None, mm=None, slot=None, src=None):
        x = _t((T, K), f32) if x is None else x
        topk = _t((T, k), i32) if topk is None else topk
        a = _t((G, max_m, K), u8) if a is None else a
        sfa = _t((G, max_m, K // 128), f32) if sfa is None else sfa
        mm = _t((G,), i32) if mm is None else mm
        slot = _t((T, k), i32) if slot is None else slot
        src = _t((G, max_m), i32) if src is None else src
        return lib.moe_dispatch_masked_fp8(*(ctypes.byref(D(t)) for t in (x, topk, a, sfa, mm, slot, src)), 0, None)

    assert dispatch(x=_t((T, K), i32)) == binding.DG_INVALID_ARG  # x dtype
    assert dispatch(topk=_t((T, k), f32)) == binding.DG_INVALID_ARG  # topk dtype
    assert dispatch(topk=_t((T + 1, k), i32)) == binding.DG_INVALID_ARG  # T mismatch
    assert dispatch(a=_t((G, max_m, K + 128), u8)) == binding.DG_INVALID_ARG  # K mismatch
    assert dispatch(sfa=_t((G, max_m, 1), f32)) == binding.DG_INVALID_ARG  # scale blocks
    assert dispatch(mm=_t((G + 1,), i32)) == binding.DG_INVALID_ARG  # masked_m length
    assert dispatch(slot=_t((T, k + 1), i32)) == binding.DG_INVALID_ARG  # slot shape
    assert dispatch(src=_t((G, max_m - 1), i32)) == binding.DG_INVALID_ARG  # src shape
    assert dispatch(topk=_t((T, 2 * k), i32)[:, :k]) == binding.DG_INVALID_ARG  # not contiguous
    assert "contiguous" in binding.last_error()
    assert dispatch(x=_t((T, K + 2), f32)[:, :K]) == binding.DG_INVALID_ARG  # x rows not 16-B aligned
    shared = torch.empty(G * max_m + 64, dtype=i32)
    assert dispatch(mm=shared[:G], src=shared[:G * max_m].view(G, max_m)) == binding.DG_INVALID_ARG  # overlap
    assert "overlaps" in binding.last_error()
    # no experts: nothing to do
    assert dispatch(a=_t((0, max_m, K), u8), sfa=_t((0, max_m, 2), f32), mm=_t((0,), i32), src=_t((0, max_m), i32)) == 0

    def combine(d=None, slot=None, w=None, y=None):
        d = _t((G, max_m, N), bf) if d is None else d
        slot = _t((T, k), i32) if slot is None else slot
        w = _t((T, k), f32) if w is None else w
        y = _t((T, N), bf) if y is None else y
        return lib.moe_combine(*(ctypes.byref(D(t)) for t in (d, slot, w, y)), None)

    assert combine(d=_t((G, max_m, N), f32)) == binding.DG_INVALID_ARG  # d dtype
    assert combine(w=_t((T, k), bf)) == binding.DG_INVALID_ARG  # weights dtype
    assert combine(w=_t((T, k + 1), f32)) == binding.DG_INVALID_ARG  # weights shape
    assert combine(y=_t((T, N + 1), bf)) == binding.DG_INVALID_ARG  # y shape
    assert combine(slot=_t((T, 2 * k), i32)[:, :k]) == binding.DG_INVALID_ARG  # not contiguous
    buf = torch.empty(G * max_m * N, dtype=bf)
    assert combine(d=buf.view(G, max_m, N), y=buf[:T * N].view(T, N)) == binding.DG_INVALID_ARG  # y overlaps d
    # no tokens: nothing to do
    assert combine(slot=_t((0, k), i32), w=_t((0, k), f32), y=_t((0, N), bf)) == 0


def test_moe_dispatch_contiguous_validation_errors(lib):
    D = binding.describe
    f32, u8, i32 = torch.float32, torch.uint8, torch.int32
    T, K, k, G, Mcap = 16, 256, 4, 8, 1024

    def dispatch(x=None, topk=None, a=None, sfa=None, lay=None, cnt=None, slot=None, align=128):
        x = _t((T, K), f32) if x is None else x
        topk = _t((T, k), i32) if topk is None else topk
        a = _t((Mcap, K), u8) if a is None else a
        sfa = _t((Mcap, K // 128), f32) if sfa is None else sfa
        lay = _t((Mcap // 128,), i32) if lay is None else lay
        cnt = _t((G,), i32) if cnt is None else cnt
        slot = _t((T, k), i32) if slot is None else slot
        return lib.moe_dispatch_contiguous_fp8(*(ctypes.byref(D(t)) for t in (x, topk, a, sfa, lay, cnt, slot)), align, 0,
                                               None)

    assert dispatch(a=_t((1000, K), u8), sfa=_t((1000, 2), f32), lay=_t((7,), i32)) == binding.DG_INVALID_ARG  # Mcap % 128
    assert "multiple of 128" in binding.last_error()
    assert dispatch(lay=_t((Mcap // 128 + 1,), i32)) == binding.DG_INVALID_ARG  # layout length
    assert dispatch(align=192) == binding.DG_INVALID_ARG  # granule
    assert "align" in binding.last_error()
    assert dispatch(sfa=_t((Mcap, 1), f32)) == binding.DG_INVALID_ARG  # scale blocks
    assert dispatch(cnt=_t((G,), f32)) == binding.DG_INVALID_ARG  # counts dtype
    assert dispatch(slot=_t((T, k + 1), i32)) == binding.DG_INVALID_ARG  # slot shape
    assert dispatch(a=_t((Mcap, K + 128), u8)) == binding.DG_INVALID_ARG  # K mismatch
    shared = torch.empty(Mcap, dtype=i32)
    assert dispatch(lay=shared[:Mcap // 128], cnt=shared[:G]) == binding.DG_INVALID_ARG  # overlap
    # nothing to route into and no experts: nothing to do
    assert dispatch(a=_t((0, K), u8), sfa=_t((0, 2), f32), lay=_t((0,), i32), cnt=_t((0,), i32)) == 0
