"""Seeded random sweep of the GEMM calls against the oracle.

Each case draws its shape and options from a generator seeded by its own
index, so a failing case names everything needed to rerun it alone:
  * ragged M and N across the launch plans (128-row tiles, 192 x 192,
    256 x 192 and 256 x 256 tiles);
  * K from one 128-wide block (64-wide for BF16) to many;
  * FP32, UE8M0 and packed UE8M0 scales, block or per-row B scales;
  * BF16 or F32 outputs with or without an accumulate input C (also in
    place), padded output rows;
  * random masked_m (clamped and negative values included) and random
    contiguous layouts (runs of one group, skipped blocks, ids past G);
  * the per-token and per-block casts and the MoE dispatch and combine on
    random shapes and routings.
Inputs carry a power-of-two magnitude per row (per 128-row block for
block-scaled B) and per 128-column block, so a scale read from the wrong
row or block shows.  The GEMMs are those of "DeepGEMM: clean and efficient
FP8 GEMM kernels" (dense, contiguous and masked grouped forms) and
"DeepInside DeepGEMM" (layouts, output dtypes, the accumulate form);
tolerances are those of the other parity tests."""

import numpy as np
import pytest

import oracle
from moe_grouped_gemm_x128_amd import synth

from helpers import (SENTINEL_BF16, assert_bf16_close, assert_f32_close, fp8_bound_terms, fp8_rounding_count, say,
                     to_dev, to_host)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SWEEP_SEED = 20261203
FORMS = {"dense": 1, "mn": 2, "masked": 3, "contig": 4, "bf16_dense": 5, "bf16_masked": 6, "bf16_contig": 7,
         "fp8_out": 8, "cast": 9, "moe": 10}


def _mg():
    import moe_grouped_gemm_x128_amd as mg

    return mg


def _rng(form, i):
    return np.random.default_rng([SWEEP_SEED, FORMS[form], i])


def _loguni(rng, lo, hi):
    """An integer in [lo, hi], log-uniformly distributed."""
    v = int(round(float(np.exp(rng.uniform(np.log(lo), np.log(hi + 1))))))
    return min(hi, max(lo, v))


def _pick(rng, options):
    return options[int(rng.integers(len(options)))]


def _spread(x, rng, rows_per_mag=1):
    """x [.., R, K] times 2^e, e uniform in [-6, 6], one e per row (or per
    rows_per_mag rows) and per 128 columns; exact in float32."""
    R, K = x.shape[-2], x.shape[-1]
    lead = x.shape[:-2]
    e = rng.integers(-6, 7, size=lead + (-(-R // rows_per_mag), -(-K // 128)))
    e = np.repeat(np.repeat(e, rows_per_mag, axis=-2)[..., :R, :], 128, axis=-1)[..., :K]
    return (x * np.exp2(e)).astype(np.float32)


def _inputs(rng, seed, shape, rows_per_mag=1):
    return _spread(synth.normal_f32(seed, shape), rng, rows_per_mag)


def _out(shape, kind, pad):
    """Output buffer with `pad` extra columns per row; BF16 filled with the
    sentinel, F32 with NaN; returns (buffer, view)."""
    full = shape[:-1] + (shape[-1] + pad,)
    if kind == "f32":
        buf = torch.full(full, float("nan"), dtype=torch.float32, device="cuda")
    else:
        buf = torch.full(full, SENTINEL_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    return buf, buf[..., :shape[-1]]


def _accumulate_input(rng, seed, shape, c_kind, d):
    """C for the accumulate form: None, a BF16 or F32 tensor, or d itself
    holding C (in place).  Returns (c, its float64 values, its stored form)."""
    if c_kind is None:
        return None, None, None
    xc = synth.normal_f32(seed, shape) * np.float32(4.0)
    as_bf16 = c_kind == "bf16" or (c_kind == "inplace" and d.dtype == torch.bfloat16)
    if as_bf16:
        bits = synth.bf16_bits_from_f32(xc)
        cref, stored = oracle.bf16_decode(bits), bits
        cdev = to_dev(bits.view(np.int16)).view(torch.bfloat16)
    else:
        cref, stored = xc.astype(np.float64), xc
        cdev = to_dev(xc)
    if c_kind == "inplace":
        d.copy_(cdev)
        return d, cref, stored
    return cdev, cref, stored


def _untouched(got, written, d_kind, c_kind, stored, what):
    if c_kind == "inplace":
        assert np.array_equal(got[~written], stored[~written]), f"{what}: rows outside the groups changed"
    elif d_kind == "f32":
        assert np.isnan(got[~written]).all(), f"{what}: rows outside the groups written"
    else:
        assert np.all(got[~written] == SENTINEL_BF16), f"{what}: rows outside the groups written"


def _pad_untouched(buf, n, what):
    if buf.shape[-1] > n:
        pad = to_host(buf[..., n:])
        ok = np.isnan(pad).all() if buf.dtype == torch.float32 else np.all(pad == SENTINEL_BF16)
        assert ok, f"{what}: row padding written"


def _cast_a(x, ue8m0, m_major):
    """Per-token cast on the device: codes and F32 scales [rows, K/128],
    M-major (a transposed view) or K-major."""
    mg = _mg()
    R, K = x.shape[-2], x.shape[-1]
    q = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
    if m_major and x.ndim == 2:
        sf = torch.empty((K // 128, R), dtype=torch.float32, device="cuda").t()
    else:
        sf = torch.empty(x.shape[:-1] + (K // 128,), dtype=torch.float32, device="cuda")
    mg.per_token_cast_to_fp8(to_dev(x), q, sf, ue8m0)
    return q, sf


def _cast_b(x, ue8m0, rowb):
    """B codes with 128 x 128 block scales, or one scale per row (rowb)."""
    if rowb:
        return _cast_a(x, ue8m0, False)
    mg = _mg()
    N, K = x.shape[-2], x.shape[-1]
    q = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
    sf = torch.empty(x.shape[:-2] + (-(-N // 128), K // 128), dtype=torch.float32, device="cuda")
    mg.per_block_cast_to_fp8(to_dev(x), q, sf, ue8m0)
    return q, sf


def _pack(sf):
    """Packed UE8M0 scales of F32 power-of-two scales: [.., ceil(KB/4)] int32."""
    mg = _mg()
    sf = sf.contiguous()
    out = torch.empty(sf.shape[:-1] + (-(-sf.shape[-1] // 4),), dtype=torch.int32, device="cuda")
    mg.pack_ue8m0_to_int(sf, out)
    return out


def _oracle_operands(xa, xb, ue8m0, rowb, a, b, what):
    ra, rsfa = oracle.per_token_cast_to_fp8(xa, ue8m0)
    rb, rsfb = (oracle.per_token_cast_to_fp8 if rowb else oracle.per_block_cast_to_fp8)(xb, ue8m0)
    assert np.array_equal(to_host(a), ra), f"{what}: A codes differ from the oracle's cast"
    assert np.array_equal(to_host(b), rb), f"{what}: B codes differ from the oracle's cast"
    return ra, rsfa, rb, rsfb


def _check(got, ref, S, Gt, written, d_kind, nround, what):
    """BF16 d: the tolerance of every BF16 output; F32 d: the FP32 bound
    (Gt, the FP8 group term, None for BF16 GEMMs)."""
    if written is not None:
        got, ref = got[written], ref[written]
        S = S[written] if S is not None else None
        Gt = Gt[written] if Gt is not None else None
    if d_kind == "f32":
        assert_f32_close(got, ref, S, nround, what, G=Gt)
    else:
        assert_bf16_close(got, ref, what)


# ---------------------------------------------------------------------------
# case generators (host only)
# ---------------------------------------------------------------------------

def dense_case(i):
    rng = _rng("dense", i)
    u = rng.random()
    if u < 0.2:
        M, N, K = _loguni(rng, 1, 128), _loguni(rng, 1, 3000), 128 * int(rng.integers(1, 17))
    elif u < 0.75:
        M, N, K = _loguni(rng, 129, 1300), _loguni(rng, 1, 1500), 128 * int(rng.integers(1, 13))
    else:
        M, N, K = int(rng.integers(1500, 4097)), int(rng.integers(1500, 4097)), 128 * int(rng.integers(1, 3))
    return dict(M=M, N=N, K=K, scales=_pick(rng, ["f32", "ue8m0", "packed"]), rowb=bool(rng.random() < 0.3),
                d_kind=_pick(rng, ["bf16", "f32"]), c_kind=_pick(rng, [None, "bf16", "f32", "inplace"]),
                pad=int(rng.integers(0, 9)), a_m_major=bool(rng.random() < 0.5))


def mn_case(i):
    rng = _rng("mn", i)
    big = rng.random() < 0.25
    hi = 256 if big else 64
    return dict(M=16 * int(rng.integers(1, hi + 1)), N=16 * int(rng.integers(1, hi + 1)),
                K=128 * int(rng.integers(1, 3 if big else 11)), layout=_pick(rng, ["NN", "TN", "TT"]),
                packed=bool(rng.random() < 0.4), c_bf16=bool(rng.random() < 0.4),
                pad_a=16 * int(rng.integers(0, 3)), pad_b=16 * int(rng.integers(0, 3)),
                d_kind=_pick(rng, ["bf16", "f32"]), rowb=bool(rng.random() < 0.3))


def _masked_m(rng, G, max_m):
    mm = []
    for _ in range(G):
        u = rng.random()
        if u < 0.1:
            mm.append(0)
        elif u < 0.25:
            mm.append(max_m)
        elif u < 0.32:
            mm.append(max_m + int(rng.integers(1, 100)))
        elif u < 0.37:
            mm.append(-int(rng.integers(1, 5)))
        else:
            mm.append(int(rng.integers(1, max_m + 1)))
    return mm


def masked_case(i, bf16=False):
    rng = _rng("bf16_masked" if bf16 else "masked", i)
    kunit = 64 if bf16 else 128
    if rng.random() < 0.25:  # the 256 x 256 tile: many groups of up to 256 rows, wide N
        G, max_m = int(rng.integers(12, 33)), int(rng.integers(129, 257))
        N, K = _pick(rng, [4096, 7168]), kunit * int(rng.integers(1, 3))
    else:
        G, max_m = int(rng.integers(1, 9)), _loguni(rng, 1, 400)
        N, K = _loguni(rng, 16, 2200), kunit * int(rng.integers(1, 9))
    case = dict(G=G, max_m=max_m, N=N, K=K, mm=_masked_m(rng, G, max_m), pad=int(rng.integers(0, 5)))
    if bf16:
        case.update(d_kind=_pick(rng, ["bf16", "f32"]), c_kind=_pick(rng, [None, "bf16", "f32", "inplace"]))
    else:
        case.update(scales=_pick(rng, ["f32", "ue8m0", "packed"]), rowb=bool(rng.random() < 0.25),
                    d_kind=_pick(rng, ["bf16", "f32"]), c_kind=_pick(rng, [None, "bf16", "f32", "inplace"]))
    return case


def _layout(rng, G, nblocks):
    out = []
    while len(out) < nblocks:
        u = rng.random()
        g = -1 if u < 0.15 else (G + int(rng.integers(0, 4)) if u < 0.2 else int(rng.integers(0, G)))
        out += [g] * int(rng.geometric(0.3))
    return out[:nblocks]


def contig_case(i, bf16=False):
    rng = _rng("bf16_contig" if bf16 else "contig", i)
    kunit = 64 if bf16 else 128
    if rng.random() < 0.2:  # the 256 x 256 tile
        G, nblocks, N, K = int(rng.integers(1, 9)), int(rng.integers(24, 65)), _pick(rng, [4096, 3000]), kunit
    else:
        G, nblocks = int(rng.integers(1, 9)), _loguni(rng, 1, 48)
        N, K = _loguni(rng, 16, 2200), kunit * int(rng.integers(1, 9))
    case = dict(G=G, N=N, K=K, layout=_layout(rng, G, nblocks), pad=int(rng.integers(0, 5)))
    if bf16:
        case.update(d_kind=_pick(rng, ["bf16", "f32"]), c_kind=_pick(rng, [None, "bf16", "f32", "inplace"]))
    else:
        case.update(scales=_pick(rng, ["f32", "ue8m0", "packed"]), rowb=bool(rng.random() < 0.25),
                    d_kind=_pick(rng, ["bf16", "f32"]), c_kind=_pick(rng, [None, "bf16", "f32", "inplace"]))
    return case


def bf16_dense_case(i):
    rng = _rng("bf16_dense", i)
    if rng.random() < 0.25:
        M, N, K = int(rng.integers(1500, 4097)), int(rng.integers(1500, 4097)), 64 * int(rng.integers(1, 5))
    else:
        M, N, K = _loguni(rng, 1, 1300), _loguni(rng, 1, 2200), 64 * int(rng.integers(1, 25))
    return dict(M=M, N=N, K=K, d_kind=_pick(rng, ["bf16", "f32"]),
                c_kind=_pick(rng, [None, "bf16", "f32", "inplace"]), pad=int(rng.integers(0, 9)))


def fp8_out_case(i):
    rng = _rng("fp8_out", i)
    M = _loguni(rng, 1, 1300) if rng.random() < 0.8 else int(rng.integers(1500, 4097))
    N = _loguni(rng, 1, 2200) if M < 1500 else int(rng.integers(1500, 4097))
    K = 128 * int(rng.integers(1, 3 if M >= 1500 else 9))
    return dict(M=M, N=N, K=K, c_kind=_pick(rng, [None, "bf16", "f32"]), ue8m0=bool(rng.random() < 0.5),
                in_ue8m0=bool(rng.random() < 0.5), q_pad=4 * int(rng.integers(0, 3)),
                sf_m_major=bool(rng.random() < 0.5), rowb=bool(rng.random() < 0.3))


N_DENSE, N_MN, N_MASKED, N_CONTIG, N_BF16, N_BF16_GROUPED, N_FP8_OUT = 32, 18, 20, 20, 12, 12, 14


# ---------------------------------------------------------------------------
# FP8 GEMMs
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("i", range(N_DENSE))
def test_sweep_dense(i):
    cs = dense_case(i)
    M, N, K = cs["M"], cs["N"], cs["K"]
    what = f"sweep dense {i} {cs}"
    say(what)
    mg = _mg()
    rng = _rng("dense", 1000 + i)
    ue8m0 = cs["scales"] != "f32"
    xa = _inputs(rng, 60000 + 4 * i, (M, K))
    xb = _inputs(rng, 60001 + 4 * i, (N, K), 1 if cs["rowb"] else 128)
    a, sfa = _cast_a(xa, ue8m0, cs["a_m_major"])
    b, sfb = _cast_b(xb, ue8m0, cs["rowb"])
    if cs["scales"] == "packed":
        sfa, sfb = _pack(sfa), _pack(sfb)
    buf, d = _out((M, N), cs["d_kind"], cs["pad"])
    c, cref, stored = _accumulate_input(rng, 60002 + 4 * i, (M, N), cs["c_kind"], d)
    mg.fp8_gemm_nt(a, b, sfa, sfb, c, d)
    torch.cuda.synchronize()
    ra, rsfa, rb, rsfb = _oracle_operands(xa, xb, ue8m0, cs["rowb"], a, b, what)
    ref = oracle.fp8_gemm_nt(ra, rb, rsfa, rsfb, cref)
    S = Gt = None
    if cs["d_kind"] == "f32":
        S, Gt = fp8_bound_terms(oracle.fp8_gemm_nt, ra, rb, rsfa, rsfb)
        S = S if cref is None else S + np.abs(cref)
    _pad_untouched(buf, N, what)
    _check(to_host(d), ref, S, Gt, None, cs["d_kind"], fp8_rounding_count(K), what)


def _stored_mn(codes, pad):
    """K-major codes [R, K] stored MN-major: a row-major [K, R + pad] buffer
    (NaN codes in the padding) whose first R columns hold the transpose."""
    R, K = codes.shape
    buf = torch.full((K, R + pad), 0x7F, dtype=torch.uint8, device="cuda")
    buf[:, :R] = codes.t()
    return buf[:, :R]


@pytest.mark.parametrize("i", range(N_MN))
def test_sweep_mn_major(i):
    cs = mn_case(i)
    M, N, K = cs["M"], cs["N"], cs["K"]
    what = f"sweep MN-major {i} {cs}"
    say(what)
    mg = _mg()
    rng = _rng("mn", 1000 + i)
    xa = _inputs(rng, 61000 + 4 * i, (M, K))
    xb = _inputs(rng, 61001 + 4 * i, (N, K), 1 if cs["rowb"] else 128)
    a, sfa = _cast_a(xa, cs["packed"], True)
    b, sfb = _cast_b(xb, cs["packed"], cs["rowb"])
    if cs["packed"]:
        sfa, sfb = _pack(sfa), _pack(sfb)
    a_st, b_st = _stored_mn(a, cs["pad_a"]), _stored_mn(b, cs["pad_b"])
    c, cref = None, None
    if cs["c_bf16"]:
        bits = synth.bf16_bits_from_f32(synth.normal_f32(61002 + 4 * i, (M, N)) * np.float32(4.0))
        c, cref = to_dev(bits.view(np.int16)).view(torch.bfloat16), oracle.bf16_decode(bits)
    dt = torch.float32 if cs["d_kind"] == "f32" else torch.bfloat16
    d = torch.empty((M, N), dtype=dt, device="cuda")
    fn = {"NN": lambda: mg.fp8_gemm_nn(a, b_st, sfa, sfb, c, d),
          "TN": lambda: mg.fp8_gemm_tn(a_st, b_st, sfa, sfb, c, d),
          "TT": lambda: mg.fp8_gemm_tt(a_st, b, sfa, sfb, c, d)}[cs["layout"]]
    fn()
    dref = torch.empty((M, N), dtype=dt, device="cuda")
    mg.fp8_gemm_nt(a, b, sfa, sfb, c, dref)
    torch.cuda.synchronize()
    bits_view = torch.int32 if dt == torch.float32 else torch.int16
    assert torch.equal(d.view(bits_view), dref.view(bits_view)), f"{what}: differs from fp8_gemm_nt"
    ra, rsfa, rb, rsfb = _oracle_operands(xa, xb, cs["packed"], cs["rowb"], a, b, what)
    ref = oracle.fp8_gemm_nt(ra, rb, rsfa, rsfb, cref)
    S = Gt = None
    if cs["d_kind"] == "f32":
        S, Gt = fp8_bound_terms(oracle.fp8_gemm_nt, ra, rb, rsfa, rsfb)
        S = S if cref is None else S + np.abs(cref)
    _check(to_host(d), ref, S, Gt, None, cs["d_kind"], fp8_rounding_count(K), what)


@pytest.mark.parametrize("i", range(N_MASKED))
def test_sweep_masked(i):
    cs = masked_case(i)
    G, max_m, N, K = cs["G"], cs["max_m"], cs["N"], cs["K"]
    what = f"sweep masked {i} {cs}"
    say(what)
    mg = _mg()
    rng = _rng("masked", 1000 + i)
    ue8m0 = cs["scales"] != "f32"
    xa = _inputs(rng, 62000 + 4 * i, (G, max_m, K))
    xb = _inputs(rng, 62001 + 4 * i, (G, N, K), 1 if cs["rowb"] else 128)
    a, sfa = _cast_a(xa, ue8m0, False)
    b, sfb = _cast_b(xb, ue8m0, cs["rowb"])
    if cs["scales"] == "packed":
        sfa, sfb = _pack(sfa), _pack(sfb)
    buf, d = _out((G, max_m, N), cs["d_kind"], cs["pad"])
    c, cref, stored = _accumulate_input(rng, 62002 + 4 * i, (G, max_m, N), cs["c_kind"], d)
    mm = np.array(cs["mm"], dtype=np.int32)
    mg.m_grouped_fp8_gemm_nt_masked(a, b, sfa, sfb, d, to_dev(mm), max_m, c=c)
    torch.cuda.synchronize()
    ra, rsfa, rb, rsfb = _oracle_operands(xa, xb, ue8m0, cs["rowb"], a, b, what)
    ref, written = oracle.m_grouped_fp8_gemm_nt_masked(ra, rb, rsfa, rsfb, mm, max_m)
    S = Gt = None
    if cs["d_kind"] == "f32":
        S, Gt = fp8_bound_terms(oracle.m_grouped_fp8_gemm_nt_masked, ra, rb, rsfa, rsfb, mm, max_m)
    if cref is not None:
        ref = ref + cref
        S = S + np.abs(cref) if S is not None else None
    got = to_host(d)
    _untouched(got, written, cs["d_kind"], cs["c_kind"], stored, what)
    _pad_untouched(buf, N, what)
    _check(got, ref, S, Gt, written, cs["d_kind"], fp8_rounding_count(K), what)


@pytest.mark.parametrize("i", range(N_CONTIG))
def test_sweep_contiguous(i):
    cs = contig_case(i)
    G, N, K = cs["G"], cs["N"], cs["K"]
    layout = np.array(cs["layout"], dtype=np.int32)
    Msum = 128 * layout.size
    what = f"sweep contiguous {i} {cs}"
    say(what)
    mg = _mg()
    rng = _rng("contig", 1000 + i)
    ue8m0 = cs["scales"] != "f32"
    xa = _inputs(rng, 63000 + 4 * i, (Msum, K))
    xb = _inputs(rng, 63001 + 4 * i, (G, N, K), 1 if cs["rowb"] else 128)
    a, sfa = _cast_a(xa, ue8m0, bool(rng.random() < 0.5))
    b, sfb = _cast_b(xb, ue8m0, cs["rowb"])
    if cs["scales"] == "packed":
        sfa, sfb = _pack(sfa), _pack(sfb)
    buf, d = _out((Msum, N), cs["d_kind"], cs["pad"])
    c, cref, stored = _accumulate_input(rng, 63002 + 4 * i, (Msum, N), cs["c_kind"], d)
    mg.m_grouped_fp8_gemm_nt_contiguous(a, b, sfa, sfb, d, to_dev(layout), c=c)
    torch.cuda.synchronize()
    ra, rsfa, rb, rsfb = _oracle_operands(xa, xb, ue8m0, cs["rowb"], a, b, what)
    ref_layout = np.where(layout < G, layout, -1)
    ref, written = oracle.m_grouped_fp8_gemm_nt_contiguous(ra, rb, rsfa, rsfb, ref_layout)
    S = Gt = None
    if cs["d_kind"] == "f32":
        S, Gt = fp8_bound_terms(oracle.m_grouped_fp8_gemm_nt_contiguous, ra, rb, rsfa, rsfb, ref_layout)
    if cref is not None:
        ref = ref + cref
        S = S + np.abs(cref) if S is not None else None
    got = to_host(d)
    _untouched(got, written, cs["d_kind"], cs["c_kind"], stored, what)
    _pad_untouched(buf, N, what)
    _check(got, ref, S, Gt, written, cs["d_kind"], fp8_rounding_count(K), what)


@pytest.mark.parametrize("i", range(N_FP8_OUT))
def test_sweep_fp8_out(i):
    from test_gpu_fp8_out import run_case

    cs = fp8_out_case(i)
    say(f"sweep fp8 out {i} {cs}")
    run_case(cs["M"], cs["N"], cs["K"], c_kind=cs["c_kind"], ue8m0=cs["ue8m0"], in_ue8m0=cs["in_ue8m0"],
             q_pad=cs["q_pad"], sf_m_major=cs["sf_m_major"], seed=64000 + 4 * i, rowb=cs["rowb"])


# ---------------------------------------------------------------------------
# BF16 GEMMs
# ---------------------------------------------------------------------------

def _bf16_inputs(rng, seed, shape):
    return synth.bf16_bits_from_f32(_inputs(rng, seed, shape))


def _dev_bf16(bits):
    return to_dev(bits.view(np.int16)).view(torch.bfloat16)


def _abs_bf16(bits):
    return bits & np.uint16(0x7FFF)


@pytest.mark.parametrize("i", range(N_BF16))
def test_sweep_bf16_dense(i):
    cs = bf16_dense_case(i)
    M, N, K = cs["M"], cs["N"], cs["K"]
    what = f"sweep bf16 dense {i} {cs}"
    say(what)
    mg = _mg()
    rng = _rng("bf16_dense", 1000 + i)
    ab = _bf16_inputs(rng, 65000 + 4 * i, (M, K))
    bb = _bf16_inputs(rng, 65001 + 4 * i, (N, K))
    buf, d = _out((M, N), cs["d_kind"], cs["pad"])
    c, cref, _ = _accumulate_input(rng, 65002 + 4 * i, (M, N), cs["c_kind"], d)
    mg.bf16_gemm_nt(_dev_bf16(ab), _dev_bf16(bb), c, d)
    torch.cuda.synchronize()
    ref = oracle.bf16_gemm_nt(ab, bb, cref)
    S = None
    if cs["d_kind"] == "f32":
        S = oracle.bf16_gemm_nt(_abs_bf16(ab), _abs_bf16(bb))
        S = S if cref is None else S + np.abs(cref)
    _pad_untouched(buf, N, what)
    _check(to_host(d), ref, S, None, None, cs["d_kind"], K, what)


@pytest.mark.parametrize("i", range(N_BF16_GROUPED))
def test_sweep_bf16_masked(i):
    cs = masked_case(i, bf16=True)
    G, max_m, N, K = cs["G"], cs["max_m"], cs["N"], cs["K"]
    what = f"sweep bf16 masked {i} {cs}"
    say(what)
    mg = _mg()
    rng = _rng("bf16_masked", 1000 + i)
    ab = _bf16_inputs(rng, 66000 + 4 * i, (G, max_m, K))
    bb = _bf16_inputs(rng, 66001 + 4 * i, (G, N, K))
    buf, d = _out((G, max_m, N), cs["d_kind"], cs["pad"])
    c, cref, stored = _accumulate_input(rng, 66002 + 4 * i, (G, max_m, N), cs["c_kind"], d)
    mm = np.array(cs["mm"], dtype=np.int32)
    mg.m_grouped_bf16_gemm_nt_masked(_dev_bf16(ab), _dev_bf16(bb), d, to_dev(mm), max_m, c=c)
    torch.cuda.synchronize()
    ref, written = oracle.m_grouped_bf16_gemm_nt_masked(ab, bb, mm, max_m)
    S = None
    if cs["d_kind"] == "f32":
        S, _ = oracle.m_grouped_bf16_gemm_nt_masked(_abs_bf16(ab), _abs_bf16(bb), mm, max_m)
    if cref is not None:
        ref = ref + cref
        S = S + np.abs(cref) if S is not None else None
    got = to_host(d)
    _untouched(got, written, cs["d_kind"], cs["c_kind"], stored, what)
    _pad_untouched(buf, N, what)
    _check(got, ref, S, None, written, cs["d_kind"], K, what)


@pytest.mark.parametrize("i", range(N_BF16_GROUPED))
def test_sweep_bf16_contiguous(i):
    cs = contig_case(i, bf16=True)
    G, N, K = cs["G"], cs["N"], cs["K"]
    layout = np.array(cs["layout"], dtype=np.int32)
    Msum = 128 * layout.size
    what = f"sweep bf16 contiguous {i} {cs}"
    say(what)
    mg = _mg()
    rng = _rng("bf16_contig", 1000 + i)
    ab = _bf16_inputs(rng, 67000 + 4 * i, (Msum, K))
    bb = _bf16_inputs(rng, 67001 + 4 * i, (G, N, K))
    buf, d = _out((Msum, N), cs["d_kind"], cs["pad"])
    c, cref, stored = _accumulate_input(rng, 67002 + 4 * i, (Msum, N), cs["c_kind"], d)
    mg.m_grouped_bf16_gemm_nt_contiguous(_dev_bf16(ab), _dev_bf16(bb), d, to_dev(layout), c=c)
    torch.cuda.synchronize()
    ref_layout = np.where(layout < G, layout, -1)
    ref, written = oracle.m_grouped_bf16_gemm_nt_contiguous(ab, bb, ref_layout)
    S = None
    if cs["d_kind"] == "f32":
        S, _ = oracle.m_grouped_bf16_gemm_nt_contiguous(_abs_bf16(ab), _abs_bf16(bb), ref_layout)
    if cref is not None:
        ref = ref + cref
        S = S + np.abs(cref) if S is not None else None
    got = to_host(d)
    _untouched(got, written, cs["d_kind"], cs["c_kind"], stored, what)
    _pad_untouched(buf, N, what)
    _check(got, ref, S, None, written, cs["d_kind"], K, what)


# ---------------------------------------------------------------------------
# the casts and the MoE steps either side of the grouped GEMMs
# ---------------------------------------------------------------------------

def cast_case(i):
    rng = _rng("cast", i)
    G = int(rng.integers(2, 5)) if rng.random() < 0.25 else 0  # 0: a 2-D tensor
    return dict(block=bool(rng.random() < 0.4), G=G, R=_loguni(rng, 1, 600 if G else 3000),
                K=8 * _loguni(rng, 1, 1024), bf16=bool(rng.random() < 0.4), mn=bool(rng.random() < 0.3),
                ue8m0=bool(rng.random() < 0.4), sf_mn=bool(rng.random() < 0.5), zero_rows=bool(rng.random() < 0.3))


def moe_case(i):
    rng = _rng("moe", i)
    G = int(rng.integers(1, 41))
    return dict(T=_loguni(rng, 1, 2000), k=int(rng.integers(1, min(8, G) + 1)), G=G, max_m=_loguni(rng, 1, 300),
                K=8 * _loguni(rng, 1, 900), N=_loguni(rng, 1, 3000), p_none=float(rng.choice([0.0, 0.05, 0.2])),
                x_bf16=bool(rng.random() < 0.4), ue8m0=bool(rng.random() < 0.4), align=_pick(rng, [128, 256]),
                cap=float(rng.uniform(0.5, 1.5)))


N_CAST, N_MOE = 24, 12


@pytest.mark.parametrize("i", range(N_CAST))
def test_sweep_cast(i):
    """Per-token and per-block casts against the oracle, codes and scales bit
    for bit: F32 or BF16 sources, K-major or MN-major, 2-D or 3-D, ragged K,
    scales K-major or M-major, magnitudes over 2^-20 .. 2^11 with all-zero
    rows (the amax floor)."""
    cs = cast_case(i)
    what = f"sweep cast {i} {cs}"
    say(what)
    mg = _mg()
    rng = _rng("cast", 1000 + i)
    lead = (cs["G"],) if cs["G"] else ()
    R, K = cs["R"], cs["K"]
    x = synth.normal_f32(68000 + 4 * i, lead + (R, K))
    e = rng.integers(-20, 12, size=lead + (R, -(-K // 128)))
    x = (x * np.exp2(np.repeat(e, 128, axis=-1)[..., :K])).astype(np.float32)
    if cs["zero_rows"]:
        x[..., rng.integers(0, R, size=max(1, R // 8)), :] = 0.0
    if cs["bf16"]:
        bits = synth.bf16_bits_from_f32(x)
        x = oracle.bf16_decode(bits).astype(np.float32)
        stored = np.ascontiguousarray(np.swapaxes(bits, -1, -2)) if cs["mn"] else bits
        src = to_dev(stored.view(np.int16)).view(torch.bfloat16)
    else:
        src = to_dev(np.ascontiguousarray(np.swapaxes(x, -1, -2)) if cs["mn"] else x)
    if cs["mn"]:
        src = src.transpose(-1, -2)  # the logical [.., R, K] view of a tensor stored [.., K, R]
    q = torch.full(lead + (R, K), 0x55, dtype=torch.uint8, device="cuda")
    if cs["block"]:
        sf = torch.full(lead + (-(-R // 128), -(-K // 128)), float("nan"), dtype=torch.float32, device="cuda")
        mg.per_block_cast_to_fp8(src, q, sf, cs["ue8m0"])
        rq, rsf = oracle.per_block_cast_to_fp8(x, cs["ue8m0"])
    else:
        if cs["sf_mn"] and not lead:
            sf = torch.full((-(-K // 128), R), float("nan"), dtype=torch.float32, device="cuda").t()
        else:
            sf = torch.full(lead + (R, -(-K // 128)), float("nan"), dtype=torch.float32, device="cuda")
        mg.per_token_cast_to_fp8(src, q, sf, cs["ue8m0"])
        rq, rsf = oracle.per_token_cast_to_fp8(x, cs["ue8m0"])
    torch.cuda.synchronize()
    assert np.array_equal(to_host(q), rq), f"{what}: codes"
    assert np.array_equal(to_host(sf).view(np.uint32), rsf.view(np.uint32)), f"{what}: scales"


@pytest.mark.parametrize("i", range(N_MOE))
def test_sweep_moe_dispatch_and_combine(i):
    """MoE dispatch into the masked and the contiguous layouts (routing
    tables, codes and scales bit for bit, untouched rows) and the combine
    (within its FP32-sum bound), against the oracle."""
    from test_gpu_moe import _check_dispatch, _combine_bound, _contig_buffers, _dispatch_buffers

    cs = moe_case(i)
    T, k, G, max_m, K, N = cs["T"], cs["k"], cs["G"], cs["max_m"], cs["K"], cs["N"]
    what = f"sweep moe {i} {cs}"
    say(what)
    mg = _mg()
    x = synth.normal_f32(69000 + 4 * i, (T, K))
    topk, w = synth.moe_routing(69001 + 4 * i, T, G, k, cs["p_none"])
    if cs["x_bf16"]:
        xb = synth.bf16_bits_from_f32(x)
        xd = to_dev(xb.view(np.int16)).view(torch.bfloat16)
        x = oracle.bf16_decode(xb).astype(np.float32)
    else:
        xd = to_dev(x)
    # masked layout
    outs = _dispatch_buffers(T, K, k, G, max_m)
    mg.moe_dispatch_masked_fp8(xd, to_dev(topk), *outs, use_ue8m0=cs["ue8m0"])
    torch.cuda.synchronize()
    _, rslot = _check_dispatch(x, topk, G, max_m, cs["ue8m0"], outs, what)
    # contiguous layout: a capacity around the routed rows, in whole 128-row blocks
    align = cs["align"]
    Mcap = 128 * max(1, int(cs["cap"] * (T * k + (align - 1) * G) / 128))
    couts = _contig_buffers(T, K, k, G, Mcap)
    mg.moe_dispatch_contiguous_fp8(xd, to_dev(topk), *couts, align=align, use_ue8m0=cs["ue8m0"])
    torch.cuda.synchronize()
    a, sfa, layout, counts, slot = (to_host(t) for t in couts)
    ra, rsfa, owned, rlayout, rcounts, rcslot = oracle.moe_dispatch_contiguous_fp8(x, topk, G, Mcap, cs["ue8m0"],
                                                                                   align=align)
    assert np.array_equal(counts, rcounts) and np.array_equal(layout, rlayout), f"{what}: contiguous tables"
    assert np.array_equal(slot, rcslot), f"{what}: contiguous slots"
    assert np.array_equal(a[owned], ra[owned]), f"{what}: contiguous codes"
    assert np.array_equal(sfa[owned].view(np.uint32), rsfa[owned].view(np.uint32)), f"{what}: contiguous scales"
    assert np.all(a[~owned] == 0x55) and np.all(np.isnan(sfa[~owned])), f"{what}: contiguous padding rows written"
    # combine over the masked slots
    d_bits = synth.bf16_bits_from_f32(synth.normal_f32(69002 + 4 * i, (G, max_m, N)))
    y = torch.full((T, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    mg.moe_combine(to_dev(d_bits.view(np.int16)).view(torch.bfloat16), to_dev(rslot), to_dev(w), y)
    torch.cuda.synchronize()
    got = oracle.bf16_decode(to_host(y))
    y_ref = oracle.moe_combine(d_bits, rslot, w)
    assert np.all(np.isfinite(got)), f"{what}: combine output not written"
    bound = _combine_bound(d_bits, rslot, w, y_ref)
    assert np.all(np.abs(got - y_ref) <= bound * (1 + 1e-6)), f"{what}: combine outside the bound"
