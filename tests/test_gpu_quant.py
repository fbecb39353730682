"""GPU parity of the FP8 quantizers and the UE8M0 pack: bit-exact against
the oracle (codes, FP32 scales, packed words, invalid counts)."""

import numpy as np
import pytest

import oracle
from moe_grouped_gemm_x128_amd import synth

from helpers import say, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _lib():
    import moe_grouped_gemm_x128_amd as mg

    return mg


def gpu_per_token(x, ue8m0=False, sf_mn_major=False, bf16=False):
    mg = _lib()
    xt = to_dev(x)
    if bf16:
        xt = xt.to(torch.bfloat16)
    q = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
    nkb = -(-x.shape[-1] // 128)
    if sf_mn_major and x.ndim == 2:
        sf = torch.empty((nkb, x.shape[0]), dtype=torch.float32, device="cuda").t()
    else:
        sf = torch.empty(x.shape[:-1] + (nkb,), dtype=torch.float32, device="cuda")
    mg.per_token_cast_to_fp8(xt, q, sf, ue8m0)
    torch.cuda.synchronize()
    return to_host(q), to_host(sf.contiguous())


def gpu_per_block(x, ue8m0=False):
    mg = _lib()
    q = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
    sf = torch.empty(x.shape[:-2] + (-(-x.shape[-2] // 128), -(-x.shape[-1] // 128)), dtype=torch.float32, device="cuda")
    mg.per_block_cast_to_fp8(to_dev(x), q, sf, ue8m0)
    torch.cuda.synchronize()
    return to_host(q), to_host(sf)


@pytest.mark.parametrize("shape", [(128, 512), (5, 300), (2, 70, 384), (1, 128)])
@pytest.mark.parametrize("ue8m0", [False, True])
def test_per_token_bit_exact(shape, ue8m0):
    say(f"per_token shape={shape} ue8m0={ue8m0}")
    x = synth.normal_f32(101, shape) * np.float32(1.7)
    q, sf = gpu_per_token(x, ue8m0)
    rq, rsf = oracle.per_token_cast_to_fp8(x, ue8m0)
    assert np.array_equal(sf.view(np.uint32), rsf.view(np.uint32))
    assert np.array_equal(q, rq)


def test_per_token_mn_major_scales_and_zero_block():
    say("per_token MN-major sf, zero block")
    x = synth.normal_f32(102, (96, 384))
    x[3, 128:256] = 0.0
    q, sf = gpu_per_token(x, sf_mn_major=True)
    rq, rsf = oracle.per_token_cast_to_fp8(x)
    assert np.array_equal(sf.view(np.uint32), rsf.view(np.uint32))
    assert np.array_equal(q, rq)


def test_per_token_bf16_input():
    say("per_token bf16 input")
    xb = synth.bf16_bits_from_f32(synth.normal_f32(103, (64, 256)))
    x32 = oracle.bf16_decode(xb).astype(np.float32)  # exact: bf16 values are binary32 values
    q, sf = gpu_per_token(x32, bf16=True)
    rq, rsf = oracle.per_token_cast_to_fp8(x32)
    assert np.array_equal(sf.view(np.uint32), rsf.view(np.uint32))
    assert np.array_equal(q, rq)


def test_per_token_rounding_corners():
    """Blocks whose maximum is 448, so s = 1 exactly and q = e4m3(x): every
    midpoint between adjacent codes (ties to even), one binary32 ulp either
    side of it, the subnormal band, negative values rounding to -0, and the
    saturation band."""
    say("per_token rounding corners")
    pos = oracle.e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    vals = np.concatenate([
        mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(500)),
        pos.astype(np.float32), np.float32([2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11, 1e-7, 0.0]),
    ]).astype(np.float32)
    vals = np.concatenate([vals, -vals])
    per = 127  # values per block, position 0 holds the 448 that fixes s = 1
    nblk = -(-vals.size // per)
    x = np.zeros((nblk, 128), dtype=np.float32)
    x[:, 0] = 448.0
    flat = np.zeros(nblk * per, dtype=np.float32)
    flat[: vals.size] = vals
    x[:, 1:] = flat.reshape(nblk, per)
    q, sf = gpu_per_token(x)
    rq, rsf = oracle.per_token_cast_to_fp8(x)
    assert np.all(rsf == 1.0)
    assert np.array_equal(sf.view(np.uint32), rsf.view(np.uint32))
    bad = np.argwhere(q != rq)
    assert bad.size == 0, [(float(x[tuple(i)]), int(q[tuple(i)]), int(rq[tuple(i)])) for i in bad[:8]]


@pytest.mark.parametrize("shape", [(256, 512), (200, 300), (2, 130, 260), (2112, 256)])
@pytest.mark.parametrize("ue8m0", [False, True])
def test_per_block_bit_exact(shape, ue8m0):
    say(f"per_block shape={shape} ue8m0={ue8m0}")
    x = synth.normal_f32(104, shape) * np.float32(0.3)
    q, sf = gpu_per_block(x, ue8m0)
    rq, rsf = oracle.per_block_cast_to_fp8(x, ue8m0)
    assert np.array_equal(sf.view(np.uint32), rsf.view(np.uint32))
    assert np.array_equal(q, rq)


def test_per_token_full_size_sampled_rows():
    """Contiguous-prefill activations [32768, 7168], quantized in one launch;
    sampled rows compared bit-exactly."""
    say("per_token full size [32768, 7168] sampled rows")
    x = synth.normal_f32(301, (32768, 7168))
    q, sf = gpu_per_token(x)
    rows = np.random.default_rng(0).choice(32768, size=64, replace=False)
    rows = np.concatenate([rows, [0, 32767]])
    rq, rsf = oracle.per_token_cast_to_fp8(x[rows])
    assert np.array_equal(sf[rows].view(np.uint32), rsf.view(np.uint32))
    assert np.array_equal(q[rows], rq)


# ---------------------------------------------------------------------------
# pack_ue8m0_to_int
# ---------------------------------------------------------------------------

def gpu_pack(x, with_counter=True):
    mg = _lib()
    xt = to_dev(x)
    out = torch.empty(x.shape[:-1] + (-(-x.shape[-1] // 4),), dtype=torch.int32, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda") if with_counter else None
    mg.pack_ue8m0_to_int(xt, out, cnt)
    torch.cuda.synchronize()
    return to_host(out), (int(cnt.item()) if with_counter else None)


@pytest.mark.parametrize("shape", [(3, 5, 16), (128, 4), (7, 13), (1000,)])
def test_pack_valid_powers_of_two(shape):
    say(f"pack shape={shape}")
    e = np.random.default_rng(1).integers(1, 255, size=shape)
    x = np.ldexp(1.0, e - 127).astype(np.float32)
    out, bad = gpu_pack(x)
    ref, rbad = oracle.pack_ue8m0_to_int(x)
    assert np.array_equal(out, ref) and bad == rbad == 0


def test_pack_invalid_inputs_counted_on_device():
    say("pack invalid inputs")
    rng = np.random.default_rng(2)
    x = rng.standard_normal((33, 56)).astype(np.float32)  # mostly invalid: mantissas, signs
    x[0] = np.ldexp(1.0, rng.integers(-20, 20, size=56)).astype(np.float32)
    x[1, :4] = np.float32([-0.0, 0.0, -1.0, 2.0 ** -127])
    out, bad = gpu_pack(x)
    ref, rbad = oracle.pack_ue8m0_to_int(x)
    assert np.array_equal(out, ref)
    assert bad == rbad and rbad > 1000
    out2, none = gpu_pack(x, with_counter=False)
    assert np.array_equal(out2, ref) and none is None


def test_pack_golden_examples_on_device():
    import os

    say("pack golden examples")
    path = os.path.join(os.path.dirname(__file__), "golden", "ue8m0_pack_examples.txt")
    rows = []
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#"):
            lhs, packed, invalid = [p.strip() for p in line.split("|")]
            rows.append((np.array([int(t, 16) for t in lhs.split()], dtype=np.uint32), int(packed), int(invalid)))
    x = np.stack([r[0] for r in rows]).view(np.float32)
    out, bad = gpu_pack(x)
    assert [int(v) for v in out[:, 0]] == [r[1] for r in rows]
    assert bad == sum(r[2] for r in rows)
