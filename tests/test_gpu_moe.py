"""GPU parity of the MoE dispatch (routing into the masked layout with the
per-token FP8 cast) and combine, against the oracle (oracle/moe.py).

Routing tables (masked_m, slot, the valid rows of src) and the cast bytes and
scales are compared bit for bit; rows past masked_m must stay untouched.
The combine is compared with the oracle's float64 sum: an FP32 sum of k
products, rounded once to BF16, lies within 2^-8 |y| + (k + 1) 2^-24 sum_j
|w_j d_j| of it.  The whole chain (dispatch -> masked FP8 GEMM -> combine)
is compared with the oracle's chain within the GEMM's tolerance carried
through the weighted sum."""

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


def _dispatch_buffers(T, K, k, G, max_m):
    a = torch.full((G, max_m, K), 0x55, dtype=torch.uint8, device="cuda")
    sfa = torch.full((G, max_m, -(-K // 128)), float("nan"), dtype=torch.float32, device="cuda")
    masked_m = torch.full((G,), -7, dtype=torch.int32, device="cuda")
    slot = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    src = torch.full((G, max_m), -7, dtype=torch.int32, device="cuda")
    return a, sfa, masked_m, slot, src


def _check_dispatch(x, topk, G, max_m, ue8m0, outs, what):
    a, sfa, masked_m, slot, src = (to_host(t) for t in outs)
    ra, rsfa, rmm, rslot, rsrc = oracle.moe_dispatch_fp8(x, topk, G, max_m, ue8m0)
    assert np.array_equal(masked_m, rmm), f"{what}: masked_m"
    assert np.array_equal(slot, rslot), f"{what}: slot"
    for e in range(G):
        n = int(rmm[e])
        assert np.array_equal(src[e, :n], rsrc[e, :n]), f"{what}: src of expert {e}"
        assert np.all(src[e, n:] == -7), f"{what}: src rows past masked_m written (expert {e})"
        assert np.array_equal(a[e, :n], ra[e, :n]), f"{what}: codes of expert {e}"
        assert np.array_equal(sfa[e, :n].view(np.uint32), rsfa[e, :n].view(np.uint32)), f"{what}: scales of expert {e}"
        assert np.all(a[e, n:] == 0x55) and np.all(np.isnan(sfa[e, n:])), f"{what}: rows past masked_m written"
    return rmm, rslot


@pytest.mark.parametrize("T,k,G,max_m,K,p_none,x_bf16,ue8m0", [
    (768, 8, 32, 256, 7168, 0.0, False, False),   # the decode shape
    (300, 6, 8, 200, 384, 0.1, True, False),      # over capacity (about 225 per expert), ids routed nowhere
    (50, 4, 5, 64, 200, 0.0, False, True),        # partial last K-block, UE8M0 scales
    (1, 1, 1, 1, 128, 0.0, True, True),
    (4097, 2, 3, 2048, 256, 0.0, False, False),   # several routing passes, capacity reached (about 2731)
    (64, 10, 12, 64, 272, 0.05, True, False),      # more choices per token than destinations held in registers
])
def test_dispatch_matches_oracle(T, k, G, max_m, K, p_none, x_bf16, ue8m0):
    say(f"moe_dispatch_masked_fp8 T={T} k={k} G={G} max_m={max_m} K={K} bf16={x_bf16} ue8m0={ue8m0}")
    mg = _mg()
    x = synth.normal_f32(611, (T, K))
    topk, _ = synth.moe_routing(612, T, G, k, p_none)
    if T > 1:
        topk[0, 0] = G  # an id past the last expert: routed nowhere
    if x_bf16:
        xb = synth.bf16_bits_from_f32(x)
        xd = to_dev(xb.view(np.int16)).view(torch.bfloat16)
        x = oracle.bf16_decode(xb).astype(np.float32)
    else:
        xd = to_dev(x)
    outs = _dispatch_buffers(T, K, k, G, max_m)
    mg.moe_dispatch_masked_fp8(xd, to_dev(topk), *outs, use_ue8m0=ue8m0)
    torch.cuda.synchronize()
    _check_dispatch(x, topk, G, max_m, ue8m0, outs, f"dispatch T={T}")


def test_dispatch_no_tokens_clears_masked_m():
    say("moe_dispatch_masked_fp8 T=0")
    mg = _mg()
    G, max_m, K, k = 4, 16, 256, 2
    outs = _dispatch_buffers(0, K, k, G, max_m)
    mg.moe_dispatch_masked_fp8(torch.empty((0, K), dtype=torch.float32, device="cuda"),
                               torch.empty((0, k), dtype=torch.int32, device="cuda"), *outs)
    torch.cuda.synchronize()
    assert to_host(outs[2]).tolist() == [0] * G


def _combine_bound(d_bits, slot, w, y_ref):
    D = oracle.bf16_decode(d_bits).reshape(-1, d_bits.shape[-1])
    T, k = slot.shape
    absum = np.zeros_like(y_ref)
    for j in range(k):
        ok = slot[:, j] >= 0
        absum[ok] += np.abs(w[ok, j].astype(np.float64))[:, None] * np.abs(D[slot[ok, j]])
    return REL_TOL * np.abs(y_ref) + (k + 1) * 2.0 ** -24 * absum


@pytest.mark.parametrize("T,k,G,max_m,N,d_pad", [(768, 8, 32, 256, 4096, 0), (100, 3, 6, 40, 1000, 8),
                                                 (33, 4, 5, 16, 77, 3), (1, 1, 1, 1, 8, 0)])
def test_combine_matches_oracle(T, k, G, max_m, N, d_pad):
    say(f"moe_combine T={T} k={k} G={G} max_m={max_m} N={N} pad={d_pad}")
    mg = _mg()
    topk, w = synth.moe_routing(621, T, G, k, 0.1)
    _, slot, _, _ = oracle.moe_route(topk, G, max_m)
    d_bits = synth.bf16_bits_from_f32(synth.normal_f32(622, (G, max_m, N)))
    dbuf = torch.zeros((G, max_m, N + d_pad), dtype=torch.int16, device="cuda")
    dbuf[:, :, :N] = to_dev(d_bits.view(np.int16))
    d = dbuf.view(torch.bfloat16)[:, :, :N]
    y = torch.full((T, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    mg.moe_combine(d, to_dev(slot), to_dev(w), y)
    torch.cuda.synchronize()
    got = oracle.bf16_decode(to_host(y))
    y_ref = oracle.moe_combine(d_bits, slot, w)
    bound = _combine_bound(d_bits, slot, w, y_ref)
    err = np.abs(got - y_ref)
    assert np.all(np.isfinite(got)), "unwritten combine output"
    assert np.all(err <= bound * (1 + 1e-6)), f"combine: {int((err > bound).sum())} outside the bound"


def test_combine_one_choice_weight_one_is_exact():
    """k = 1, weight 1: y is the selected BF16 row itself, bit for bit; a
    dropped token gives a zero row."""
    mg = _mg()
    G, max_m, N, T = 3, 8, 520, 10
    say(f"moe_combine exact rows G={G} max_m={max_m} N={N}")
    d_bits = synth.bf16_bits_from_f32(synth.normal_f32(631, (G, max_m, N)))
    slot = np.array([[s] for s in (0, 5, 23, 9, -1, 17, 1, 2, 3, 22)], dtype=np.int32)
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    mg.moe_combine(to_dev(d_bits.view(np.int16)).view(torch.bfloat16), to_dev(slot),
                   torch.ones((T, 1), dtype=torch.float32, device="cuda"), y)
    torch.cuda.synchronize()
    got = to_host(y)
    rows = d_bits.reshape(G * max_m, N)
    for t in range(T):
        if slot[t, 0] >= 0:
            assert np.array_equal(got[t], rows[slot[t, 0]]), t
        else:
            assert not got[t].any(), t


def test_moe_chain_dispatch_gemm_combine():
    """dispatch -> masked FP8 GEMM -> combine on a reduced decode shape,
    against the oracle's chain (route, cast, float64 GEMM, float64 sum)."""
    mg = _mg()
    T, k, G, max_m, N, K = 192, 4, 8, 128, 512, 1024
    say(f"moe chain T={T} k={k} G={G} max_m={max_m} N={N} K={K}")
    x = synth.normal_f32(641, (T, K))
    xb = synth.normal_f32(642, (G, N, K))
    topk, w = synth.moe_routing(643, T, G, k)
    a, sfa, masked_m, slot, src = _dispatch_buffers(T, K, k, G, max_m)
    mg.moe_dispatch_masked_fp8(to_dev(x), to_dev(topk), a, sfa, masked_m, slot, src)
    qb = torch.empty((G, N, K), dtype=torch.uint8, device="cuda")
    sfb = torch.empty((G, N // 128, K // 128), dtype=torch.float32, device="cuda")
    mg.per_block_cast_to_fp8(to_dev(xb), qb, sfb)
    d = torch.zeros((G, max_m, N), dtype=torch.bfloat16, device="cuda")
    mg.m_grouped_fp8_gemm_nt_masked(a, qb, sfa, sfb, d, masked_m, max_m)
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    mg.moe_combine(d, slot, to_dev(w), y)
    torch.cuda.synchronize()
    ra, rsfa, rmm, rslot, _ = oracle.moe_dispatch_fp8(x, topk, G, max_m)
    rb, rsfb = oracle.per_block_cast_to_fp8(xb)
    D, _ = oracle.m_grouped_fp8_gemm_nt_masked(ra, rb, rsfa, rsfb, rmm, max_m)
    rows = D.reshape(G * max_m, N)
    y_ref = np.zeros((T, N))
    band = np.zeros((T, N))
    rms = float(np.sqrt(np.mean(np.concatenate([D[e, :rmm[e]].ravel() for e in range(G)]) ** 2)))
    for j in range(k):
        ok = rslot[:, j] >= 0
        wj = w[ok, j].astype(np.float64)[:, None]
        y_ref[ok] += wj * rows[rslot[ok, j]]
        band[ok] += wj * (ABS_RMS_TOL * rms + REL_TOL * np.abs(rows[rslot[ok, j]]))
    got = oracle.bf16_decode(to_host(y))
    err = np.abs(got - y_ref)
    # the GEMM's band carried through the weighted sum, then one BF16 rounding
    bound = band * (1 + REL_TOL) + REL_TOL * np.abs(y_ref) + 1e-6 * (np.abs(y_ref) + band)
    assert np.all(err <= bound), f"chain: {int((err > bound).sum())} outside the bound"


# ---------------------------------------------------------------------------
# contiguous layout (prefill)
# ---------------------------------------------------------------------------

def _contig_buffers(T, K, k, G, Mcap):
    a = torch.full((Mcap, K), 0x55, dtype=torch.uint8, device="cuda")
    sfa = torch.full((Mcap, -(-K // 128)), float("nan"), dtype=torch.float32, device="cuda")
    layout = torch.full((Mcap // 128,), -7, dtype=torch.int32, device="cuda")
    counts = torch.full((G,), -7, dtype=torch.int32, device="cuda")
    slot = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    return a, sfa, layout, counts, slot


@pytest.mark.parametrize("T,k,G,Mcap,K,p_none,x_bf16,align", [
    (4096, 8, 32, 36864, 7168, 0.0, False, 128),  # a prefill routing: every pair fits
    (4096, 8, 32, 40960, 7168, 0.0, False, 256),  # the same in 256-row granules
    (50, 3, 7, 512, 200, 0.1, True, 128),         # regions past the capacity: experts 4..6 dropped
    (50, 3, 7, 1024, 200, 0.1, True, 256),        # (256: experts 4..6 dropped as well)
    (1, 1, 1, 128, 128, 0.0, False, 256),         # a region larger than the capacity
    (0, 2, 4, 256, 256, 0.0, False, 128),         # no tokens: counts 0, every block -1
])
def test_dispatch_contiguous_matches_oracle(T, k, G, Mcap, K, p_none, x_bf16, align):
    say(f"moe_dispatch_contiguous_fp8 T={T} k={k} G={G} Mcap={Mcap} K={K} bf16={x_bf16} align={align}")
    mg = _mg()
    x = synth.normal_f32(651, (T, K))
    topk, _ = synth.moe_routing(652, T, G, k, p_none)
    if x_bf16:
        xb = synth.bf16_bits_from_f32(x)
        xd = to_dev(xb.view(np.int16)).view(torch.bfloat16)
        x = oracle.bf16_decode(xb).astype(np.float32)
    else:
        xd = to_dev(x)
    outs = _contig_buffers(T, K, k, G, Mcap)
    mg.moe_dispatch_contiguous_fp8(xd, to_dev(topk), *outs, align=align)
    torch.cuda.synchronize()
    a, sfa, layout, counts, slot = (to_host(t) for t in outs)
    ra, rsfa, owned, rlayout, rcounts, rslot = oracle.moe_dispatch_contiguous_fp8(x, topk, G, Mcap, align=align)
    assert np.array_equal(counts, rcounts) and np.array_equal(layout, rlayout) and np.array_equal(slot, rslot)
    assert np.array_equal(a[owned], ra[owned]), "codes"
    assert np.array_equal(sfa[owned].view(np.uint32), rsfa[owned].view(np.uint32)), "scales"
    assert np.all(a[~owned] == 0x55) and np.all(np.isnan(sfa[~owned])), "padding rows written"


@pytest.mark.parametrize("align", [128, 256])
def test_moe_chain_contiguous_dispatch_gemm_combine(align):
    """dispatch (contiguous) -> contiguous FP8 GEMM -> combine, against the
    oracle's chain."""
    mg = _mg()
    T, k, G, N, K = 512, 4, 8, 512, 1024
    Mcap = -(-(T * k + (align - 1) * G) // 128) * 128
    say(f"moe contiguous chain T={T} k={k} G={G} Mcap={Mcap} N={N} K={K}")
    x = synth.normal_f32(661, (T, K))
    xb = synth.normal_f32(662, (G, N, K))
    topk, w = synth.moe_routing(663, T, G, k)
    a, sfa, layout, counts, slot = _contig_buffers(T, K, k, G, Mcap)
    mg.moe_dispatch_contiguous_fp8(to_dev(x), to_dev(topk), a, sfa, layout, counts, slot, align=align)
    qb = torch.empty((G, N, K), dtype=torch.uint8, device="cuda")
    sfb = torch.empty((G, N // 128, K // 128), dtype=torch.float32, device="cuda")
    mg.per_block_cast_to_fp8(to_dev(xb), qb, sfb)
    d = torch.zeros((Mcap, N), dtype=torch.bfloat16, device="cuda")
    mg.m_grouped_fp8_gemm_nt_contiguous(a, qb, sfa, sfb, d, layout)
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    mg.moe_combine(d.view(1, Mcap, N), slot, to_dev(w), y)
    torch.cuda.synchronize()
    ra, rsfa, owned, rlayout, _, rslot = oracle.moe_dispatch_contiguous_fp8(x, topk, G, Mcap, align=align)
    rb, rsfb = oracle.per_block_cast_to_fp8(xb)
    rows = np.zeros((Mcap, N))
    for e in range(G):
        sel = owned & (np.repeat(rlayout, 128) == e)
        rows[sel] = oracle.fp8_gemm_nt(ra[sel], rb[e], rsfa[sel], rsfb[e])
    rms = float(np.sqrt(np.mean(rows[owned] ** 2)))
    y_ref = np.zeros((T, N))
    band = np.zeros((T, N))
    for j in range(k):
        ok = rslot[:, j] >= 0
        wj = w[ok, j].astype(np.float64)[:, None]
        y_ref[ok] += wj * rows[rslot[ok, j]]
        band[ok] += wj * (ABS_RMS_TOL * rms + REL_TOL * np.abs(rows[rslot[ok, j]]))
    got = oracle.bf16_decode(to_host(y))
    bound = band * (1 + REL_TOL) + REL_TOL * np.abs(y_ref) + 1e-6 * (np.abs(y_ref) + band)
    err = np.abs(got - y_ref)
    assert np.all(err <= bound), f"contiguous chain: {int((err > bound).sum())} outside the bound"


def test_moe_decode_chain_graph_replay():
    """dispatch -> masked FP8 GEMM -> combine captured once in a hipGraph and
    replayed with new routing and tokens written before each replay (the
    fused MoE path's graph compatibility, "DeepGEMM CUDA Graph Compatibility
    for Masked Grouped GEMMs", last section); every replay equals an eager
    run of the same calls, bit for bit."""
    mg = _mg()
    T, k, G, max_m, N, K = 256, 4, 16, 128, 512, 1024
    say(f"moe decode chain graph replay T={T} k={k} G={G} max_m={max_m} N={N} K={K}")
    qb = torch.empty((G, N, K), dtype=torch.uint8, device="cuda")
    sfb = torch.empty((G, N // 128, K // 128), dtype=torch.float32, device="cuda")
    mg.per_block_cast_to_fp8(to_dev(synth.normal_f32(671, (G, N, K))), qb, sfb)
    x = torch.empty((T, K), dtype=torch.float32, device="cuda")
    topk = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")

    def buffers():
        a, sfa, masked_m, slot, src = _dispatch_buffers(T, K, k, G, max_m)
        d = torch.zeros((G, max_m, N), dtype=torch.bfloat16, device="cuda")
        y = torch.zeros((T, N), dtype=torch.bfloat16, device="cuda")
        return a, sfa, masked_m, slot, src, d, y

    def calls(bufs, stream=None):
        a, sfa, masked_m, slot, src, d, y = bufs
        mg.moe_dispatch_masked_fp8(x, topk, a, sfa, masked_m, slot, src, stream=stream)
        mg.m_grouped_fp8_gemm_nt_masked(a, qb, sfa, sfb, d, masked_m, max_m, stream=stream)
        mg.moe_combine(d, slot, w, y, stream=stream)

    gbufs = buffers()
    x.copy_(to_dev(synth.normal_f32(672, (T, K))))
    t0, w0 = synth.moe_routing(673, T, G, k)
    topk.copy_(to_dev(t0))
    w.copy_(to_dev(w0))
    calls(gbufs)  # eager warm-up
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            calls(gbufs, stream=stream)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    for r in range(3):
        x.copy_(to_dev(synth.normal_f32(680 + r, (T, K))))
        tr, wr = synth.moe_routing(690 + r, T, G, k, 0.2 * r)
        topk.copy_(to_dev(tr))
        w.copy_(to_dev(wr))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ebufs = buffers()
        calls(ebufs)
        torch.cuda.synchronize()
        y_g, y_e = gbufs[6], ebufs[6]
        assert torch.equal(y_g.view(torch.int16), y_e.view(torch.int16)), f"replay {r}: combine output"
        assert torch.equal(gbufs[2], ebufs[2]) and torch.equal(gbufs[3], ebufs[3]), f"replay {r}: routing"
        # and the routing against the oracle
        rmm, rslot, _, _ = oracle.moe_route(tr, G, max_m)
        assert np.array_equal(to_host(gbufs[2]), rmm) and np.array_equal(to_host(gbufs[3]), rslot), f"replay {r}"


def test_dispatch_scales_m_major_per_expert():
    """The dispatch writing A's scales M-major per expert ([G, K/128, max_m]
    seen through a transposed view, the layout of the MoE decode benchmark):
    the same codes, scales and routing as the oracle."""
    say("moe_dispatch_masked_fp8, scales M-major per expert")
    mg = _mg()
    T, k, G, max_m, K = 96, 4, 8, 64, 1024
    x = synth.normal_f32(651, (T, K))
    topk, _ = synth.moe_routing(652, T, G, k, 0.05)
    a, _, masked_m, slot, src = _dispatch_buffers(T, K, k, G, max_m)
    sfa = torch.full((G, K // 128, max_m), float("nan"), dtype=torch.float32, device="cuda").transpose(1, 2)
    assert sfa.stride() == (K // 128 * max_m, 1, max_m)
    outs = (a, sfa, masked_m, slot, src)
    mg.moe_dispatch_masked_fp8(to_dev(x), to_dev(topk), *outs)
    torch.cuda.synchronize()
    _check_dispatch(x, topk, G, max_m, False, outs, "dispatch, M-major scales")
