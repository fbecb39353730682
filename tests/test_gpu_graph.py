"""Masked grouped GEMMs captured once in a hipGraph and replayed with new
masked_m contents written between replays (64 experts, max_m 128,
N 7168, K 2048).

The captured graph holds, per replay: the per-token UE8M0 cast of the
activations, pack_ue8m0_to_int of both scale tensors, the masked FP8 GEMM
on the packed scales, and the masked BF16 GEMM on the same shapes.  Replay
0 has every masked_m = 0, replay 1 every masked_m = 128, the rest are
seeded uniform draws.  Every replay is checked against the oracle on
sampled experts, rows and column blocks, every untouched row is checked
against the sentinel, and the replayed outputs are compared bit for bit
with an eager run of the same calls."""

import numpy as np
import pytest

import oracle
from moe_grouped_gemm_x128_amd import synth

from helpers import (SENTINEL_BF16, assert_bf16_close, assert_f32_close, fp8_bound_terms, fp8_rounding_count, say,
                     to_dev, to_host)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CHECK_GROUPS = (0, 1, 21, 42, 63)


def _mg():
    import moe_grouped_gemm_x128_amd as mg

    return mg


def test_masked_graph_replay_with_new_masked_m():
    cfg = synth.MASKED_GRAPH
    G, max_m, N, K = cfg["G"], cfg["max_m"], cfg["N"], cfg["K"]
    KB = K // 128
    say(f"graph setup G={G} max_m={max_m} N={N} K={K}")
    mg = _mg()

    xa = synth.normal_f32(cfg["seed_a"], (G, max_m, K))
    xa_dev = to_dev(xa)
    xb_dev = torch.empty((G, N, K), dtype=torch.float32, device="cuda")
    xb_keep = {}
    for g, chunk in enumerate(synth.normal_f32_chunks(cfg["seed_b"], (G, N, K))):
        xb_dev[g].copy_(torch.from_numpy(chunk))
        if g in CHECK_GROUPS:
            xb_keep[g] = chunk
    # weights: quantized once, outside the graph (static across replays)
    qb = torch.empty((G, N, K), dtype=torch.uint8, device="cuda")
    sfb = torch.empty((G, N // 128, KB), dtype=torch.float32, device="cuda")
    mg.per_block_cast_to_fp8(xb_dev, qb, sfb, True)
    b16 = xb_dev.to(torch.bfloat16)
    a16 = xa_dev.to(torch.bfloat16)
    del xb_dev
    torch.cuda.synchronize()

    qa = torch.empty((G, max_m, K), dtype=torch.uint8, device="cuda")
    sfa = torch.empty((G, max_m, KB), dtype=torch.float32, device="cuda")
    pa = torch.empty((G, max_m, KB // 4), dtype=torch.int32, device="cuda")
    pb = torch.empty((G, N // 128, KB // 4), dtype=torch.int32, device="cuda")
    d8 = torch.empty((G, max_m, N), dtype=torch.bfloat16, device="cuda")
    d16 = torch.empty((G, max_m, N), dtype=torch.bfloat16, device="cuda")
    masked_m = torch.zeros(G, dtype=torch.int32, device="cuda")

    def step():
        mg.per_token_cast_to_fp8(xa_dev, qa, sfa, True)
        mg.pack_ue8m0_to_int(sfa, pa)
        mg.pack_ue8m0_to_int(sfb, pb)
        mg.m_grouped_fp8_gemm_nt_masked(qa, qb, pa, pb, d8, masked_m, max_m)
        mg.m_grouped_bf16_gemm_nt_masked(a16, b16, d16, masked_m, max_m)

    def fill_sentinel():
        d8.view(torch.int16).fill_(SENTINEL_BF16)
        d16.view(torch.int16).fill_(SENTINEL_BF16)

    # warm-up, then capture on a side stream
    fill_sentinel()
    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graph.capture_begin()
        step()
        graph.capture_end()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    # oracle quantization of the checked experts (A rows are sampled per replay)
    rq_b, rsf_b = {}, {}
    for g in CHECK_GROUPS:
        rq_b[g], rsf_b[g] = oracle.per_block_cast_to_fp8(xb_keep[g], True)
    a16_bits = to_host(a16)
    b16_bits = {g: synth.bf16_bits_from_f32(xb_keep[g]) for g in CHECK_GROUPS}
    ref_pb = {g: oracle.pack_ue8m0_to_int(rsf_b[g])[0] for g in CHECK_GROUPS}
    pb_host = None

    draws = [np.zeros(G, np.int32), np.full(G, max_m, np.int32)]
    draws += [synth.masked_m_uniform(cfg["seed_m"] + r, G, max_m) for r in range(2, 6)]
    for r, mm in enumerate(draws):
        say(f"graph replay {r}: sum(masked_m)={int(mm.sum())}")
        masked_m.copy_(torch.from_numpy(mm))
        fill_sentinel()
        graph.replay()
        torch.cuda.synchronize()
        g8, g16 = to_host(d8), to_host(d16)
        # eager run of the same calls: identical bits
        fill_sentinel()
        step()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(d8), g8), f"replay {r}: FP8 replay differs from eager"
        assert np.array_equal(to_host(d16), g16), f"replay {r}: BF16 replay differs from eager"
        if pb_host is None:
            pb_host = to_host(pb)
            for g in CHECK_GROUPS:
                assert np.array_equal(pb_host[g], ref_pb[g])
        for g in range(G):
            v = int(mm[g])
            assert np.all(g8[g, v:] == SENTINEL_BF16) and np.all(g16[g, v:] == SENTINEL_BF16), (r, g)
        for g in CHECK_GROUPS:
            v = int(mm[g])
            if v == 0:
                continue
            rows = np.unique(np.concatenate([np.random.default_rng(100 * r + g).choice(v, size=min(12, v), replace=False), [v - 1]]))
            ra, rsfa = oracle.per_token_cast_to_fp8(xa[g, rows], True)
            rpa, _ = oracle.pack_ue8m0_to_int(rsfa)
            ua = oracle.scales_from_packed_ue8m0(rpa, KB)
            ub = oracle.scales_from_packed_ue8m0(ref_pb[g], KB)
            for nb in (0, 27, 55):
                cols = slice(nb * 128, nb * 128 + 128)
                ref8 = oracle.fp8_gemm_nt(ra, rq_b[g][cols], ua, ub[nb:nb + 1])
                assert_bf16_close(g8[g, rows][:, cols], ref8, f"replay {r} fp8 g={g} nb={nb}")
                ref16 = oracle.bf16_decode(a16_bits[g, rows]) @ oracle.bf16_decode(b16_bits[g][cols]).T
                assert_bf16_close(g16[g, rows][:, cols], ref16, f"replay {r} bf16 g={g} nb={nb}")


def test_every_entry_point_replays_under_capture():
    """One graph holding the casts, the pack, the dense FP8 GEMM with an
    accumulate input, the contiguous FP8 GEMM and the dense and contiguous
    BF16 GEMMs; replayed three times with new contents written into the
    input buffers between replays, every replay bit-identical to an eager
    run of the same calls on the same inputs."""
    mg = _mg()
    M, N, K, G = 256, 384, 512, 2
    layout = torch.tensor([1, -1, 0, 1], dtype=torch.int32, device="cuda")
    Msum = 4 * 128
    xa = torch.empty((M, K), device="cuda")
    xb = torch.empty((N, K), device="cuda")
    xg = torch.empty((Msum, K), device="cuda")
    xgb = torch.empty((G, N, K), device="cuda")
    cin = torch.empty((M, N), device="cuda")
    qa = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sfa = torch.empty((K // 128, M), dtype=torch.float32, device="cuda").t()
    qb = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sfb = torch.empty((N // 128, K // 128), dtype=torch.float32, device="cuda")
    qg = torch.empty((Msum, K), dtype=torch.uint8, device="cuda")
    sfg = torch.empty((Msum, K // 128), dtype=torch.float32, device="cuda")
    qgb = torch.empty((G, N, K), dtype=torch.uint8, device="cuda")
    sfgb = torch.empty((G, N // 128, K // 128), dtype=torch.float32, device="cuda")
    psf = torch.empty((N // 128, 1), dtype=torch.int32, device="cuda")
    outs = {k: torch.empty(s, dtype=torch.bfloat16, device="cuda")
            for k, s in [("d8", (M, N)), ("g8", (Msum, N)), ("d16", (M, N)), ("g16", (Msum, N))]}

    def step():
        mg.per_token_cast_to_fp8(xa, qa, sfa)
        mg.per_block_cast_to_fp8(xb, qb, sfb)
        mg.per_token_cast_to_fp8(xg, qg, sfg)
        mg.per_block_cast_to_fp8(xgb, qgb, sfgb)
        mg.pack_ue8m0_to_int(sfb, psf)
        mg.fp8_gemm_nt(qa, qb, sfa, sfb, cin, outs["d8"])
        mg.m_grouped_fp8_gemm_nt_contiguous(qg, qgb, sfg, sfgb, outs["g8"], layout)
        mg.bf16_gemm_nt(xa.to(torch.bfloat16), xb.to(torch.bfloat16), None, outs["d16"])
        mg.m_grouped_bf16_gemm_nt_contiguous(xg.to(torch.bfloat16), xgb.to(torch.bfloat16), outs["g16"], layout)

    def fill(seed):
        for i, t in enumerate((xa, xb, xg, xgb, cin)):
            t.copy_(torch.from_numpy(synth.normal_f32(seed + i, tuple(t.shape))))
        for o in outs.values():
            o.view(torch.int16).fill_(SENTINEL_BF16)

    fill(700)
    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graph.capture_begin()
        step()
        graph.capture_end()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for r in range(3):
        say(f"all-entry-point graph replay {r}")
        fill(710 + 10 * r)
        graph.replay()
        torch.cuda.synchronize()
        got = {k: to_host(v).copy() for k, v in outs.items()}
        got["psf"] = to_host(psf).copy()
        fill(710 + 10 * r)
        step()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert np.array_equal(to_host(v), got[k]), f"replay {r}: {k} differs from eager"
        assert np.array_equal(to_host(psf), got["psf"])
        assert np.all(got["g8"][128:256] == SENTINEL_BF16) and np.all(got["g16"][128:256] == SENTINEL_BF16)
    # the replayed dense FP8 result against the oracle on the last inputs
    ra, rsfa = oracle.per_token_cast_to_fp8(to_host(xa))
    rb, rsfb = oracle.per_block_cast_to_fp8(to_host(xb))
    ref = oracle.fp8_gemm_nt(ra, rb, rsfa, rsfb, c=to_host(cin).astype(np.float64))
    assert_bf16_close(got["d8"], ref, "replayed dense FP8 with C")


def test_two_launch_plan_replays_under_capture():
    """The BF16 GEMM whose launch plan is two launches over column ranges
    (4000 x 7100 x 4096: 256 x 256 tiles on [0, 4096), 256 x 192 on the
    rest) captured once and replayed with new inputs; every replay
    bit-identical to an eager run."""
    mg = _mg()
    from moe_grouped_gemm_x128_amd import binding

    M, N, K = 4000, 7100, 4096
    c = binding.query_config(binding.DG_KIND_BF16_DENSE, 1, M, N, K)
    assert (c["n_split"], c["block_n2"]) == (4096, 192)
    a = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    b = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    d = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def fill(seed):
        a.copy_(torch.from_numpy(synth.normal_f32(seed, (M, K))))
        b.copy_(torch.from_numpy(synth.normal_f32(seed + 1, (N, K))))
        d.view(torch.int16).fill_(SENTINEL_BF16)

    fill(730)
    mg.bf16_gemm_nt(a, b, None, d)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graph.capture_begin()
        mg.bf16_gemm_nt(a, b, None, d)
        graph.capture_end()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for r in range(2):
        say(f"two-launch plan graph replay {r}")
        fill(740 + 10 * r)
        graph.replay()
        torch.cuda.synchronize()
        got = to_host(d).copy()
        fill(740 + 10 * r)
        mg.bf16_gemm_nt(a, b, None, d)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(d), got), f"replay {r} differs from eager"
        assert not np.any(got == SENTINEL_BF16), "elements left unwritten"


def test_layouts_and_accumulate_forms_replay_under_capture():
    """The NN / TN / TT GEMMs on FP8 operands stored MN-major, the masked
    grouped GEMM with an F32 accumulate input and F32 output, the contiguous
    grouped GEMM with a BF16 accumulate input and the dense GEMM with FP8
    output, captured in one graph and replayed three times with new
    operands written between replays (casts and transposed copies run
    eagerly, outside the graph): every replay bit-identical to eager calls,
    the MN-major results equal to the NT GEMM's, and the masked result
    within the F32 bound of the oracle's C + A . B^T."""
    mg = _mg()
    M, N, K, G, max_m = 256, 384, 512, 2, 128
    layout = torch.tensor([1, 0, 0, -1], dtype=torch.int32, device="cuda")
    Msum = 4 * 128
    masked_m = torch.tensor([100, 37], dtype=torch.int32, device="cuda")
    dev = "cuda"
    xa, xb = torch.empty((M, K), device=dev), torch.empty((N, K), device=dev)
    xga, xgb = torch.empty((G * max_m, K), device=dev), torch.empty((G, N, K), device=dev)
    xc = torch.empty((Msum, K), device=dev)
    qa, qb = torch.empty((M, K), dtype=torch.uint8, device=dev), torch.empty((N, K), dtype=torch.uint8, device=dev)
    sfa = torch.empty((K // 128, M), dtype=torch.float32, device=dev).t()
    sfb = torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev)
    a_t = torch.empty((K, M), dtype=torch.uint8, device=dev)  # A stored [K, M]
    b_t = torch.empty((K, N), dtype=torch.uint8, device=dev)  # B stored [K, N]
    qga = torch.empty((G * max_m, K), dtype=torch.uint8, device=dev)
    sfga = torch.empty((G * max_m, K // 128), dtype=torch.float32, device=dev)
    qgb = torch.empty((G, N, K), dtype=torch.uint8, device=dev)
    sfgb = torch.empty((G, N // 128, K // 128), dtype=torch.float32, device=dev)
    qc = torch.empty((Msum, K), dtype=torch.uint8, device=dev)
    sfc = torch.empty((Msum, K // 128), dtype=torch.float32, device=dev)
    cm = torch.empty((G, max_m, N), dtype=torch.float32, device=dev)
    cc = torch.empty((Msum, N), dtype=torch.bfloat16, device=dev)
    outs = {
        "nn": torch.empty((M, N), dtype=torch.bfloat16, device=dev),
        "tn": torch.empty((M, N), dtype=torch.bfloat16, device=dev),
        "tt": torch.empty((M, N), dtype=torch.bfloat16, device=dev),
        "dm": torch.empty((G, max_m, N), dtype=torch.float32, device=dev),
        "dc": torch.empty((Msum, N), dtype=torch.bfloat16, device=dev),
        "q": torch.empty((M, N), dtype=torch.uint8, device=dev),
        "sfq": torch.empty((M, N // 128), dtype=torch.float32, device=dev),
    }
    a3, sfa3 = qga.view(G, max_m, K), sfga.view(G, max_m, K // 128)

    def step():
        mg.fp8_gemm_nn(qa, b_t, sfa, sfb, None, outs["nn"])
        mg.fp8_gemm_tn(a_t, b_t, sfa, sfb, None, outs["tn"])
        mg.fp8_gemm_tt(a_t, qb, sfa, sfb, None, outs["tt"])
        mg.m_grouped_fp8_gemm_nt_masked(a3, qgb, sfa3, sfgb, outs["dm"], masked_m, max_m, c=cm)
        mg.m_grouped_fp8_gemm_nt_contiguous(qc, qgb, sfc, sfgb, outs["dc"], layout, c=cc)
        mg.fp8_gemm_nt_fp8_out(qa, qb, sfa, sfb, None, outs["q"], outs["sfq"])

    def fill(seed):
        for i, t in enumerate((xa, xb, xga, xgb, xc, cm)):
            t.copy_(torch.from_numpy(synth.normal_f32(seed + i, tuple(t.shape))))
        cc.copy_(torch.from_numpy(synth.normal_f32(seed + 9, tuple(cc.shape))))
        mg.per_token_cast_to_fp8(xa, qa, sfa)
        mg.per_block_cast_to_fp8(xb, qb, sfb)
        mg.per_token_cast_to_fp8(xga, qga, sfga)
        mg.per_block_cast_to_fp8(xgb, qgb, sfgb)
        mg.per_token_cast_to_fp8(xc, qc, sfc)
        a_t.copy_(qa.t())
        b_t.copy_(qb.t())
        for o in outs.values():
            o.view(torch.uint8).fill_(0x5A)

    fill(800)
    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graph.capture_begin()
        step()
        graph.capture_end()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    nt = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    for r in range(3):
        say(f"layouts / accumulate graph replay {r}")
        fill(810 + 10 * r)
        graph.replay()
        torch.cuda.synchronize()
        got = {k: to_host(v).copy() for k, v in outs.items()}
        fill(810 + 10 * r)
        step()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert np.array_equal(to_host(v), got[k]), f"replay {r}: {k} differs from eager"
        mg.fp8_gemm_nt(qa, qb, sfa, sfb, None, nt)
        torch.cuda.synchronize()
        for k in ("nn", "tn", "tt"):
            assert np.array_equal(got[k], to_host(nt)), f"replay {r}: {k} differs from the NT GEMM"
        # rows past masked_m and skipped blocks keep the fill pattern
        assert np.all(got["dm"][0, 100:].view(np.uint8) == 0x5A) and np.all(got["dm"][1, 37:].view(np.uint8) == 0x5A)
        assert np.all(got["dc"][384:].view(np.uint8) == 0x5A)
    # the last replay's masked result against the oracle (F32 output: C + A . B^T)
    ra, rsfa = oracle.per_token_cast_to_fp8(to_host(xga).reshape(G, max_m, K))
    rb, rsfb = oracle.per_block_cast_to_fp8(to_host(xgb))
    cmh = to_host(cm).astype(np.float64)
    for g, m in enumerate((100, 37)):
        ref = cmh[g, :m] + oracle.fp8_gemm_nt(ra[g, :m], rb[g], rsfa[g, :m], rsfb[g])
        S, Gt = fp8_bound_terms(oracle.fp8_gemm_nt, ra[g, :m], rb[g], rsfa[g, :m], rsfb[g])
        assert_f32_close(got["dm"][g, :m], ref, S + np.abs(cmh[g, :m]), fp8_rounding_count(K), f"masked F32 group {g}",
                         G=Gt)


def test_row_scale_and_output_forms_replay_under_capture():
    """One graph with the forms that take one B scale per row and the F32
    and FP8 outputs: the dense FP8 GEMM (row scales, F32 d), the FP8-output
    GEMM (row scales, the 256 x 128 tile), the TT layout (row scales, F32 d)
    and the masked BF16 GEMM's accumulate form (BF16 C, F32 d); replayed
    three times with new inputs, each replay bit-identical to an eager run."""
    mg = _mg()
    M, N, K = 256, 384, 512
    G, max_m, Kb = 2, 128, 256
    xa = torch.empty((M, K), device="cuda")
    xb = torch.empty((N, K), device="cuda")
    xm = torch.empty((G, max_m, Kb), device="cuda")
    xmb = torch.empty((G, N, Kb), device="cuda")
    xc = torch.empty((G, max_m, N), device="cuda")
    masked_m = torch.tensor([100, 37], dtype=torch.int32, device="cuda")
    qa = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sfa = torch.empty((K // 128, M), dtype=torch.float32, device="cuda").t()
    qb = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sfb = torch.empty((N, K // 128), dtype=torch.float32, device="cuda")  # one scale per row of B
    a_st = torch.empty((K, M), dtype=torch.uint8, device="cuda")  # A stored MN-major
    outs = {"d32": torch.empty((M, N), dtype=torch.float32, device="cuda"),
            "q8": torch.empty((M, N), dtype=torch.uint8, device="cuda"),
            "sfq": torch.empty((M, N // 128), dtype=torch.float32, device="cuda"),
            "tt32": torch.empty((M, N), dtype=torch.float32, device="cuda"),
            "m32": torch.empty((G, max_m, N), dtype=torch.float32, device="cuda")}

    def step():
        mg.per_token_cast_to_fp8(xa, qa, sfa)
        mg.per_token_cast_to_fp8(xb, qb, sfb)
        mg.fp8_gemm_nt(qa, qb, sfa, sfb, None, outs["d32"])
        mg.fp8_gemm_nt_fp8_out(qa, qb, sfa, sfb, None, outs["q8"], outs["sfq"])
        a_st.copy_(qa.t())
        mg.fp8_gemm_tt(a_st, qb, sfa, sfb, None, outs["tt32"])
        mg.m_grouped_bf16_gemm_nt_masked(xm.to(torch.bfloat16), xmb.to(torch.bfloat16), outs["m32"], masked_m, max_m,
                                         c=xc.to(torch.bfloat16))

    def fill(seed):
        for i, t in enumerate((xa, xb, xm, xmb, xc)):
            t.copy_(torch.from_numpy(synth.normal_f32(seed + i, tuple(t.shape))))
        for o in outs.values():
            o.view(torch.uint8).fill_(0x5A)

    fill(900)
    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graph.capture_begin()
        step()
        graph.capture_end()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for r in range(3):
        say(f"row-scale / output-form graph replay {r}")
        fill(910 + 10 * r)
        graph.replay()
        torch.cuda.synchronize()
        got = {k: to_host(v).copy() for k, v in outs.items()}
        fill(910 + 10 * r)
        step()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert np.array_equal(to_host(v).view(np.uint8), got[k].view(np.uint8)), f"replay {r}: {k} differs from eager"
        # the TT layout equals the NT GEMM; rows past masked_m keep the fill
        assert np.array_equal(got["tt32"].view(np.uint32), got["d32"].view(np.uint32))
        assert np.all(got["m32"][0, 100:].view(np.uint8) == 0x5A) and np.all(got["m32"][1, 37:].view(np.uint8) == 0x5A)
    # the last replay's F32 dense result against the oracle
    ra, rsfa = oracle.per_token_cast_to_fp8(to_host(xa))
    rb, rsfb = oracle.per_token_cast_to_fp8(to_host(xb))
    S, Gt = fp8_bound_terms(oracle.fp8_gemm_nt, ra, rb, rsfa, rsfb)
    assert_f32_close(got["d32"], oracle.fp8_gemm_nt(ra, rb, rsfa, rsfb), S, fp8_rounding_count(K),
                     "replayed dense FP8, row scales, F32 d", G=Gt)
