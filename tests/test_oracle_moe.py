"""Pins of the oracle's MoE dispatch and combine: a hand-worked routing
example (tests/golden/moe_route_example.txt), an independent vectorised
construction of the routing on random inputs (stable order of flat indices
per expert), capacity overflow, the gather of the dispatch in a closed form,
and the combine against brute force and its closed forms."""

import os

import numpy as np
import pytest

import oracle
from moe_grouped_gemm_x128_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "moe_route_example.txt")


def _golden():
    rec = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        key, rest = line.split(None, 1)
        rows = [[int(v) for v in r.split()] for r in rest.split("|")]
        scalar = key in ("G", "max_m") or key.endswith("_Mcap") or key.endswith("_align")
        rec[key] = rows[0][0] if scalar else np.array(rows if len(rows) > 1 else rows[0])
    return rec


def test_route_hand_worked_example():
    g = _golden()
    masked_m, slot, src, counts = oracle.moe_route(g["topk"], g["G"], g["max_m"])
    assert masked_m.tolist() == g["masked_m"].tolist()
    assert counts.tolist() == g["counts"].tolist()
    assert slot.tolist() == g["slot"].tolist()
    assert src.tolist() == g["src"].tolist()


def _route_vectorised(topk, G, max_m):
    """The same routing built another way: for each expert, the flat indices
    t*k + j routed to it in increasing order (np.flatnonzero) are its rows."""
    T, k = topk.shape
    flat = topk.reshape(-1)
    slot = np.full(T * k, -1, dtype=np.int64)
    src = np.full((G, max_m), -1, dtype=np.int64)
    counts = np.zeros(G, dtype=np.int64)
    for e in range(G):
        idx = np.flatnonzero(flat == e)
        counts[e] = idx.size
        keep = idx[:max_m]
        slot[keep] = e * max_m + np.arange(keep.size)
        src[e, :keep.size] = keep // k
    return np.minimum(counts, max_m), slot.reshape(T, k), src, counts


@pytest.mark.parametrize("T,k,G,max_m,seed", [(64, 8, 32, 256, 1), (300, 4, 8, 128, 2), (50, 6, 5, 40, 3),
                                              (1, 1, 1, 1, 4)])
def test_route_matches_vectorised_construction(T, k, G, max_m, seed):
    rng = np.random.default_rng(seed)
    topk = rng.integers(-1, G + 1, size=(T, k))  # includes ids outside [0, G)
    want = _route_vectorised(topk, G, max_m)
    got = oracle.moe_route(topk, G, max_m)
    for w, g_ in zip(want, got):
        assert np.array_equal(np.asarray(w), np.asarray(g_))


def test_route_capacity_overflow():
    # every token to expert 1, capacity 3: rows 0..2 are tokens 0..2, the rest dropped
    topk = np.ones((7, 1), dtype=np.int64)
    masked_m, slot, src, counts = oracle.moe_route(topk, 2, 3)
    assert masked_m.tolist() == [0, 3] and counts.tolist() == [0, 7]
    assert slot[:, 0].tolist() == [3, 4, 5, -1, -1, -1, -1]
    assert src.tolist() == [[-1, -1, -1], [0, 1, 2]]


def test_dispatch_round_robin_closed_form():
    """k = 1 and token t to expert t mod G: expert e's row r is token
    r*G + e, cast per token."""
    G, max_m, T, K = 4, 8, 27, 256
    x = synth.normal_f32(61, (T, K))
    topk = (np.arange(T) % G)[:, None]
    a, sfa, masked_m, slot, src = oracle.moe_dispatch_fp8(x, topk, G, max_m)
    for e in range(G):
        n = len(range(e, T, G))
        assert masked_m[e] == min(n, max_m)
        for r in range(masked_m[e]):
            q, s = oracle.per_token_cast_to_fp8(x[r * G + e][None])
            assert np.array_equal(a[e, r], q[0]) and np.array_equal(sfa[e, r], s[0])
        assert not a[e, masked_m[e]:].any()


def test_combine_brute_force_and_closed_forms():
    rng = np.random.default_rng(5)
    G, max_m, N, T, k = 3, 4, 40, 6, 3
    d_bits = synth.bf16_bits_from_f32(rng.standard_normal((G, max_m, N)).astype(np.float32))
    slot = rng.integers(-1, G * max_m, size=(T, k)).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    y = oracle.moe_combine(d_bits, slot, w)
    D = oracle.bf16_decode(d_bits).reshape(G * max_m, N)
    for t in range(T):
        for n in range(N):
            ref = 0.0
            for j in range(k):
                if slot[t, j] >= 0:
                    ref += float(w[t, j]) * float(D[slot[t, j], n])
            assert abs(y[t, n] - ref) <= 1e-12 * max(1.0, abs(ref))
    # one choice of weight 1: y is that row exactly; all slots dropped: y = 0
    s1 = np.array([[5], [-1]], dtype=np.int32)
    y1 = oracle.moe_combine(d_bits, s1, np.ones((2, 1), np.float32))
    assert np.array_equal(y1[0], D[5]) and not y1[1].any()


def test_route_contiguous_hand_worked_example():
    g = _golden()
    for pre in ("c_", "c2_", "c3_"):
        counts, slot, layout, _ = oracle.moe_route_contiguous(g["topk"], g["G"], g[pre + "Mcap"], g.get(pre + "align", 128))
        assert counts.tolist() == g["counts"].tolist()
        assert layout.tolist() == g[pre + "layout"].tolist()
        assert slot.tolist() == g[pre + "slot"].tolist()


@pytest.mark.parametrize("align", [128, 256])
@pytest.mark.parametrize("T,k,G,Mcap,seed", [(300, 8, 16, 4096, 1), (300, 8, 16, 1024, 2), (40, 3, 7, 1024, 3)])
def test_route_contiguous_matches_vectorised_construction(T, k, G, Mcap, seed, align):
    rng = np.random.default_rng(seed)
    topk = rng.integers(-1, G + 1, size=(T, k))
    flat = topk.reshape(-1)
    counts = np.array([(flat == e).sum() for e in range(G)])
    start = np.concatenate([[0], np.cumsum(-(-counts // align) * align)[:-1]])
    slot = np.full(T * k, -1)
    layout = np.full(Mcap // 128, -1)
    for e in range(G):
        idx = np.flatnonzero(flat == e)
        rows = start[e] + np.arange(idx.size)
        slot[idx[rows < Mcap]] = rows[rows < Mcap]
        nb = -(-counts[e] // align) * align // 128
        layout[start[e] // 128:min(start[e] // 128 + nb, Mcap // 128)] = e
    got = oracle.moe_route_contiguous(topk, G, Mcap, align)
    assert np.array_equal(got[0], counts)
    assert np.array_equal(got[1], slot.reshape(T, k))
    assert np.array_equal(got[2], layout)
    # every owned row belongs to a block of its own expert
    for t in range(T):
        for j in range(k):
            if got[1][t, j] >= 0:
                assert got[2][got[1][t, j] // 128] == topk[t, j]


def test_dispatch_contiguous_rows_are_the_tokens_casts():
    x = synth.normal_f32(71, (20, 256))
    topk, _ = synth.moe_routing(72, 20, 5, 3)
    a, sfa, owned, layout, counts, slot = oracle.moe_dispatch_contiguous_fp8(x, topk, 5, 1024)
    q, s = oracle.per_token_cast_to_fp8(x)
    for t in range(20):
        for row in slot[t]:
            assert row >= 0 and np.array_equal(a[row], q[t]) and np.array_equal(sfa[row], s[t])
    assert owned.sum() == 60 and not a[~owned].any()
