"""MoE dispatch into the masked layout and combine (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The steps either side of the masked grouped GEMM on one GPU ("DeepGEMM
tested by Novita AI", the masked layout for decode: each expert owns a
padded buffer of max_m rows of which masked_m[e] are valid; "DeepGEMM CUDA
Graph Compatibility for Masked Grouped GEMMs", last section: the fused MoE
path chains the input casting and the masked GEMM calls under the same
stateless launch model).  The pages name the steps, not their definition;
the reading taken:

  * Route: topk_idx [T, k] holds the expert of each (token, choice); a
    value outside [0, G) routes nowhere.  Pairs routed to expert e take its
    rows 0, 1, 2, ... in row-major (t, j) order; pairs beyond max_m rows are
    dropped.  masked_m[e] = min(count_e, max_m); slot[t, j] = e * max_m +
    row (or -1: not routed or dropped); src[e, row] = t.
  * Cast: row r < masked_m[e] of expert e's buffer is token src[e, r]
    cast per token to FP8 exactly as per_token_cast_to_fp8 casts it.
  * Combine: y[t] = sum over j with slot[t, j] >= 0 of w[t, j] * D[slot[t,
    j]], where D is the masked GEMM's BF16 output [G, max_m, N].
  * Contiguous layout (prefill, "DeepGEMM tested by Novita AI", contiguous
    layout: groups concatenated along M in 128-row blocks, a group id per
    block): expert e's pairs fill a region of ceil(count_e / align) * align
    rows (align 128 or 256: whole blocks, or whole 256-row tiles) that
    starts where expert e - 1's region ends; rows past the capacity Mcap are
    dropped; blocks past the last region get id -1.  slot[t, j] is
    the row in the concatenated buffer (or -1); rows of a region past its
    count are padding that no token owns.

Pins: tests/test_oracle_moe.py (a hand-worked routing example with its
expected table, capacity overflow, invariants on random routings, and the
combine's closed forms).
"""

import numpy as np

from .formats import bf16_decode
from .quant import per_token_cast_to_fp8


def moe_route(topk_idx, G, max_m):
    """Returns (masked_m int32 [G], slot int32 [T, k], src int32 [G, max_m]
    with -1 where no token was placed, counts int64 [G] before capping)."""
    topk = np.asarray(topk_idx, dtype=np.int64)
    T, k = topk.shape
    counts = np.zeros(G, dtype=np.int64)
    slot = np.full((T, k), -1, dtype=np.int32)
    src = np.full((G, max_m), -1, dtype=np.int32)
    for t in range(T):
        for j in range(k):
            e = int(topk[t, j])
            if e < 0 or e >= G:
                continue
            row = int(counts[e])
            counts[e] += 1
            if row < max_m:
                slot[t, j] = e * max_m + row
                src[e, row] = t
    masked_m = np.minimum(counts, max_m).astype(np.int32)
    return masked_m, slot, src, counts


def moe_dispatch_fp8(x, topk_idx, G, max_m, use_ue8m0=False):
    """Route, then cast the routed tokens into the expert buffers.

    x float32 [T, K].  Returns (a uint8 [G, max_m, K], sfa float32
    [G, max_m, ceil(K/128)], masked_m, slot, src); rows past masked_m[e] are
    zero in a and sfa (the device leaves them untouched)."""
    x = np.asarray(x, dtype=np.float32)
    T, K = x.shape
    masked_m, slot, src, _ = moe_route(topk_idx, G, max_m)
    nkb = -(-K // 128)
    a = np.zeros((G, max_m, K), dtype=np.uint8)
    sfa = np.zeros((G, max_m, nkb), dtype=np.float32)
    for e in range(G):
        n = int(masked_m[e])
        if n:
            a[e, :n], sfa[e, :n] = per_token_cast_to_fp8(x[src[e, :n]], use_ue8m0)
    return a, sfa, masked_m, slot, src


def moe_combine(d_bits, slot, topk_weights):
    """y [T, N] float64 = sum_j w[t, j] * D[slot[t, j]] over slot >= 0.

    d_bits uint16 [G, max_m, N] (BF16 patterns), slot int32 [T, k],
    topk_weights float32 [T, k]."""
    D = bf16_decode(d_bits)
    G, max_m, N = D.shape
    rows = D.reshape(G * max_m, N)
    slot = np.asarray(slot, dtype=np.int64)
    w = np.asarray(topk_weights, dtype=np.float64)
    T, k = slot.shape
    y = np.zeros((T, N), dtype=np.float64)
    for j in range(k):
        ok = slot[:, j] >= 0
        y[ok] += w[ok, j][:, None] * rows[slot[ok, j]]
    return y


def moe_route_contiguous(topk_idx, G, Mcap, align=128):
    """Returns (counts int64 [G] before capping, slot int32 [T, k],
    grouped_layout int32 [Mcap / 128], start int64 [G] first row of each
    expert's region)."""
    topk = np.asarray(topk_idx, dtype=np.int64)
    T, k = topk.shape
    counts = np.zeros(G, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = int(topk[t, j])
            if 0 <= e < G:
                counts[e] += 1
    blocks = -(-counts // align) * (align // 128)
    start = np.concatenate([[0], np.cumsum(blocks)[:-1]]) * 128
    layout = np.full(Mcap // 128, -1, dtype=np.int32)
    for e in range(G):
        b0 = start[e] // 128
        for b in range(b0, min(b0 + blocks[e], Mcap // 128)):
            layout[b] = e
    slot = np.full((T, k), -1, dtype=np.int32)
    seen = np.zeros(G, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = int(topk[t, j])
            if e < 0 or e >= G:
                continue
            row = start[e] + seen[e]
            seen[e] += 1
            if row < Mcap:
                slot[t, j] = row
    return counts, slot, layout, start


def moe_dispatch_contiguous_fp8(x, topk_idx, G, Mcap, use_ue8m0=False, align=128):
    """Route into the contiguous layout and cast the routed tokens.

    Returns (a uint8 [Mcap, K], sfa float32 [Mcap, ceil(K/128)], owned bool
    [Mcap] (rows a token was cast into), grouped_layout, counts, slot)."""
    x = np.asarray(x, dtype=np.float32)
    T, K = x.shape
    counts, slot, layout, _ = moe_route_contiguous(topk_idx, G, Mcap, align)
    a = np.zeros((Mcap, K), dtype=np.uint8)
    sfa = np.zeros((Mcap, -(-K // 128)), dtype=np.float32)
    owned = np.zeros(Mcap, dtype=bool)
    q, sf = per_token_cast_to_fp8(x, use_ue8m0) if T else (np.zeros((0, K), np.uint8), None)
    for t in range(T):
        for row in slot[t]:
            if row >= 0:
                a[row], sfa[row], owned[row] = q[t], sf[t], True
    return a, sfa, owned, layout, counts, slot
