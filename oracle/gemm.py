"""Block-scaled FP8 GEMMs and the masked BF16 GEMM, in float64 (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Definition followed ("DeepInside DeepGEMM", section 2 NT layout and section 4
example; "DeepGEMM tested by Novita AI", section "Technological Innovations",
per-block promotion): with A [M, K] and B [N, K] holding E4M3 codes, sfa
[M, ceil(K/128)] one scale per row per 128-wide K-block and sfb
[ceil(N/128), ceil(K/128)] one scale per 128x128 block of B,

    P_kb[m, n] = sum_{k in block kb} dec(A[m, k]) * dec(B[n, k])
    D[m, n]    = sum_kb P_kb[m, n] * (sfa[m, kb] * sfb[n // 128, kb])

and D is returned as float64 (no bf16 rounding: the comparison allows for
the device's bf16 output).  sfb may instead hold one scale per row of B,
[N, ceil(K/128)] (the per-row b_sf of the dense example in "DeepInside
DeepGEMM", section 4), and then

    D[m, n]    = sum_kb P_kb[m, n] * (sfa[m, kb] * sfb[n, kb]);

the form is told by the row count of sfb (N rows with N != ceil(N/128);
for N = 1 the two forms coincide).

Exactness: every E4M3 value is an integer multiple of 2^-9 below 2^9, so a
product is an integer multiple of 2^-18 below 2^18 and a 128-term block sum
is an integer multiple of 2^-18 below 2^25; P_kb is therefore exact in
float64 whatever order the matmul library sums in.  sfa*sfb (two binary32
values) is exact in float64.  Only the final multiply and the sum over
blocks round, at float64 precision.

Pins: tests/test_oracle_gemm.py (pure-Python brute force on tiny shapes,
also for the NN / TN / TT storage layouts, the closed form for one-hot B
with power-of-two scales, numpy float64 matmul when every scale is 1, and
the masked/contiguous invariants).
"""

import numpy as np

from .formats import e4m3_decode, bf16_decode, bf16_round, ue8m0_decode
from .quant import per_token_cast_to_fp8

BLOCK = 128


def _scaled_block_gemm(a, b, sfa, sfb):
    """D = sum_kb (A_kb B_kb^T) * (sfa[:, kb] outer sfb-per-column[:, kb])."""
    A = e4m3_decode(a)
    B = e4m3_decode(b)
    M, K = A.shape
    N = B.shape[0]
    sfa = np.asarray(sfa, dtype=np.float64)
    sfb = np.asarray(sfb, dtype=np.float64)
    nkb = -(-K // BLOCK)
    nnb = -(-N // BLOCK)
    if sfb.shape[0] == N and N != nnb:
        scale_row = np.arange(N)  # one scale per row of B
    elif sfb.shape[0] == nnb:
        scale_row = np.arange(N) // BLOCK  # one scale per 128-row block of B
    else:
        raise ValueError(f"sfb has {sfb.shape[0]} rows; expected {nnb} (128x128 blocks) or {N} (per row)")
    D = np.zeros((M, N), dtype=np.float64)
    for kb in range(nkb):
        ks = slice(kb * BLOCK, (kb + 1) * BLOCK)
        P = A[:, ks] @ B[:, ks].T
        D += P * (sfa[:, kb][:, None] * sfb[scale_row, kb][None, :])
    return D


def fp8_gemm_nt(a, b, sfa, sfb, c=None):
    """Dense D = C + A . B^T with block scales.

    a uint8 [M, K], b uint8 [N, K] (E4M3 codes), sfa float [M, ceil(K/128)],
    sfb float [ceil(N/128), ceil(K/128)] or, one per row, [N, ceil(K/128)],
    optional c [M, N] (float64).
    Returns float64 [M, N].
    """
    D = _scaled_block_gemm(np.asarray(a), np.asarray(b), sfa, sfb)
    if c is not None:
        D = D + np.asarray(c, dtype=np.float64)
    return D


def fp8_gemm_nn(a, b_kn, sfa, sfb, c=None):
    """The NN layout ("DeepInside DeepGEMM", section 2: NT, NN, TN and TT):
    A stored [M, K], B stored [K, N]; D[m, n] = C + sum_k A[m, k] B[k, n] with
    the same block scales (sfa per row of A and 128-wide K-block, sfb per
    128 columns of D and K-block)."""
    return fp8_gemm_nt(a, np.asarray(b_kn).T, sfa, sfb, c)


def fp8_gemm_tn(a_km, b_kn, sfa, sfb, c=None):
    """The TN layout: A stored [K, M], B stored [K, N]."""
    return fp8_gemm_nt(np.asarray(a_km).T, np.asarray(b_kn).T, sfa, sfb, c)


def fp8_gemm_tt(a_km, b, sfa, sfb, c=None):
    """The TT layout: A stored [K, M], B stored [N, K]."""
    return fp8_gemm_nt(np.asarray(a_km).T, b, sfa, sfb, c)


def fp8_gemm_nt_fp8_out(a, b, sfa, sfb, c=None, use_ue8m0=False):
    """The dense GEMM with its output cast to FP8 ("DeepInside DeepGEMM",
    section 5: the FP8 cast of a tensor belongs in the kernel that produces
    it, not in a separate helper).  The reading taken: the output is what
    the BF16 GEMM returns, cast per token as per_token_cast_to_fp8 casts a
    BF16 tensor -- D = C + A . B^T (fp8_gemm_nt), rounded once to bfloat16,
    then 1x128 blocks per row, s = amax/448 (UE8M0: rounded up to a power of
    two), q = e4m3(x / s).

    Returns (q uint8 [M, N] E4M3 codes, sf float32 [M, ceil(N/128)]).
    Pins: tests/test_oracle_gemm.py (hand-built products with a known block
    maximum of 448, where the code of each element follows from its value,
    including a value whose code changes if the BF16 rounding is skipped).
    """
    D = bf16_round(fp8_gemm_nt(a, b, sfa, sfb, c))
    return per_token_cast_to_fp8(D.astype(np.float32), use_ue8m0)


def m_grouped_fp8_gemm_nt_contiguous(a, b, sfa, sfb, grouped_layout):
    """Groups concatenated along M ("DeepGEMM tested by Novita AI", contiguous
    layout section).  Row m uses group g = grouped_layout[m // 128]; a block
    with g < 0 is skipped.

    a [Msum, K], b [G, N, K], sfa [Msum, nkb], sfb [G, nnb, nkb].
    Returns (D float64 [Msum, N], written bool [Msum]); rows with
    written=False are left to the caller's contents.
    """
    a = np.asarray(a)
    layout = np.asarray(grouped_layout, dtype=np.int64)
    Msum = a.shape[0]
    N = b.shape[1]
    D = np.zeros((Msum, N), dtype=np.float64)
    written = np.zeros(Msum, dtype=bool)
    for blk, g in enumerate(layout):
        if g < 0:
            continue
        rows = slice(blk * BLOCK, min((blk + 1) * BLOCK, Msum))
        D[rows] = _scaled_block_gemm(a[rows], b[g], sfa[rows], sfb[g])
        written[rows] = True
    return D, written


def _valid_rows(masked_m, max_m):
    """Rows computed for each group: masked_m clamped to [0, max_m]."""
    return [int(min(max(int(v), 0), max_m)) for v in np.asarray(masked_m).reshape(-1)]


def m_grouped_fp8_gemm_nt_masked(a, b, sfa, sfb, masked_m, max_m):
    """Masked grouped GEMM ("DeepGEMM CUDA Graph Compatibility for Masked
    Grouped GEMMs", section "Tensor-Based Metadata Arguments"): group g
    computes only its first masked_m[g] rows of a padded [max_m, K] buffer.

    a [G, max_m, K], b [G, N, K], sfa [G, max_m, nkb], sfb [G, nnb, nkb].
    Returns (D float64 [G, max_m, N], written bool [G, max_m]).
    """
    G = b.shape[0]
    N = b.shape[1]
    D = np.zeros((G, max_m, N), dtype=np.float64)
    written = np.zeros((G, max_m), dtype=bool)
    for g, v in enumerate(_valid_rows(masked_m, max_m)):
        if v == 0:
            continue
        D[g, :v] = _scaled_block_gemm(a[g, :v], b[g], sfa[g, :v], sfb[g])
        written[g, :v] = True
    return D, written


def m_grouped_bf16_gemm_nt_masked(a_bits, b_bits, masked_m, max_m):
    """Masked grouped BF16 GEMM: D[g, m] = A[g, m] . B[g]^T for m < masked_m[g]
    (same page and section; signature of its capture example).

    a_bits uint16 [G, max_m, K], b_bits uint16 [G, N, K] (bfloat16 patterns).
    Returns (D float64 [G, max_m, N], written bool [G, max_m]).
    """
    G = b_bits.shape[0]
    N = b_bits.shape[1]
    D = np.zeros((G, max_m, N), dtype=np.float64)
    written = np.zeros((G, max_m), dtype=bool)
    for g, v in enumerate(_valid_rows(masked_m, max_m)):
        if v == 0:
            continue
        D[g, :v] = bf16_decode(a_bits[g, :v]) @ bf16_decode(b_bits[g]).T
        written[g, :v] = True
    return D, written


def bf16_gemm_nt(a_bits, b_bits, c=None):
    """Dense BF16 GEMM D = C + A . B^T ("DeepGEMM: Why DeepSeek Built Its Own
    BLAS Kernels", its table of primitives: the BF16 GEMM next to FP8; NT
    layout and accumulate form as for fp8_gemm_nt).

    a_bits uint16 [M, K], b_bits uint16 [N, K] (bfloat16 patterns), optional
    c [M, N] (float64).  Returns float64 [M, N].
    """
    D = bf16_decode(a_bits) @ bf16_decode(b_bits).T
    if c is not None:
        D = D + np.asarray(c, dtype=np.float64)
    return D


def m_grouped_bf16_gemm_nt_contiguous(a_bits, b_bits, grouped_layout):
    """Contiguous grouped BF16 GEMM: row m uses B[g] with g =
    grouped_layout[m // 128]; a block with g < 0 is skipped (same layout as
    m_grouped_fp8_gemm_nt_contiguous, without scales).

    a_bits uint16 [Msum, K], b_bits uint16 [G, N, K].
    Returns (D float64 [Msum, N], written bool [Msum]).
    """
    layout = np.asarray(grouped_layout, dtype=np.int64)
    Msum = a_bits.shape[0]
    N = b_bits.shape[1]
    D = np.zeros((Msum, N), dtype=np.float64)
    written = np.zeros(Msum, dtype=bool)
    for blk, g in enumerate(layout):
        if g < 0:
            continue
        rows = slice(blk * 128, min((blk + 1) * 128, Msum))
        D[rows] = bf16_decode(a_bits[rows]) @ bf16_decode(b_bits[g]).T
        written[rows] = True
    return D, written


def scales_from_packed_ue8m0(packed, n):
    """Unpack int32 words of four UE8M0 bytes back to float64 scales [..., n]
    (byte j of word i is the exponent of element 4i + j)."""
    words = np.asarray(packed, dtype=np.int32).view(np.uint32)
    out = np.empty(words.shape[:-1] + (n,), dtype=np.float64)
    for j in range(n):
        out[..., j] = ue8m0_decode((words[..., j // 4] >> np.uint32(8 * (j % 4))) & np.uint32(0xFF))
    return out
