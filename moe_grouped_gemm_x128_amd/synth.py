"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module only draws random numbers and builds index metadata; it holds
none of the quantization or GEMM arithmetic.  All draws use numpy's PCG64
(``numpy.random.default_rng(seed)``).

Workloads are DeepSeek-V3-shaped MoE and dense GEMMs, the shapes the pages
benchmark ("DeepGEMM tested by Novita AI": contiguous layout for prefill,
masked layout for decode).  Values are N(0, 1) float32; there are no real
activations or weights here.
"""

import numpy as np

# ----------------------------------------------------------------------------
# workload definitions (sizes only)
# ----------------------------------------------------------------------------

DENSE_SMALL = dict(M=128, N=256, K=512, seed_a=101, seed_b=102)

# dense M=4096 shapes (N, K); seeds 201+2i / 202+2i
DENSE_V3_SHAPES = [(2112, 7168), (24576, 1536), (7168, 16384), (4096, 7168), (7168, 2048)]
DENSE_V3_M = 4096

# contiguous grouped prefill: 4 groups x 8192 rows; two (N, K) weight shapes
CONTIG = dict(G=4, rows_per_group=8192, shapes=[(4096, 7168), (7168, 2048)], seed_a=301, seed_b=302)

# masked grouped decode: 32 experts, 256-row padded buffer, mean 192 valid rows
MASKED = dict(G=32, max_m=256, shapes=[(4096, 7168), (7168, 2048)], seed_a=401, seed_b=402, seed_m=403)

# masked grouped decode under graph replay: 64 experts, 128-row buffer
MASKED_GRAPH = dict(G=64, max_m=128, N=7168, K=2048, seed_a=501, seed_b=502, seed_m=503)

# MoE decode around the masked GEMM: 768 tokens, each to 8 of 32 experts
# (mean 192 rows per expert, the masked decode's centre), 256-row buffers
MOE_DECODE = dict(T=768, k=8, G=32, max_m=256, N=4096, K=7168, seed_x=601, seed_b=602, seed_r=603)

# MoE prefill around the contiguous GEMM: 4096 tokens, each to 8 of 32 experts
# (1024 rows per expert on average), capacity T * k + 127 * G rounded to 128
MOE_PREFILL = dict(T=4096, k=8, G=32, N=4096, K=7168, seed_x=671, seed_b=672, seed_r=673)


def dense_v3_seeds(i):
    return 201 + 2 * i, 202 + 2 * i


# ----------------------------------------------------------------------------
# draws
# ----------------------------------------------------------------------------

def normal_f32(seed, shape):
    """N(0, 1) float32 array of the given shape from PCG64(seed)."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal(size=shape, dtype=np.float32)


def normal_f32_chunks(seed, shape):
    """Yield the same values as normal_f32(seed, shape), one leading-index
    slice at a time (keeps host memory bounded for multi-GB tensors)."""
    rng = np.random.default_rng(seed)
    for _ in range(shape[0]):
        yield rng.standard_normal(size=shape[1:], dtype=np.float32)


def masked_m_decode(seed, G, centre=192, lo=0.7, hi=1.3):
    """masked_m[g] = floor(centre * U(lo, hi)), one draw per group."""
    rng = np.random.default_rng(seed)
    return np.floor(centre * rng.uniform(lo, hi, size=G)).astype(np.int32)


def masked_m_uniform(seed, G, max_m):
    """masked_m[g] uniform over the integers 0..max_m inclusive."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, max_m + 1, size=G, dtype=np.int32)


def contiguous_layout(G, rows_per_group, block=128):
    """Group id of every 128-row block when G groups of rows_per_group rows
    are concatenated in order."""
    per = rows_per_group // block
    return np.repeat(np.arange(G, dtype=np.int32), per)


def shuffled_layout(seed, G, nblocks, p_skip=0.15):
    """Random group id per block, with about p_skip of the blocks marked -1
    (padding that the kernel must leave untouched)."""
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, G, size=nblocks, dtype=np.int32)
    ids[rng.uniform(size=nblocks) < p_skip] = -1
    return ids


def moe_routing(seed, T, G, k, p_none=0.0):
    """Routing of T tokens: each picks k distinct experts of G uniformly
    (topk_idx int32 [T, k]) with positive weights summing to 1 per token
    (float32 [T, k]); a fraction p_none of the choices is set to -1 (routed
    nowhere, as a token whose expert lives on another GPU)."""
    if k > G:
        raise ValueError(f"k = {k} distinct experts out of G = {G}")
    rng = np.random.default_rng(seed)
    idx = np.argsort(rng.uniform(size=(T, G)), axis=1)[:, :k].astype(np.int32)
    w = rng.uniform(0.05, 1.0, size=(T, k))
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    if p_none > 0:
        idx[rng.uniform(size=(T, k)) < p_none] = -1
    return idx, w


def bf16_bits_from_f32(x):
    """bfloat16 bit patterns (uint16) of float32 values, rounded to nearest
    even by torch's own CPU conversion (input preparation only)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)
