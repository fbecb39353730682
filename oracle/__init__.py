"""CPU oracle for the block-scaled FP8 (grouped) GEMM path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package imports this
package; only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import, call or execute it.  It shares no code,
tables, constants or helpers with the HIP library: every bit pattern is
decoded here from the format definitions, and every result is computed in
float64 from the plain definition of the operation.

Modules
  formats  -- OCP E4M3 ("fn") decode/encode, bf16 decode and rounding,
              UE8M0 decode.
  quant    -- per-token (1x128) and per-block (128x128) FP8 quantizers and
              the UE8M0 packing of four scales into one int32.
  gemm     -- dense, contiguous-grouped and masked-grouped FP8 GEMMs with
              fine-grained scales, the dense one with its output cast
              per token to FP8, and the dense, contiguous-grouped and
              masked-grouped BF16 GEMMs.
  moe      -- the steps either side of the masked grouped GEMM: routing of
              (token, choice) pairs into expert buffers with the per-token
              cast, and the weighted combine of the GEMM's rows per token.

Sources (the pages this follows):
  * "DeepInside DeepGEMM: Unpacking DeepSeek's Unified Tensor Core Library
    for SM90 and SM100", section 2 (NT layout, FP32 scaling factors, packed
    UE8M0 four to an int), section 4 (the fp8_gemm_nt example with per
    128-wide K-block scale factors and D = C + A @ B.T) and section 5 (the
    FP8 cast of a tensor fused into the kernel that produces it).
  * "DeepGEMM CUDA Graph Compatibility for Masked Grouped GEMMs", section
    "Tensor-Based Metadata Arguments" (masked_m on the device,
    max_m_per_group) and the capture example.
  * "[GH-ISSUE #414] pack_ue8m0_to_int is not CUDA Graph capture safe",
    sections "Summary" (validity predicate) and "Expected behavior" (the
    packing expression).
  * "DeepGEMM tested by Novita AI", section "Technological Innovations"
    (per-block promotion of the MMA result into an FP32 accumulator) and the
    sections on the contiguous and masked grouped layouts.

Every function is pinned by ``tests/test_oracle_*.py`` (marked "not gpu")
against closed forms, library routines, brute force and invariants; see the
docstring of each function for its pin.
"""

from .formats import (
    E4M3_MAX,
    e4m3_decode,
    e4m3_encode,
    bf16_decode,
    bf16_round,
    ue8m0_decode,
)
from .quant import per_token_cast_to_fp8, per_block_cast_to_fp8, pack_ue8m0_to_int, AMAX_FLOOR
from .gemm import (
    bf16_gemm_nt,
    fp8_gemm_nn,
    fp8_gemm_nt,
    fp8_gemm_nt_fp8_out,
    fp8_gemm_tn,
    fp8_gemm_tt,
    m_grouped_bf16_gemm_nt_contiguous,
    m_grouped_fp8_gemm_nt_contiguous,
    m_grouped_fp8_gemm_nt_masked,
    m_grouped_bf16_gemm_nt_masked,
    scales_from_packed_ue8m0,
)
from .moe import moe_route, moe_dispatch_fp8, moe_combine, moe_route_contiguous, moe_dispatch_contiguous_fp8

__all__ = [
    "E4M3_MAX",
    "AMAX_FLOOR",
    "e4m3_decode",
    "e4m3_encode",
    "bf16_decode",
    "bf16_round",
    "ue8m0_decode",
    "per_token_cast_to_fp8",
    "per_block_cast_to_fp8",
    "pack_ue8m0_to_int",
    "bf16_gemm_nt",
    "m_grouped_bf16_gemm_nt_contiguous",
    "fp8_gemm_nn",
    "fp8_gemm_nt",
    "fp8_gemm_nt_fp8_out",
    "fp8_gemm_tn",
    "fp8_gemm_tt",
    "m_grouped_fp8_gemm_nt_contiguous",
    "m_grouped_fp8_gemm_nt_masked",
    "m_grouped_bf16_gemm_nt_masked",
    "scales_from_packed_ue8m0",
    "moe_route",
    "moe_dispatch_fp8",
    "moe_combine",
    "moe_route_contiguous",
    "moe_dispatch_contiguous_fp8",
]
