"""Block-scaled FP8 (grouped) GEMM library for MI355X (gfx950).

The compute path is the HIP library ``libdgmi.so`` built from ``csrc/``
(``python -m moe_grouped_gemm_x128_amd.build``); this package holds its thin
ctypes binding (same names and argument order as ``include/dgmi.h``) and the
seeded synthetic input generators.  Importing the package loads nothing; the
library is opened on first use and a missing library raises.
"""

from .binding import (  # noqa: F401
    DgmiError,
    load_library,
    last_error,
    dgmi_init,
    fp8_gemm_nt,
    fp8_gemm_nt_fp8_out,
    fp8_gemm_nn,
    fp8_gemm_tn,
    fp8_gemm_tt,
    m_grouped_fp8_gemm_nt_contiguous,
    m_grouped_fp8_gemm_nt_masked,
    m_grouped_bf16_gemm_nt_masked,
    bf16_gemm_nt,
    m_grouped_bf16_gemm_nt_contiguous,
    per_token_cast_to_fp8,
    per_block_cast_to_fp8,
    pack_ue8m0_to_int,
    moe_dispatch_masked_fp8,
    moe_dispatch_contiguous_fp8,
    moe_combine,
    query_config,
)
