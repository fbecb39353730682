// Internal definitions shared by the HIP kernels and the host-side ABI of
// libdgmi (gfx950 only).  Not part of the public interface (include/dgmi.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dgmi {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Scale-factor storage of the FP8 GEMMs: FP32 or packed UE8M0, and the flag
// SF_ROWB when B carries one scale per row (per 1x128 block) instead of one
// per 128x128 block.
enum ScaleFmt : int { SF_F32 = 0, SF_UE8M0 = 1, SF_ROWB = 2 };

// Tile scheduling of the GEMM kernel.
enum GemmMode : int { MODE_DENSE = 0, MODE_CONTIG = 1, MODE_MASKED = 2 };

// Arguments of one GEMM launch (block-scaled FP8, or BF16 without scales).
// The A and B operands are addressed in BYTES: lda, ldb and their group
// strides are byte strides and k_bytes is the row length in bytes (K for
// FP8, 2K for BF16).  Scale strides are in elements (32-bit words); d
// strides in BF16 elements.  "gs" is the stride between groups (masked: per
// expert buffer; contiguous: per B).
struct GemmParams {
  const uint8_t* a;
  const uint8_t* b;
  const void* sfa;  // FP8 only
  const void* sfb;  // FP8 only
  uint16_t* d;
  const void* c;        // dense only: optional accumulate input C [M, N] (BF16 or F32), may be d
  int64_t ldc;          // row stride of c in elements
  int32_t c_f32;        // c holds F32 (else BF16)
  const int32_t* meta;  // masked_m [G] or grouped_layout [M/128]; unused for dense
  int64_t lda, a_gs;
  int64_t ldb, b_gs;
  int64_t sfa_sm, sfa_sk, sfa_gs;
  int64_t sfb_sn, sfb_sk, sfb_gs;
  int64_t ldd, d_gs;
  int32_t M;       // dense: M; contiguous: Msum; masked: max_m
  int32_t N, k_bytes, G;
  int32_t tiles_m, tiles_n;
};

// float -> bfloat16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// 2^(e-127) for an unsigned E8M0 exponent byte (byte 0 is the subnormal 2^-127).
__device__ __forceinline__ float ue8m0_to_f32(uint32_t e) {
  return e == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(e << 23);
}

}  // namespace dgmi
