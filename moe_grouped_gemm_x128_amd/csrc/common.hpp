// Internal definitions shared by the HIP kernels and the host-side ABI of
// libdgmi (gfx950 only).  Not part of the public interface (include/dgmi.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dgmi {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

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
  const void* c;        // optional accumulate input C shaped like D (BF16 or F32), may be d
  int64_t ldc;          // row stride of c in elements
  int64_t c_gs;         // masked: stride of c between groups, in elements
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
  // FP8 output (dense only): D cast per token to E4M3 q [M, N] (row stride
  // ldq bytes) with FP32 scales sfq [M, ceil(N/128)] (strides in elements)
  uint8_t* q;
  float* sfq;
  int64_t ldq, sfq_sm, sfq_sn;
  int32_t q_ue8m0;
  int32_t d_f32;  // d holds F32 (row stride ldd in F32 elements; d_gs in BF16-sized units, 2 per element)
  // dense FP8 only: A / B stored MN-major ([K, M] / [K, N], rows contiguous);
  // lda / ldb are then the byte strides between consecutive K-rows
  int32_t a_mn, b_mn;
};

// Output of a GEMM: BF16 D, D cast per token to FP8, or the FP32 D itself.
enum GemmOut : int { OUT_BF16 = 0, OUT_FP8 = 1, OUT_F32 = 2 };

// float -> bfloat16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Four floats -> four bfloat16 (bits, little-endian in two words), rounded to
// nearest even by the hardware conversion (two v_cvt_pk_bf16_f32): the
// values of f32_to_bf16_rne for every non-NaN input; NaN stays NaN.
__device__ __forceinline__ i32x2 to_bf16x4_bits(f32x4 v) {
  return __builtin_bit_cast(i32x2, __builtin_convertvector(v, bf16x4));
}

// The same four values rounded by f32_to_bf16_rne (integer arithmetic).
__device__ __forceinline__ i32x2 to_bf16x4_bits_int(f32x4 v) {
  return i32x2{(int)((uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16)),
               (int)((uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16))};
}

// 2^(e-127) for an unsigned E8M0 exponent byte (byte 0 is the subnormal 2^-127).
__device__ __forceinline__ float ue8m0_to_f32(uint32_t e) {
  return e == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(e << 23);
}

// ---------------------------------------------------------------------------
// FP8 (E4M3) casting of a 1x128 or 128x128 block (the quantizers, and the
// GEMM epilogue that writes FP8 output):
//   amax = max |x| over the block, floored at 1e-4
//   s    = amax / 448 (correctly rounded), or the next power of two (UE8M0)
//   q    = e4m3(clamp(x / s, -448, 448)) with the correctly rounded quotient
// ---------------------------------------------------------------------------

// Block scale from the block maximum.
__device__ __forceinline__ float block_scale(float amax, int ue8m0) {
  amax = fmaxf(amax, 1e-4f);
  float s = __fdiv_rn(amax, 448.0f);
  if (ue8m0) {
    uint32_t u = __float_as_uint(s);  // s is a positive normal number
    if (u & 0x007fffffu) u = (u & 0x7f800000u) + 0x00800000u;
    s = __uint_as_float(u);
  }
  return s;
}

// The correctly rounded binary32 quotient x / s, given r = RN(1 / s) (one
// correctly rounded division per block): y = RN(x r) is within one ulp of
// x / s, the residual x - y s is exact with an FMA, and RN(y + r (x - y s))
// is the correctly rounded quotient (Markstein's correction step) whenever
// it is a normal number.  Smaller quotients (below 2^-126) encode to E4M3
// zero whichever way they round, so the FP8 bytes are those of x / s.  The
// sign is copied from x (s > 0): the correction would turn -0 into +0.
struct Recip {
  float s, r;
};
__device__ __forceinline__ Recip recip_of(float s) { return Recip{s, __fdiv_rn(1.0f, s)}; }
__device__ __forceinline__ float quot(float x, Recip d) {
  const float y = x * d.r;
  const float e = __builtin_fmaf(-y, d.s, x);
  return __builtin_copysignf(__builtin_fmaf(e, d.r, y), x);
}

// Four values -> four E4M3 bytes (little-endian in one word), x / s rounded
// to nearest even by the hardware conversion after clamping to +-448.
__device__ __forceinline__ uint32_t encode4(const float v[4], Recip d) {
  float t[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) t[j] = fminf(fmaxf(quot(v[j], d), -448.0f), 448.0f);
  // bytes 0-1, then 2-3 (the first conversion's old word only supplies
  // bits 16-31, which the second overwrites)
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(t[0], t[1], __float_as_int(t[0]), false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(t[2], t[3], w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ uint32_t encode1(float v, Recip d) {
  float t = fminf(fmaxf(quot(v, d), -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(t, 0.0f, 0, false) & 0xffu;
}

}  // namespace dgmi
