// FP8 quantizers (per-token 1x128 and per-block 128x128) and the UE8M0
// packing kernel, gfx950.
//
// What they compute ("DeepInside DeepGEMM", sections 2 and 5: FP32 scaling
// factors per block, packed UE8M0 scales four to an int, and the FP8
// casting helpers that feed fp8_gemm_nt):
//   amax = max |x| over the block, floored at 1e-4
//   s    = amax / 448                      (correctly rounded binary32 division)
//   s    = smallest power of two >= s      (UE8M0 scales only)
//   q    = e4m3(clamp(x / s, -448, 448))   (round to nearest even)
// Packing ("[GH-ISSUE #414] pack_ue8m0_to_int is not CUDA Graph capture
// safe", section "Expected behavior"): the exponent byte of four
// consecutive scales per int32; the value check of the issue's Summary is a
// device-side count, never a host synchronisation.
//
// All three are HBM-bound streaming kernels: one read of x and one write of
// q per element, with the block reduction held in registers.

#include "common.hpp"
#include "launch.hpp"

namespace dgmi {

namespace {

__device__ __forceinline__ float load_elem(const float* p) { return *p; }
__device__ __forceinline__ float load_elem(const uint16_t* p) { return bf16_to_f32(*p); }

// Four consecutive elements starting at p (16-B aligned for f32, 8-B for bf16).
__device__ __forceinline__ void load4(const float* p, float v[4]) {
  float4 t = *reinterpret_cast<const float4*>(p);
  v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
}
__device__ __forceinline__ void load4(const uint16_t* p, float v[4]) {
  uint2 t = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(t.x << 16);
  v[1] = __uint_as_float(t.x & 0xffff0000u);
  v[2] = __uint_as_float(t.y << 16);
  v[3] = __uint_as_float(t.y & 0xffff0000u);
}

// block_scale, Recip, quot, encode4 and encode1: common.hpp (shared with the
// GEMM epilogue that writes FP8 output).

// ---------------------------------------------------------------------------
// per-token: eight lanes per 1x128 block, 16 elements per lane in four
// chunks of four that lie 32 elements apart, so that each load instruction
// reads 128 contiguous bytes (F32) per block.  The block's scale and
// reciprocal (two correctly rounded divisions, executed by every lane) are
// spread over 16 elements per lane: the cast is bound by instruction issue,
// not by HBM, at four elements per lane.
// ---------------------------------------------------------------------------
constexpr int TOKEN_LANES = 8;     // lanes per block
constexpr int TOKEN_GROUPS = 256 / TOKEN_LANES;  // blocks per workgroup
constexpr int SCATTER_K = 8;  // destinations per token held in registers

// SCATTER (MoE dispatch): x is [T, K] (G = 1, R = T) and each token's
// codes and scales go to every row its slots name instead of row r of q.
// Its stores outnumber its loads (one per destination), so there each lane
// holds 16 consecutive elements: its codes leave as one 16-byte store per
// destination and a block's eight lanes write 128 contiguous bytes.
template <bool SCATTER>
__device__ __forceinline__ int chunk_offset(int c, int sub) {
  return SCATTER ? sub * 16 + c * 4 : c * 32 + sub * 4;
}

template <typename TIn, bool SCATTER = false, class Args = QuantArgs>
__global__ __launch_bounds__(256) void per_token_kernel(Args p) {
  const TIn* __restrict__ x = static_cast<const TIn*>(p.x);
  const int sub = threadIdx.x & (TOKEN_LANES - 1);
  const int KB = (p.K + 127) / 128;
  const int64_t total = (int64_t)p.G * p.R * KB;
  const int64_t grp = (int64_t)blockIdx.x * TOKEN_GROUPS + (threadIdx.x / TOKEN_LANES);
  if (grp >= total) return;  // whole 8-lane groups only; the shuffles below stay within a group
  const int kb = (int)(grp % KB);
  const int64_t rr = grp / KB;
  const int r = (int)(rr % p.R);
  const int g = (int)(rr / p.R);
  const TIn* xr = x + g * p.sx_g + r * p.sx_r;
  uint8_t* qr = p.q + g * p.sq_g + r * p.sq_r;
  // SCATTER: the destinations of this token's first SCATTER_K slots, read
  // once (q row offset in bytes, scale row offset in elements; -1: none)
  int64_t dq[SCATTER_K], ds[SCATTER_K];
  if constexpr (SCATTER) {
#pragma unroll
    for (int j = 0; j < SCATTER_K; ++j) {
      const int32_t sl = j < p.k ? p.slot[(int64_t)r * p.k + j] : -1;
      dq[j] = ds[j] = -1;
      if (sl >= 0 && sl < p.rows) {
        if (p.flat) {  // q and sf hold their groups back to back: no division
          dq[j] = (int64_t)sl * p.sq_r;
          ds[j] = (int64_t)sl * p.ssf_r;
        } else {
          const int e = sl / p.max_m, row = sl % p.max_m;
          dq[j] = e * p.sq_g + row * p.sq_r;
          ds[j] = e * p.ssf_g + row * p.ssf_r;
        }
      }
    }
  }

  float v[4][4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int k0 = kb * 128 + chunk_offset<SCATTER>(c, sub);
    if (k0 + 3 < p.K) {
      load4(xr + k0, v[c]);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[c][j] = (k0 + j < p.K) ? load_elem(xr + k0 + j) : 0.0f;
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[c][0]), fabsf(v[c][1])), fmaxf(fabsf(v[c][2]), fabsf(v[c][3]))));
#pragma unroll
  for (int off = TOKEN_LANES / 2; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, TOKEN_LANES));
  const float s = block_scale(amax, p.ue8m0);
  const Recip d = recip_of(s);

  if constexpr (SCATTER) {
    // cast once (elements past K are zeros and their bytes are not stored),
    // store to each destination row
    const int k0 = kb * 128 + sub * 16;
    uint32_t w[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) w[c] = encode4(v[c], d);
    const bool whole = p.qvec && k0 + 15 < p.K;
    auto put = [&](int64_t oq) {
      uint8_t* qd = p.q + oq + k0;
      if (whole) {
        *reinterpret_cast<i32x4*>(qd) = i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
      } else {
        for (int i = 0; i < 16; ++i)
          if (k0 + i < p.K) qd[i] = (uint8_t)(w[i / 4] >> (8 * (i % 4)));
      }
    };
#pragma unroll
    for (int j = 0; j < SCATTER_K; ++j)
      if (dq[j] >= 0) put(dq[j]);
    for (int j = SCATTER_K; j < p.k; ++j) {  // more choices per token than SCATTER_K
      const int32_t sl = p.slot[(int64_t)r * p.k + j];
      if (sl < 0 || sl >= p.rows) continue;  // routed nowhere or dropped
      const int e = sl / p.max_m, row = sl % p.max_m;
      put(e * p.sq_g + row * p.sq_r);
    }
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int k0 = kb * 128 + c * 32 + sub * 4;
      if (k0 + 3 < p.K) {
        *reinterpret_cast<uint32_t*>(qr + k0) = encode4(v[c], d);
      } else {
        for (int j = 0; j < 4; ++j)
          if (k0 + j < p.K) qr[k0 + j] = (uint8_t)encode1(v[c][j], d);
      }
    }
  }
  if (sub == 0) {
    if constexpr (SCATTER) {
#pragma unroll
      for (int j = 0; j < SCATTER_K; ++j)
        if (ds[j] >= 0) p.sf[ds[j] + kb * p.ssf_k] = s;
      for (int j = SCATTER_K; j < p.k; ++j) {
        const int32_t sl = p.slot[(int64_t)r * p.k + j];
        if (sl < 0 || sl >= p.rows) continue;
        const int e = sl / p.max_m, row = sl % p.max_m;
        p.sf[e * p.ssf_g + row * p.ssf_r + kb * p.ssf_k] = s;
      }
    } else {
      p.sf[g * p.ssf_g + r * p.ssf_r + kb * p.ssf_k] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// per-block: one workgroup (256 threads) per 128x128 block; thread t owns
// columns 4*(t%32)..+3 of rows t/32 + 8j, j = 0..15 (64 values in registers)
// ---------------------------------------------------------------------------
template <typename TIn>
__global__ __launch_bounds__(256) void per_block_kernel(QuantArgs p) {
  __shared__ float red[4];
  const TIn* __restrict__ x = static_cast<const TIn*>(p.x);
  const int NB = (p.R + 127) / 128, KB = (p.K + 127) / 128;
  int blk = blockIdx.x;
  const int kb = blk % KB;
  blk /= KB;
  const int nb = blk % NB;
  const int g = blk / NB;
  const int tid = threadIdx.x;
  const int c0 = kb * 128 + (tid & 31) * 4;
  const int rbase = nb * 128 + (tid >> 5);
  const TIn* xg = x + g * p.sx_g;
  const bool full_cols = c0 + 3 < p.K;

  float v[16][4];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int r = rbase + 8 * j;
    if (r < p.R && full_cols) {
      load4(xg + (int64_t)r * p.sx_r + c0, v[j]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[j][e] = (r < p.R && c0 + e < p.K) ? load_elem(xg + (int64_t)r * p.sx_r + c0 + e) : 0.0f;
    }
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[j][0]), fabsf(v[j][1])), fmaxf(fabsf(v[j][2]), fabsf(v[j][3]))));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = block_scale(amax, p.ue8m0);
  const Recip d = recip_of(s);

  uint8_t* qg = p.q + g * p.sq_g;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int r = rbase + 8 * j;
    if (r >= p.R) continue;
    uint8_t* qr = qg + (int64_t)r * p.sq_r;
    if (full_cols) {
      *reinterpret_cast<uint32_t*>(qr + c0) = encode4(v[j], d);
    } else {
      for (int e = 0; e < 4; ++e)
        if (c0 + e < p.K) qr[c0 + e] = (uint8_t)encode1(v[j][e], d);
    }
  }
  if (tid == 0) p.sf[g * p.ssf_g + nb * p.ssf_r + kb * p.ssf_k] = s;
}

// ---------------------------------------------------------------------------
// UE8M0 pack: one thread per output int32
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pack_ue8m0_kernel(PackArgs p) {
  const int64_t total = (int64_t)p.G * p.R * p.nw;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int bad = 0;
  if (i < total) {
    const int w = (int)(i % p.nw);
    const int64_t rr = i / p.nw;
    const int r = (int)(rr % p.R);
    const int g = (int)(rr / p.R);
    const float* xr = p.x + g * p.sx_g + r * p.sx_r;
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = 4 * w + j;
      if (k < p.n) {
        const uint32_t bits = __float_as_uint(xr[k]);
        word |= ((bits >> 23) & 0xffu) << (8 * j);
        bad += ((bits >> 31) != 0u || (bits & 0x007fffffu) != 0u) ? 1 : 0;
      }
    }
    p.out[g * p.so_g + r * p.so_r + w] = (int32_t)word;
  }
  if (p.invalid != nullptr) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) bad += __shfl_xor(bad, off, 64);
    if ((threadIdx.x & 63) == 0 && bad != 0) atomicAdd(p.invalid, bad);
  }
}

// ---------------------------------------------------------------------------
// Casts of an MN-major x: element (g, r, k) at x[g * sx_g + k * sx_k + r]
// (the transpose of a row-major [K, R] tensor), written K-major as the NT
// GEMM reads it ("DeepInside DeepGEMM", section 5: transposition and FP8
// casting fused into one producer instead of separate helpers).  One
// workgroup per 128 (K) x TR (rows) tile.  Each thread loads 4 x 4 blocks
// (four consecutive rows at four consecutive k: loads run along the rows,
// coalesced) and keeps them in registers; the block maximum is reduced from
// registers (per-token: over the 16 threads holding the same rows, through
// shuffles and an LDS exchange between the four waves; per-block: over the
// workgroup).  encode4 on a column of a 4 x 4 block gives one row's four
// consecutive codes as one word, so only the codes pass through LDS, as
// [r][k] bytes, and each row leaves as contiguous 16-byte pieces.  The scale
// and codes are those of the row-major casts above, bit for bit.
// ---------------------------------------------------------------------------
template <typename TIn, bool PER_BLOCK>
__global__ __launch_bounds__(256) void cast_mn_kernel(QuantTArgs p) {
  constexpr int TR = PER_BLOCK ? 128 : 64;  // rows of the tile
  constexpr int RQ = TR / 4;                // row quads
  constexpr int NB = 128 * TR / 16 / 256;   // 4 x 4 blocks per thread (2 or 4)
  constexpr int KQS = 256 / RQ;             // k-quad stride between a thread's blocks
  constexpr int P = 128 + 16;               // LDS row pitch of the codes (bytes)
  __shared__ __attribute__((aligned(16))) uint8_t codes[TR * P];
  __shared__ float part[4 * 64];
  const TIn* __restrict__ x = static_cast<const TIn*>(p.x);
  const int RB = (p.R + TR - 1) / TR, KB = (p.K + 127) / 128;
  int blk = blockIdx.x;
  const int kb = blk % KB;
  blk /= KB;
  const int rb = blk % RB;
  const int g = blk / RB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r0 = rb * TR, k0 = kb * 128;
  const TIn* xg = x + g * p.sx_g;
  const int rq = tid % RQ;  // rows 4 rq .. 4 rq + 3 of the tile

  // phase 1: NB blocks of 4 k x 4 rows (v[b][kk][j]: k = 4 kq + kk, row 4 rq + j)
  float v[NB][4][4];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int kq = tid / RQ + KQS * b;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int gk = k0 + 4 * kq + kk, gr = r0 + 4 * rq;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[b][kk][j] = 0.0f;
      if (gk < p.K) {
        const TIn* src = xg + (int64_t)gk * p.sx_k + gr;
        if (p.vec && gr + 3 < p.R) {
          load4(src, v[b][kk]);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (gr + j < p.R) v[b][kk][j] = load_elem(src + j);
        }
      }
    }
  }
  // block maxima: per row (per-token) or over the tile (per-block)
  float m[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int j = 0; j < 4; ++j) m[j] = fmaxf(m[j], fabsf(v[b][kk][j]));
  float amax[4];
  if constexpr (PER_BLOCK) {
    float t = fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3]));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) t = fmaxf(t, __shfl_xor(t, off, 64));
    if (lane == 0) part[wave] = t;
    __syncthreads();
    const float a = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
#pragma unroll
    for (int j = 0; j < 4; ++j) amax[j] = a;
  } else {
    // the 16 threads of row quad rq: lanes rq, rq + 16, rq + 32, rq + 48 of each wave
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m[j] = fmaxf(m[j], __shfl_xor(m[j], 16, 64));
      m[j] = fmaxf(m[j], __shfl_xor(m[j], 32, 64));
    }
    if (lane < 16) {
#pragma unroll
      for (int j = 0; j < 4; ++j) part[wave * 64 + 4 * rq + j] = m[j];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rr = 4 * rq + j;
      amax[j] = fmaxf(fmaxf(part[rr], part[64 + rr]), fmaxf(part[128 + rr], part[192 + rr]));
    }
  }
  float sc[4];
  Recip d[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    sc[j] = block_scale(amax[j], p.ue8m0);
    d[j] = recip_of(sc[j]);
  }
  // phase 2: codes of row 4 rq + j at k = 4 kq .. 4 kq + 3 as one word into LDS
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int kq = tid / RQ + KQS * b;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float col[4] = {v[b][0][j], v[b][1][j], v[b][2][j], v[b][3][j]};
      *reinterpret_cast<uint32_t*>(codes + (4 * rq + j) * P + 4 * kq) = encode4(col, d[j]);
    }
  }
  // scales: per row (the thread of k-quad 0 of the row quad), or one per tile
  if constexpr (PER_BLOCK) {
    if (tid == 0) p.sf[g * p.ssf_g + (int64_t)rb * p.ssf_r + kb * p.ssf_k] = sc[0];
  } else {
    if (tid < RQ) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (r0 + 4 * rq + j < p.R) p.sf[g * p.ssf_g + (int64_t)(r0 + 4 * rq + j) * p.ssf_r + kb * p.ssf_k] = sc[j];
    }
  }
  __syncthreads();
  // phase 3: each row's 128 codes as eight 16-byte pieces
#pragma unroll
  for (int i = 0; i < TR * 8 / 256; ++i) {
    const int piece = tid + 256 * i;
    const int r = piece / 8, kp = (piece % 8) * 16;
    const int gr = r0 + r, gk = k0 + kp;
    if (gr >= p.R || gk >= p.K) continue;
    const i32x4 w = *reinterpret_cast<const i32x4*>(codes + r * P + kp);
    uint8_t* qd = p.q + g * p.sq_g + (int64_t)gr * p.sq_r + gk;
    if (p.qvec && gk + 16 <= p.K) {
      *reinterpret_cast<i32x4*>(qd) = w;
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (gk + e < p.K) qd[e] = (uint8_t)((uint32_t)w[e / 4] >> (8 * (e & 3)));
    }
  }
}

}  // namespace

hipError_t launch_cast_mn(const QuantTArgs& p, bool per_block, hipStream_t stream) {
  const int TR = per_block ? 128 : 64;
  const int64_t blocks = (int64_t)p.G * ((p.R + TR - 1) / TR) * ((p.K + 127) / 128);
  if (blocks == 0) return hipSuccess;
  const dim3 g((unsigned)blocks), b(256);
  if (per_block) {
    if (p.x_bf16) cast_mn_kernel<uint16_t, true><<<g, b, 0, stream>>>(p);
    else cast_mn_kernel<float, true><<<g, b, 0, stream>>>(p);
  } else {
    if (p.x_bf16) cast_mn_kernel<uint16_t, false><<<g, b, 0, stream>>>(p);
    else cast_mn_kernel<float, false><<<g, b, 0, stream>>>(p);
  }
  return hipGetLastError();
}

hipError_t launch_per_token(const QuantArgs& p, hipStream_t stream) {
  const int64_t KB = (p.K + 127) / 128;
  const int64_t blocks = ((int64_t)p.G * p.R * KB + TOKEN_GROUPS - 1) / TOKEN_GROUPS;
  if (blocks == 0) return hipSuccess;
  if (p.x_bf16)
    per_token_kernel<uint16_t><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(p);
  else
    per_token_kernel<float><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_per_token_scatter(const QuantScatterArgs& p, hipStream_t stream) {
  const int64_t KB = (p.K + 127) / 128;
  const int64_t blocks = ((int64_t)p.G * p.R * KB + TOKEN_GROUPS - 1) / TOKEN_GROUPS;
  if (blocks == 0) return hipSuccess;
  if (p.x_bf16)
    per_token_kernel<uint16_t, true, QuantScatterArgs><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(p);
  else
    per_token_kernel<float, true, QuantScatterArgs><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_per_block(const QuantArgs& p, hipStream_t stream) {
  const int64_t blocks = (int64_t)p.G * ((p.R + 127) / 128) * ((p.K + 127) / 128);
  if (blocks == 0) return hipSuccess;
  if (p.x_bf16)
    per_block_kernel<uint16_t><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(p);
  else
    per_block_kernel<float><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_pack_ue8m0(const PackArgs& p, hipStream_t stream) {
  const int64_t total = (int64_t)p.G * p.R * p.nw;
  if (total == 0) return hipSuccess;
  pack_ue8m0_kernel<<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace dgmi
