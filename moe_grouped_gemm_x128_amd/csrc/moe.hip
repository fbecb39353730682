// The steps either side of the masked grouped GEMM on one GPU, gfx950:
// routing of (token, choice) pairs into per-expert buffers (the masked
// layout of "DeepGEMM tested by Novita AI", decode section: max_m rows per
// expert, masked_m[e] of them valid), whose per-token FP8 cast is the
// quantizer's own kernel casting each token once and storing its codes into
// every row the routing gives it ("DeepInside DeepGEMM", section 5: the cast
// done by the kernel that produces the tensor), and the weighted combine of
// the GEMM's output rows per token.
//
//   route:   pairs routed to expert e take its rows 0, 1, ... in row-major
//            (token, choice) order; pairs beyond max_m rows are dropped;
//            ids outside [0, G) route nowhere.
//            masked_m[e] = min(count, max_m); slot[t, j] = e * max_m + row
//            or -1; src[e, row] = t.
//   combine: y[t] = sum over j with a valid slot of w[t, j] * d[slot[t, j]]
//            (FP32, j in increasing order, one FMA per term), BF16 out.
//
// Routing is deterministic without atomics or scratch memory: one workgroup
// per expert scans every pair (the routing table is small and stays in L2)
// and ranks its matches with a workgroup-wide prefix sum.

#include "common.hpp"
#include "launch.hpp"

namespace dgmi {

namespace {

enum RouteMode : int { ROUTE_MASKED = 0, ROUTE_COUNT = 1, ROUTE_CONTIG = 2 };

constexpr int ROUTE_THREADS = 1024;
constexpr int ROUTE_PER_THREAD = 8;  // consecutive pairs per thread per pass (8192 per pass)

// Sum of v over the workgroup (every thread gets it).
__device__ __forceinline__ int64_t block_sum(int64_t v, int64_t* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  int64_t total = 0;
#pragma unroll
  for (int w = 0; w < ROUTE_THREADS / 64; ++w) total += red[w];
  __syncthreads();
  return total;
}

// MODE: ROUTE_MASKED (rows of expert e's own buffer, capacity max_m),
// ROUTE_COUNT (counts[e] only), ROUTE_CONTIG (rows of the concatenated
// buffer: expert e's region of ceil(count / align) * align rows starts after
// the regions of experts 0..e-1, from counts; capacity mcap rows; the region's
// blocks get id e in layout, blocks past the last region -1).  One workgroup
// per expert (ROUTE_CONTIG: at least one, for the layout).
template <int MODE>
__global__ __launch_bounds__(ROUTE_THREADS) void moe_route_kernel(const MoeRouteArgs p) {
  __shared__ int wave_sum[ROUTE_THREADS / 64];
  __shared__ int64_t red[ROUTE_THREADS / 64];
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n = (int64_t)p.T * p.k;
  int64_t start = 0;  // ROUTE_CONTIG: first row of e's region
  if constexpr (MODE == ROUTE_CONTIG) {
    int64_t before = 0, all = 0;
    for (int f = tid; f < p.G; f += ROUTE_THREADS) {
      const int64_t rows = ((int64_t)p.counts[f] + p.align - 1) / p.align * p.align;
      all += rows;
      before += f < e ? rows : 0;
    }
    start = block_sum(before, red);
    const int64_t total = block_sum(all, red);
    const int64_t nblk = p.mcap / 128;
    if (e < p.G) {
      const int64_t b0 = start / 128, b1 = (start + ((int64_t)p.counts[e] + p.align - 1) / p.align * p.align) / 128;
      for (int64_t b = b0 + tid; b < b1 && b < nblk; b += ROUTE_THREADS) p.layout[b] = e;
    }
    if (e == 0)
      for (int64_t b = total / 128 + tid; b < nblk; b += ROUTE_THREADS) p.layout[b] = -1;
    if (e >= p.G) return;  // (no experts: the layout only)
  }
  int count = 0;  // pairs routed to e so far (the same in every thread)
  for (int64_t base = 0; base < n; base += (int64_t)ROUTE_THREADS * ROUTE_PER_THREAD) {
    const int64_t i0 = base + (int64_t)tid * ROUTE_PER_THREAD;
    int v[ROUTE_PER_THREAD];
    if (p.vec && i0 + ROUTE_PER_THREAD <= n) {
#pragma unroll
      for (int q = 0; q < ROUTE_PER_THREAD; q += 4) {
        const i32x4 t4 = *reinterpret_cast<const i32x4*>(p.topk + i0 + q);
        v[q] = t4[0];
        v[q + 1] = t4[1];
        v[q + 2] = t4[2];
        v[q + 3] = t4[3];
      }
    } else {
#pragma unroll
      for (int q = 0; q < ROUTE_PER_THREAD; ++q) v[q] = i0 + q < n ? p.topk[i0 + q] : -1;
    }
    int mine = 0;
#pragma unroll
    for (int q = 0; q < ROUTE_PER_THREAD; ++q) mine += v[q] == e ? 1 : 0;
    // inclusive prefix of `mine` over the wave, then over the waves
    int incl = mine;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int up = __shfl_up(incl, off, 64);
      if (lane >= off) incl += up;
    }
    if (lane == 63) wave_sum[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < ROUTE_THREADS / 64; ++w) {
      const int s = wave_sum[w];
      before += w < wave ? s : 0;
      total += s;
    }
    __syncthreads();  // every wave has read wave_sum before the next pass writes it
    int rank = count + before + incl - mine;
    if constexpr (MODE != ROUTE_COUNT) {
#pragma unroll
      for (int q = 0; q < ROUTE_PER_THREAD; ++q) {
        const int64_t i = i0 + q;
        if (v[q] == e) {
          if constexpr (MODE == ROUTE_MASKED) {
            if (rank < p.max_m) {
              p.slot[i] = e * p.max_m + rank;
              p.src[(int64_t)e * p.max_m + rank] = (int32_t)(i / p.k);
            } else {
              p.slot[i] = -1;  // over capacity: dropped
            }
          } else {
            const int64_t row = start + rank;
            p.slot[i] = row < p.mcap ? (int32_t)row : -1;  // past the capacity: dropped
          }
          ++rank;
        } else if (e == 0 && i < n && (v[q] < 0 || v[q] >= p.G)) {
          p.slot[i] = -1;  // routed nowhere
        }
      }
    }
    count += total;
  }
  if (tid == 0) {
    if constexpr (MODE == ROUTE_MASKED) p.masked_m[e] = count < p.max_m ? count : p.max_m;
    if constexpr (MODE == ROUTE_COUNT) p.counts[e] = count;
  }
}

constexpr int COMBINE_THREADS = 256;  // 8 columns per thread

__global__ __launch_bounds__(COMBINE_THREADS) void moe_combine_kernel(const MoeCombineArgs p) {
  const int t = blockIdx.x / p.col_blocks;
  const int c0 = ((blockIdx.x % p.col_blocks) * COMBINE_THREADS + threadIdx.x) * 8;
  if (c0 >= p.N) return;
  const bool full = p.vec && c0 + 8 <= p.N;
  f32x4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
  const int64_t rows = (int64_t)p.G * p.max_m;
  for (int j = 0; j < p.k; ++j) {
    const int32_t s = p.slot[(int64_t)t * p.k + j];
    if (s < 0 || s >= rows) continue;  // not routed, dropped, or not a row of d
    const float w = p.w[(int64_t)t * p.k + j];
    const uint16_t* row = p.d + (int64_t)(s / p.max_m) * p.sd_g + (int64_t)(s % p.max_m) * p.sd_r + c0;
    if (full) {
      const i32x4 v = *reinterpret_cast<const i32x4*>(row);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        acc0[2 * h] = __builtin_fmaf(w, __uint_as_float((uint32_t)v[h] << 16), acc0[2 * h]);
        acc0[2 * h + 1] = __builtin_fmaf(w, __uint_as_float((uint32_t)v[h] & 0xffff0000u), acc0[2 * h + 1]);
        acc1[2 * h] = __builtin_fmaf(w, __uint_as_float((uint32_t)v[h + 2] << 16), acc1[2 * h]);
        acc1[2 * h + 1] = __builtin_fmaf(w, __uint_as_float((uint32_t)v[h + 2] & 0xffff0000u), acc1[2 * h + 1]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (c0 + e < p.N) {
          const float x = bf16_to_f32(row[e]);
          if (e < 4) acc0[e] = __builtin_fmaf(w, x, acc0[e]);
          else acc1[e - 4] = __builtin_fmaf(w, x, acc1[e - 4]);
        }
      }
    }
  }
  const i32x2 lo = to_bf16x4_bits(acc0), hi = to_bf16x4_bits(acc1);
  uint16_t* yrow = p.y + (int64_t)t * p.sy + c0;
  if (full && p.y_vec) {
    *reinterpret_cast<i32x4*>(yrow) = i32x4{lo[0], lo[1], hi[0], hi[1]};
  } else {
    const uint32_t wds[4] = {(uint32_t)lo[0], (uint32_t)lo[1], (uint32_t)hi[0], (uint32_t)hi[1]};
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (c0 + e < p.N) yrow[e] = (uint16_t)(wds[e / 2] >> (16 * (e & 1)));
  }
}

}  // namespace

hipError_t launch_moe_route(const MoeRouteArgs& p, hipStream_t stream) {
  if (p.G == 0) return hipSuccess;
  moe_route_kernel<ROUTE_MASKED><<<dim3((unsigned)p.G), dim3(ROUTE_THREADS), 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_moe_route_contiguous(const MoeRouteArgs& p, hipStream_t stream) {
  if (p.G > 0) {
    moe_route_kernel<ROUTE_COUNT><<<dim3((unsigned)p.G), dim3(ROUTE_THREADS), 0, stream>>>(p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  moe_route_kernel<ROUTE_CONTIG><<<dim3((unsigned)(p.G > 0 ? p.G : 1)), dim3(ROUTE_THREADS), 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_moe_combine(const MoeCombineArgs& p, hipStream_t stream) {
  if (p.T == 0 || p.N == 0) return hipSuccess;
  MoeCombineArgs q = p;
  q.col_blocks = (p.N + COMBINE_THREADS * 8 - 1) / (COMBINE_THREADS * 8);
  moe_combine_kernel<<<dim3((unsigned)((int64_t)p.T * q.col_blocks)), dim3(COMBINE_THREADS), 0, stream>>>(q);
  return hipGetLastError();
}

}  // namespace dgmi
