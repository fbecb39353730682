// Masked grouped BF16 GEMM for gfx950 ("DeepGEMM CUDA Graph Compatibility
// for Masked Grouped GEMMs": m_grouped_bf16_gemm_nt_masked(a, b, d,
// masked_m, max_m_per_group), capture example and section "Tensor-Based
// Metadata Arguments").
//
//   D[g, m, :] = A[g, m, :] . B[g]^T   for m < clamp(masked_m[g], 0, max_m)
//
// BF16 operands on v_mfma_f32_16x16x32_bf16, FP32 accumulation in the MFMA
// accumulators, BF16 out (round to nearest even).  The grid is
// G x ceil(max_m/BM) x ceil(N/BN), fixed by the shapes; masked_m is read on
// the device only: a tile starting at or past masked_m[g] exits at once,
// fragments wholly past it skip their MFMAs, and rows past it are never
// stored.  The K loop stages 64-element (128-byte) K slices of the A and B
// tiles through double-buffered LDS with the same swizzled 128-byte rows as
// the FP8 kernel.

#include "common.hpp"
#include "launch.hpp"

namespace dgmi {

namespace {

constexpr int BKE = 64;  // K elements per stage (128 bytes per row)

__device__ __forceinline__ int lds_off(int r, int c) { return r * 128 + ((c ^ (r & 7)) << 4); }

template <int BM, int BN, int WM, int WN>
struct TileShape {
  static constexpr int NT = WM * WN * 64;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 16, FN = TN / 16;
  static constexpr int ACH = BM * 8 / NT, BCH = BN * 8 / NT;
  static constexpr int STAGE = (BM + BN) * 128;
  static_assert((BM * 8) % NT == 0 && (BN * 8) % NT == 0, "tile rows must split evenly over threads");
};

__device__ __forceinline__ bf16x8 as_bf16x8(i32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM* WN * 64) void bf16_masked_kernel(const Bf16GemmParams p) {
  using T = TileShape<BM, BN, WM, WN>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * T::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  int bid = blockIdx.x;
  const int per = p.tiles_m * p.tiles_n;
  const int g = bid / per;
  bid -= g * per;
  const int tm = bid / p.tiles_n, tn = bid - (bid / p.tiles_n) * p.tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  int v = p.masked_m[g];
  v = v < 0 ? 0 : (v > p.max_m ? p.max_m : v);
  if (m0 >= v) return;
  const int row_lim = v;

  const uint8_t* A = reinterpret_cast<const uint8_t*>(p.a + (int64_t)g * p.a_gs);
  const uint8_t* B = reinterpret_cast<const uint8_t*>(p.b + (int64_t)g * p.b_gs);
  uint16_t* D = p.d + (int64_t)g * p.d_gs;
  const int64_t lda_b = p.lda * 2, ldb_b = p.ldb * 2;

  const uint8_t* asrc[T::ACH];
  int aoff[T::ACH];
#pragma unroll
  for (int j = 0; j < T::ACH; ++j) {
    const int q = tid + j * T::NT, r = q >> 3, c = q & 7;
    asrc[j] = A + (int64_t)min(m0 + r, row_lim - 1) * lda_b + c * 16;
    aoff[j] = lds_off(r, c);
  }
  const uint8_t* bsrc[T::BCH];
  int boff[T::BCH];
#pragma unroll
  for (int j = 0; j < T::BCH; ++j) {
    const int q = tid + j * T::NT, r = q >> 3, c = q & 7;
    bsrc[j] = B + (int64_t)min(n0 + r, p.N - 1) * ldb_b + c * 16;
    boff[j] = BM * 128 + lds_off(r, c);
  }

  f32x4 acc[T::FM][T::FN];
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fragments of this wave that hold at least one valid row
  const int wave_row0 = m0 + wm * T::TM;
  const int fm_live = min(T::FM, max(0, (row_lim - wave_row0 + 15) / 16));

  i32x4 ra[T::ACH], rb[T::BCH];
  auto gload = [&](int ks) {
    const int64_t off = (int64_t)ks * 128;
#pragma unroll
    for (int j = 0; j < T::ACH; ++j) ra[j] = *reinterpret_cast<const i32x4*>(asrc[j] + off);
#pragma unroll
    for (int j = 0; j < T::BCH; ++j) rb[j] = *reinterpret_cast<const i32x4*>(bsrc[j] + off);
  };
  auto lstore = [&](int st) {
    uint8_t* base = smem + st * T::STAGE;
#pragma unroll
    for (int j = 0; j < T::ACH; ++j) *reinterpret_cast<i32x4*>(base + aoff[j]) = ra[j];
#pragma unroll
    for (int j = 0; j < T::BCH; ++j) *reinterpret_cast<i32x4*>(base + boff[j]) = rb[j];
  };

  const int KS = p.K / BKE;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int ks = 0; ks < KS; ++ks) {
    const int st = ks & 1;
    const bool more = ks + 1 < KS;
    if (more) gload(ks + 1);
    const uint8_t* As = smem + st * T::STAGE;
    const uint8_t* Bs = As + BM * 128;
    const int fr = lane & 15;
    const int fc = lane >> 4;  // 16-B chunk within each 32-element half
    i32x4 b0[T::FN], b1[T::FN];
#pragma unroll
    for (int j = 0; j < T::FN; ++j) {
      const int r = wn * T::TN + j * 16 + fr;
      b0[j] = *reinterpret_cast<const i32x4*>(Bs + lds_off(r, fc));
      b1[j] = *reinterpret_cast<const i32x4*>(Bs + lds_off(r, 4 + fc));
    }
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
      if (i < fm_live) {
        const int r = wm * T::TM + i * 16 + fr;
        const i32x4 a0 = *reinterpret_cast<const i32x4*>(As + lds_off(r, fc));
        const i32x4 a1 = *reinterpret_cast<const i32x4*>(As + lds_off(r, 4 + fc));
#pragma unroll
        for (int j = 0; j < T::FN; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a0), as_bf16x8(b0[j]), acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a1), as_bf16x8(b1[j]), acc[i][j], 0, 0, 0);
        }
      }
    }
    if (more) lstore(st ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < T::FM; ++i) {
#pragma unroll
    for (int j = 0; j < T::FN; ++j) {
      const int col = n0 + wn * T::TN + j * 16 + (lane & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = wave_row0 + i * 16 + (lane >> 4) * 4 + e;
        if (row < row_lim && col < p.N) D[(int64_t)row * p.ldd + col] = f32_to_bf16_rne(acc[i][j][e]);
      }
    }
  }
}

}  // namespace

TileCfg bf16_masked_config(int64_t G, int64_t max_m, int64_t N, int64_t K) {
  (void)G; (void)max_m; (void)N; (void)K;
  TileCfg c;
  c.bm = 128;
  c.bn = 128;
  c.threads = 256;
  c.lds_bytes = 2 * (128 + 128) * 128;
  c.variant = 0;
  return c;
}

int64_t bf16_masked_grid(const TileCfg& cfg, int64_t G, int64_t max_m, int64_t N) {
  return G * ((max_m + cfg.bm - 1) / cfg.bm) * ((N + cfg.bn - 1) / cfg.bn);
}

hipError_t launch_bf16_masked(Bf16GemmParams p, hipStream_t stream) {
  const TileCfg cfg = bf16_masked_config(p.G, p.max_m, p.N, p.K);
  p.tiles_m = (p.max_m + cfg.bm - 1) / cfg.bm;
  p.tiles_n = (p.N + cfg.bn - 1) / cfg.bn;
  const int64_t grid = bf16_masked_grid(cfg, p.G, p.max_m, p.N);
  if (grid == 0) return hipSuccess;
  bf16_masked_kernel<128, 128, 2, 2><<<dim3((unsigned)grid), dim3(256), 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace dgmi
