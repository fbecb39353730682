// Block-scaled FP8 GEMM for gfx950: dense, contiguous-grouped and
// masked-grouped scheduling over one kernel body.
//
// What it computes ("DeepInside DeepGEMM", sections 2 and 4; "DeepGEMM
// tested by Novita AI", section "Technological Innovations"):
//   D[m, n] = sum_kb P_kb[m, n] * sfa[m, kb] * sfb[n / 128, kb],
//   P_kb    = A[m, kb*128 : kb*128+128] . B[n, same]^T
// Each 128-wide K-block is exactly one v_mfma_f32_16x16x128_f8f6f4 per
// 16x16 output fragment, computed into a fresh FP32 partial; the partial is
// then promoted into the FP32 accumulator with one FMA per element using the
// product of the row scale and the 128x128 block scale.  Output is BF16
// (round to nearest even).
//
// Schedulers ("DeepGEMM CUDA Graph Compatibility for Masked Grouped GEMMs",
// sections "Stateless Kernel Architecture" and "Tensor-Based Metadata
// Arguments"): the grid is a function of the shapes only.
//   dense      -- tiles of [M, N]
//   contiguous -- tiles of [Msum, N]; each 128-row block reads its group id
//                 from grouped_layout on the device, negative = skip
//   masked     -- G x tiles of [max_m, N]; a tile whose first row is at or
//                 beyond masked_m[g] exits at once, rows beyond masked_m[g]
//                 are never stored
//
// Data path per workgroup (BM x BN tile, WM x WN waves of 64 lanes):
//   HBM -> registers (16-B loads, coalesced along K) -> LDS (double
//   buffered, 128-B rows with the 16-B chunk index XOR-swizzled by the row)
//   -> MFMA operand fragments (two ds_read_b128 per 16x128 fragment).
// A row scales are staged through LDS with the tiles; the B block scale of
// a wave is one uniform value per K-block.

#include "common.hpp"
#include "launch.hpp"

namespace dgmi {

namespace {

constexpr int BK = 128;  // K-block = scale block = K of one MFMA

// Byte offset in a tile of 16-byte chunk c (0..7) of row r.
__device__ __forceinline__ int lds_off(int r, int c) { return r * 128 + ((c ^ (r & 7)) << 4); }

template <int BM, int BN, int WM, int WN>
struct TileShape {
  static constexpr int NT = WM * WN * 64;
  static constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
  static constexpr int FM = TM / 16, FN = TN / 16;  // 16x16 fragments per wave
  static constexpr int ACH = BM * 8 / NT;           // 16-B chunks per thread per stage
  static constexpr int BCH = BN * 8 / NT;
  static constexpr int STAGE = (BM + BN) * BK;      // bytes of one LDS stage
  static_assert((BM * 8) % NT == 0 && (BN * 8) % NT == 0, "tile rows must split evenly over threads");
  static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be whole fragments");
  static_assert(TN <= 128 && 128 % TN == 0, "a wave's columns must lie in one 128-column scale block");
  static_assert(BM <= NT, "one thread per tile row stages the A scales");
};

template <int SF>
__device__ __forceinline__ float load_scale(const void* base, int64_t idx_row, int kb, int64_t s_row, int64_t s_k) {
  if (SF == SF_F32) {
    return static_cast<const float*>(base)[idx_row * s_row + (int64_t)kb * s_k];
  } else {
    const uint32_t w = static_cast<const uint32_t*>(base)[idx_row * s_row + (int64_t)(kb >> 2) * s_k];
    return ue8m0_to_f32((w >> ((kb & 3) * 8)) & 0xffu);
  }
}

template <int BM, int BN, int WM, int WN, int MODE, int SF>
__global__ __launch_bounds__(WM* WN * 64) void fp8_gemm_kernel(const Fp8GemmParams p) {
  using T = TileShape<BM, BN, WM, WN>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * T::STAGE];
  __shared__ __attribute__((aligned(16))) float ssa[2][BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // ---- tile decode (depends on device metadata only through early exits)
  int bid = blockIdx.x;
  int g = 0;
  if (MODE == MODE_MASKED) {
    const int per = p.tiles_m * p.tiles_n;
    g = bid / per;
    bid -= g * per;
  }
  const int tm = bid / p.tiles_n, tn = bid - (bid / p.tiles_n) * p.tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;

  int row_lim = p.M;  // rows [0, row_lim) may be read and written
  int npass = 1;
  int pg[2] = {0, 0}, plo[2] = {0, 0}, phi[2] = {BM, BM};
  if (MODE == MODE_MASKED) {
    int v = p.meta[g];
    v = v < 0 ? 0 : (v > p.M ? p.M : v);
    if (m0 >= v) return;
    row_lim = v;
  } else if (MODE == MODE_CONTIG) {
    const int nblk = p.M / 128;
    const int b0 = m0 / 128;
    int g0 = p.meta[b0];
    if (g0 >= p.G) g0 = -1;
    int g1 = g0;
    if (BM == 256) {
      g1 = (b0 + 1 < nblk) ? p.meta[b0 + 1] : -1;
      if (g1 >= p.G) g1 = -1;
    }
    if (g0 == g1) {
      if (g0 < 0) return;
      pg[0] = g0;
    } else {
      npass = 0;
      if (g0 >= 0) { pg[npass] = g0; plo[npass] = 0; phi[npass] = 128; ++npass; }
      if (g1 >= 0) { pg[npass] = g1; plo[npass] = 128; phi[npass] = 256; ++npass; }
      if (npass == 0) return;
    }
  }

  const int KB = p.K / BK;
  const int NB = (p.N + 127) / 128;
  const int nb_wave = __builtin_amdgcn_readfirstlane(min((n0 + wn * T::TN) / 128, NB - 1));
  const uint8_t* A = p.a + (MODE == MODE_MASKED ? (int64_t)g * p.a_gs : 0);
  const int64_t sfa_g = (MODE == MODE_MASKED) ? (int64_t)g * p.sfa_gs : 0;
  uint16_t* D = p.d + (MODE == MODE_MASKED ? (int64_t)g * p.d_gs : 0);

  // per-thread global sources and LDS destinations of the tile loads
  const uint8_t* asrc[T::ACH];
  int aoff[T::ACH];
#pragma unroll
  for (int j = 0; j < T::ACH; ++j) {
    const int q = tid + j * T::NT, r = q >> 3, c = q & 7;
    asrc[j] = A + (int64_t)min(m0 + r, row_lim - 1) * p.lda + c * 16;
    aoff[j] = lds_off(r, c);
  }
  int boff[T::BCH];
  int brow[T::BCH];
#pragma unroll
  for (int j = 0; j < T::BCH; ++j) {
    const int q = tid + j * T::NT, r = q >> 3, c = q & 7;
    brow[j] = min(n0 + r, p.N - 1);
    boff[j] = BM * BK + lds_off(r, c);
  }
  const int64_t sa_row = min(m0 + (tid < BM ? tid : 0), row_lim - 1);

  for (int pass = 0; pass < npass; ++pass) {
    const int gg = (MODE == MODE_MASKED) ? g : pg[pass];
    const uint8_t* B = p.b + (int64_t)gg * p.b_gs;
    const void* sfa = static_cast<const char*>(p.sfa) + sfa_g * (SF == SF_F32 ? 4 : 4);
    const void* sfb = static_cast<const char*>(p.sfb) + (int64_t)gg * p.sfb_gs * 4;

    f32x4 acc[T::FM][T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int j = 0; j < T::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    i32x4 ra[T::ACH], rb[T::BCH];
    float rsa = 0.f, rsb = 0.f;
    auto gload = [&](int kb) {
#pragma unroll
      for (int j = 0; j < T::ACH; ++j) ra[j] = *reinterpret_cast<const i32x4*>(asrc[j] + (int64_t)kb * BK);
#pragma unroll
      for (int j = 0; j < T::BCH; ++j)
        rb[j] = *reinterpret_cast<const i32x4*>(B + (int64_t)brow[j] * p.ldb + (int64_t)kb * BK + ((tid + j * T::NT) & 7) * 16);
      if (tid < BM) rsa = load_scale<SF>(sfa, sa_row, kb, p.sfa_sm, p.sfa_sk);
      rsb = load_scale<SF>(sfb, nb_wave, kb, p.sfb_sn, p.sfb_sk);
    };
    auto lstore = [&](int st) {
      uint8_t* base = smem + st * T::STAGE;
#pragma unroll
      for (int j = 0; j < T::ACH; ++j) *reinterpret_cast<i32x4*>(base + aoff[j]) = ra[j];
#pragma unroll
      for (int j = 0; j < T::BCH; ++j) *reinterpret_cast<i32x4*>(base + boff[j]) = rb[j];
      if (tid < BM) ssa[st][tid] = rsa;
    };

    gload(0);
    lstore(0);
    float sb_cur = rsb;
    __syncthreads();

    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    for (int kb = 0; kb < KB; ++kb) {
      const int st = kb & 1;
      const bool more = kb + 1 < KB;
      if (more) gload(kb + 1);

      const uint8_t* As = smem + st * T::STAGE;
      const uint8_t* Bs = As + BM * BK;
      const int fr = lane & 15;          // fragment row (A) / column (B)
      const int fc = (lane >> 4) * 2;    // first of the lane's two 16-B K chunks
      i32x8 bf[T::FN];
#pragma unroll
      for (int j = 0; j < T::FN; ++j) {
        const int r = wn * T::TN + j * 16 + fr;
        const i32x4 lo = *reinterpret_cast<const i32x4*>(Bs + lds_off(r, fc));
        const i32x4 hi = *reinterpret_cast<const i32x4*>(Bs + lds_off(r, fc + 1));
        bf[j] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int i = 0; i < T::FM; ++i) {
        const int r = wm * T::TM + i * 16 + fr;
        const i32x4 lo = *reinterpret_cast<const i32x4*>(As + lds_off(r, fc));
        const i32x4 hi = *reinterpret_cast<const i32x4*>(As + lds_off(r, fc + 1));
        const i32x8 af = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        const f32x4 s = *reinterpret_cast<const f32x4*>(&ssa[st][wm * T::TM + i * 16 + (lane >> 4) * 4]) * sb_cur;
#pragma unroll
        for (int j = 0; j < T::FN; ++j) {
          const f32x4 part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], zero, 0, 0, 0, 0, 0, 0);
          acc[i][j] += part * s;
        }
      }
      if (more) {
        lstore(st ^ 1);
        sb_cur = rsb;
      }
      __syncthreads();
    }

    // ---- epilogue: BF16 out, rows < row_lim of this pass, columns < N
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
#pragma unroll
      for (int j = 0; j < T::FN; ++j) {
        const int col = n0 + wn * T::TN + j * 16 + (lane & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int rl = wm * T::TM + i * 16 + (lane >> 4) * 4 + e;
          const int row = m0 + rl;
          if (rl >= plo[pass] && rl < phi[pass] && row < row_lim && col < p.N)
            D[(int64_t)row * p.ldd + col] = f32_to_bf16_rne(acc[i][j][e]);
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_tile(const Fp8GemmParams& p, int mode, int sf_fmt, int64_t grid, hipStream_t stream) {
  const dim3 g((unsigned)grid), b(WM * WN * 64);
#define DGMI_LAUNCH(MODE_, SF_) fp8_gemm_kernel<BM, BN, WM, WN, MODE_, SF_><<<g, b, 0, stream>>>(p)
  if (sf_fmt == SF_F32) {
    if (mode == MODE_DENSE) DGMI_LAUNCH(MODE_DENSE, SF_F32);
    else if (mode == MODE_CONTIG) DGMI_LAUNCH(MODE_CONTIG, SF_F32);
    else DGMI_LAUNCH(MODE_MASKED, SF_F32);
  } else {
    if (mode == MODE_DENSE) DGMI_LAUNCH(MODE_DENSE, SF_UE8M0);
    else if (mode == MODE_CONTIG) DGMI_LAUNCH(MODE_CONTIG, SF_UE8M0);
    else DGMI_LAUNCH(MODE_MASKED, SF_UE8M0);
  }
#undef DGMI_LAUNCH
  return hipGetLastError();
}

}  // namespace

TileCfg fp8_gemm_config(int mode, int64_t G, int64_t M, int64_t N, int64_t K) {
  (void)mode; (void)G; (void)M; (void)N; (void)K;
  TileCfg c;
  c.bm = 128;
  c.bn = 128;
  c.threads = 256;
  c.lds_bytes = 2 * (128 + 128) * BK + 2 * 128 * 4;
  c.variant = 0;
  return c;
}

int64_t fp8_gemm_grid(const TileCfg& cfg, int mode, int64_t G, int64_t M, int64_t N) {
  const int64_t tm = (M + cfg.bm - 1) / cfg.bm, tn = (N + cfg.bn - 1) / cfg.bn;
  return (mode == MODE_MASKED ? G : 1) * tm * tn;
}

hipError_t launch_fp8_gemm(Fp8GemmParams p, int mode, int sf_fmt, hipStream_t stream) {
  const TileCfg cfg = fp8_gemm_config(mode, p.G, p.M, p.N, p.K);
  p.tiles_m = (p.M + cfg.bm - 1) / cfg.bm;
  p.tiles_n = (p.N + cfg.bn - 1) / cfg.bn;
  const int64_t grid = fp8_gemm_grid(cfg, mode, p.G, p.M, p.N);
  if (grid == 0) return hipSuccess;
  return launch_tile<128, 128, 2, 2>(p, mode, sf_fmt, grid, stream);
}

}  // namespace dgmi
