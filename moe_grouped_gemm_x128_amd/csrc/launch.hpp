// Kernel launchers of libdgmi, called by the host-side ABI (abi.cpp) after
// it has validated every argument.  Internal interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace dgmi {

// Quantizer arguments.  x is viewed as [G, R, K] (R = rows, or N for the
// per-block cast); strides in elements.  sf is [G, R or ceil(R/128), ceil(K/128)].
struct QuantArgs {
  const void* x;
  int32_t x_bf16;
  int64_t sx_g, sx_r;
  uint8_t* q;
  int64_t sq_g, sq_r;
  float* sf;
  int64_t ssf_g, ssf_r, ssf_k;
  int32_t G, R, K;
  int32_t ue8m0;
};

// Casts of an MN-major x: element (g, r, k) at x[g * sx_g + k * sx_k + r]
// (sx_r unused); vec: 16-byte (f32) / 8-byte (bf16) loads along r are
// aligned; qvec: q rows take 16-byte stores.
struct QuantTArgs : QuantArgs {
  int64_t sx_k;
  int32_t vec, qvec;
};

// Per-token cast of the tokens x [T, K] (G = 1, R = T) into the rows their
// slots name: slot[t * k + j] = e * max_m + row in [0, rows) selects row
// `row` of group e of q and sf (strides sq_g / sq_r, ssf_g / ssf_r); other
// values are skipped.
struct QuantScatterArgs : QuantArgs {
  const int32_t* slot;
  int32_t k, max_m, rows;
  int32_t flat;  // sq_g == max_m * sq_r and ssf_g == max_m * ssf_r
  int32_t qvec;  // q, sq_r and sq_g are multiples of 16 bytes
};

// MoE routing into the masked layout (moe.hip): topk [T, k] contiguous,
// slot [T, k] contiguous, src [G, max_m] contiguous, masked_m [G].
struct MoeRouteArgs {
  const int32_t* topk;
  int32_t T, k, G, max_m;
  int32_t vec;  // topk is 16-byte aligned: 16-byte loads
  int32_t* masked_m;
  int32_t* slot;
  int32_t* src;
  // contiguous layout: counts [G] (written by the count pass, then read),
  // layout [mcap / 128], capacity mcap rows (a multiple of 128)
  int32_t* counts;
  int32_t* layout;
  int64_t mcap;
  int32_t align;  // region granule in rows: 128 or 256
};

// MoE combine (moe.hip): d BF16 [G, max_m, N] (strides in elements), slot and
// w [T, k] contiguous, y BF16 [T, N] (row stride sy).
struct MoeCombineArgs {
  const uint16_t* d;
  int64_t sd_g, sd_r;
  int32_t G, max_m, N;
  const int32_t* slot;
  const float* w;
  int32_t T, k;
  uint16_t* y;
  int64_t sy;
  int32_t vec, y_vec;  // 16-byte loads of d rows, 16-byte stores of y rows
  int32_t col_blocks;  // set by the launcher
};

struct PackArgs {
  const float* x;
  int64_t sx_g, sx_r;
  int32_t* out;
  int64_t so_g, so_r;
  int32_t G, R, n, nw;
  int32_t* invalid;
};

// Tile configuration of a GEMM launch (a pure function of the shapes).
struct TileCfg {
  int bm, bn, threads, lds_bytes;
  int variant;  // index of the kernel instance
};

hipError_t launch_per_token(const QuantArgs& p, hipStream_t stream);
hipError_t launch_per_token_scatter(const QuantScatterArgs& p, hipStream_t stream);
hipError_t launch_cast_mn(const QuantTArgs& p, bool per_block, hipStream_t stream);
hipError_t launch_moe_route(const MoeRouteArgs& p, hipStream_t stream);
hipError_t launch_moe_route_contiguous(const MoeRouteArgs& p, hipStream_t stream);
hipError_t launch_moe_combine(const MoeCombineArgs& p, hipStream_t stream);
hipError_t launch_per_block(const QuantArgs& p, hipStream_t stream);
hipError_t launch_pack_ue8m0(const PackArgs& p, hipStream_t stream);

// Launch plan of a GEMM: one launch over all N columns, or two launches on
// the same stream, cfg[0] over columns [0, n_split) and cfg[1] over
// [n_split, N) (n_split a multiple of 256).
struct GemmPlan {
  TileCfg cfg[2];
  int64_t n_split;
  int parts;
};

// Contiguous layouts of more 128-row blocks than this take 128-row tiles: the
// 256-row tiles list their tile starts in LDS (4 bytes a block).
constexpr int64_t RUNS_MAX_BLOCKS = 8192;

// GEMMs: the plan for (mode, G, M, N, K) and the grid of each launch (pure
// functions of the shapes), and the launchers.
GemmPlan fp8_gemm_plan(int mode, int64_t G, int64_t M, int64_t N, int64_t K, int sf_fmt);
GemmPlan bf16_gemm_plan(int mode, int64_t G, int64_t M, int64_t N, int64_t K);
int64_t gemm_grid(const TileCfg& cfg, int mode, int64_t G, int64_t M, int64_t N);
int64_t plan_grid(const GemmPlan& plan, int part, int mode, int64_t G, int64_t M, int64_t N);
// static LDS of one workgroup of launch `part` (0 past the plan's launches)
int plan_lds(const GemmPlan& plan, int part, int mode);
// sf_fmt: SF_F32 or SF_UE8M0, plus SF_ROWB for one B scale per row of B;
// an MN-major A or B (p.a_mn, p.b_mn: dense, block scales, BF16 d) takes the
// plan of fp8_mn_gemm_plan
hipError_t launch_fp8_gemm(GemmParams p, int mode, int sf_fmt, hipStream_t stream);
GemmPlan fp8_mn_gemm_plan();
// Dense FP8 GEMM whose output D is cast per token to FP8 (p.q, p.sfq) in the
// epilogue; sf_fmt SF_F32 or SF_UE8M0, plus SF_ROWB for one B scale per row.
GemmPlan fp8_out_gemm_plan(int64_t M, int64_t N, int sf_fmt);
hipError_t launch_fp8_gemm_fp8_out(GemmParams p, int sf_fmt, hipStream_t stream);
// BF16 GEMMs: same kernel body; byte strides in p, no scales
hipError_t launch_bf16_gemm(GemmParams p, int mode, hipStream_t stream);

}  // namespace dgmi
