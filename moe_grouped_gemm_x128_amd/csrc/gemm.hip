// GEMM kernels of libdgmi for gfx950: the block-scaled FP8 GEMM (dense,
// contiguous-grouped and masked-grouped scheduling) and the masked BF16 GEMM,
// over one kernel body.
//
// What the FP8 kind computes ("DeepInside DeepGEMM", sections 2 and 4;
// "DeepGEMM tested by Novita AI", section "Technological Innovations"):
//   D[m, n] = sum_kb P_kb[m, n] * sfa[m, kb] * sfb[n / 128, kb],
//   P_kb    = A[m, kb*128 : kb*128+128] . B[n, same]^T
// Each 128-wide K-block is exactly one v_mfma_f32_16x16x128_f8f6f4 per
// 16x16 output fragment, computed into a fresh FP32 partial; the partial is
// then promoted into the FP32 accumulator with one FMA per element using the
// product of the row scale and the 128x128 block scale.  With power-of-two
// UE8M0 scales the promote is the MFMA's own: v_mfma_scale_f32_16x16x128_
// f8f6f4 multiplies by 2^(e-127) per A row and per B row and accumulates in
// place (the SM100 recipe of "DeepInside DeepGEMM", section 2, on CDNA4).
// Output is BF16 (round to nearest even).
//
// The BF16 kind ("DeepGEMM CUDA Graph Compatibility for Masked Grouped
// GEMMs", the masked BF16 call of its capture example) computes
// D = A . B^T on v_mfma_f32_16x16x32_bf16 with the FP32 accumulator in the
// MFMA itself; no scales.  Both kinds move 128-byte K-slices of every row
// (128 FP8 or 64 BF16 elements), so they share the data path below.
//
// Schedulers ("DeepGEMM CUDA Graph Compatibility for Masked Grouped GEMMs",
// sections "Stateless Kernel Architecture" and "Tensor-Based Metadata
// Arguments"): the grid is a function of the shapes only.
//   dense      -- tiles of [M, N]
//   contiguous -- tiles of [Msum, N]; each 128-row block reads its group id
//                 from grouped_layout on the device, negative = skip.  A
//                 256-row tile whose two 128-row blocks belong to different
//                 groups computes its first block; a second copy of the grid
//                 (blocks total..2*total-1) computes the second block of
//                 such tiles and exits at once everywhere else.
//   masked     -- G x tiles of [max_m, N]; a tile whose first row is at or
//                 beyond masked_m[g] exits at once, rows beyond masked_m[g]
//                 are never stored
//
// Data path per workgroup (BM x BN tile, WM x WN waves of 64 lanes,
// S = STAGES LDS stages of one K-slice each):
//   * HBM -> LDS with buffer loads that write LDS directly (no register
//     staging): each wave instruction fills 8 tile rows of 128 bytes; the
//     16-byte chunk c of row r is stored at slot c ^ h(r), so the 16 rows of
//     an MFMA fragment read at one chunk hit distinct banks.
//   * One continuous software pipeline over fragment groups (below): two
//     barriers per K-slice.  After the first (second fragment group) the B
//     tile of slice kb+S is loaded into the B part of the slice's stage;
//     after the second (before the last group) its A tile, so S-1 slices of
//     A and nearly S of B are always in flight.
//   * The MFMA takes the B fragment as its first operand: the 16x16 result
//     then holds, per lane, one output row (m = lane % 16) and four output
//     columns.  The B fragment rows are permuted so that the four fragments
//     of a wave give every lane 16 consecutive columns: one row scale per
//     lane per fragment row, and the BF16 epilogue stores 2 x 16 bytes per
//     lane per fragment row, straight from registers.
//   * Tile order is XCD-aware: workgroups are dealt to the 8 XCDs round
//     robin, so the block index is remapped to give each XCD a contiguous
//     band of tiles (its L2 then holds the shared A rows / B columns).

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace dgmi {

namespace {

constexpr int BK = 128;  // bytes of one K-slice per row (= one FP8 scale block)
constexpr int NUM_XCD = 8;

enum Kind : int { KIND_FP8 = 0, KIND_BF16 = 1 };

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediate that waits for vmcnt <= n only (gfx9 encoding: vmcnt
// bits [3:0] and [15:14], expcnt [6:4] and lgkmcnt [11:8] left at "no wait").
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
// ... and additionally lgkmcnt(0)
constexpr int vmcnt_lgkm0(int n) { return vmcnt_only(n) & ~(15 << 8); }

// LDS swizzle: 16-byte chunk c of tile row r is stored at slot c ^ h(r),
// with h linear over GF(2) in the row bits:
//   h(r) = (b0 ^ b3 ^ b5) | b1 << 1 | (b2 ^ b4) << 2.
// The MFMA fragment reads touch 16 rows at one chunk: A fragments rows
// r0 + 0..15 (bits 0-3 vary), B fragments the permuted rows of the epilogue
// layout (bits 0, 1, 4, 5 vary).  h is a bijection on the varying bits in
// both cases, for every group of 8 lanes and for every 16 lanes split by
// row parity, so the reads are free of bank conflicts with 32 or with 64
// four-byte banks.
__device__ __host__ constexpr int swz(int r) { return ((r ^ (r >> 3) ^ (r >> 5)) & 1) | (r & 2) | ((((r >> 2) ^ (r >> 4)) & 1) << 2); }
// Byte offset in a tile of 16-byte chunk c (0..7) of tile row r.
__device__ __forceinline__ int lds_off(int r, int c) { return r * 128 + ((c ^ swz(r)) << 4); }

template <int BM_, int BN_, int WM_, int WN_, int STAGES_>
struct TileShape {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, STAGES = STAGES_;
  static constexpr int NW = WM * WN;
  static constexpr int NT = NW * 64;
  static constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
  static constexpr int FM = TM / 16, FN = TN / 16;  // 16x16 fragments per wave
  static constexpr int A_LOADS = BM / (8 * NW);     // LDS-DMA instructions per wave per stage
  static constexpr int B_LOADS = BN / (8 * NW);
  static constexpr int LOADS = A_LOADS + B_LOADS;
  static constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK, STAGE = (BM + BN) * BK;
  static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "tile rows must split into 8-row wave loads");
  static_assert(FN == 4, "the epilogue packs four fragments into 16 consecutive columns");
  static_assert(TN == 64 && 128 % TN == 0, "a wave's columns must lie in one 128-column scale block");
  static constexpr int NBT = (BN + 127) / 128;      // 128-column scale blocks per tile
  static_assert(BM + NBT <= NT, "one thread per tile row stages the A scales, one per column block the B scale");
  static_assert(STAGES >= 2 && STAGES <= 3, "two or three LDS stages");
  static_assert(FM >= 3, "a K-slice has an early point (group 1) before its late point (last group)");
  template <int KIND>
  static constexpr int lds_bytes() { return STAGES * STAGE + (KIND == KIND_FP8 ? STAGES * NT * 4 : 0); }
};

// Raw 32-bit scale word of row/column-block idx_row for K-block kb: the FP32
// bits, or the packed UE8M0 word holding it (decoded by scale_value).
template <int SF>
__device__ __forceinline__ uint32_t load_scale_raw(const void* base, int64_t idx_row, int kb, int64_t s_row, int64_t s_k) {
  const uint32_t* p = static_cast<const uint32_t*>(base);
  return SF == SF_F32 ? p[idx_row * s_row + (int64_t)kb * s_k] : p[idx_row * s_row + (int64_t)(kb >> 2) * s_k];
}
template <int SF>
__device__ __forceinline__ float scale_value(uint32_t raw, int kb) {
  return SF == SF_F32 ? __uint_as_float(raw) : ue8m0_to_f32((raw >> ((kb & 3) * 8)) & 0xffu);
}

// Tile index of this workgroup after the XCD remap: the hardware deals
// block b to XCD b % 8; XCD x receives the contiguous tile range starting at
// x*q + min(x, r) (q = total / 8, r = total % 8).
__device__ __forceinline__ int xcd_remap(int b, int total) {
  const int q = total / NUM_XCD, r = total % NUM_XCD;
  const int x = b % NUM_XCD, local = b / NUM_XCD;
  return x * q + min(x, r) + local;
}

// Linear tile t -> (tm, tn), walking bands of `gm` tile rows column by column
// so that consecutive tiles share B columns and nearby A rows.
__device__ __forceinline__ void band_order(int t, int tiles_m, int tiles_n, int gm, int& tm, int& tn) {
  const int band = t / (gm * tiles_n);
  const int first = band * gm;
  const int rows = min(gm, tiles_m - first);
  const int in_band = t - band * gm * tiles_n;
  tm = first + in_band % rows;
  tn = in_band / rows;
}

__device__ __forceinline__ bf16x8 lo_bf16(const i32x8& v) { return __builtin_bit_cast(bf16x8, i32x4{v[0], v[1], v[2], v[3]}); }
__device__ __forceinline__ bf16x8 hi_bf16(const i32x8& v) { return __builtin_bit_cast(bf16x8, i32x4{v[4], v[5], v[6], v[7]}); }

template <class T, int KIND, int SF, int MODE>
__global__ __launch_bounds__(T::NT) void gemm_kernel(const GemmParams p) {
  constexpr int S = T::STAGES;
  constexpr bool FP8 = KIND == KIND_FP8;
  // one array per stage and operand, so that the compiler can tell the
  // LDS-DMA target of one from the fragment reads of another (it would
  // otherwise drain every load in flight before those reads)
  __shared__ __attribute__((aligned(16))) uint8_t lds_a0[T::A_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t lds_a1[T::A_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t lds_a2[S > 2 ? T::A_BYTES : 16];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b0[T::B_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b1[T::B_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b2[S > 2 ? T::B_BYTES : 16];
  // FP8: per stage, A row scales in slots [0, BM), B block scales in
  // [BM, BM + NBT); one slot per thread so the stores need no branch
  __shared__ __attribute__((aligned(16))) float ssc[FP8 ? S : 1][FP8 ? T::NT : 1];
  auto stage_a = [&](int s) -> uint8_t* { return s == 0 ? lds_a0 : (s == 1 ? lds_a1 : lds_a2); };
  auto stage_b = [&](int s) -> uint8_t* { return s == 0 ? lds_b0 : (s == 1 ? lds_b1 : lds_b2); };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / T::WN, wn = wave % T::WN;

  // ---- tile decode (device metadata only gates early exits, never the grid)
  const int per_group = p.tiles_m * p.tiles_n;
  const int total = (MODE == MODE_MASKED ? p.G : 1) * per_group;
  int bid = blockIdx.x;
  bool second = false;  // contiguous, 256-row tiles: second copy of the grid
  if (MODE == MODE_CONTIG && T::BM == 256 && bid >= total) {
    second = true;
    bid -= total;
  }
  int t = xcd_remap(bid, total);
  int g = 0;
  if (MODE == MODE_MASKED) {
    g = t / per_group;
    t -= g * per_group;
  }
  int tm, tn;
  band_order(t, p.tiles_m, p.tiles_n, MODE == MODE_MASKED ? p.tiles_m : 8, tm, tn);
  const int m0 = __builtin_amdgcn_readfirstlane(tm * T::BM), n0 = __builtin_amdgcn_readfirstlane(tn * T::BN);

  int row_lim = p.M;        // rows [0, row_lim) may be read and written
  int lo = 0, hi = T::BM;   // tile rows this workgroup stores
  if (MODE == MODE_MASKED) {
    int v = __builtin_amdgcn_readfirstlane(p.meta[g]);
    v = v < 0 ? 0 : (v > p.M ? p.M : v);
    if (m0 >= v) return;
    row_lim = v;
  } else if (MODE == MODE_CONTIG) {
    const int nblk = p.M / 128;
    const int b0 = m0 / 128;
    int g0 = __builtin_amdgcn_readfirstlane(p.meta[b0]);
    if (g0 < 0 || g0 >= p.G) g0 = -1;
    int g1 = g0;
    if (T::BM == 256) {
      g1 = (b0 + 1 < nblk) ? __builtin_amdgcn_readfirstlane(p.meta[b0 + 1]) : -1;
      if (g1 < 0 || g1 >= p.G) g1 = -1;
    }
    if (second) {
      if (g0 == g1 || g0 < 0 || g1 < 0) return;  // no second block to do
      g = g1; lo = 128;
    } else if (g0 == g1) {
      if (g0 < 0) return;
      g = g0;
    } else if (g0 >= 0) {
      g = g0; hi = 128;
    } else {
      g = g1; lo = 128;
    }
  }
  g = __builtin_amdgcn_readfirstlane(g);

  const int KB = __builtin_amdgcn_readfirstlane(p.k_bytes / BK);
  const int NB = (p.N + 127) / 128;
  const uint8_t* A = p.a + (MODE == MODE_MASKED ? (int64_t)g * p.a_gs : 0);
  const uint8_t* B = p.b + (MODE == MODE_DENSE ? 0 : (int64_t)g * p.b_gs);
  uint16_t* D = p.d + (MODE == MODE_MASKED ? (int64_t)g * p.d_gs : 0);

  // LDS-DMA sources.  Instruction j of this wave fills tile rows
  // [8(j*NW+wave), +8); lane l writes slot l%8 of row l/8 and so reads chunk
  // (slot ^ h(row)).  Instruction j uses its own buffer resource, starting
  // j*8*NW rows into the tile and covering only the rows that exist (rows <
  // min(row_lim, m0 + hi) for A, < N for B): the hardware range check on the
  // per-lane offset returns zeros past them, so no clamping and no memory
  // traffic for those rows, and the per-lane offset is the same for every j
  // whose h term matches (one register per operand on 8-wave tiles).
  // Row (g8*8 + lrow) has h = lrow ^ h(g8*8) by linearity, so lane l reads
  // chunk (l%8) ^ (l/8) ^ h(g8*8), the last term uniform per instruction.
  const int lrow = lane >> 3, lslot = lane & 7;
  const int a_rows = __builtin_amdgcn_readfirstlane(max(0, min(min(row_lim - m0, hi), T::BM)));
  const int b_rows = __builtin_amdgcn_readfirstlane(max(0, min(p.N - n0, T::BN)));
  const uint32_t a_vrow = (uint32_t)((wave * 8 + lrow) * p.lda), b_vrow = (uint32_t)((wave * 8 + lrow) * p.ldb);
  const uint32_t vchunk = (uint32_t)(lslot ^ lrow);
  const int a_jstep = T::NW * 8 * (int)p.lda, b_jstep = T::NW * 8 * (int)p.ldb;
  const uint8_t* const a_tile = A + (int64_t)m0 * p.lda;
  const uint8_t* const b_tile = B + (int64_t)n0 * p.ldb;
  const int a_bytes = a_rows * (int)p.lda, b_bytes = b_rows * (int)p.ldb;

  auto issue_a_one = [&](uint8_t* stage, int kb, int j) {
    const uint32_t hu = (uint32_t)swz((j * T::NW + wave) * 8);
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a_tile + (int64_t)j * a_jstep), (short)0, max(0, a_bytes - j * a_jstep), 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(stage + (j * T::NW + wave) * 1024), 16,
                                             a_vrow + ((vchunk ^ hu) << 4), kb * BK, 0, 0);
  };
  auto issue_b_one = [&](uint8_t* stage, int kb, int j) {
    const uint32_t hu = (uint32_t)swz((j * T::NW + wave) * 8);
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(b_tile + (int64_t)j * b_jstep), (short)0, max(0, b_bytes - j * b_jstep), 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(stage + (j * T::NW + wave) * 1024), 16,
                                             b_vrow + ((vchunk ^ hu) << 4), kb * BK, 0, 0);
  };
  auto issue_a = [&](uint8_t* stage, int kb) {
#pragma unroll
    for (int j = 0; j < T::A_LOADS; ++j) issue_a_one(stage, kb, j);
  };
  auto issue_b = [&](uint8_t* stage, int kb) {
#pragma unroll
    for (int j = 0; j < T::B_LOADS; ++j) issue_b_one(stage, kb, j);
  };
  auto issue_loads = [&](int st, int kb) {
    issue_a(stage_a(st), kb);
    issue_b(stage_b(st), kb);
  };

  // Scale staged by this thread (FP8): A row m0 + tid (tid < BM), B column
  // block n0/128 + (tid - BM) (BM <= tid < BM + NBT), else a harmless
  // duplicate of row 0.
  const bool sc_is_b = tid >= T::BM && tid < T::BM + T::NBT;
  const int64_t sc_row = sc_is_b ? (int64_t)min(n0 / 128 + (tid - T::BM), NB - 1)
                                 : (int64_t)max(0, min(m0 + (tid < T::BM ? tid : 0), row_lim - 1));
  const void* sfa = static_cast<const float*>(p.sfa) + (MODE == MODE_MASKED ? (int64_t)g * p.sfa_gs : 0);
  const void* sfb = static_cast<const float*>(p.sfb) + (MODE == MODE_DENSE ? 0 : (int64_t)g * p.sfb_gs);
  const void* sc_base = sc_is_b ? sfb : sfa;
  const int64_t sc_srow = sc_is_b ? p.sfb_sn : p.sfa_sm, sc_sk = sc_is_b ? p.sfb_sk : p.sfa_sk;
  auto load_sc = [&](int kb) -> uint32_t {
    if constexpr (FP8) return load_scale_raw<SF>(sc_base, sc_row, kb, sc_srow, sc_sk);
    else return 0u;
  };
  auto store_sc = [&](int slot, uint32_t raw, int kb) {
    if constexpr (FP8) ssc[slot][tid] = scale_value<SF>(raw, kb);
  };

  // fragment-read geometry: MFMA row j of B fragment f is tile column
  // (j/4)*16 + f*4 + j%4, so lane group q = lane/16 ends up with columns
  // 16q .. 16q+15 of the wave tile (4 per fragment).
  // With h linear, lds_off(r0 + x, c) = (lds_off(x, c) ^ (h(r0) << 4)) + r0*128
  // whenever r0 has no bits below 4 in common with x; fragment offsets are
  // therefore a per-lane base XOR a compile-time constant, plus an immediate.
  const int fr = lane & 15;
  const int kc = (lane >> 4) * 2;  // first of the lane's two 16-B K chunks
  const int a_base = lds_off(wm * T::TM + fr, kc);                                  // fragment 0, chunk kc
  const int b_base = lds_off(wn * T::TN + (fr >> 2) * 16 + (fr & 3), kc);  // fragment 0, chunk kc

  // a wave whose rows all lie outside the rows to compute skips its MFMAs
  // (masked decode past masked_m; the unused half of a contiguous tile)
  const int wrow0 = wm * T::TM;
  const bool live = wrow0 < hi && wrow0 + T::TM > lo && m0 + wrow0 < row_lim;
  f32x4 acc[T::FM][T::FN];
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- prologue: K-slices 0..S-1 in flight, slice 0 landed.
  // The wait before the first barrier counts the loads issued after the
  // slice-0 tiles (the next slice's scale and the tiles of slices 1..S-1);
  // the fences keep the issue order that count assumes (the compiler would
  // otherwise hoist the scale loads above the tile loads and leave the last
  // slice-0 tile load in flight at the barrier).
  issue_loads(0, 0);
  __builtin_amdgcn_sched_barrier(0);
  const uint32_t rs0 = load_sc(0);
  uint32_t rs = load_sc(min(1, KB - 1));  // scale of the next slice to stage
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s = 1; s < S; ++s) {
    issue_loads(s, min(s, KB - 1));
    __builtin_amdgcn_sched_barrier(0);
  }
  store_sc(0, rs0, 0);
  __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0((FP8 ? 1 : 0) + (S - 1) * T::LOADS));
  __builtin_amdgcn_s_barrier();

  // Early point of K-slice kb (start of its second fragment group): every
  // wave has its B fragments of the slice in registers, so after a barrier
  // the B part of stage kb % S is free and the B tile of slice kb+S is
  // loaded into it, most of a slice before the A tile (B is the operand that
  // streams from HBM in the grouped decode shapes; A is shared and cached).
  auto early_sync = [&]() {
    __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(63));  // this wave's LDS reads are done
    __builtin_amdgcn_s_barrier();
  };
  auto early_point = [&](uint8_t* cur_b, int kb) {
    early_sync();
    issue_b(cur_b, min(kb + S, KB - 1));
    __builtin_amdgcn_sched_barrier(0);
  };
  // Late point of K-slice kb (before its last fragment group): stage the
  // scales of slice kb+1, wait for its tiles, barrier -- after it every wave
  // is done with stage kb % S and slice kb+1 is visible -- then load the A
  // tile of slice kb+S into stage kb % S.  The scale load goes first (vmcnt
  // counts in issue order).  Loads issued after the tiles of slice kb+1 that
  // may stay in flight: the B tile of slice kb+2 for two stages; the A tile
  // of slice kb+2 and the B tile of slice kb+3 for three.
  constexpr int LATE_VM = S == 2 ? T::B_LOADS : (S - 2) * T::LOADS;
  auto late_sync = [&](int kb, int slot) {
    store_sc(slot, rs, kb + 1);
    __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(LATE_VM));
    __builtin_amdgcn_s_barrier();
    rs = load_sc(min(kb + 2, KB - 1));
    __builtin_amdgcn_sched_barrier(0);
  };
  auto late_point = [&](uint8_t* cur_a, int kb, int slot) {
    late_sync(kb, slot);
    issue_a(cur_a, min(kb + S, KB - 1));
    __builtin_amdgcn_sched_barrier(0);
  };
  // In the K loop the tile loads of a point are not issued in a burst after
  // its barrier but one after each MFMA of the group that follows it (load j
  // after MFMA j % FN): a burst from all waves at once stalls their MFMA
  // issue behind the address unit (measured: 9% fewer cycles per K-slice).
  // The issue order, and so every vmcnt count above, is unchanged.
  auto spread_loads = [&](int i, int f, uint8_t* cur_a, uint8_t* cur_b, int kb) {
    if (i == 1) {
#pragma unroll
      for (int j = 0; j < T::B_LOADS; ++j)
        if (j % T::FN == f) issue_b_one(cur_b, min(kb + S, KB - 1), j);
    }
    if (i + 1 == T::FM) {
#pragma unroll
      for (int j = 0; j < T::A_LOADS; ++j)
        if (j % T::FN == f) issue_a_one(cur_a, min(kb + S, KB - 1), j);
    }
  };

  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  auto b_frag = [&](const uint8_t* stage, int f) {
    const int off = (b_base ^ (swz(f * 4) << 4)) + f * 4 * 128;  // rows +4f
    const i32x4 l = *reinterpret_cast<const i32x4*>(stage + off);
    const i32x4 h = *reinterpret_cast<const i32x4*>(stage + (off ^ 16));
    return i32x8{l[0], l[1], l[2], l[3], h[0], h[1], h[2], h[3]};
  };
  auto a_frag = [&](const uint8_t* stage, int i) {
    const int off = (a_base ^ (swz(i * 16) << 4)) + i * 16 * 128;  // rows +16i
    const i32x4 l = *reinterpret_cast<const i32x4*>(stage + off);
    const i32x4 h = *reinterpret_cast<const i32x4*>(stage + (off ^ 16));
    return i32x8{l[0], l[1], l[2], l[3], h[0], h[1], h[2], h[3]};
  };
  const int sa_row0 = wm * T::TM + fr;             // this lane's scale slot for fragment row 0
  const int sb_slot = T::BM + (wn * T::TN) / 128;  // this wave's B block scale slot

  // ---- K loop: one continuous software pipeline over fragment groups.
  // Group (kb, i) issues the FN MFMAs of A fragment i of slice kb and (FP8)
  // interleaved, the promote FMAs of the previous group (its partials are a
  // whole group old, so no FMA waits on an MFMA in flight), while the LDS
  // reads for the next group are in flight.  The barrier sits before the
  // last group of each slice: by then every wave has read all it needs of
  // the current stage (the last A fragment is already in registers), so the
  // last group streams in the next slice's B fragments, first A fragment and
  // scales, and the next slice starts with no bubble.  Scheduling fences
  // keep exactly this order (the compiler would otherwise pair each MFMA
  // with its own FMAs and serialise on the MFMA latency).
  // A fragments (and their row scales) are read PF fragment groups ahead
  // of their MFMAs; the next slice's first PF are read right after the late
  // barrier.
  constexpr int PF = 1;
  static_assert(PF == 1 || PF == 2, "prefetch depth");
  auto kloop = [&]() {
    i32x8 bf[T::FN];
    i32x8 af, af1;             // A fragments of the current and (PF = 2) the next group
    float sa = 0.f, sa1 = 0.f, sb = 0.f;  // raw row scales of those groups / block scale of the slice
    f32x4 P[2][T::FN];         // partials of the current and the previous group
    float s_prev = 0.f;        // combined scale of the previous group (the first promote adds 0 * 0)
#pragma unroll
    for (int f = 0; f < T::FN; ++f) P[(T::FM - 1) & 1][f] = zero;
#pragma unroll
    for (int f = 0; f < T::FN; ++f) bf[f] = b_frag(lds_b0, f);
    af = a_frag(lds_a0, 0);
    af1 = PF == 2 ? a_frag(lds_a0, 1) : af;
    if constexpr (FP8) {
      sa = ssc[0][sa_row0];
      sa1 = PF == 2 ? ssc[0][sa_row0 + 16] : sa;
      sb = ssc[0][sb_slot];
    }

    auto kblock = [&](auto st_tag, int kb) {
      constexpr int ST = decltype(st_tag)::value;
      constexpr int NX = (ST + 1) % S;
      uint8_t* cur_a = ST == 0 ? lds_a0 : (ST == 1 ? lds_a1 : lds_a2);
      uint8_t* cur_b = ST == 0 ? lds_b0 : (ST == 1 ? lds_b1 : lds_b2);
      uint8_t* nxt_a = NX == 0 ? lds_a0 : (NX == 1 ? lds_a1 : lds_a2);
      uint8_t* nxt_b = NX == 0 ? lds_b0 : (NX == 1 ? lds_b1 : lds_b2);
#pragma unroll
      for (int i = 0; i < T::FM; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        if (i == 1) early_sync();
        const float s_cur = sa * sb;
        // the A fragment / row scale that become current after this group
        // (n0) and, for PF = 2, the one after (n1)
        i32x8 n0 = af1, n1 = af1;
        float ns0 = sa1, ns1 = sa1, nsb = sb;
        if (i + 1 < T::FM) {
          if (PF == 1) {
            if constexpr (FP8) ns0 = ssc[ST][sa_row0 + (i + 1) * 16];
            n0 = a_frag(cur_a, i + 1);
          } else if (i + 2 < T::FM) {
            if constexpr (FP8) ns1 = ssc[ST][sa_row0 + (i + 2) * 16];
            n1 = a_frag(cur_a, i + 2);
          }
        } else {
          late_sync(kb, NX);
          if constexpr (FP8) {
            ns0 = ssc[NX][sa_row0];
            if (PF == 2) ns1 = ssc[NX][sa_row0 + 16];
            nsb = ssc[NX][sb_slot];
          }
          n0 = a_frag(nxt_a, 0);
        }
        if constexpr (FP8 && SF == SF_UE8M0) {
          // power-of-two scales go into the MFMA itself: its scale operands
          // multiply by 2^(e-127) per A row (the lane's row) and per B row
          // (one 128-column block per wave), and it accumulates in place
          const int ea = (int)(__float_as_uint(sa) >> 23), eb = (int)(__float_as_uint(sb) >> 23);
#pragma unroll
          for (int f = 0; f < T::FN; ++f) {
            __builtin_amdgcn_sched_barrier(0);
            acc[i][f] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[f], af, acc[i][f], 0, 0, 0, eb, 0, ea);
            spread_loads(i, f, cur_a, cur_b, kb);
            if (i + 1 == T::FM) bf[f] = b_frag(nxt_b, f);  // last use of bf[f] in this slice
          }
        } else if constexpr (FP8) {
          // the promote of the previous group: i-1 of this slice, or the
          // last group of the previous slice
#pragma unroll
          for (int f = 0; f < T::FN; ++f) {
            __builtin_amdgcn_sched_barrier(0);
            P[i & 1][f] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[f], af, zero, 0, 0, 0, 0, 0, 0);
            spread_loads(i, f, cur_a, cur_b, kb);
            __builtin_amdgcn_sched_barrier(0);
            if (i > 0) acc[i - 1][f] += P[(i - 1) & 1][f] * s_prev;
            else acc[T::FM - 1][f] += P[(T::FM - 1) & 1][f] * s_prev;
            if (i + 1 == T::FM) bf[f] = b_frag(nxt_b, f);  // last use of bf[f] in this slice
          }
        } else {
          // two K=32 halves per 128-byte slice; the four fragments between
          // the two MFMAs of one accumulator hide the MFMA latency
#pragma unroll
          for (int f = 0; f < T::FN; ++f) {
            __builtin_amdgcn_sched_barrier(0);
            acc[i][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo_bf16(bf[f]), lo_bf16(af), acc[i][f], 0, 0, 0);
            spread_loads(i, f, cur_a, cur_b, kb);
          }
#pragma unroll
          for (int f = 0; f < T::FN; ++f) {
            __builtin_amdgcn_sched_barrier(0);
            acc[i][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi_bf16(bf[f]), hi_bf16(af), acc[i][f], 0, 0, 0);
          }
          if (i + 1 == T::FM) {
#pragma unroll
            for (int f = 0; f < T::FN; ++f) bf[f] = b_frag(nxt_b, f);
          }
        }
        if (PF == 2 && i + 1 == T::FM) {
          __builtin_amdgcn_sched_barrier(0);
          n1 = a_frag(nxt_a, 1);  // after the B fragments the next group 0 waits for
        }
        s_prev = s_cur;
        if (PF == 1) {
          af = n0;
          sa = ns0;
        } else {
          af = i + 1 < T::FM ? af1 : n0;
          sa = i + 1 < T::FM ? sa1 : ns0;
          af1 = n1;
          sa1 = ns1;
        }
        sb = nsb;
      }
    };

    int kb = 0;
    for (; kb + S <= KB; kb += S) {
      kblock(std::integral_constant<int, 0>{}, kb);
      kblock(std::integral_constant<int, 1>{}, kb + 1);
      if constexpr (S > 2) kblock(std::integral_constant<int, 2>{}, kb + 2);
    }
    if (kb < KB) kblock(std::integral_constant<int, 0>{}, kb);
    if constexpr (S > 2) {
      if (kb + 1 < KB) kblock(std::integral_constant<int, 1>{}, kb + 1);
    }
    if constexpr (FP8 && SF == SF_F32) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int f = 0; f < T::FN; ++f) acc[T::FM - 1][f] += P[(T::FM - 1) & 1][f] * s_prev;
    }
  };

  if (live) {
    kloop();
  } else {
    // this wave computes nothing: it still takes part in the scale staging,
    // loads and barriers of every K-slice, without MFMAs
    for (int kb = 0; kb < KB; ++kb) {
      early_point(stage_b(kb % S), kb);
      late_point(stage_a(kb % S), kb, (kb + 1) % S);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // drain the redundant last loads before LDS is reused or freed
  if (!live) return;

  // ---- epilogue: BF16, row m = lane%16 of each fragment row, 16 consecutive columns per lane
  const int col0 = n0 + wn * T::TN + (lane >> 4) * 16;
  const bool vec_ok = ((p.ldd & 7) == 0) && ((reinterpret_cast<uintptr_t>(D) & 15) == 0);
#pragma unroll
  for (int i = 0; i < T::FM; ++i) {
    const int rl = wm * T::TM + i * 16 + fr;
    const int row = m0 + rl;
    if (rl < lo || rl >= hi || row >= row_lim) continue;
    if (MODE == MODE_DENSE && p.c != nullptr) {
      // D = C + A . B^T ("DeepInside DeepGEMM", section 4): C is added to the
      // FP32 accumulator before the BF16 rounding (read before d is written,
      // so c may be d itself)
      const int cc = col0;
      if (p.c_f32) {
        const float* crow = static_cast<const float*>(p.c) + (int64_t)row * p.ldc;
        const bool cvec = ((p.ldc & 3) == 0) && ((reinterpret_cast<uintptr_t>(p.c) & 15) == 0) && cc + 16 <= p.N;
#pragma unroll
        for (int f = 0; f < T::FN; ++f) {
          if (cvec) {
            const f32x4 cv = *reinterpret_cast<const f32x4*>(crow + cc + 4 * f);
            acc[i][f] += cv;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (cc + 4 * f + e < p.N) acc[i][f][e] += crow[cc + 4 * f + e];
          }
        }
      } else {
        const uint16_t* crow = static_cast<const uint16_t*>(p.c) + (int64_t)row * p.ldc;
        const bool cvec = ((p.ldc & 7) == 0) && ((reinterpret_cast<uintptr_t>(p.c) & 15) == 0) && cc + 16 <= p.N;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (cvec) {
            const i32x4 cv = *reinterpret_cast<const i32x4*>(crow + cc + 8 * h);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              acc[i][2 * h + w / 2][2 * (w & 1)] += __uint_as_float((uint32_t)cv[w] << 16);
              acc[i][2 * h + w / 2][2 * (w & 1) + 1] += __uint_as_float((uint32_t)cv[w] & 0xffff0000u);
            }
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (cc + 8 * h + e < p.N) acc[i][2 * h + e / 4][e & 3] += bf16_to_f32(crow[cc + 8 * h + e]);
          }
        }
      }
    }
    uint32_t packed[8];
#pragma unroll
    for (int f = 0; f < T::FN; ++f) {
      packed[2 * f] = (uint32_t)f32_to_bf16_rne(acc[i][f][0]) | ((uint32_t)f32_to_bf16_rne(acc[i][f][1]) << 16);
      packed[2 * f + 1] = (uint32_t)f32_to_bf16_rne(acc[i][f][2]) | ((uint32_t)f32_to_bf16_rne(acc[i][f][3]) << 16);
    }
    uint16_t* drow = D + (int64_t)row * p.ldd;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = col0 + 8 * h;
      if (vec_ok && c + 8 <= p.N) {
        *reinterpret_cast<i32x4*>(drow + c) =
            i32x4{(int)packed[4 * h], (int)packed[4 * h + 1], (int)packed[4 * h + 2], (int)packed[4 * h + 3]};
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (c + e < p.N) drow[c + e] = (uint16_t)(packed[4 * h + e / 2] >> (16 * (e & 1)));
      }
    }
  }
}

using TileL = TileShape<256, 256, 2, 4, 2>;  // 512 threads, wave tile 128 x 64, 2 x 64 KB stages
using TileW = TileShape<128, 256, 2, 4, 3>;  // 512 threads, wave tile  64 x 64, 3 x 48 KB stages
using TileS = TileShape<128, 128, 2, 2, 3>;  // 256 threads, wave tile  64 x 64, 3 x 32 KB stages
using TileT = TileShape<256, 128, 4, 2, 3>;  // 512 threads, wave tile  64 x 64, 3 x 48 KB stages

enum Variant : int { VAR_L = 0, VAR_W = 1, VAR_S = 2, VAR_T = 3 };

template <class T, int KIND>
hipError_t launch_tile(const GemmParams& p, int mode, int sf_fmt, int64_t grid, hipStream_t stream) {
  const dim3 g((unsigned)grid), b(T::NT);
  if constexpr (KIND == KIND_BF16) {
    if (mode == MODE_DENSE) gemm_kernel<T, KIND_BF16, SF_F32, MODE_DENSE><<<g, b, 0, stream>>>(p);
    else if (mode == MODE_CONTIG) gemm_kernel<T, KIND_BF16, SF_F32, MODE_CONTIG><<<g, b, 0, stream>>>(p);
    else gemm_kernel<T, KIND_BF16, SF_F32, MODE_MASKED><<<g, b, 0, stream>>>(p);
    return hipGetLastError();
  }
#define DGMI_LAUNCH(MODE_, SF_) gemm_kernel<T, KIND_FP8, SF_, MODE_><<<g, b, 0, stream>>>(p)
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

template <class T, int KIND>
TileCfg make_cfg(int variant) {
  TileCfg c;
  c.bm = T::BM;
  c.bn = T::BN;
  c.threads = T::NT;
  c.lds_bytes = T::template lds_bytes<KIND>();
  c.variant = variant;
  return c;
}

template <int KIND>
hipError_t launch_variant(const TileCfg& cfg, const GemmParams& p, int mode, int sf_fmt, int64_t grid,
                          hipStream_t stream) {
  switch (cfg.variant) {
    case VAR_L: return launch_tile<TileL, KIND>(p, mode, sf_fmt, grid, stream);
    case VAR_W: return launch_tile<TileW, KIND>(p, mode, sf_fmt, grid, stream);
    case VAR_T: return launch_tile<TileT, KIND>(p, mode, sf_fmt, grid, stream);
    default: return launch_tile<TileS, KIND>(p, mode, sf_fmt, grid, stream);
  }
}

}  // namespace

// Tile choice, a pure function of the shapes.  Rows <= 128 (small dense M,
// decode buffers of up to 128 rows per expert) use 128-row tiles with three
// stages; everything else the 256 x 256 tile with two stages (three do not
// fit in LDS), which measured fastest on all the large dense and grouped
// shapes.
TileCfg fp8_gemm_config(int mode, int64_t G, int64_t M, int64_t N, int64_t K) {
  (void)mode; (void)G; (void)K;
  if (M <= 128) return N <= 128 ? make_cfg<TileS, KIND_FP8>(VAR_S) : make_cfg<TileW, KIND_FP8>(VAR_W);
  return make_cfg<TileL, KIND_FP8>(VAR_L);
}

int64_t gemm_grid(const TileCfg& cfg, int mode, int64_t G, int64_t M, int64_t N) {
  const int64_t tm = (M + cfg.bm - 1) / cfg.bm, tn = (N + cfg.bn - 1) / cfg.bn;
  const int64_t tiles = (mode == MODE_MASKED ? G : 1) * tm * tn;
  // contiguous 256-row tiles: a second copy for tiles split between two groups
  return (mode == MODE_CONTIG && cfg.bm == 256) ? 2 * tiles : tiles;
}

hipError_t launch_fp8_gemm(GemmParams p, int mode, int sf_fmt, hipStream_t stream) {
  const TileCfg cfg = fp8_gemm_config(mode, p.G, p.M, p.N, p.k_bytes);
  p.tiles_m = (p.M + cfg.bm - 1) / cfg.bm;
  p.tiles_n = (p.N + cfg.bn - 1) / cfg.bn;
  const int64_t grid = gemm_grid(cfg, mode, p.G, p.M, p.N);
  if (grid == 0) return hipSuccess;
  return launch_variant<KIND_FP8>(cfg, p, mode, sf_fmt, grid, stream);
}

// BF16 GEMMs: the same tile choice as the FP8 GEMM (a K-slice is 64 BF16
// elements instead of 128 FP8 ones, the bytes per tile are the same).
TileCfg bf16_gemm_config(int mode, int64_t G, int64_t M, int64_t N, int64_t K) {
  (void)mode; (void)G; (void)K;
  if (M <= 128) return N <= 128 ? make_cfg<TileS, KIND_BF16>(VAR_S) : make_cfg<TileW, KIND_BF16>(VAR_W);
  return make_cfg<TileL, KIND_BF16>(VAR_L);
}

hipError_t launch_bf16_gemm(GemmParams p, int mode, hipStream_t stream) {
  const TileCfg cfg = bf16_gemm_config(mode, p.G, p.M, p.N, p.k_bytes / 2);
  p.tiles_m = (p.M + cfg.bm - 1) / cfg.bm;
  p.tiles_n = (p.N + cfg.bn - 1) / cfg.bn;
  const int64_t grid = gemm_grid(cfg, mode, p.G, p.M, p.N);
  if (grid == 0) return hipSuccess;
  return launch_variant<KIND_BF16>(cfg, p, mode, SF_F32, grid, stream);
}

}  // namespace dgmi
