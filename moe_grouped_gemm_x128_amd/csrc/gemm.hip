// GEMM kernels of libdgmi for gfx950: the block-scaled FP8 GEMM (dense,
// contiguous-grouped and masked-grouped scheduling) and the masked BF16 GEMM,
// over one kernel body.
//
// What the FP8 kind computes ("DeepInside DeepGEMM", sections 2 and 4;
// "DeepGEMM tested by Novita AI", section "Technological Innovations"):
//   D[m, n] = sum_kb P_kb[m, n] * sfa[m, kb] * sfb[n / 128, kb],
//   P_kb    = A[m, kb*128 : kb*128+128] . B[n, same]^T
// (or sfb[n, kb] with one scale per row of B, section 4's example call)
// Each 128-wide K-block is exactly one v_mfma_f32_16x16x128_f8f6f4 per
// 16x16 output fragment, computed into a fresh FP32 partial; the partial is
// then promoted into the FP32 accumulator with one FMA per element using the
// product of the row scale and the 128x128 block scale.  With power-of-two
// UE8M0 scales the promote is the MFMA's own: v_mfma_scale_f32_16x16x128_
// f8f6f4 multiplies by 2^(e-127) per A row and per B row and accumulates in
// place (the SM100 recipe of "DeepInside DeepGEMM", section 2, on CDNA4).
// Output is BF16 (round to nearest even), the FP32 accumulator itself, or
// (dense) FP8 cast per token in the epilogue; an accumulate input C is added
// to the FP32 accumulator first.
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
//                 from grouped_layout on the device, negative = skip.  With
//                 256-row tiles each run of blocks of one group is cut into
//                 tiles from its first block (two blocks a tile, one at the
//                 run's end); each workgroup lists the tile starts with a
//                 block-wide scan of grouped_layout, the grid holds one
//                 workgroup per block and column tile, and those past the
//                 listed tiles exit at once.
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
//     columns.  On 64-column wave tiles the B fragment rows are permuted so
//     that the four fragments of a wave give every lane 16 consecutive
//     columns: one row scale per lane per fragment row, one block scale per
//     wave, and the BF16 epilogue stores 2 x 16 bytes per lane per fragment
//     row, straight from registers.  The 48-column wave tiles of the
//     256 x 192 tile keep MFMA order (4 columns per lane and fragment, one
//     block scale per fragment, 8-byte stores).
//   * Block sizes per shape ("DeepGEMM tested by Novita AI", section
//     "Technological Innovations of DeepGEMM", item "Support for Arbitrary
//     Matrix Sizes"): a 256 x 192 tile, alone or (BF16) beside the
//     256 x 256 one in a second launch over the last columns, when that
//     fills the last round of workgroups better, and for the dense GEMMs a
//     192 x 192 tile where a problem fits one round of it (plan_large's
//     cost model).  MN-major operands take the 256 x 192 tile.
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
// layout (bits 0, 1, 4, 5 vary) or, on 48-column wave tiles, rows r0 + 0..15
// like A (r0 a multiple of 16).  h is a bijection on the varying bits in
// both cases, for every group of 8 lanes and for every 16 lanes split by
// row parity, so the reads are free of bank conflicts with 32 or with 64
// four-byte banks.
__device__ __host__ constexpr int swz(int r) { return ((r ^ (r >> 3) ^ (r >> 5)) & 1) | (r & 2) | ((((r >> 2) ^ (r >> 4)) & 1) << 2); }
// Byte offset in a tile of 16-byte chunk c (0..7) of tile row r.
__device__ __forceinline__ int lds_off(int r, int c) { return r * 128 + ((c ^ swz(r)) << 4); }

// MN-major operands (the operand stored [K, rows], rows contiguous): a stage
// holds the slice's 128 K-rows of 256 bytes each (the tile's rows, padded to
// 256), and the 16-byte chunk c of K-row k is stored at slot c ^ hmn(k),
//   hmn(k) = (k & 7) | ((k >> 5) & 1) << 3.
// The transposing fragment reads (ds_read_b64_tr_b8) of one 16-lane group
// touch K-rows 8 apart in an aligned run of 8 at one chunk: (k & 7) spreads
// them over 8 slots; the two 16-lane groups served together differ in bit 5
// of k, and the last term puts them on the other half of the banks.
constexpr int MN_ROW = 256;
__device__ __host__ constexpr int hmn(int k) { return (k & 7) | (((k >> 5) & 1) << 3); }

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
  // Column layouts.  PERM (64-column wave tiles, tile starts at multiples of
  // 128): the B rows are permuted so that a lane holds 16 consecutive
  // columns, and a wave's columns lie in one 128-column scale block.
  // Otherwise fragment f holds columns 16f..16f+15 of the wave tile in MFMA
  // order (4 consecutive columns per lane), and each fragment takes the scale
  // of its own 128-column block (a 16-column fragment never straddles one
  // when the tile starts at a multiple of 16).
  static constexpr bool PERM = TN == 64;
  static_assert(PERM ? FN == 4 : TN % 16 == 0, "wave tile columns");
  static constexpr int NSB = PERM ? 1 : FN;         // B block scales a wave uses per K-slice
  static constexpr int NBT = (BN + 127) / 128 + (PERM ? 0 : 1);  // 128-column scale blocks a tile touches
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
  return (SF & SF_UE8M0) == 0 ? p[idx_row * s_row + (int64_t)kb * s_k] : p[idx_row * s_row + (int64_t)(kb >> 2) * s_k];
}
template <int SF>
__device__ __forceinline__ float scale_value(uint32_t raw, int kb) {
  return (SF & SF_UE8M0) == 0 ? __uint_as_float(raw) : ue8m0_to_f32((raw >> ((kb & 3) * 8)) & 0xffu);
}

// Tile starts of a contiguous layout with 256-row tiles.  A run is a
// maximal sequence of blocks of one group; the blocks at even offsets in it
// start tiles.  Every thread takes one block a pass (NW*64 blocks a pass);
// per wave, ballots give the run starts and tile starts among its lanes, and
// the waves' masks, shared in LDS, give each lane its run's start (the
// latest one at or before it, or the carry from earlier passes) and each
// tile start its place in the list.  Entry j of the list: first block x 2 +
// (the next block belongs to the tile), and grp[j] its group.  Returns the
// number of tiles; every thread calls it, the lists are complete on return.
template <int NW>
__device__ __forceinline__ int contig_tile_list(int nblk, const int* layout, int G, int* list, int* grp,
                                                uint64_t* ws_rs, int* ws_cnt) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t below = (1ull << lane) - 1;  // lanes before this one
  int count = 0, carry = -1;                  // tiles so far; latest run start so far
  for (int base = 0; base < nblk; base += NW * 64) {
    // the block's group and its neighbours' (ids outside [0, G) skip a
    // block); the loads are clamped into the layout, so all three issue at
    // once, and the selects put -1 where a neighbour does not exist
    const int b = base + tid, bc = min(b, nblk - 1);
    const int v = layout[bc], vp = layout[max(bc - 1, 0)], vn = layout[min(bc + 1, nblk - 1)];
    auto valid = [G](int x) { return x >= 0 && x < G ? x : -1; };
    const int gb = b < nblk ? valid(v) : -1;
    const int gp = b > 0 && b < nblk ? valid(vp) : -1;
    const int gn = b + 1 < nblk ? valid(vn) : -1;
    const uint64_t m_rs = __ballot(gb >= 0 && gb != gp);  // run starts
    if (lane == 0) ws_rs[wave] = m_rs;
    __syncthreads();
    // this lane's run start: the latest in its own wave at or before it,
    // else the latest in the earlier waves, else the carry (run starts grow
    // with the block index)
    int before = carry, last = carry;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint64_t x = ws_rs[w];
      const int h = x != 0 ? base + w * 64 + 63 - __clzll(x) : -1;
      last = max(last, h);
      before = w < wave ? max(before, h) : before;
    }
    const uint64_t mine = m_rs & (below | (1ull << lane));
    const int rs = mine != 0 ? b - lane + 63 - __clzll(mine) : before;
    const bool starts = gb >= 0 && ((b - rs) & 1) == 0;
    const uint64_t m_st = __ballot(starts);
    if (lane == 0) ws_cnt[wave] = __popcll(m_st);
    __syncthreads();
    int off = count, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int c = ws_cnt[w];
      off += w < wave ? c : 0;
      tot += c;
    }
    if (starts) {
      const int j = off + __popcll(m_st & below);
      list[j] = 2 * b + (gn == gb ? 1 : 0);
      grp[j] = gb;
    }
    count += tot;
    carry = last;
  }
  __syncthreads();
  return count;
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


// One FP8 block product of a 16x16 fragment over 128 K values, P = B . A^T
// added to c, with no scaling (the FP32-scale kinds promote P themselves).
// The f8f6f4 matrix core has no builtin of its own without scales: the
// scaled builtin with literal zero scale operands is what the backend lowers
// to the unscaled v_mfma_f32_16x16x128_f8f6f4.  The zeros must stay literals
// inside this helper -- a non-constant scale operand selects the scaled
// instruction, where a scale byte of 0 multiplies by 2^-127 and would zero
// every product.
__device__ __forceinline__ f32x4 mfma_fp8_unscaled(const i32x8& b, const i32x8& a, const f32x4& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, c, 0, 0, 0, /*scale_b=*/0, 0, /*scale_a=*/0);
}

__device__ __forceinline__ bf16x8 lo_bf16(const i32x8& v) { return __builtin_bit_cast(bf16x8, i32x4{v[0], v[1], v[2], v[3]}); }
__device__ __forceinline__ bf16x8 hi_bf16(const i32x8& v) { return __builtin_bit_cast(bf16x8, i32x4{v[4], v[5], v[6], v[7]}); }

// Epilogue of the unpermuted column layout: fragment f of wave column wn
// holds tile columns wn*TN + 16f + 4q .. +3 in lane group q = lane/16, row
// m = lane%16 of each fragment row.  Optional C (dense only) is added to the
// FP32 accumulator before the BF16 rounding; c may alias d (each element of
// C is read before the same thread writes it).  8-byte stores of four BF16.
template <class T, int OUT>
__device__ __forceinline__ void epilogue_cols4(const GemmParams& p, uint16_t* D, f32x4 (&acc)[T::FM][T::FN], int m0,
                                               int n0, int wm, int wn, int lane, int lo, int hi, int row_lim,
                                               const void* cbase) {
  const int fr = lane & 15;
  const int colq = n0 + wn * T::TN + (lane >> 4) * 4;
  const bool vec_ok = ((p.ldd & 3) == 0) && ((reinterpret_cast<uintptr_t>(D) & 7) == 0);
  const bool has_c = cbase != nullptr;
#pragma unroll
  for (int i = 0; i < T::FM; ++i) {
    const int rl = wm * T::TM + i * 16 + fr;
    const int row = m0 + rl;
    if (rl < lo || rl >= hi || row >= row_lim) continue;
    uint16_t* drow = D + (int64_t)row * p.ldd;
#pragma unroll
    for (int f = 0; f < T::FN; ++f) {
      const int c = colq + 16 * f;
      f32x4 v = acc[i][f];
      if (has_c) {
        if (p.c_f32) {
          const float* crow = static_cast<const float*>(cbase) + (int64_t)row * p.ldc;
          if (((p.ldc & 3) == 0) && ((reinterpret_cast<uintptr_t>(cbase) & 15) == 0) && c + 4 <= p.N) {
            v += *reinterpret_cast<const f32x4*>(crow + c);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (c + e < p.N) v[e] += crow[c + e];
          }
        } else {
          const uint16_t* crow = static_cast<const uint16_t*>(cbase) + (int64_t)row * p.ldc;
          if (((p.ldc & 3) == 0) && ((reinterpret_cast<uintptr_t>(cbase) & 7) == 0) && c + 4 <= p.N) {
            const i32x2 cv = *reinterpret_cast<const i32x2*>(crow + c);
            v[0] += __uint_as_float((uint32_t)cv[0] << 16);
            v[1] += __uint_as_float((uint32_t)cv[0] & 0xffff0000u);
            v[2] += __uint_as_float((uint32_t)cv[1] << 16);
            v[3] += __uint_as_float((uint32_t)cv[1] & 0xffff0000u);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (c + e < p.N) v[e] += bf16_to_f32(crow[c + e]);
          }
        }
      }
      if constexpr (OUT == OUT_F32) {
        // the FP32 values themselves (dense): one 16-byte store of 4 columns
        float* frow = reinterpret_cast<float*>(D) + (int64_t)row * p.ldd;
        if (((p.ldd & 3) == 0) && ((reinterpret_cast<uintptr_t>(D) & 15) == 0) && c + 4 <= p.N) {
          *reinterpret_cast<f32x4*>(frow + c) = v;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (c + e < p.N) frow[c + e] = v[e];
        }
        continue;
      }
      const i32x2 wv = to_bf16x4_bits(v);
      const uint32_t w0 = (uint32_t)wv[0], w1 = (uint32_t)wv[1];
      if (vec_ok && c + 4 <= p.N) {
        *reinterpret_cast<i32x2*>(drow + c) = i32x2{(int)w0, (int)w1};
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (c + e < p.N) drow[c + e] = (uint16_t)((e < 2 ? w0 : w1) >> (16 * (e & 1)));
      }
    }
  }
}

// Adds C[row, cc .. cc+15] to one row of a wave's accumulators in the
// permuted layout (16 consecutive columns per lane; columns >= N untouched).
template <class T>
__device__ __forceinline__ void add_c_perm(const GemmParams& p, f32x4 (&acc)[T::FN], int row, int cc) {
  static_assert(T::FN == 4, "16 columns per lane");
  if (p.c_f32) {
    const float* crow = static_cast<const float*>(p.c) + (int64_t)row * p.ldc;
    const bool cvec = ((p.ldc & 3) == 0) && ((reinterpret_cast<uintptr_t>(p.c) & 15) == 0) && cc + 16 <= p.N;
#pragma unroll
    for (int f = 0; f < T::FN; ++f) {
      if (cvec) {
        const f32x4 cv = *reinterpret_cast<const f32x4*>(crow + cc + 4 * f);
        acc[f] += cv;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (cc + 4 * f + e < p.N) acc[f][e] += crow[cc + 4 * f + e];
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
          acc[2 * h + w / 2][2 * (w & 1)] += __uint_as_float((uint32_t)cv[w] << 16);
          acc[2 * h + w / 2][2 * (w & 1) + 1] += __uint_as_float((uint32_t)cv[w] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (cc + 8 * h + e < p.N) acc[2 * h + e / 4][e & 3] += bf16_to_f32(crow[cc + 8 * h + e]);
      }
    }
  }
}

// FP8-output epilogue (dense, 64-column wave tiles in the permuted layout):
// D is rounded to BF16 (C added first, as in the BF16 epilogue) and cast per
// token exactly as per_token_cast_to_fp8 casts a BF16 tensor: per row and
// 128-column block, amax over the block (the 16 columns of each of four lanes
// of a wave, and of its neighbouring wave, exchanged through LDS), s =
// amax/448 or its UE8M0 round-up, q = e4m3(x / s).  ("DeepInside DeepGEMM",
// section 5: the FP8 cast fused into the kernel that produces the tensor.)
template <class T>
__device__ __forceinline__ void epilogue_fp8(const GemmParams& p, f32x4 (&acc)[T::FM][T::FN], uint8_t* lds, int m0,
                                             int n0, int wm, int wn, int lane, int row_lim) {
  static_assert(T::PERM && T::WN % 2 == 0 && T::BN % 128 == 0 && T::BM * T::WN * 4 <= T::B_BYTES,
                "a 128-column block is the 64 columns of two neighbouring waves");
  const int fr = lane & 15;
  const int col0 = n0 + wn * T::TN + (lane >> 4) * 16;  // this lane's 16 consecutive columns
  float* xch = reinterpret_cast<float*>(lds);  // [BM][WN] wave maxima per row
  float wmax[T::FM];
  // every wave is past its K loop (its LDS reads and loads drained) before
  // the stages are reused; the barriers order the LDS exchange (fenced, so
  // the compiler keeps the LDS accesses on their side)
  __syncthreads();
#pragma unroll
  for (int i = 0; i < T::FM; ++i) {
    const int rl = wm * T::TM + i * 16 + fr;
    const int row = m0 + rl;
    if (p.c != nullptr && row < row_lim) add_c_perm<T>(p, acc[i], row, col0);
    // the BF16 value of D (the hardware conversion rounds to nearest even,
    // as the BF16 epilogue does).  Columns past N hold +0 (B rows past N load
    // as zeros, C is not added there) or NaN (a non-finite B scale), and
    // neither changes the block maximum: fmaxf passes over NaN.
    float m = 0.0f;
#pragma unroll
    for (int f = 0; f < T::FN; ++f) {
      acc[i][f] = __builtin_convertvector(__builtin_convertvector(acc[i][f], bf16x4), f32x4);
#pragma unroll
      for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(acc[i][f][e]));
    }
    m = fmaxf(m, __shfl_xor(m, 16, 64));
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    wmax[i] = m;
    if ((lane >> 4) == 0) xch[rl * T::WN + wn] = m;
  }
  __syncthreads();
  const bool vec_ok = ((p.ldq & 15) == 0) && ((reinterpret_cast<uintptr_t>(p.q) & 15) == 0);
  const int blk = (n0 + (wn & ~1) * T::TN) / 128;  // this wave pair's 128-column block
#pragma unroll
  for (int i = 0; i < T::FM; ++i) {
    const int rl = wm * T::TM + i * 16 + fr;
    const int row = m0 + rl;
    if (row >= row_lim || blk * 128 >= p.N) continue;
    const float amax = fmaxf(wmax[i], xch[rl * T::WN + (wn ^ 1)]);
    const float s = block_scale(amax, p.q_ue8m0);
    const Recip d = recip_of(s);
    uint32_t w[T::FN];
#pragma unroll
    for (int f = 0; f < T::FN; ++f) {
      const float v[4] = {acc[i][f][0], acc[i][f][1], acc[i][f][2], acc[i][f][3]};
      w[f] = encode4(v, d);
    }
    uint8_t* qrow = p.q + (int64_t)row * p.ldq;
    if (vec_ok && col0 + 16 <= p.N) {
      *reinterpret_cast<i32x4*>(qrow + col0) = i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
    } else {
      // q rows are 4-byte aligned
#pragma unroll
      for (int f = 0; f < T::FN; ++f) {
        const int c = col0 + 4 * f;
        if (c + 4 <= p.N) {
          *reinterpret_cast<uint32_t*>(qrow + c) = w[f];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (c + e < p.N) qrow[c + e] = (uint8_t)(w[f] >> (8 * e));
        }
      }
    }
    if ((lane >> 4) == 0 && (wn & 1) == 0) p.sfq[(int64_t)row * p.sfq_sm + (int64_t)blk * p.sfq_sn] = s;
  }
}

// LAY: bit 0 -- A is MN-major (stored [K, M], rows contiguous), bit 1 -- B is
// MN-major (stored [K, N]); dense FP8 with BF16 output on tiles whose B
// fragments keep MFMA column order ("DeepInside DeepGEMM", section 2: the
// NN, TN and TT layouts besides NT).
template <class T, int KIND, int SF, int MODE, int OUT = OUT_BF16, int LAY = 0>
__global__ __launch_bounds__(T::NT) void gemm_kernel(const GemmParams p) {
  constexpr int S = T::STAGES;
  constexpr bool FP8 = KIND == KIND_FP8;
  constexpr bool A_MN = (LAY & 1) != 0, B_MN = (LAY & 2) != 0;
  static_assert(LAY == 0 || (FP8 && MODE == MODE_DENSE && OUT != OUT_FP8 && !T::PERM && T::NW == 8 &&
                             T::BM <= MN_ROW && T::BN <= MN_ROW),
                "MN-major operands: dense FP8, BF16 or F32 output, MFMA column order, 8 waves");
  // stage bytes and LDS-DMA instructions per wave per stage of each operand
  // (an MN-major stage is 128 K-rows of 256 bytes: four K-rows per instruction)
  constexpr int A_STAGE = A_MN ? BK * MN_ROW : T::A_BYTES, B_STAGE = B_MN ? BK * MN_ROW : T::B_BYTES;
  constexpr int A_LD = A_MN ? BK * MN_ROW / (1024 * T::NW) : T::A_LOADS;
  constexpr int B_LD = B_MN ? BK * MN_ROW / (1024 * T::NW) : T::B_LOADS;
  constexpr int LD_ALL = A_LD + B_LD;
  constexpr bool UE8 = FP8 && (SF & SF_UE8M0) != 0;
  // one B scale per row of B ("DeepInside DeepGEMM", section 4: the per-row
  // b_sf of its dense example): the promote scales each output column by
  // its own row's scale; the UE8M0 MFMA takes the scale of the B row each
  // lane supplies
  constexpr bool ROWB = FP8 && (SF & SF_ROWB) != 0;
  constexpr bool ROWB_F32 = ROWB && !UE8;
  static_assert(!ROWB || T::BM + T::BN <= T::NT, "one thread per tile row of A and of B stages its scale");
  // B scales a lane uses per K-slice: one per wave (or per fragment) for
  // block scales, one per fragment (its own B row) for UE8M0 row scales;
  // FP32 row scales are 4-vectors per fragment (below)
  constexpr int NSB = ROWB ? (UE8 ? T::FN : 1) : T::NSB;
  // one array per stage and operand, so that the compiler can tell the
  // LDS-DMA target of one from the fragment reads of another (it would
  // otherwise drain every load in flight before those reads)
  __shared__ __attribute__((aligned(16))) uint8_t lds_a0[A_STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t lds_a1[A_STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t lds_a2[S > 2 ? A_STAGE : 16];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b0[B_STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b1[B_STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b2[S > 2 ? B_STAGE : 16];
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
  // group of a 128-row block of the contiguous layout; ids outside [0, G)
  // skip the block
  auto group_of = [&](int blk) {
    const int v = p.meta[blk];
    return (v < 0 || v >= p.G) ? -1 : v;
  };
  // Contiguous layout with 256-row tiles: a block at an even offset in its
  // run of equal group ids starts a tile of the run's next two blocks (one
  // at the run's end), so tiles never straddle groups.  Every workgroup
  // scans grouped_layout and builds the list of those tile starts, in block
  // order, in the first two A stages (free until the prologue).  The grid holds
  // one workgroup per 128-row block and column tile: the first
  // (list length) x tiles_n take the listed tiles in the usual XCD-banded
  // order, the rest -- all after them in dispatch order -- exit at once.
  constexpr bool RUNS = MODE == MODE_CONTIG && T::BM == 256;
  int tm, tn, g = 0, hi = T::BM;
  if constexpr (RUNS) {
    static_assert(A_STAGE >= 4 * RUNS_MAX_BLOCKS, "the tile lists fit the first two A stages");
    __shared__ uint64_t ws_rs[T::NW];
    __shared__ int ws_cnt[T::NW];
    int* list = reinterpret_cast<int*>(lds_a0);
    int* grp = reinterpret_cast<int*>(lds_a1);
    const int count = contig_tile_list<T::NW>(p.M / 128, p.meta, p.G, list, grp, ws_rs, ws_cnt);
    const int total_c = count * p.tiles_n;
    if ((int)blockIdx.x >= total_c) return;
    int j;
    band_order(xcd_remap(blockIdx.x, total_c), count, p.tiles_n, 8, j, tn);
    const int e = __builtin_amdgcn_readfirstlane(list[j]);
    tm = e >> 1;  // the tile's first 128-row block
    g = __builtin_amdgcn_readfirstlane(grp[j]);
    if ((e & 1) == 0) hi = 128;  // one block: the run's last
    __syncthreads();  // every wave has read the lists before the prologue loads into these stages
  } else {
    int t = xcd_remap(blockIdx.x, total);
    if (MODE == MODE_MASKED) {
      g = t / per_group;
      t -= g * per_group;
    }
    band_order(t, p.tiles_m, p.tiles_n, MODE == MODE_MASKED ? p.tiles_m : 8, tm, tn);
  }
  const int m0 = __builtin_amdgcn_readfirstlane(RUNS ? tm * 128 : tm * T::BM);
  const int n0 = __builtin_amdgcn_readfirstlane(tn * T::BN);

  int row_lim = p.M;  // rows [0, row_lim) may be read and written
  const int lo = 0;   // tile rows [lo, hi) are stored
  if (MODE == MODE_MASKED) {
    int v = __builtin_amdgcn_readfirstlane(p.meta[g]);
    v = v < 0 ? 0 : (v > p.M ? p.M : v);
    if (m0 >= v) return;
    row_lim = v;
  } else if (MODE == MODE_CONTIG && !RUNS) {
    const int gb = __builtin_amdgcn_readfirstlane(group_of(m0 / 128));
    if (gb < 0) return;
    g = gb;
  }
  g = __builtin_amdgcn_readfirstlane(g);

  const int KB = __builtin_amdgcn_readfirstlane(p.k_bytes / BK);
  const int NB = (p.N + 127) / 128;
  const uint8_t* A = p.a + (MODE == MODE_MASKED ? (int64_t)g * p.a_gs : 0);
  const uint8_t* B = p.b + (MODE == MODE_DENSE ? 0 : (int64_t)g * p.b_gs);
  uint16_t* D = p.d + (MODE == MODE_MASKED ? (int64_t)g * p.d_gs : 0);
  // accumulate input C, shaped like D (per group for the masked form)
  const void* C = p.c == nullptr ? nullptr
                                 : static_cast<const void*>(static_cast<const uint8_t*>(p.c) +
                                                            (MODE == MODE_MASKED ? (int64_t)g * p.c_gs * (p.c_f32 ? 4 : 2)
                                                                                 : 0));

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
  const uint32_t a_vrow = A_MN ? 0u : (uint32_t)((wave * 8 + lrow) * p.lda);
  const uint32_t b_vrow = B_MN ? 0u : (uint32_t)((wave * 8 + lrow) * p.ldb);
  const uint32_t vchunk = (uint32_t)(lslot ^ lrow);
  const int a_jstep = A_MN ? 0 : T::NW * 8 * (int)p.lda, b_jstep = B_MN ? 0 : T::NW * 8 * (int)p.ldb;
  const uint8_t* const a_tile = A + (int64_t)m0 * p.lda;
  const uint8_t* const b_tile = B + (int64_t)n0 * p.ldb;
  const int a_bytes = A_MN ? 0 : a_rows * (int)p.lda, b_bytes = B_MN ? 0 : b_rows * (int)p.ldb;

  // MN-major operand (stored [K, R] with K-rows ld bytes apart, R = M or N):
  // instruction j fills K-rows [4(j NW + wave), +4) of the stage, lane l the
  // 16-byte slot l % 16 of K-row 4(j NW + wave) + l / 16, from the tile's
  // logical chunk (l % 16) ^ hmn(row).  One buffer resource per operand
  // starts at column r0 of K-row 0 and ends after the operand's last valid
  // byte, so columns past R in the last K-row read zeros (in earlier K-rows
  // they only feed output rows or columns that are never stored); the lane
  // offset carries the K-row, slice included (the host keeps K x ld below
  // 2^31), so a slice's loads need no scalar address work.
  const int k_rows = KB * BK;
  auto mn_rsrc = [&](const uint8_t* base, int64_t ld, int r0, int r_valid) {
    const int64_t avail = (int64_t)(k_rows - 1) * ld + (r_valid - r0);
    const int nrec = (int)max((int64_t)0, min(avail, (int64_t)0x7fffffff));
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + r0), (short)0, nrec, 0x00020000);
  };
  const __amdgpu_buffer_rsrc_t a_mn_rsrc = mn_rsrc(A, A_MN ? p.lda : 0, m0, min(row_lim, m0 + hi));
  const __amdgpu_buffer_rsrc_t b_mn_rsrc = mn_rsrc(B, B_MN ? p.ldb : 0, n0, p.N);
  // CH: 16-byte chunks of the tile's rows per K-row (16, or 12 on a 192-row
  // side).  A lane whose logical chunk lies past them gets an offset beyond
  // the resource (at least 2^31), so the range check turns its load into
  // zeros with no memory access; no fragment read touches its slot.
  auto issue_mn_one = [&](auto ch_tag, uint8_t* stage, __amdgpu_buffer_rsrc_t rsrc, int64_t ld, int kb, int j) {
    constexpr int CH = decltype(ch_tag)::value;
    const int krow = 4 * (j * T::NW + wave) + (lane >> 4);  // K-row in the slice
    const int chunk = (lane & 15) ^ hmn(krow);
    uint32_t voff = (uint32_t)(kb * BK + krow) * (uint32_t)ld + (uint32_t)(chunk << 4);
    if constexpr (CH < 16) voff = chunk < CH ? voff : 0x80000000u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(stage + (j * T::NW + wave) * 1024), 16, voff, 0, 0, 0);
  };
  auto issue_a_one = [&](uint8_t* stage, int kb, int j) {
    if constexpr (A_MN) {
      issue_mn_one(std::integral_constant<int, T::BM / 16>{}, stage, a_mn_rsrc, p.lda, kb, j);
      return;
    }
    const uint32_t hu = (uint32_t)swz((j * T::NW + wave) * 8);
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a_tile + (int64_t)j * a_jstep), (short)0, max(0, a_bytes - j * a_jstep), 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(stage + (j * T::NW + wave) * 1024), 16,
                                             a_vrow + ((vchunk ^ hu) << 4), kb * BK, 0, 0);
  };
  auto issue_b_one = [&](uint8_t* stage, int kb, int j) {
    if constexpr (B_MN) {
      issue_mn_one(std::integral_constant<int, T::BN / 16>{}, stage, b_mn_rsrc, p.ldb, kb, j);
      return;
    }
    const uint32_t hu = (uint32_t)swz((j * T::NW + wave) * 8);
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(b_tile + (int64_t)j * b_jstep), (short)0, max(0, b_bytes - j * b_jstep), 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(stage + (j * T::NW + wave) * 1024), 16,
                                             b_vrow + ((vchunk ^ hu) << 4), kb * BK, 0, 0);
  };
  auto issue_a = [&](uint8_t* stage, int kb) {
#pragma unroll
    for (int j = 0; j < A_LD; ++j) issue_a_one(stage, kb, j);
  };
  auto issue_b = [&](uint8_t* stage, int kb) {
#pragma unroll
    for (int j = 0; j < B_LD; ++j) issue_b_one(stage, kb, j);
  };
  auto issue_loads = [&](int st, int kb) {
    issue_a(stage_a(st), kb);
    issue_b(stage_b(st), kb);
  };

  // Scale staged by this thread (FP8): A row m0 + tid (tid < BM), B column
  // block n0/128 + (tid - BM) (BM <= tid < BM + NBT) or, with row scales, B
  // row n0 + (tid - BM) (BM <= tid < BM + BN), else a harmless duplicate of
  // row 0.
  const bool sc_is_b = tid >= T::BM && tid < T::BM + (ROWB ? T::BN : T::NBT);
  const int64_t sc_row = sc_is_b ? (ROWB ? (int64_t)min(n0 + (tid - T::BM), p.N - 1)
                                         : (int64_t)min(n0 / 128 + (tid - T::BM), NB - 1))
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
  // Without the permutation (PERM false) fragment f reads tile rows
  // wn*TN + 16f + 0..15; its offsets are kept per fragment (the row base is
  // a multiple of 16 but its bits can overlap those of 16f).
  const int fr = lane & 15;
  const int kc = (lane >> 4) * 2;  // first of the lane's two 16-B K chunks
  const int a_base = lds_off(wm * T::TM + fr, kc);                                  // fragment 0, chunk kc
  const int b_base = lds_off(wn * T::TN + (fr >> 2) * 16 + (fr & 3), kc);  // fragment 0, chunk kc (PERM)
  int b_offs[T::PERM ? 1 : T::FN];
#pragma unroll
  for (int f = 0; f < (T::PERM ? 1 : T::FN); ++f) b_offs[f] = lds_off(wn * T::TN + 16 * f + fr, kc);

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
  __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0((FP8 ? 1 : 0) + (S - 1) * LD_ALL));
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
  constexpr int LATE_VM = S == 2 ? B_LD : (S - 2) * LD_ALL;
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
      for (int j = 0; j < B_LD; ++j)
        if (j % T::FN == f) issue_b_one(cur_b, min(kb + S, KB - 1), j);
    }
    if (i + 1 == T::FM) {
#pragma unroll
      for (int j = 0; j < A_LD; ++j)
        if (j % T::FN == f) issue_a_one(cur_a, min(kb + S, KB - 1), j);
    }
  };

  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  // MN-major fragment (16 rows from tile row r0, the lane's 32 K-bytes):
  // four transposing reads.  Lane s of each 16-lane group reads 8 bytes of
  // K-row 32q + 8t + s/2 (q = lane / 16, t = 0..3) at tile columns
  // r0 + 8 (s & 1) .. +7; the group's 16 reads, transposed, hand lane s the
  // bytes of tile row r0 + s at K 32q + 8t .. +7 -- the K-contiguous order of
  // the MFMA operand.  hmn of those K-rows is (s / 2) | (q & 1) << 3 for all t.
  const int mn_s = lane & 15, mn_q = lane >> 4;
  const int mn_h = (mn_s >> 1) | ((mn_q & 1) << 3);
  const int mn_k0 = (32 * mn_q + (mn_s >> 1)) * MN_ROW + 8 * (mn_s & 1);
  auto mn_frag = [&](const uint8_t* stage, int r0) {
    typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
    const int off = mn_k0 + ((((r0 >> 4) ^ mn_h)) << 4);
    i32x8 r;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(stage + off + t * 8 * MN_ROW));
      r[2 * t] = v[0];
      r[2 * t + 1] = v[1];
    }
    return r;
  };
  auto b_frag = [&](const uint8_t* stage, int f) {
    if constexpr (B_MN) return mn_frag(stage, wn * T::TN + 16 * f);
    const int off = T::PERM ? (b_base ^ (swz(f * 4) << 4)) + f * 4 * 128  // rows +4f
                            : b_offs[T::PERM ? 0 : f];
    const i32x4 l = *reinterpret_cast<const i32x4*>(stage + off);
    const i32x4 h = *reinterpret_cast<const i32x4*>(stage + (off ^ 16));
    return i32x8{l[0], l[1], l[2], l[3], h[0], h[1], h[2], h[3]};
  };
  auto a_frag = [&](const uint8_t* stage, int i) {
    if constexpr (A_MN) return mn_frag(stage, wm * T::TM + 16 * i);
    const int off = (a_base ^ (swz(i * 16) << 4)) + i * 16 * 128;  // rows +16i
    const i32x4 l = *reinterpret_cast<const i32x4*>(stage + off);
    const i32x4 h = *reinterpret_cast<const i32x4*>(stage + (off ^ 16));
    return i32x8{l[0], l[1], l[2], l[3], h[0], h[1], h[2], h[3]};
  };
  const int sa_row0 = wm * T::TM + fr;  // this lane's scale slot for fragment row 0
  // B scale slots: block scales -- slot BM + x holds column block n0/128 + x
  // (one per wave, or one per fragment); UE8M0 row scales -- slot BM + r
  // holds B row n0 + r, the row this lane supplies to fragment f; FP32 row
  // scales -- the four output columns of this lane in fragment f, from slot
  // sbv_slot[f] on
  int sb_slot[NSB];
#pragma unroll
  for (int f = 0; f < NSB; ++f)
    sb_slot[f] = T::BM + (ROWB ? (T::PERM ? wn * T::TN + (fr >> 2) * 16 + 4 * f + (fr & 3) : wn * T::TN + 16 * f + fr)
                               : (T::PERM ? (wn * T::TN) / 128 : ((n0 & 127) + wn * T::TN + 16 * f) / 128));
  int sbv_slot[ROWB_F32 ? T::FN : 1];
#pragma unroll
  for (int f = 0; f < (ROWB_F32 ? T::FN : 1); ++f)
    sbv_slot[f] = T::BM + (T::PERM ? wn * T::TN + 16 * (lane >> 4) + 4 * f : wn * T::TN + 16 * f + 4 * (lane >> 4));
  auto read_sbv = [&](int st, int f) { return *reinterpret_cast<const f32x4*>(&ssc[st][sbv_slot[f]]); };

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
  // barrier.  Two groups ahead where a group has fewer than four MFMAs, so
  // that the LDS read latency still has as many MFMAs to hide behind.
  constexpr int PF = T::FN < 4 ? 2 : 1;
  static_assert(PF == 1 || PF == 2, "prefetch depth");
  auto kloop = [&]() {
    i32x8 bf[T::FN];
    i32x8 af, af1;             // A fragments of the current and (PF = 2) the next group
    float sa = 0.f, sa1 = 0.f;  // row scales of those groups
    float sb[NSB];              // B scale(s) of the slice (1 for FP32 row scales)
    f32x4 P[2][T::FN];          // partials of the current and the previous group
    float s_prev[NSB];          // combined scale(s) of the previous group (the first promote adds 0 * 0)
    // FP32 row scales of the lane's output columns, per fragment: of this
    // slice and of the previous one (whose last group is promoted in this
    // slice's first group)
    f32x4 sbv[ROWB_F32 ? T::FN : 1], sbv_prev[ROWB_F32 ? T::FN : 1];
#pragma unroll
    for (int f = 0; f < NSB; ++f) sb[f] = s_prev[f] = 0.f;
#pragma unroll
    for (int f = 0; f < (ROWB_F32 ? T::FN : 1); ++f) sbv[f] = sbv_prev[f] = zero;
#pragma unroll
    for (int f = 0; f < T::FN; ++f) P[(T::FM - 1) & 1][f] = zero;
#pragma unroll
    for (int f = 0; f < T::FN; ++f) bf[f] = b_frag(lds_b0, f);
    af = a_frag(lds_a0, 0);
    af1 = PF == 2 ? a_frag(lds_a0, 1) : af;
    if constexpr (FP8) {
      sa = ssc[0][sa_row0];
      sa1 = PF == 2 ? ssc[0][sa_row0 + 16] : sa;
      if constexpr (ROWB_F32) {
        sb[0] = 1.0f;
#pragma unroll
        for (int f = 0; f < T::FN; ++f) sbv[f] = read_sbv(0, f);
      } else {
#pragma unroll
        for (int f = 0; f < NSB; ++f) sb[f] = ssc[0][sb_slot[f]];
      }
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
        float s_cur[NSB];
#pragma unroll
        for (int f = 0; f < NSB; ++f) s_cur[f] = sa * sb[f];
        // the A fragment / row scale that become current after this group
        // (n0) and, for PF = 2, the one after (n1)
        i32x8 n0 = af1, n1 = af1;
        float ns0 = sa1, ns1 = sa1, nsb[NSB];
#pragma unroll
        for (int f = 0; f < NSB; ++f) nsb[f] = sb[f];
        f32x4 nsbv[ROWB_F32 ? T::FN : 1];
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
            if constexpr (ROWB_F32) {
#pragma unroll
              for (int f = 0; f < T::FN; ++f) nsbv[f] = read_sbv(NX, f);
            } else {
#pragma unroll
              for (int f = 0; f < NSB; ++f) nsb[f] = ssc[NX][sb_slot[f]];
            }
          }
          n0 = a_frag(nxt_a, 0);
        }
        if constexpr (UE8) {
          // power-of-two scales go into the MFMA itself: its scale operands
          // multiply by 2^(e-127) per A row (the lane's row) and per B row
          // (the fragment's 128-column block), and it accumulates in place
          const int ea = (int)(__float_as_uint(sa) >> 23);
#pragma unroll
          for (int f = 0; f < T::FN; ++f) {
            __builtin_amdgcn_sched_barrier(0);
            const int eb = (int)(__float_as_uint(sb[NSB == 1 ? 0 : f]) >> 23);
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
            P[i & 1][f] = mfma_fp8_unscaled(bf[f], af, zero);
            spread_loads(i, f, cur_a, cur_b, kb);
            __builtin_amdgcn_sched_barrier(0);
            const float sp = s_prev[NSB == 1 ? 0 : f];
            if constexpr (ROWB_F32) {
              if (i > 0) acc[i - 1][f] += P[(i - 1) & 1][f] * (sbv[f] * sp);
              else acc[T::FM - 1][f] += P[(T::FM - 1) & 1][f] * (sbv_prev[f] * sp);
            } else {
              if (i > 0) acc[i - 1][f] += P[(i - 1) & 1][f] * sp;
              else acc[T::FM - 1][f] += P[(T::FM - 1) & 1][f] * sp;
            }
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
#pragma unroll
        for (int f = 0; f < NSB; ++f) s_prev[f] = s_cur[f];
        if (PF == 1) {
          af = n0;
          sa = ns0;
        } else {
          af = i + 1 < T::FM ? af1 : n0;
          sa = i + 1 < T::FM ? sa1 : ns0;
          af1 = n1;
          sa1 = ns1;
        }
#pragma unroll
        for (int f = 0; f < NSB; ++f) sb[f] = nsb[f];
        if constexpr (ROWB_F32) {
          if (i + 1 == T::FM) {
#pragma unroll
            for (int f = 0; f < T::FN; ++f) {
              sbv_prev[f] = sbv[f];
              sbv[f] = nsbv[f];
            }
          }
        }
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
    if constexpr (FP8 && !UE8) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int f = 0; f < T::FN; ++f) {
        if constexpr (ROWB_F32) acc[T::FM - 1][f] += P[(T::FM - 1) & 1][f] * (sbv_prev[f] * s_prev[0]);
        else acc[T::FM - 1][f] += P[(T::FM - 1) & 1][f] * s_prev[T::NSB == 1 ? 0 : f];
      }
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
  if (!live) {
    if constexpr (OUT == OUT_FP8) {
      // the FP8 epilogue's two barriers (the rows of this wave are past M,
      // and so are those of its partner wave, so nothing here is read)
      __syncthreads();
      __syncthreads();
    }
    return;
  }

  if constexpr (OUT == OUT_FP8) {
    epilogue_fp8<T>(p, acc, lds_b0, m0, n0, wm, wn, lane, row_lim);
  } else if constexpr (!T::PERM) {
    epilogue_cols4<T, OUT>(p, D, acc, m0, n0, wm, wn, lane, lo, hi, row_lim, C);
  } else {
    // ---- epilogue: BF16, row m = lane%16 of each fragment row, 16 consecutive columns per lane
    const int col0 = n0 + wn * T::TN + (lane >> 4) * 16;
    const bool vec_ok = ((p.ldd & 7) == 0) && ((reinterpret_cast<uintptr_t>(D) & 15) == 0);
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
      const int rl = wm * T::TM + i * 16 + fr;
      const int row = m0 + rl;
      if (rl < lo || rl >= hi || row >= row_lim) continue;
      if (C != nullptr) {
        // D = C + A . B^T ("DeepInside DeepGEMM", section 4): C is added to the
        // FP32 accumulator before the BF16 rounding (read before d is written,
        // so c may be d itself)
        const int cc = col0;
        if (p.c_f32) {
          const float* crow = static_cast<const float*>(C) + (int64_t)row * p.ldc;
          const bool cvec = ((p.ldc & 3) == 0) && ((reinterpret_cast<uintptr_t>(C) & 15) == 0) && cc + 16 <= p.N;
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
          const uint16_t* crow = static_cast<const uint16_t*>(C) + (int64_t)row * p.ldc;
          const bool cvec = ((p.ldc & 7) == 0) && ((reinterpret_cast<uintptr_t>(C) & 15) == 0) && cc + 16 <= p.N;
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
      if constexpr (OUT == OUT_F32) {
        // the FP32 values themselves (dense): four 16-byte stores of 4 columns
        float* frow = reinterpret_cast<float*>(D) + (int64_t)row * p.ldd;
        const bool f_ok = ((p.ldd & 3) == 0) && ((reinterpret_cast<uintptr_t>(D) & 15) == 0);
#pragma unroll
        for (int f = 0; f < T::FN; ++f) {
          const int c = col0 + 4 * f;
          if (f_ok && c + 4 <= p.N) {
            *reinterpret_cast<f32x4*>(frow + c) = acc[i][f];
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (c + e < p.N) frow[c + e] = acc[i][f][e];
          }
        }
        continue;
      }
      uint32_t packed[8];
#pragma unroll
      for (int f = 0; f < T::FN; ++f) {
        // (the contiguous kernels keep the integer rounding: with the
        // hardware conversion the 256 x 256 UE8M0 one spills in its K loop)
        const i32x2 wv = MODE == MODE_CONTIG ? to_bf16x4_bits_int(acc[i][f]) : to_bf16x4_bits(acc[i][f]);
        packed[2 * f] = (uint32_t)wv[0];
        packed[2 * f + 1] = (uint32_t)wv[1];
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
}

using TileL = TileShape<256, 256, 2, 4, 2>;  // 512 threads, wave tile 128 x 64, 2 x 64 KB stages
using TileW = TileShape<128, 256, 2, 4, 3>;  // 512 threads, wave tile  64 x 64, 3 x 48 KB stages
using TileS = TileShape<128, 128, 2, 2, 3>;  // 256 threads, wave tile  64 x 64, 3 x 32 KB stages
using TileT = TileShape<256, 128, 4, 2, 3>;  // 512 threads, wave tile  64 x 64, 3 x 48 KB stages
using TileN = TileShape<256, 192, 2, 4, 2>;  // 512 threads, wave tile 128 x 48, 2 x 56 KB stages
using TileQ = TileShape<192, 192, 2, 4, 2>;  // 512 threads, wave tile  96 x 48, 2 x 48 KB stages (dense only)

enum Variant : int { VAR_L = 0, VAR_W = 1, VAR_S = 2, VAR_T = 3, VAR_N = 4, VAR_Q = 5 };

// Launch one tile configuration.  ROWB: whether the per-row B scale kernels
// exist for this tile (they need a thread per tile row of A and of B and the
// registers for per-lane column scales: the 256 x 192 and 128-row tiles).
template <class T, int KIND, bool ROWB>
hipError_t launch_tile(const GemmParams& p, int mode, int sf_fmt, int64_t grid, hipStream_t stream) {
  const dim3 g((unsigned)grid), b(T::NT);
  if (p.d_f32) {
    // FP32 D: every kind, form and scale format
    if constexpr (KIND == KIND_BF16) {
      if (mode == MODE_DENSE) gemm_kernel<T, KIND_BF16, SF_F32, MODE_DENSE, OUT_F32><<<g, b, 0, stream>>>(p);
      else if (mode == MODE_CONTIG) gemm_kernel<T, KIND_BF16, SF_F32, MODE_CONTIG, OUT_F32><<<g, b, 0, stream>>>(p);
      else gemm_kernel<T, KIND_BF16, SF_F32, MODE_MASKED, OUT_F32><<<g, b, 0, stream>>>(p);
    } else {
#define DGMI_LAUNCH_F32(SF_)                                                                                 \
  do {                                                                                                       \
    if (mode == MODE_DENSE) gemm_kernel<T, KIND_FP8, SF_, MODE_DENSE, OUT_F32><<<g, b, 0, stream>>>(p);     \
    else if (mode == MODE_CONTIG) gemm_kernel<T, KIND_FP8, SF_, MODE_CONTIG, OUT_F32><<<g, b, 0, stream>>>(p); \
    else gemm_kernel<T, KIND_FP8, SF_, MODE_MASKED, OUT_F32><<<g, b, 0, stream>>>(p);                       \
  } while (0)
      if (sf_fmt == SF_F32) {
        DGMI_LAUNCH_F32(SF_F32);
      } else if (sf_fmt == SF_UE8M0) {
        DGMI_LAUNCH_F32(SF_UE8M0);
      } else if constexpr (ROWB) {
        if (sf_fmt == (SF_F32 | SF_ROWB)) DGMI_LAUNCH_F32(SF_F32 | SF_ROWB);
        else DGMI_LAUNCH_F32(SF_UE8M0 | SF_ROWB);
      } else {
        return hipErrorInvalidValue;  // the launch plan never picks this tile for row scales
      }
#undef DGMI_LAUNCH_F32
    }
    return hipGetLastError();
  }
  if constexpr (KIND == KIND_BF16) {
    if (mode == MODE_DENSE) gemm_kernel<T, KIND_BF16, SF_F32, MODE_DENSE><<<g, b, 0, stream>>>(p);
    else if (mode == MODE_CONTIG) gemm_kernel<T, KIND_BF16, SF_F32, MODE_CONTIG><<<g, b, 0, stream>>>(p);
    else gemm_kernel<T, KIND_BF16, SF_F32, MODE_MASKED><<<g, b, 0, stream>>>(p);
    return hipGetLastError();
  } else {
#define DGMI_LAUNCH(SF_)                                                                           \
  do {                                                                                             \
    if (mode == MODE_DENSE) gemm_kernel<T, KIND_FP8, SF_, MODE_DENSE><<<g, b, 0, stream>>>(p);     \
    else if (mode == MODE_CONTIG) gemm_kernel<T, KIND_FP8, SF_, MODE_CONTIG><<<g, b, 0, stream>>>(p); \
    else gemm_kernel<T, KIND_FP8, SF_, MODE_MASKED><<<g, b, 0, stream>>>(p);                       \
  } while (0)
    if (sf_fmt == SF_F32) {
      DGMI_LAUNCH(SF_F32);
    } else if (sf_fmt == SF_UE8M0) {
      DGMI_LAUNCH(SF_UE8M0);
    } else if constexpr (ROWB) {
      if (sf_fmt == (SF_F32 | SF_ROWB)) DGMI_LAUNCH(SF_F32 | SF_ROWB);
      else DGMI_LAUNCH(SF_UE8M0 | SF_ROWB);
    } else {
      return hipErrorInvalidValue;  // the launch plan never picks this tile for row scales
    }
#undef DGMI_LAUNCH
    return hipGetLastError();
  }
}

// Launch one tile configuration of the dense FP8 GEMM with FP8 output.
// ROWB: whether the tile also takes one B scale per row (not the 256 x 256
// tile, which has no registers for the per-lane column scales).
template <class T, bool ROWB>
hipError_t launch_tile_fp8_out(const GemmParams& p, int sf_fmt, int64_t grid, hipStream_t stream) {
  const dim3 g((unsigned)grid), b(T::NT);
  if (sf_fmt == SF_F32) {
    gemm_kernel<T, KIND_FP8, SF_F32, MODE_DENSE, OUT_FP8><<<g, b, 0, stream>>>(p);
  } else if (sf_fmt == SF_UE8M0) {
    gemm_kernel<T, KIND_FP8, SF_UE8M0, MODE_DENSE, OUT_FP8><<<g, b, 0, stream>>>(p);
  } else if constexpr (ROWB) {
    if (sf_fmt == (SF_F32 | SF_ROWB)) gemm_kernel<T, KIND_FP8, SF_F32 | SF_ROWB, MODE_DENSE, OUT_FP8><<<g, b, 0, stream>>>(p);
    else if (sf_fmt == (SF_UE8M0 | SF_ROWB)) gemm_kernel<T, KIND_FP8, SF_UE8M0 | SF_ROWB, MODE_DENSE, OUT_FP8><<<g, b, 0, stream>>>(p);
    else return hipErrorInvalidValue;
  } else {
    return hipErrorInvalidValue;  // the launch plan never picks this tile for row scales
  }
  return hipGetLastError();
}

// Launch the 192 x 192 tile: the dense GEMMs only (FP8 with block or row
// scales, FP32 or UE8M0, or BF16; BF16 or FP32 output).  Its 192-row tiles do not
// align with the 128-row blocks of the grouped layouts.
template <int KIND>
hipError_t launch_tile_q(const GemmParams& p, int mode, int sf_fmt, int64_t grid, hipStream_t stream) {
  if constexpr (KIND == KIND_FP8) {
    if (mode != MODE_DENSE) return hipErrorInvalidValue;
    const dim3 g((unsigned)grid), b(TileQ::NT);
    if (sf_fmt == (SF_F32 | SF_ROWB)) {
      if (p.d_f32) gemm_kernel<TileQ, KIND_FP8, SF_F32 | SF_ROWB, MODE_DENSE, OUT_F32><<<g, b, 0, stream>>>(p);
      else gemm_kernel<TileQ, KIND_FP8, SF_F32 | SF_ROWB, MODE_DENSE><<<g, b, 0, stream>>>(p);
    } else if (sf_fmt == (SF_UE8M0 | SF_ROWB)) {
      if (p.d_f32) gemm_kernel<TileQ, KIND_FP8, SF_UE8M0 | SF_ROWB, MODE_DENSE, OUT_F32><<<g, b, 0, stream>>>(p);
      else gemm_kernel<TileQ, KIND_FP8, SF_UE8M0 | SF_ROWB, MODE_DENSE><<<g, b, 0, stream>>>(p);
    } else if (sf_fmt != SF_F32 && sf_fmt != SF_UE8M0) {
      return hipErrorInvalidValue;
    } else if (p.d_f32) {
      if (sf_fmt == SF_F32) gemm_kernel<TileQ, KIND_FP8, SF_F32, MODE_DENSE, OUT_F32><<<g, b, 0, stream>>>(p);
      else gemm_kernel<TileQ, KIND_FP8, SF_UE8M0, MODE_DENSE, OUT_F32><<<g, b, 0, stream>>>(p);
    } else {
      if (sf_fmt == SF_F32) gemm_kernel<TileQ, KIND_FP8, SF_F32, MODE_DENSE><<<g, b, 0, stream>>>(p);
      else gemm_kernel<TileQ, KIND_FP8, SF_UE8M0, MODE_DENSE><<<g, b, 0, stream>>>(p);
    }
    return hipGetLastError();
  } else {
    if (mode != MODE_DENSE) return hipErrorInvalidValue;
    const dim3 g((unsigned)grid), b(TileQ::NT);
    if (p.d_f32) gemm_kernel<TileQ, KIND_BF16, SF_F32, MODE_DENSE, OUT_F32><<<g, b, 0, stream>>>(p);
    else gemm_kernel<TileQ, KIND_BF16, SF_F32, MODE_DENSE><<<g, b, 0, stream>>>(p);
    return hipGetLastError();
  }
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
    case VAR_L: return launch_tile<TileL, KIND, false>(p, mode, sf_fmt, grid, stream);
    case VAR_W: return launch_tile<TileW, KIND, true>(p, mode, sf_fmt, grid, stream);
    case VAR_T: return launch_tile<TileT, KIND, false>(p, mode, sf_fmt, grid, stream);
    case VAR_N: return launch_tile<TileN, KIND, true>(p, mode, sf_fmt, grid, stream);
    case VAR_Q: return launch_tile_q<KIND>(p, mode, sf_fmt, grid, stream);
    default: return launch_tile<TileS, KIND, true>(p, mode, sf_fmt, grid, stream);
  }
}

// Launch plan for problems above 128 rows, a pure function of the shapes.
// The 256 x 256 tile computes whole rounds of one tile per CU; when its tile
// count leaves the last round partly idle, the 256 x 192 tile may take all
// columns, or columns [n_split, N) in a second launch after the 256 x 256
// tile's [0, n_split).  Cost model, in K-loop slices of the 256 x 256 tile
// (both kinds move 128 bytes of K per slice), from per-wave cycle stamps of
// the FP8 kernel on 4096 x {4096, 3072, 2112} x {7168, 2048}: a 256 x 192
// slice costs 0.88 of one (2320 against 2640 cycles); every round adds 7
// (prologue and epilogue, about 18.6K cycles); a second launch adds 5.7 (the
// first launch's tail and the launch gap, about 15K cycles).  A round costs
// rounds(tiles) * (KB * slice + 7).  E.g. M = 4096: N = 2112, K = 7168 goes
// to 176 tiles of 256 x 192 (63 -> 56.3); BF16 N = 7168, K = 16384 (256
// slices) splits at 4096 (526 -> 501); N = 7168, K = 2048 stays on 256 x 256.
// The dense FP8 GEMM may also take 192 x 192 tiles (slice 0.75 from the same
// stamps-and-timing fit: 4096 x 2112 x 7168 on 242 tiles of 192 x 192 took
// 70.3 us against 80.9 us on 176 of 256 x 192, builds alternated).
// Only the BF16 kind splits: the FP8 kernel runs at the power limit, and in
// a partly idle last round its busy CUs clock higher (2.03 GHz with 176 of
// 256 busy, 1.86 with all), which recovers what the second launch would
// save.  Measured on 4096 x 7168 x 16384, one box, builds alternated: FP8
// split 390.7 against 391.6 us back to back and 387.6 against 380.4 us in
// the benchmark's step; BF16 split 3% faster in both.
constexpr int NUM_CU = 256;
// Cost model constants, in K-loop slices of the 256 x 256 tile (above).
constexpr double SLICE_256x192 = 0.88, SLICE_192x192 = 0.75, PER_ROUND = 7.0, PER_LAUNCH = 5.7;

// Cost of one launch of `tiles` tiles of KB slices each, at `slice` per slice:
// whole rounds of one tile per CU.
double launch_cost(int64_t tiles, int64_t KB, double slice) {
  const int64_t rounds = (tiles + NUM_CU - 1) / NUM_CU;
  return (double)rounds * ((double)KB * slice + PER_ROUND);
}

// Whether the dense 192 x 192 tile costs less than `other` (one launch).
bool dense_q_wins(int64_t M, int64_t N, int64_t KB, double other) {
  return launch_cost(((M + 191) / 192) * ((N + 191) / 192), KB, SLICE_192x192) < other;
}

template <int KIND>
GemmPlan plan_large(int mode, int64_t G, int64_t M, int64_t N, int64_t KB) {
  const int64_t units = (mode == MODE_MASKED ? G : 1) * ((M + 255) / 256);
  auto cost = [&](int64_t cols, int64_t bn, double slice) {
    return launch_cost(units * ((cols + bn - 1) / bn), KB, slice);
  };
  GemmPlan best;
  best.parts = 1;
  best.n_split = N;
  best.cfg[0] = make_cfg<TileL, KIND>(VAR_L);
  double best_cost = cost(N, 256, 1.0);
  const double only_n = cost(N, 192, SLICE_256x192);
  if (only_n < best_cost) {
    best_cost = only_n;
    best.cfg[0] = make_cfg<TileN, KIND>(VAR_N);
  }
  if (mode == MODE_DENSE && dense_q_wins(M, N, KB, best_cost)) {
    // 192 x 192 tiles (dense only: they do not align with the grouped layouts' 128-row blocks)
    best_cost = launch_cost(((M + 191) / 192) * ((N + 191) / 192), KB, SLICE_192x192);
    best.cfg[0] = make_cfg<TileQ, KIND>(VAR_Q);
  }
  for (int64_t n1 = 256; KIND == KIND_BF16 && n1 < N; n1 += 256) {
    const double c = cost(n1, 256, 1.0) + cost(N - n1, 192, SLICE_256x192) + PER_LAUNCH;
    if (c < best_cost) {
      best_cost = c;
      best.parts = 2;
      best.n_split = n1;
      best.cfg[0] = make_cfg<TileL, KIND>(VAR_L);
      best.cfg[1] = make_cfg<TileN, KIND>(VAR_N);
    }
  }
  return best;
}

template <int KIND>
hipError_t launch_plan(const GemmPlan& plan, GemmParams p, int mode, int sf_fmt, hipStream_t stream) {
  for (int part = 0; part < plan.parts; ++part) {
    GemmParams q = p;
    const int64_t n_off = part == 0 ? 0 : plan.n_split;
    const int64_t n_len = plan.parts == 1 ? p.N : (part == 0 ? plan.n_split : p.N - plan.n_split);
    if (n_off > 0) {
      // columns [n_off, N): B rows, the B scale rows of their 128-column
      // blocks (n_off is a multiple of 256), D and C columns
      q.b = p.b + n_off * p.ldb;
      if (KIND == KIND_FP8) q.sfb = static_cast<const uint32_t*>(p.sfb) + (n_off / 128) * p.sfb_sn;
      q.d = p.d + n_off * (p.d_f32 ? 2 : 1);  // (F32 D: two BF16-sized units per element)
      if (p.c != nullptr) q.c = static_cast<const uint8_t*>(p.c) + n_off * (p.c_f32 ? 4 : 2);
    }
    q.N = (int32_t)n_len;
    const TileCfg& cfg = plan.cfg[part];
    q.tiles_m = (q.M + cfg.bm - 1) / cfg.bm;
    q.tiles_n = (q.N + cfg.bn - 1) / cfg.bn;
    const int64_t grid = gemm_grid(cfg, mode, q.G, q.M, q.N);
    if (grid == 0) continue;
    const hipError_t e = launch_variant<KIND>(cfg, q, mode, sf_fmt, grid, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

// Tile choice, a pure function of the shapes.  Rows <= 128 (small dense M,
// decode buffers of up to 128 rows per expert) use 128-row tiles with three
// stages (one launch); everything else 256-row tiles with two stages (three
// do not fit in LDS): the 256 x 256 tile, which measured fastest on all the
// large dense and grouped shapes whose tiles fill whole rounds of the CUs,
// with the 256 x 192 tile taking all or part of the columns when that fills
// the last round better, or (dense only) the 192 x 192 tile where a problem
// fits one round of it (plan_large, dense_q_wins).  One B scale per row of B
// takes the 256 x 192 or 192 x 192 tile above 128 rows.
GemmPlan fp8_gemm_plan(int mode, int64_t G, int64_t M, int64_t N, int64_t K, int sf_fmt) {
  // rows <= 128, or a contiguous layout too long for the 256-row tiles' list
  const bool rows128 = M <= 128 || (mode == MODE_CONTIG && M / 128 > RUNS_MAX_BLOCKS);
  if (!rows128 && (sf_fmt & SF_ROWB)) {
    // row scales: the 256 x 192 tile (the 256 x 256 FP32 kernel has no
    // registers left for per-lane column scales)
    GemmPlan p;
    p.parts = 1;
    p.n_split = N;
    p.cfg[0] = make_cfg<TileN, KIND_FP8>(VAR_N);
    if (mode == MODE_DENSE) {  // or 192 x 192 tiles where they cost less (plan_large's model)
      const int64_t KB = (K + 127) / 128;
      if (dense_q_wins(M, N, KB, launch_cost(((M + 255) / 256) * ((N + 191) / 192), KB, SLICE_256x192)))
        p.cfg[0] = make_cfg<TileQ, KIND_FP8>(VAR_Q);
    }
    return p;
  }
  if (rows128) {
    GemmPlan p;
    p.parts = 1;
    p.n_split = N;
    p.cfg[0] = N <= 128 ? make_cfg<TileS, KIND_FP8>(VAR_S) : make_cfg<TileW, KIND_FP8>(VAR_W);
    return p;
  }
  return plan_large<KIND_FP8>(mode, G, M, N, (K + BK - 1) / BK);
}

int64_t gemm_grid(const TileCfg& cfg, int mode, int64_t G, int64_t M, int64_t N) {
  const int64_t tm = (M + cfg.bm - 1) / cfg.bm, tn = (N + cfg.bn - 1) / cfg.bn;
  // contiguous 256-row tiles: one workgroup per 128-row block (at most one
  // tile starts there) and column tile; those past the listed tiles exit
  if (mode == MODE_CONTIG && cfg.bm == 256) return (M / 128) * tn;
  return (mode == MODE_MASKED ? G : 1) * tm * tn;
}

int64_t plan_grid(const GemmPlan& plan, int part, int mode, int64_t G, int64_t M, int64_t N) {
  if (part >= plan.parts) return 0;
  const int64_t n_len = plan.parts == 1 ? N : (part == 0 ? plan.n_split : N - plan.n_split);
  return gemm_grid(plan.cfg[part], mode, G, M, n_len);
}

int plan_lds(const GemmPlan& plan, int part, int mode) {
  if (part >= plan.parts) return 0;
  const TileCfg& c = plan.cfg[part];
  // contiguous 256-row tiles: the run scan's wave masks (8 bytes) and tile
  // counts (4 bytes) per wave, beside the stages
  return c.lds_bytes + ((mode == MODE_CONTIG && c.bm == 256) ? (c.threads / 64) * 12 : 0);
}

// Dense FP8 GEMM with an MN-major A and/or B: one launch of the 256 x 192
// tile, whose 48-column wave tiles keep the MFMA's column order (the
// transposing B fragment reads hand each 8-lane run 8 consecutive columns,
// which the permuted order of the 64-column wave tiles does not keep).
GemmPlan fp8_mn_gemm_plan() {
  GemmPlan p;
  p.parts = 1;
  p.n_split = 0;
  p.cfg[0] = make_cfg<TileN, KIND_FP8>(VAR_N);
  p.cfg[0].lds_bytes = 2 * 2 * BK * MN_ROW + 2 * TileN::NT * 4;  // both operands MN-major (the largest)
  return p;
}

hipError_t launch_fp8_gemm_mn(GemmParams p, int sf_fmt, hipStream_t stream) {
  p.tiles_m = (p.M + TileN::BM - 1) / TileN::BM;
  p.tiles_n = (p.N + TileN::BN - 1) / TileN::BN;
  const dim3 g((unsigned)((int64_t)p.tiles_m * p.tiles_n)), b(TileN::NT);
  const int lay = (p.a_mn ? 1 : 0) | (p.b_mn ? 2 : 0);
  if (sf_fmt != SF_F32 && sf_fmt != SF_UE8M0 && sf_fmt != (SF_F32 | SF_ROWB) && sf_fmt != (SF_UE8M0 | SF_ROWB))
    return hipErrorInvalidValue;
#define DGMI_LAUNCH_MN_SF(SF_, LAY_)                                                                            \
  do {                                                                                                          \
    if (p.d_f32) gemm_kernel<TileN, KIND_FP8, SF_, MODE_DENSE, OUT_F32, LAY_><<<g, b, 0, stream>>>(p);         \
    else gemm_kernel<TileN, KIND_FP8, SF_, MODE_DENSE, OUT_BF16, LAY_><<<g, b, 0, stream>>>(p);                \
  } while (0)
#define DGMI_LAUNCH_MN(LAY_)                                                                                    \
  do {                                                                                                          \
    if (sf_fmt == SF_F32) DGMI_LAUNCH_MN_SF(SF_F32, LAY_);                                                      \
    else if (sf_fmt == SF_UE8M0) DGMI_LAUNCH_MN_SF(SF_UE8M0, LAY_);                                             \
    else if (sf_fmt == (SF_F32 | SF_ROWB)) DGMI_LAUNCH_MN_SF(SF_F32 | SF_ROWB, LAY_);                           \
    else DGMI_LAUNCH_MN_SF(SF_UE8M0 | SF_ROWB, LAY_);                                                           \
  } while (0)
  if (lay == 1) DGMI_LAUNCH_MN(1);
  else if (lay == 2) DGMI_LAUNCH_MN(2);
  else if (lay == 3) DGMI_LAUNCH_MN(3);
  else return hipErrorInvalidValue;
#undef DGMI_LAUNCH_MN
#undef DGMI_LAUNCH_MN_SF
  return hipGetLastError();
}

hipError_t launch_fp8_gemm(GemmParams p, int mode, int sf_fmt, hipStream_t stream) {
  if (p.a_mn || p.b_mn) {
    if (mode != MODE_DENSE) return hipErrorInvalidValue;
    return launch_fp8_gemm_mn(p, sf_fmt, stream);
  }
  return launch_plan<KIND_FP8>(fp8_gemm_plan(mode, p.G, p.M, p.N, p.k_bytes, sf_fmt), p, mode, sf_fmt, stream);
}

// Dense FP8 GEMM with FP8 output: the tiles whose waves cover 64 columns
// (a 128-column block is two neighbouring waves), one launch: 256 x 256
// above 128 rows, the 128-row tiles below.
GemmPlan fp8_out_gemm_plan(int64_t M, int64_t N, int sf_fmt) {
  GemmPlan p;
  p.parts = 1;
  p.n_split = N;
  if (M > 128) {
    // one B scale per row: the 256 x 128 tile (wave tile 64 x 64, 64 columns
    // per wave as the FP8 epilogue needs, registers to spare)
    p.cfg[0] = (sf_fmt & SF_ROWB) ? make_cfg<TileT, KIND_FP8>(VAR_T) : make_cfg<TileL, KIND_FP8>(VAR_L);
  } else {
    p.cfg[0] = N <= 128 ? make_cfg<TileS, KIND_FP8>(VAR_S) : make_cfg<TileW, KIND_FP8>(VAR_W);
  }
  return p;
}

hipError_t launch_fp8_gemm_fp8_out(GemmParams p, int sf_fmt, hipStream_t stream) {
  const TileCfg cfg = fp8_out_gemm_plan(p.M, p.N, sf_fmt).cfg[0];
  p.tiles_m = (p.M + cfg.bm - 1) / cfg.bm;
  p.tiles_n = (p.N + cfg.bn - 1) / cfg.bn;
  const int64_t grid = gemm_grid(cfg, MODE_DENSE, 1, p.M, p.N);
  if (grid == 0) return hipSuccess;
  switch (cfg.variant) {
    case VAR_L: return launch_tile_fp8_out<TileL, false>(p, sf_fmt, grid, stream);
    case VAR_T: return launch_tile_fp8_out<TileT, true>(p, sf_fmt, grid, stream);
    case VAR_W: return launch_tile_fp8_out<TileW, true>(p, sf_fmt, grid, stream);
    default: return launch_tile_fp8_out<TileS, true>(p, sf_fmt, grid, stream);
  }
}

// BF16 GEMMs: the same tile choice as the FP8 GEMM (a K-slice is 64 BF16
// elements instead of 128 FP8 ones, the bytes per tile are the same).
GemmPlan bf16_gemm_plan(int mode, int64_t G, int64_t M, int64_t N, int64_t K) {
  if (M <= 128 || (mode == MODE_CONTIG && M / 128 > RUNS_MAX_BLOCKS)) {
    GemmPlan p;
    p.parts = 1;
    p.n_split = N;
    p.cfg[0] = N <= 128 ? make_cfg<TileS, KIND_BF16>(VAR_S) : make_cfg<TileW, KIND_BF16>(VAR_W);
    return p;
  }
  return plan_large<KIND_BF16>(mode, G, M, N, (2 * K + BK - 1) / BK);
}

hipError_t launch_bf16_gemm(GemmParams p, int mode, hipStream_t stream) {
  return launch_plan<KIND_BF16>(bf16_gemm_plan(mode, p.G, p.M, p.N, p.k_bytes / 2), p, mode, SF_F32, stream);
}

}  // namespace dgmi
