/*
 * dgmi.h -- C ABI of the block-scaled FP8 (grouped) GEMM library for MI355X.
 *
 * The library (libdgmi.so) computes DeepGEMM-style FP8 GEMMs with
 * fine-grained scaling on gfx950: E4M3 operands, one FP32 scale per 1x128
 * K-block of each activation row and one per 128x128 block of the weights
 * (or the same scales as power-of-two UE8M0 exponents packed four to an
 * int32), each 128-wide K-block contracted on the matrix cores and promoted
 * into an FP32 accumulator multiplied by both scales, BF16 out.
 *   "DeepInside DeepGEMM: Unpacking DeepSeek's Unified Tensor Core Library
 *    for SM90 and SM100", section 2 (NT layout, FP32 or packed UE8M0 scale
 *    factors) and section 4 (fp8_gemm_nt(a, b, a_sf, b_sf, c, bf16)).
 *
 * Conventions shared by every entry point
 *   - Every buffer is device memory allocated and owned by the caller,
 *     outputs included.  The library never allocates, frees, synchronises,
 *     reads device memory on the host, or keeps a pointer after returning
 *     ("DeepGEMM CUDA Graph Compatibility for Masked Grouped GEMMs",
 *     sections "Eliminating Host-Side Allocation" and "Tensor-Based
 *     Metadata Arguments").
 *   - Each call validates shapes/dtypes/strides on the host, then enqueues
 *     its kernels on `stream` (NULL = the null stream) and returns.  The
 *     launch configuration depends only on the shapes, never on device
 *     data, so every entry point except dgmi_init may be captured into a
 *     hipGraph and replayed (same page, section "Stateless Kernel
 *     Architecture").  Device faults surface at the caller's next sync.
 *   - Tensors are described by dg_tensor: shape and strides in ELEMENTS.
 *     The innermost (last) stride of every data operand must be 1.
 *   - On error nothing is launched, the call returns a non-zero status and
 *     dg_last_error() describes it.  Calls are reentrant and thread-safe.
 */
#ifndef DGMI_H
#define DGMI_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
enum {
  DG_F32 = 0,  /* IEEE binary32 */
  DG_BF16 = 1, /* bfloat16 */
  DG_E4M3 = 2, /* OCP FP8 E4M3 ("fn": max 448, no inf), one byte */
  DG_I32 = 3   /* int32: masked_m, grouped_layout, packed UE8M0 scales */
};

/* status codes */
enum {
  DG_OK = 0,
  DG_INVALID_ARG = 1,   /* null / dtype / ndim / shape / stride / alignment / aliasing */
  DG_UNSUPPORTED = 2,   /* legal but not implemented (K % 128 != 0; GEMM operand row strides of 8 MiB or more) */
  DG_LAUNCH_FAILED = 3  /* the HIP runtime rejected a launch */
};

typedef struct dg_tensor {
  void* data;        /* device pointer, caller-owned */
  int32_t dtype;     /* DG_* element type */
  int32_t ndim;      /* 1..4 */
  int64_t shape[4];
  int64_t stride[4]; /* in elements */
} dg_tensor;

/* Message for the last non-zero status returned on this thread. */
const char* dg_last_error(void);

/* Optional eager set-up (checks that a gfx950 device is current).  Not
 * capture-safe; every other entry point works without calling it. */
int dgmi_init(void);

/*
 * D = A . B^T, block-scaled FP8, BF16 out ("DeepInside DeepGEMM", section 4:
 * the NT GEMM fp8_gemm_nt with D = C + A @ B.T).
 *   a   E4M3 [M, K]          row stride lda (elements = bytes), 16-B aligned
 *   b   E4M3 [N, K]          weights in NT layout (K contiguous)
 *   sfa F32  [M, K/128]      any strides (K-major or M-major), or
 *       I32  [M, ceil(K/512)] packed UE8M0 (byte j of word i: K-block 4i+j)
 *   sfb F32  [ceil(N/128), K/128] or I32 [ceil(N/128), ceil(K/512)]: one
 *       scale per 128x128 block of B; or F32 [N, K/128] or I32
 *       [N, ceil(K/512)]: one scale per row of B (the per-row b_sf of the
 *       section's example), told apart by the row count (for N = 1 the two
 *       forms are the same).  sfa and sfb must use the same format.
 *   c   NULL, or the accumulate input C: BF16 or F32 [M, N], any row stride
 *       (innermost stride 1), element-aligned; it may be d itself (same base,
 *       dtype and strides: an in-place D += A . B^T), any other overlap with d
 *       is rejected.  Each element of C is added to the FP32 accumulator
 *       before the BF16 rounding (same section: D = C + A @ B.T).
 *   d   BF16 [M, N], any row stride (innermost stride 1); or F32 [M, N],
 *       4-B aligned: the FP32 accumulator (C added) stored without rounding
 *       (the section's call takes the output dtype as an argument); with
 *       c = d in F32 this is the in-place D += A . B^T.  Either scale form
 *       of B goes with either output dtype.
 * D[m,n] = C[m,n] + sum_kb (sum_{k in kb} A[m,k] B[n,k]) * sfa[m,kb] * sfb[n/128,kb]
 * (sfb[n,kb] with one scale per row of B).
 * K must be a multiple of 128; M and N are arbitrary.
 * a or b may also be MN-major: the transposed view ([M, K] with strides
 * (1, lda)) of a row-major [K, M] tensor, likewise b of a [K, N] one -- the
 * layouts of fp8_gemm_nn / _tn / _tt below, with their conditions.
 */
int fp8_gemm_nt(const dg_tensor* a, const dg_tensor* b, const dg_tensor* sfa,
                const dg_tensor* sfb, const dg_tensor* c, const dg_tensor* d,
                hipStream_t stream);

/*
 * The NN, TN and TT layouts of the same GEMM ("DeepInside DeepGEMM", section
 * 2: besides NT, the NN, TN and TT layouts of the FP8 GEMM), for operands
 * already in FP8 and stored MN-major.  The first letter is A's layout, the
 * second B's, read as D = op(A) . op(B):
 *   fp8_gemm_nn  a E4M3 [M, K] (K contiguous),  b E4M3 [K, N] (N contiguous)
 *   fp8_gemm_tn  a E4M3 [K, M] (M contiguous),  b E4M3 [K, N]
 *   fp8_gemm_tt  a E4M3 [K, M],                 b E4M3 [N, K] (K contiguous)
 * so D[m,n] = C[m,n] + sum_kb (sum_{k in kb} A[m,k] B[n,k]) sfa[m,kb] sfb[n/128,kb]
 * (sfb[n,kb] with one scale per row of B) with A[m,k] and B[n,k] read from
 * the stored layouts.  sfa, sfb, c and d as for fp8_gemm_nt (sfa is
 * [M, K/128], sfb [ceil(N/128), K/128] or [N, K/128] whatever the operands'
 * layout).  An MN-major operand is row-major in its stored shape,
 * with a 16-byte aligned base and a K-row stride (bytes) that is a multiple
 * of 16, at least its row count, and small enough that K x stride < 2^31 - 256
 * (the operand is addressed with 32-bit offsets); its row count (M or N) must
 * be a multiple of 16
 * (else DG_UNSUPPORTED).  Either scale form of B (one per 128x128 block or
 * one per row), FP32 or packed UE8M0; BF16 or F32 d.  The fragments of an
 * MN-major operand are read from LDS with transposing loads; results equal
 * fp8_gemm_nt's on the same values bit for bit.
 */
int fp8_gemm_nn(const dg_tensor* a, const dg_tensor* b, const dg_tensor* sfa, const dg_tensor* sfb,
                const dg_tensor* c, const dg_tensor* d, hipStream_t stream);
int fp8_gemm_tn(const dg_tensor* a, const dg_tensor* b, const dg_tensor* sfa, const dg_tensor* sfb,
                const dg_tensor* c, const dg_tensor* d, hipStream_t stream);
int fp8_gemm_tt(const dg_tensor* a, const dg_tensor* b, const dg_tensor* sfa, const dg_tensor* sfb,
                const dg_tensor* c, const dg_tensor* d, hipStream_t stream);

/*
 * fp8_gemm_nt with its output cast to FP8 in the same kernel ("DeepInside
 * DeepGEMM", section 5: FP8 casting done by separate helpers costs HBM
 * bandwidth, and belongs in the kernel that produces the tensor): D is
 * formed and rounded to BF16 as by fp8_gemm_nt (C added first), then cast
 * per token exactly as per_token_cast_to_fp8 casts that BF16 tensor, so q
 * and sfq are bit-identical to fp8_gemm_nt followed by per_token_cast_to_fp8
 * with the same use_ue8m0.  The BF16 D is never written to memory.
 *   a, b, sfa, sfb, c  as fp8_gemm_nt (sfb one scale per 128x128 block of B
 *       or one per row of B)
 *   q   E4M3 [M, N], any row stride that is a multiple of 4 (innermost
 *       stride 1), 4-B aligned base; must not overlap any input
 *   sfq F32 [M, ceil(N/128)], any strides, 4-B aligned: the scale of each
 *       1x128 block of D (amax/448 floored as for per_token_cast_to_fp8;
 *       with use_ue8m0 rounded up to a power of two)
 * K must be a multiple of 128; M and N are arbitrary.
 */
int fp8_gemm_nt_fp8_out(const dg_tensor* a, const dg_tensor* b, const dg_tensor* sfa,
                        const dg_tensor* sfb, const dg_tensor* c, const dg_tensor* q,
                        const dg_tensor* sfq, int use_ue8m0, hipStream_t stream);

/*
 * Contiguous grouped FP8 GEMM: groups concatenated along M ("DeepGEMM tested
 * by Novita AI", section on the contiguous layout for prefill / training).
 *   a   E4M3 [Msum, K], Msum % 128 == 0
 *   b   E4M3 [G, N, K]
 *   sfa as fp8_gemm_nt with M = Msum;  sfb [G, ceil(N/128), ...] or, one
 *       per row of B, [G, N, ...]
 *   d   BF16 [Msum, N], or F32 [Msum, N] (4-B aligned): the FP32
 *       accumulator stored without rounding
 *   grouped_layout I32 [Msum/128] on the device: group id of each 128-row
 *       block; a negative id marks a block to skip (its rows of d are not
 *       written).  Ids >= G are treated as skipped as well.
 */
int m_grouped_fp8_gemm_nt_contiguous(const dg_tensor* a, const dg_tensor* b,
                                     const dg_tensor* sfa, const dg_tensor* sfb,
                                     const dg_tensor* d, const dg_tensor* grouped_layout,
                                     hipStream_t stream);

/*
 * Masked grouped FP8 GEMM for MoE decode ("DeepGEMM CUDA Graph Compatibility
 * for Masked Grouped GEMMs", section "Tensor-Based Metadata Arguments").
 *   a   E4M3 [G, max_m, K] (or [G*max_m, K])
 *   b   E4M3 [G, N, K]
 *   sfa F32 [G, max_m, K/128] (or [G*max_m, K/128]) or packed I32
 *   sfb F32 [G, ceil(N/128), K/128] or packed I32 (or one per row of B:
 *       [G, N, ...])
 *   d   BF16 [G, max_m, N] (or [G*max_m, N]), or F32 of that shape (4-B
 *       aligned): the FP32 accumulator stored without rounding
 *   masked_m I32 [G] on the device: group g computes its first
 *       clamp(masked_m[g], 0, max_m) rows; every other row of d is left
 *       untouched.  Read only by the kernels, never by the host.
 *   max_m_per_group  rows per group of the padded buffers (fixes the grid).
 */
int m_grouped_fp8_gemm_nt_masked(const dg_tensor* a, const dg_tensor* b,
                                 const dg_tensor* sfa, const dg_tensor* sfb,
                                 const dg_tensor* d, const dg_tensor* masked_m,
                                 int64_t max_m_per_group, hipStream_t stream);

/*
 * The two grouped FP8 GEMMs in the accumulate form D = C + A . B^T of
 * fp8_gemm_nt ("DeepInside DeepGEMM", section 4), the other arguments as
 * above.  c is BF16 or F32 with d's shape ([Msum, N]; [G, max_m, N] or
 * [G*max_m, N]), innermost stride 1, element-aligned; each element of C is
 * added to the FP32 accumulator before d is rounded (BF16) or stored (F32).
 * c may be d itself (same base, dtype and strides: an in-place D += A . B^T);
 * any other overlap with d is rejected.  Rows that are not computed (skipped
 * blocks, rows past masked_m) are neither read from c nor written to d.
 */
int m_grouped_fp8_gemm_nt_contiguous_acc(const dg_tensor* a, const dg_tensor* b,
                                         const dg_tensor* sfa, const dg_tensor* sfb,
                                         const dg_tensor* c, const dg_tensor* d,
                                         const dg_tensor* grouped_layout, hipStream_t stream);
int m_grouped_fp8_gemm_nt_masked_acc(const dg_tensor* a, const dg_tensor* b,
                                     const dg_tensor* sfa, const dg_tensor* sfb,
                                     const dg_tensor* c, const dg_tensor* d,
                                     const dg_tensor* masked_m, int64_t max_m_per_group,
                                     hipStream_t stream);

/*
 * Masked grouped BF16 GEMM, argument order of the pages' capture example
 * (a, b, d, masked_m, max_m_per_group): D[g,m,:] = A[g,m,:] . B[g]^T for
 * m < clamp(masked_m[g], 0, max_m), FP32 accumulation, BF16 out.
 *   a BF16 [G, max_m, K] or [G*max_m, K]; b BF16 [G, N, K]; d like a with N,
 *   BF16, or F32 (4-B aligned: the FP32 accumulator stored without rounding).
 *   Rows past masked_m are not written.  K must be a multiple of 64.
 */
int m_grouped_bf16_gemm_nt_masked(const dg_tensor* a, const dg_tensor* b,
                                  const dg_tensor* d, const dg_tensor* masked_m,
                                  int64_t max_m_per_group, hipStream_t stream);

/*
 * Dense BF16 GEMM D = C + A . B^T: the BF16 GEMM primitive ("DeepGEMM: Why
 * DeepSeek Built Its Own BLAS Kernels", its table of primitives) in the NT
 * layout and accumulate form of fp8_gemm_nt, FP32 accumulation, BF16 out.
 *   a BF16 [M, K], b BF16 [N, K] (row strides multiples of 8 elements,
 *   16-B aligned bases); c NULL or BF16/F32 [M, N] as for fp8_gemm_nt (may be
 *   d itself); d BF16 [M, N] or F32 [M, N] (4-B aligned, the FP32 accumulator
 *   stored as is), any row stride.  K must be a multiple of 64.
 */
int bf16_gemm_nt(const dg_tensor* a, const dg_tensor* b, const dg_tensor* c, const dg_tensor* d,
                 hipStream_t stream);

/*
 * Contiguous grouped BF16 GEMM: the layout of m_grouped_fp8_gemm_nt_contiguous
 * without scales.
 *   a BF16 [Msum, K] (Msum % 128 == 0), b BF16 [G, N, K], d BF16 [Msum, N]
 *   or F32 [Msum, N] (4-B aligned: the FP32 accumulator stored without rounding)
 *   grouped_layout I32 [Msum/128]: group id per 128-row block; negative ids
 *   (and ids >= G) skip the block, its rows of d are not written.
 *   K must be a multiple of 64.
 */
int m_grouped_bf16_gemm_nt_contiguous(const dg_tensor* a, const dg_tensor* b, const dg_tensor* d,
                                      const dg_tensor* grouped_layout, hipStream_t stream);

/*
 * The two grouped BF16 GEMMs in the accumulate form D = C + A . B^T of
 * bf16_gemm_nt (the accumulate form of fp8_gemm_nt, "DeepInside DeepGEMM",
 * section 4), the other arguments as above.  c is BF16 or F32 with d's
 * shape ([Msum, N]; [G, max_m, N] or [G*max_m, N]), innermost stride 1,
 * element-aligned; each element of C is added to the FP32 accumulator before
 * d is rounded (BF16) or stored (F32).  c may be d itself (same base, dtype
 * and strides: an in-place D += A . B^T); any other overlap with d is
 * rejected.  Rows that are not computed (skipped blocks, rows past masked_m)
 * are neither read from c nor written to d.
 */
int m_grouped_bf16_gemm_nt_contiguous_acc(const dg_tensor* a, const dg_tensor* b, const dg_tensor* c,
                                          const dg_tensor* d, const dg_tensor* grouped_layout, hipStream_t stream);
int m_grouped_bf16_gemm_nt_masked_acc(const dg_tensor* a, const dg_tensor* b, const dg_tensor* c,
                                      const dg_tensor* d, const dg_tensor* masked_m, int64_t max_m_per_group,
                                      hipStream_t stream);

/*
 * Per-token FP8 cast: each row of x cut into 1x128 blocks along K; block
 * scale s = amax/448 (amax floored at 1e-4; with use_ue8m0 rounded up to a
 * power of two), q = e4m3(x/s) rounded to nearest even after clamping to
 * +-448 ("DeepInside DeepGEMM", section 5: the FP8 casting helpers).
 *   x  F32 or BF16 [R, K] or [G, R, K]: K-major (innermost stride 1, 16-B
 *      aligned rows), or MN-major (stride 1 along R: the transpose of a
 *      row-major [K, R] tensor, e.g. an activation kept [K, M] for the TN
 *      GEMM), read through a transposing LDS tile ("DeepInside DeepGEMM",
 *      section 5: transposition and casting fused into the producer)
 *   q  E4M3 same shape, K-major: the operand layout of the NT GEMMs
 *   sf F32 [R, ceil(K/128)] (or [G, R, ...]) with any strides
 * The bytes do not depend on the layout of x.
 */
int per_token_cast_to_fp8(const dg_tensor* x, const dg_tensor* q, const dg_tensor* sf,
                          int use_ue8m0, hipStream_t stream);

/*
 * Per-block FP8 cast over 128x128 blocks (weights): as per_token_cast_to_fp8
 * with one scale per block.
 *   x  F32 or BF16 [N, K] or [G, N, K], K-major or MN-major as for
 *      per_token_cast_to_fp8 (a weight kept [K, N] for the NN / TT GEMMs);
 *      q E4M3 same shape, K-major
 *   sf F32 [ceil(N/128), ceil(K/128)] or [G, ...] with any strides
 */
int per_block_cast_to_fp8(const dg_tensor* x, const dg_tensor* q, const dg_tensor* sf,
                          int use_ue8m0, hipStream_t stream);

/*
 * Pack FP32 power-of-two scales into UE8M0 bytes, four per int32 ("[GH-ISSUE
 * #414] pack_ue8m0_to_int is not CUDA Graph capture safe", section "Expected
 * behavior"): byte j of out[..., i] = bits 30..23 of x[..., 4i+j]; missing
 * tail elements give zero bytes.  Shape and dtype checks stay on the host;
 * the value check of the issue's Summary (x >= 0 with a zero mantissa) is
 * done on the device without any host synchronisation: when invalid_count
 * is not NULL, the number of offending elements is ADDED to the int32 it
 * points to (device memory; the caller zeroes it).
 *   x   F32 [..., n] (1 to 3 dims, innermost stride 1)
 *   out I32 [..., ceil(n/4)] same leading shape
 */
int pack_ue8m0_to_int(const dg_tensor* x, const dg_tensor* out, int32_t* invalid_count,
                      hipStream_t stream);

/*
 * MoE dispatch into the masked layout, with the per-token FP8 cast of the
 * routed tokens ("DeepGEMM tested by Novita AI", decode section: each expert
 * owns a padded buffer of max_m rows of which masked_m[e] are valid;
 * "DeepGEMM CUDA Graph Compatibility for Masked Grouped GEMMs", last
 * section: the fused MoE path chains the input casting and the masked GEMM
 * calls; "DeepInside DeepGEMM", section 5: the cast done where the tensor
 * is produced).  Two kernels on `stream`, no allocation, no host sync.
 *   x        F32 or BF16 [T, K] tokens (16-B aligned base and row stride)
 *   topk_idx I32 [T, k] contiguous: the expert of each (token, choice); ids
 *            outside [0, G) route nowhere
 *   a        E4M3 [G, max_m, K] out (4-B aligned rows): row r of expert e is
 *            its r-th routed token, cast as per_token_cast_to_fp8 casts it;
 *            rows >= masked_m[e] are left untouched
 *   sfa      F32 [G, max_m, ceil(K/128)] out, any strides: its scales
 *   masked_m I32 [G] out: min(tokens routed to e, max_m)
 *   slot     I32 [T, k] out, contiguous: e * max_m + r where (t, j) landed,
 *            -1 if routed nowhere or dropped
 *   src      I32 [G, max_m] out, contiguous: the token of each row (rows <
 *            masked_m[e] only)
 * Pairs routed to an expert take its rows in row-major (t, j) order; those
 * beyond max_m rows are dropped (slot -1).  The outputs feed
 * m_grouped_fp8_gemm_nt_masked (a, sfa, masked_m, max_m) and moe_combine
 * (slot).  G * max_m and T * k must fit in int32 (else DG_UNSUPPORTED).
 */
int moe_dispatch_masked_fp8(const dg_tensor* x, const dg_tensor* topk_idx, const dg_tensor* a,
                            const dg_tensor* sfa, const dg_tensor* masked_m, const dg_tensor* slot,
                            const dg_tensor* src, int use_ue8m0, hipStream_t stream);

/*
 * MoE dispatch into the contiguous layout of m_grouped_fp8_gemm_nt_contiguous
 * (prefill: "DeepGEMM tested by Novita AI", contiguous layout, groups
 * concatenated along M in 128-row blocks with a group id per block), with
 * the per-token FP8 cast of the routed tokens as in moe_dispatch_masked_fp8.
 * Three kernels on `stream` (count, place, cast), no allocation, no host sync.
 *   x, topk_idx     as moe_dispatch_masked_fp8
 *   a               E4M3 [Mcap, K] out (Mcap % 128 == 0, 4-B aligned rows):
 *                   expert e's routed tokens fill a region of
 *                   ceil(count_e / align) * align rows, regions in expert
 *                   order, tokens in row-major (t, j) order; the rows of a
 *                   region past count_e are padding and left untouched
 *   sfa             F32 [Mcap, ceil(K/128)] out, any strides: their scales
 *   grouped_layout  I32 [Mcap/128] out: e for the blocks of e's region, -1
 *                   for the blocks past the last region
 *   counts          I32 [G] out: pairs routed to each expert
 *   slot            I32 [T, k] out, contiguous: the row of a where (t, j)
 *                   landed, -1 if routed nowhere or past the capacity Mcap
 *   align           128 (whole blocks), or 256 (whole 256-row tiles of the
 *                   contiguous GEMM: no region then ends in a one-block
 *                   tile, at the cost of more padding rows)
 * Mcap >= T * k + (align - 1) * G holds every routing.  The outputs feed
 * m_grouped_fp8_gemm_nt_contiguous (a, sfa, grouped_layout) and moe_combine
 * (slot, with the GEMM's [Mcap, N] output viewed as [1, Mcap, N]).
 */
int moe_dispatch_contiguous_fp8(const dg_tensor* x, const dg_tensor* topk_idx, const dg_tensor* a,
                                const dg_tensor* sfa, const dg_tensor* grouped_layout,
                                const dg_tensor* counts, const dg_tensor* slot, int32_t align,
                                int use_ue8m0, hipStream_t stream);

/*
 * MoE combine: y[t] = sum over j of topk_weights[t, j] * d[slot[t, j]], the
 * rows of the masked GEMM's output picked by moe_dispatch_masked_fp8's slot
 * table; slots outside [0, G * max_m) (not routed, dropped) add nothing.
 * FP32 sum in increasing j, one FMA per term, rounded to BF16.
 *   d            BF16 [G, max_m, N], any row/group strides (innermost 1)
 *   slot         I32 [T, k] contiguous
 *   topk_weights F32 [T, k] contiguous
 *   y            BF16 [T, N] out, any row stride; must not overlap d
 */
int moe_combine(const dg_tensor* d, const dg_tensor* slot, const dg_tensor* topk_weights,
                const dg_tensor* y, hipStream_t stream);

/* Launch configuration chosen for a GEMM (a pure function of the shapes).
 * A GEMM is one launch over all N columns, or two launches in stream order:
 * the first over columns [0, n_split), the second (block_n2 > 0) over
 * [n_split, N) with a narrower tile, when that fills the last round of
 * workgroups over the compute units better (block sizes that are not powers
 * of two: "DeepGEMM tested by Novita AI", section "Technological Innovations
 * of DeepGEMM", item "Support for Arbitrary Matrix Sizes"). */
typedef struct dg_config {
  int32_t block_m, block_n;   /* output tile of one workgroup (first launch) */
  int32_t threads;            /* workgroup size */
  int64_t grid;               /* workgroups of the first launch */
  int32_t lds_bytes;          /* static LDS per workgroup of the first launch */
  int64_t n_split;            /* columns of the first launch (N when there is one launch) */
  int32_t block_n2;           /* tile width of the second launch, 0 if none (block_m, threads as above) */
  int64_t grid2;              /* workgroups of the second launch, 0 if none */
  int32_t lds_bytes2;         /* static LDS per workgroup of the second launch */
} dg_config;

enum {
  DG_KIND_DENSE = 0, DG_KIND_CONTIGUOUS = 1, DG_KIND_MASKED = 2,            /* FP8 GEMMs */
  DG_KIND_BF16_MASKED = 3, DG_KIND_BF16_DENSE = 4, DG_KIND_BF16_CONTIGUOUS = 5, /* BF16 GEMMs */
  DG_KIND_DENSE_ROWB = 6, DG_KIND_CONTIGUOUS_ROWB = 7, DG_KIND_MASKED_ROWB = 8, /* FP8, one B scale per row */
  DG_KIND_DENSE_FP8_OUT = 9,                                                      /* fp8_gemm_nt_fp8_out */
  DG_KIND_DENSE_MN = 10,                        /* fp8_gemm_nn / _tn / _tt (an MN-major operand) */
  DG_KIND_DENSE_FP8_OUT_ROWB = 11               /* fp8_gemm_nt_fp8_out, one B scale per row */
};

/* Fill *out with the configuration `kind` would launch for these sizes
 * (M = rows: M, Msum or max_m; G = groups, 1 for dense). */
int dg_query_config(int32_t kind, int64_t G, int64_t M, int64_t N, int64_t K, dg_config* out);

#ifdef __cplusplus
}
#endif
#endif /* DGMI_H */
