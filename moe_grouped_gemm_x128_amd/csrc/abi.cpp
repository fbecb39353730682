// Host side of libdgmi: the extern "C" entry points declared in dgmi.h.
//
// Every entry point validates its descriptors on the host (dtype, rank,
// shape consistency, unit innermost stride, alignment, aliasing of the
// output), then enqueues the kernels on the caller's stream and returns.
// Nothing here allocates, synchronises or reads device memory, so each call
// can be captured into a hipGraph ("DeepGEMM CUDA Graph Compatibility for
// Masked Grouped GEMMs", sections "Eliminating Host-Side Allocation" and
// "Tensor-Based Metadata Arguments"; "[GH-ISSUE #414] pack_ue8m0_to_int is
// not CUDA Graph capture safe", section "Expected behavior": shape and dtype
// checks stay on the host, value checks never synchronise).

#include <stdarg.h>
#include <stdio.h>

#include <string>

#include "dgmi.h"
#include "launch.hpp"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return DG_OK;
}

int elem_size(int32_t dtype) {
  switch (dtype) {
    case DG_F32: return 4;
    case DG_BF16: return 2;
    case DG_E4M3: return 1;
    case DG_I32: return 4;
    default: return 0;
  }
}

const char* dtype_name(int32_t dtype) {
  switch (dtype) {
    case DG_F32: return "F32";
    case DG_BF16: return "BF16";
    case DG_E4M3: return "E4M3";
    case DG_I32: return "I32";
    default: return "?";
  }
}

// Basic well-formedness: non-null, known dtype, 1..4 dims, non-negative
// shape, non-negative strides, innermost stride 1 when `unit_inner` (for a
// tensor with elements).
int check_basic(const dg_tensor* t, const char* name, bool unit_inner) {
  if (t == nullptr) return fail(DG_INVALID_ARG, "%s: descriptor is NULL", name);
  if (elem_size(t->dtype) == 0) return fail(DG_INVALID_ARG, "%s: unknown dtype %d", name, t->dtype);
  if (t->ndim < 1 || t->ndim > 4) return fail(DG_INVALID_ARG, "%s: ndim %d not in 1..4", name, t->ndim);
  int64_t numel = 1;
  for (int i = 0; i < t->ndim; ++i) {
    if (t->shape[i] < 0) return fail(DG_INVALID_ARG, "%s: negative extent in dim %d", name, i);
    if (t->stride[i] < 0) return fail(DG_INVALID_ARG, "%s: negative stride in dim %d", name, i);
    if (t->shape[i] > INT32_MAX) return fail(DG_INVALID_ARG, "%s: extent of dim %d exceeds 2^31-1", name, i);
    numel *= t->shape[i];
  }
  if (numel > 0 && t->data == nullptr) return fail(DG_INVALID_ARG, "%s: data pointer is NULL", name);
  if (unit_inner && numel > 0 && t->shape[t->ndim - 1] > 1 && t->stride[t->ndim - 1] != 1)
    return fail(DG_INVALID_ARG, "%s: innermost stride must be 1 (got %lld)", name, (long long)t->stride[t->ndim - 1]);
  return DG_OK;
}

int check_dtype(const dg_tensor* t, const char* name, int32_t want) {
  if (t->dtype != want)
    return fail(DG_INVALID_ARG, "%s: dtype %s, expected %s", name, dtype_name(t->dtype), dtype_name(want));
  return DG_OK;
}

// Byte span [lo, hi) touched by a strided tensor (empty => lo == hi).
void span(const dg_tensor* t, uintptr_t* lo, uintptr_t* hi) {
  int64_t last = 0;
  for (int i = 0; i < t->ndim; ++i) {
    if (t->shape[i] == 0) {
      *lo = *hi = reinterpret_cast<uintptr_t>(t->data);
      return;
    }
    last += (t->shape[i] - 1) * t->stride[i];
  }
  *lo = reinterpret_cast<uintptr_t>(t->data);
  *hi = *lo + (uintptr_t)((last + 1) * elem_size(t->dtype));
}

int check_no_alias(const dg_tensor* out, const char* oname, const dg_tensor* in, const char* iname) {
  if (in == nullptr) return DG_OK;
  uintptr_t a0, a1, b0, b1;
  span(out, &a0, &a1);
  span(in, &b0, &b1);
  if (a0 < a1 && b0 < b1 && a0 < b1 && b0 < a1)
    return fail(DG_INVALID_ARG, "%s overlaps %s in memory", oname, iname);
  return DG_OK;
}

bool aligned(const void* p, int bytes) { return (reinterpret_cast<uintptr_t>(p) % bytes) == 0; }

#define DG_TRY(expr)             \
  do {                           \
    int rc_ = (expr);            \
    if (rc_ != DG_OK) return rc_; \
  } while (0)

// A matrix-like operand viewed as [G, R, C]: either 3-D, or 2-D with R = G*rows
// split by `rows_per_group` (rows_per_group <= 0: 2-D means a single group).
struct View3 {
  int64_t G, R, C;
  int64_t sg, sr;
};

int view3(const dg_tensor* t, const char* name, int64_t G_expect, int64_t rows_per_group, View3* v) {
  if (t->ndim == 3) {
    v->G = t->shape[0];
    v->R = t->shape[1];
    v->C = t->shape[2];
    v->sg = t->stride[0];
    v->sr = t->stride[1];
  } else if (t->ndim == 2) {
    if (rows_per_group > 0) {
      if (t->shape[0] != G_expect * rows_per_group)
        return fail(DG_INVALID_ARG, "%s: 2-D leading extent %lld != groups*rows %lld", name,
                    (long long)t->shape[0], (long long)(G_expect * rows_per_group));
      v->G = G_expect;
      v->R = rows_per_group;
      v->sg = rows_per_group * t->stride[0];
    } else {
      v->G = 1;
      v->R = t->shape[0];
      v->sg = 0;
    }
    v->C = t->shape[1];
    v->sr = t->stride[0];
  } else {
    return fail(DG_INVALID_ARG, "%s: expected 2 or 3 dims, got %d", name, t->ndim);
  }
  if (G_expect >= 0 && v->G != G_expect)
    return fail(DG_INVALID_ARG, "%s: %lld groups, expected %lld", name, (long long)v->G, (long long)G_expect);
  return DG_OK;
}

// Scale-factor operand of the FP8 GEMMs: F32 [.., rows, nkb] or packed I32
// [.., rows, ceil(nkb/4)]; any strides.
int check_scales(const dg_tensor* t, const char* name, int sf_fmt, int64_t G_expect, int64_t rows_per_group,
                 int64_t rows, int64_t nkb, View3* v) {
  DG_TRY(check_basic(t, name, false));
  DG_TRY(check_dtype(t, name, sf_fmt == dgmi::SF_F32 ? DG_F32 : DG_I32));
  DG_TRY(view3(t, name, G_expect, rows_per_group, v));
  const int64_t cols = sf_fmt == dgmi::SF_F32 ? nkb : (nkb + 3) / 4;
  if (v->R != rows || v->C != cols)
    return fail(DG_INVALID_ARG, "%s: shape [..,%lld,%lld], expected [..,%lld,%lld]", name, (long long)v->R,
                (long long)v->C, (long long)rows, (long long)cols);
  return DG_OK;
}

// The kernels address a tile of up to 256 rows of A or B with 32-bit buffer
// offsets (row * row stride + K offset): row strides (bytes) must stay below
// 2^31 / 256, i.e. 8 MiB.
int check_row_strides(int64_t lda_bytes, int64_t ldb_bytes, const char* fname) {
  constexpr int64_t kMax = INT32_MAX / 256;
  if (lda_bytes > kMax || ldb_bytes > kMax)
    return fail(DG_UNSUPPORTED, "%s: row strides of a and b must be below %lld bytes (got %lld, %lld)", fname,
                (long long)kMax, (long long)lda_bytes, (long long)ldb_bytes);
  return DG_OK;
}

int check_launch(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DG_LAUNCH_FAILED, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

// Common FP8 GEMM validation.  mode: dense / contig / masked.  With q != NULL
// (dense only) the output is D cast per token to FP8: q E4M3 [M, N] and sfq
// F32 [M, ceil(N/128)] take the place of d (NULL).
int fp8_gemm_common(int mode, const dg_tensor* a, const dg_tensor* b, const dg_tensor* sfa, const dg_tensor* sfb,
                    const dg_tensor* c, const dg_tensor* d, const dg_tensor* meta, int64_t max_m, hipStream_t stream,
                    const char* fname, const dg_tensor* q = nullptr, const dg_tensor* sfq = nullptr,
                    int q_ue8m0 = 0) {
  const bool fp8_out = q != nullptr;
  if (fp8_out) d = q;  // the output operand, for the shape and alias checks
  const char* dname = fp8_out ? "q" : "d";
  // An MN-major operand (dense only) is the transposed view of a row-major
  // [K, M] or [K, N] tensor: a 2-D descriptor with unit stride along its rows
  // and its K-row stride in stride[1].
  auto mn_major = [](const dg_tensor* t) {
    return t != nullptr && t->ndim == 2 && t->shape[1] > 1 && t->stride[1] != 1 &&
           (t->shape[0] <= 1 || t->stride[0] == 1);
  };
  const bool a_mn = mode == dgmi::MODE_DENSE && mn_major(a), b_mn = mode == dgmi::MODE_DENSE && mn_major(b);
  DG_TRY(check_basic(a, "a", !a_mn));
  DG_TRY(check_basic(b, "b", !b_mn));
  DG_TRY(check_basic(d, dname, true));
  DG_TRY(check_dtype(a, "a", DG_E4M3));
  DG_TRY(check_dtype(b, "b", DG_E4M3));
  // d: BF16, or F32 for the dense GEMM (the FP32 accumulator stored as is)
  const bool d_f32 = !fp8_out && d->dtype == DG_F32;
  DG_TRY(check_dtype(d, dname, fp8_out ? DG_E4M3 : (d_f32 ? DG_F32 : DG_BF16)));
  if (sfa == nullptr || sfb == nullptr) return fail(DG_INVALID_ARG, "%s: scale descriptors must not be NULL", fname);
  if (sfa->dtype != sfb->dtype) return fail(DG_INVALID_ARG, "%s: sfa and sfb must have the same dtype", fname);
  const int sf_fmt = sfa->dtype == DG_I32 ? dgmi::SF_UE8M0 : dgmi::SF_F32;

  View3 va, vb, vd, vsa, vsb;
  int64_t G = 1, rows_pg = 0;
  if (mode == dgmi::MODE_DENSE) {
    if (a->ndim != 2 || b->ndim != 2 || d->ndim != 2)
      return fail(DG_INVALID_ARG, "%s: a, b, %s must be 2-D", fname, dname);
    DG_TRY(view3(b, "b", 1, 0, &vb));
  } else {
    if (b->ndim != 3) return fail(DG_INVALID_ARG, "%s: b must be [G, N, K]", fname);
    G = b->shape[0];
    DG_TRY(view3(b, "b", G, 0, &vb));
  }
  if (mode == dgmi::MODE_MASKED) {
    if (max_m < 0) return fail(DG_INVALID_ARG, "%s: max_m_per_group must be >= 0", fname);
    rows_pg = max_m;
    DG_TRY(view3(a, "a", G, rows_pg, &va));
    DG_TRY(view3(d, "d", G, rows_pg, &vd));
  } else {
    if (a->ndim != 2 || d->ndim != 2) return fail(DG_INVALID_ARG, "%s: a and %s must be 2-D", fname, dname);
    DG_TRY(view3(a, "a", 1, 0, &va));
    DG_TRY(view3(d, dname, 1, 0, &vd));
  }
  const int64_t M = va.R, K = va.C, N = vb.R;
  if (vb.C != K) return fail(DG_INVALID_ARG, "%s: K mismatch: a has %lld, b has %lld", fname, (long long)K, (long long)vb.C);
  if (vd.R != M || vd.C != N)
    return fail(DG_INVALID_ARG, "%s: %s is [..,%lld,%lld], expected [..,%lld,%lld]", fname, dname, (long long)vd.R,
                (long long)vd.C, (long long)M, (long long)N);
  if (mode == dgmi::MODE_MASKED && M != max_m)
    return fail(DG_INVALID_ARG, "%s: a has %lld rows per group, max_m_per_group is %lld", fname, (long long)M,
                (long long)max_m);
  if (K % 128 != 0) return fail(DG_UNSUPPORTED, "%s: K = %lld is not a multiple of 128", fname, (long long)K);
  const int64_t nkb = K / 128, nnb = (N + 127) / 128;
  DG_TRY(check_scales(sfa, "sfa", sf_fmt, mode == dgmi::MODE_MASKED ? G : 1, rows_pg, M, nkb, &vsa));
  // sfb: one scale per 128x128 block of B, or one per row of B (N rows; for
  // N = 1 the two forms are the same)
  const bool rowb = sfb->ndim >= 2 && sfb->shape[sfb->ndim - 2] == N && N != nnb;
  DG_TRY(check_scales(sfb, "sfb", sf_fmt, mode == dgmi::MODE_DENSE ? 1 : G, 0, rowb ? N : nnb, nkb, &vsb));
  if (mode == dgmi::MODE_DENSE && (sfb->ndim != 2 || sfa->ndim != 2))
    return fail(DG_INVALID_ARG, "%s: sfa and sfb must be 2-D", fname);
  if (mode == dgmi::MODE_CONTIG && sfb->ndim != 3) return fail(DG_INVALID_ARG, "%s: sfb must be [G, ceil(N/128), ..]", fname);

  // MN-major operands: K-rows of M (N) bytes, 16-byte aligned, ld bytes apart
  const int64_t lda = a_mn ? a->stride[1] : va.sr, ldb = b_mn ? b->stride[1] : vb.sr;
  if (a_mn || b_mn) {
    if (fp8_out) return fail(DG_UNSUPPORTED, "%s: MN-major operands take a BF16 or F32 d", fname);
    if ((a_mn && M % 16) || (b_mn && N % 16))
      return fail(DG_UNSUPPORTED, "%s: an MN-major operand needs its row count (M or N) to be a multiple of 16",
                  fname);
    if ((a_mn && lda < M) || (b_mn && ldb < N))
      return fail(DG_UNSUPPORTED, "%s: the K-row stride of an MN-major operand must be at least its row count", fname);
    // the kernels address an MN-major operand with 32-bit offsets from its first K-row
    const int64_t lim = (int64_t(1) << 31) - 256;
    if ((a_mn && K * lda > lim) || (b_mn && K * ldb > lim))
      return fail(DG_UNSUPPORTED, "%s: an MN-major operand must span less than 2^31 bytes (K x K-row stride)", fname);
  }
  // alignment: 16-B operand rows (the kernels load 16-B chunks), 16-B output rows
  if (!aligned(a->data, 16) || !aligned(b->data, 16) || lda % 16 || ldb % 16 || va.sg % 16 || vb.sg % 16)
    return fail(DG_INVALID_ARG, "%s: a and b need 16-byte aligned bases and row/group strides", fname);
  DG_TRY(check_row_strides(a_mn ? 0 : lda, b_mn ? 0 : ldb, fname));
  if (fp8_out) {
    // q rows are written in 4-byte words (16-byte stores when 16-byte aligned)
    if (!aligned(d->data, 4) || (M > 1 && N > 0 && vd.sr % 4))
      return fail(DG_INVALID_ARG, "%s: q needs a 4-byte aligned base and row stride", fname);
    DG_TRY(check_basic(sfq, "sfq", false));
    DG_TRY(check_dtype(sfq, "sfq", DG_F32));
    if (sfq->ndim != 2 || sfq->shape[0] != M || sfq->shape[1] != nnb)
      return fail(DG_INVALID_ARG, "%s: sfq must be F32 [M, ceil(N/128)] = [%lld, %lld]", fname, (long long)M,
                  (long long)nnb);
    if (!aligned(sfq->data, 4)) return fail(DG_INVALID_ARG, "%s: sfq must be 4-byte aligned", fname);
  } else if (!aligned(d->data, d_f32 ? 4 : 2)) {
    return fail(DG_INVALID_ARG, "%s: d must be element-aligned", fname);
  }
  if (!aligned(sfa->data, 4) || !aligned(sfb->data, 4)) return fail(DG_INVALID_ARG, "%s: scales must be 4-byte aligned", fname);

  if (mode == dgmi::MODE_CONTIG) {
    if (M % 128 != 0) return fail(DG_INVALID_ARG, "%s: Msum = %lld is not a multiple of 128", fname, (long long)M);
    DG_TRY(check_basic(meta, "grouped_layout", true));
    DG_TRY(check_dtype(meta, "grouped_layout", DG_I32));
    if (meta->ndim != 1 || meta->shape[0] != M / 128)
      return fail(DG_INVALID_ARG, "%s: grouped_layout must be I32 [Msum/128 = %lld]", fname, (long long)(M / 128));
  } else if (mode == dgmi::MODE_MASKED) {
    DG_TRY(check_basic(meta, "masked_m", true));
    DG_TRY(check_dtype(meta, "masked_m", DG_I32));
    if (meta->ndim != 1 || meta->shape[0] != G)
      return fail(DG_INVALID_ARG, "%s: masked_m must be I32 [G = %lld]", fname, (long long)G);
  }
  DG_TRY(check_no_alias(d, dname, a, "a"));
  DG_TRY(check_no_alias(d, dname, b, "b"));
  DG_TRY(check_no_alias(d, dname, sfa, "sfa"));
  DG_TRY(check_no_alias(d, dname, sfb, "sfb"));
  if (meta != nullptr) DG_TRY(check_no_alias(d, dname, meta, "metadata"));
  if (fp8_out) {
    DG_TRY(check_no_alias(sfq, "sfq", a, "a"));
    DG_TRY(check_no_alias(sfq, "sfq", b, "b"));
    DG_TRY(check_no_alias(sfq, "sfq", sfa, "sfa"));
    DG_TRY(check_no_alias(sfq, "sfq", sfb, "sfb"));
    DG_TRY(check_no_alias(sfq, "sfq", q, "q"));
    DG_TRY(check_no_alias(sfq, "sfq", c, "c"));
  }
  // accumulate input: D = C + A . B^T, C BF16 or F32 with d's shape ([M, N],
  // [Msum, N], or [G, max_m, N] / [G * max_m, N]); c may be d itself (same
  // base and strides), any other overlap is rejected
  bool c_f32 = false;
  int64_t ldc = 0, c_gs = 0;
  if (c != nullptr) {
    DG_TRY(check_basic(c, "c", true));
    if (c->dtype != DG_BF16 && c->dtype != DG_F32) return fail(DG_INVALID_ARG, "%s: c must be BF16 or F32", fname);
    View3 vc;
    if (mode == dgmi::MODE_MASKED) {
      DG_TRY(view3(c, "c", G, rows_pg, &vc));
    } else {
      if (c->ndim != 2) return fail(DG_INVALID_ARG, "%s: c must be 2-D", fname);
      DG_TRY(view3(c, "c", 1, 0, &vc));
    }
    if ((mode == dgmi::MODE_MASKED && vc.G != G) || vc.R != M || vc.C != N)
      return fail(DG_INVALID_ARG, "%s: c must have the shape of %s ([..,%lld,%lld])", fname, dname, (long long)M,
                  (long long)N);
    c_f32 = c->dtype == DG_F32;
    if (!aligned(c->data, c_f32 ? 4 : 2)) return fail(DG_INVALID_ARG, "%s: c must be element-aligned", fname);
    ldc = vc.sr;
    c_gs = vc.sg;
    // (with FP8 output, c and q differ in dtype and must not overlap)
    const bool same_as_d = c->data == d->data && c->dtype == d->dtype && ldc == vd.sr && (G <= 1 || c_gs == vd.sg);
    if (!same_as_d) DG_TRY(check_no_alias(d, dname, c, "c"));
  }

  dgmi::GemmParams p = {};
  p.a = static_cast<const uint8_t*>(a->data);
  p.b = static_cast<const uint8_t*>(b->data);
  p.sfa = sfa->data;
  p.sfb = sfb->data;
  p.d = fp8_out ? nullptr : static_cast<uint16_t*>(d->data);
  p.d_f32 = d_f32 ? 1 : 0;
  if (fp8_out) {
    p.q = static_cast<uint8_t*>(q->data);
    p.ldq = vd.sr;
    p.sfq = static_cast<float*>(sfq->data);
    p.sfq_sm = sfq->stride[0];
    p.sfq_sn = sfq->stride[1];
    p.q_ue8m0 = q_ue8m0 ? 1 : 0;
  }
  p.c = c != nullptr ? c->data : nullptr;
  p.ldc = ldc;
  p.c_gs = c_gs;
  p.c_f32 = c_f32 ? 1 : 0;
  p.meta = meta ? static_cast<const int32_t*>(meta->data) : nullptr;
  p.lda = lda;
  p.a_gs = va.sg;
  p.ldb = ldb;
  p.b_gs = vb.sg;
  p.a_mn = a_mn ? 1 : 0;
  p.b_mn = b_mn ? 1 : 0;
  p.sfa_sm = vsa.sr;
  p.sfa_sk = sfa->stride[sfa->ndim - 1];
  p.sfa_gs = vsa.sg;
  p.sfb_sn = vsb.sr;
  p.sfb_sk = sfb->stride[sfb->ndim - 1];
  p.sfb_gs = vsb.sg;
  p.ldd = vd.sr;
  p.d_gs = d_f32 ? 2 * vd.sg : vd.sg;  // (the kernels step d in BF16-sized units)
  p.M = (int32_t)M;
  p.N = (int32_t)N;
  p.k_bytes = (int32_t)K;
  p.G = (int32_t)G;
  if (M == 0 || N == 0 || G == 0) return ok();
  if (K == 0) return fail(DG_UNSUPPORTED, "%s: K = 0 is not supported", fname);
  if (fp8_out)
    return check_launch(dgmi::launch_fp8_gemm_fp8_out(p, sf_fmt | (rowb ? dgmi::SF_ROWB : 0), stream), fname);
  return check_launch(dgmi::launch_fp8_gemm(p, mode, sf_fmt | (rowb ? dgmi::SF_ROWB : 0), stream), fname);
}

// Quantizer validation: x [R, K] or [G, R, K]; q same shape; sf [.., R', KB].
// x is K-major (innermost stride 1) or MN-major (stride 1 along the rows:
// the transpose of a row-major [K, R] tensor), q is K-major.
int quant_common(const dg_tensor* x, const dg_tensor* q, const dg_tensor* sf, int use_ue8m0, hipStream_t stream,
                 bool per_block, const char* fname) {
  const bool mn_major = x != nullptr && x->ndim >= 2 && x->shape[x->ndim - 1] > 1 && x->stride[x->ndim - 1] != 1 &&
                        (x->shape[x->ndim - 2] <= 1 || x->stride[x->ndim - 2] == 1);
  DG_TRY(check_basic(x, "x", !mn_major));
  DG_TRY(check_basic(q, "q", true));
  DG_TRY(check_basic(sf, "sf", false));
  if (x->dtype != DG_F32 && x->dtype != DG_BF16) return fail(DG_INVALID_ARG, "%s: x must be F32 or BF16", fname);
  DG_TRY(check_dtype(q, "q", DG_E4M3));
  DG_TRY(check_dtype(sf, "sf", DG_F32));
  if (x->ndim != q->ndim || x->ndim != sf->ndim || (x->ndim != 2 && x->ndim != 3))
    return fail(DG_INVALID_ARG, "%s: x, q and sf must all be 2-D or all 3-D", fname);
  for (int i = 0; i < x->ndim; ++i)
    if (x->shape[i] != q->shape[i]) return fail(DG_INVALID_ARG, "%s: q must have the shape of x", fname);
  View3 vx, vq, vs;
  DG_TRY(view3(x, "x", -1, 0, &vx));
  DG_TRY(view3(q, "q", vx.G, 0, &vq));
  DG_TRY(view3(sf, "sf", vx.G, 0, &vs));
  const int64_t R = vx.R, K = vx.C;
  const int64_t srows = per_block ? (R + 127) / 128 : R;
  if (vs.R != srows || vs.C != (K + 127) / 128)
    return fail(DG_INVALID_ARG, "%s: sf is [..,%lld,%lld], expected [..,%lld,%lld]", fname, (long long)vs.R,
                (long long)vs.C, (long long)srows, (long long)((K + 127) / 128));
  const int xe = elem_size(x->dtype);
  if (!mn_major && (!aligned(x->data, 16) || (vx.sr * xe) % 16 || (vx.sg * xe) % 16))
    return fail(DG_INVALID_ARG, "%s: x needs a 16-byte aligned base and row/group strides", fname);
  if (mn_major && !aligned(x->data, xe)) return fail(DG_INVALID_ARG, "%s: x must be element-aligned", fname);
  if (!aligned(q->data, 4) || vq.sr % 4 || vq.sg % 4)
    return fail(DG_INVALID_ARG, "%s: q needs a 4-byte aligned base and row/group strides", fname);
  if (!aligned(sf->data, 4)) return fail(DG_INVALID_ARG, "%s: sf must be 4-byte aligned", fname);
  DG_TRY(check_no_alias(q, "q", x, "x"));
  DG_TRY(check_no_alias(sf, "sf", x, "x"));
  DG_TRY(check_no_alias(sf, "sf", q, "q"));
  dgmi::QuantArgs p = {};
  p.x = x->data;
  p.x_bf16 = x->dtype == DG_BF16;
  p.sx_g = vx.sg;
  p.sx_r = vx.sr;
  p.q = static_cast<uint8_t*>(q->data);
  p.sq_g = vq.sg;
  p.sq_r = vq.sr;
  p.sf = static_cast<float*>(sf->data);
  p.ssf_g = vs.sg;
  p.ssf_r = vs.sr;
  p.ssf_k = sf->stride[sf->ndim - 1];
  p.G = (int32_t)vx.G;
  p.R = (int32_t)R;
  p.K = (int32_t)K;
  p.ue8m0 = use_ue8m0 ? 1 : 0;
  if (vx.G == 0 || R == 0 || K == 0) return ok();
  if (mn_major) {
    // read through a transposing LDS tile
    dgmi::QuantTArgs t = {};
    static_cast<dgmi::QuantArgs&>(t) = p;
    t.sx_k = x->stride[x->ndim - 1];
    const int64_t lb = x->dtype == DG_F32 ? 16 : 8;  // bytes of four elements
    t.vec = (aligned(x->data, (int)lb) && (t.sx_k * xe) % lb == 0 && (vx.sg * xe) % lb == 0) ? 1 : 0;
    t.qvec = (aligned(q->data, 16) && (R <= 1 || vq.sr % 16 == 0) && (vx.G <= 1 || vq.sg % 16 == 0)) ? 1 : 0;
    return check_launch(dgmi::launch_cast_mn(t, per_block, stream), fname);
  }
  return check_launch(per_block ? dgmi::launch_per_block(p, stream) : dgmi::launch_per_token(p, stream), fname);
}

// The BF16 GEMMs (dense with optional C, contiguous, masked): the same
// kernel body as the FP8 GEMM with BF16 operands and no scales.
int bf16_gemm_common(int mode, const dg_tensor* a, const dg_tensor* b, const dg_tensor* c, const dg_tensor* d,
                     const dg_tensor* meta, int64_t max_m, hipStream_t stream, const char* fname) {
  DG_TRY(check_basic(a, "a", true));
  DG_TRY(check_basic(b, "b", true));
  DG_TRY(check_basic(d, "d", true));
  DG_TRY(check_dtype(a, "a", DG_BF16));
  DG_TRY(check_dtype(b, "b", DG_BF16));
  // d: BF16, or F32 (the FP32 accumulator stored as is)
  const bool d_f32 = d->dtype == DG_F32;
  DG_TRY(check_dtype(d, "d", d_f32 ? DG_F32 : DG_BF16));
  View3 va, vb, vd;
  int64_t G = 1;
  if (mode == dgmi::MODE_DENSE) {
    if (a->ndim != 2 || b->ndim != 2 || d->ndim != 2) return fail(DG_INVALID_ARG, "%s: a, b, d must be 2-D", fname);
    DG_TRY(view3(b, "b", 1, 0, &vb));
  } else {
    if (b->ndim != 3) return fail(DG_INVALID_ARG, "%s: b must be [G, N, K]", fname);
    G = b->shape[0];
    DG_TRY(view3(b, "b", G, 0, &vb));
  }
  if (mode == dgmi::MODE_MASKED) {
    if (max_m < 0) return fail(DG_INVALID_ARG, "%s: max_m_per_group must be >= 0", fname);
    DG_TRY(view3(a, "a", G, max_m, &va));
    DG_TRY(view3(d, "d", G, max_m, &vd));
  } else {
    if (a->ndim != 2 || d->ndim != 2) return fail(DG_INVALID_ARG, "%s: a and d must be 2-D", fname);
    DG_TRY(view3(a, "a", 1, 0, &va));
    DG_TRY(view3(d, "d", 1, 0, &vd));
  }
  const int64_t M = va.R, K = va.C, N = vb.R;
  if (mode == dgmi::MODE_MASKED && M != max_m)
    return fail(DG_INVALID_ARG, "%s: a has %lld rows per group, max_m_per_group is %lld", fname, (long long)M, (long long)max_m);
  if (vb.C != K) return fail(DG_INVALID_ARG, "%s: K mismatch", fname);
  if (vd.R != M || vd.C != N) return fail(DG_INVALID_ARG, "%s: d must be [.., %lld, %lld]", fname, (long long)M, (long long)N);
  if (K % 64 != 0) return fail(DG_UNSUPPORTED, "%s: K = %lld is not a multiple of 64", fname, (long long)K);
  if (!aligned(a->data, 16) || !aligned(b->data, 16) || va.sr % 8 || vb.sr % 8 || va.sg % 8 || vb.sg % 8)
    return fail(DG_INVALID_ARG, "%s: a and b need 16-byte aligned bases and row/group strides", fname);
  DG_TRY(check_row_strides(2 * va.sr, 2 * vb.sr, fname));
  if (!aligned(d->data, d_f32 ? 4 : 2)) return fail(DG_INVALID_ARG, "%s: d must be element-aligned", fname);
  if (mode == dgmi::MODE_CONTIG) {
    if (M % 128 != 0) return fail(DG_INVALID_ARG, "%s: Msum = %lld is not a multiple of 128", fname, (long long)M);
    DG_TRY(check_basic(meta, "grouped_layout", true));
    DG_TRY(check_dtype(meta, "grouped_layout", DG_I32));
    if (meta->ndim != 1 || meta->shape[0] != M / 128)
      return fail(DG_INVALID_ARG, "%s: grouped_layout must be I32 [Msum/128 = %lld]", fname, (long long)(M / 128));
  } else if (mode == dgmi::MODE_MASKED) {
    DG_TRY(check_basic(meta, "masked_m", true));
    DG_TRY(check_dtype(meta, "masked_m", DG_I32));
    if (meta->ndim != 1 || meta->shape[0] != G) return fail(DG_INVALID_ARG, "%s: masked_m must be I32 [G]", fname);
  }
  DG_TRY(check_no_alias(d, "d", a, "a"));
  DG_TRY(check_no_alias(d, "d", b, "b"));
  if (meta != nullptr) DG_TRY(check_no_alias(d, "d", meta, "metadata"));
  bool c_f32 = false;
  int64_t ldc = 0, c_gs = 0;
  if (c != nullptr) {
    // C shaped like d: [M, N] (dense), [Msum, N] (contiguous), [G, max_m, N]
    // or [G*max_m, N] (masked, its own group stride)
    DG_TRY(check_basic(c, "c", true));
    if (c->dtype != DG_BF16 && c->dtype != DG_F32) return fail(DG_INVALID_ARG, "%s: c must be BF16 or F32", fname);
    View3 vc;
    if (mode == dgmi::MODE_MASKED) {
      DG_TRY(view3(c, "c", G, max_m, &vc));
    } else {
      if (c->ndim != 2) return fail(DG_INVALID_ARG, "%s: c must be 2-D", fname);
      DG_TRY(view3(c, "c", 1, 0, &vc));
    }
    if ((mode == dgmi::MODE_MASKED && vc.G != G) || vc.R != M || vc.C != N)
      return fail(DG_INVALID_ARG, "%s: c must have the shape of d ([..,%lld,%lld])", fname, (long long)M,
                  (long long)N);
    c_f32 = c->dtype == DG_F32;
    if (!aligned(c->data, c_f32 ? 4 : 2)) return fail(DG_INVALID_ARG, "%s: c must be element-aligned", fname);
    ldc = vc.sr;
    c_gs = vc.sg;
    const bool same_as_d = c->data == d->data && c->dtype == d->dtype && ldc == vd.sr && (G <= 1 || c_gs == vd.sg);
    if (!same_as_d) DG_TRY(check_no_alias(d, "d", c, "c"));
  }
  // the kernel addresses A and B in bytes
  dgmi::GemmParams p = {};
  p.a = static_cast<const uint8_t*>(a->data);
  p.b = static_cast<const uint8_t*>(b->data);
  p.d = static_cast<uint16_t*>(d->data);
  p.d_f32 = d_f32 ? 1 : 0;
  p.c = c != nullptr ? c->data : nullptr;
  p.ldc = ldc;
  p.c_gs = c_gs;
  p.c_f32 = c_f32 ? 1 : 0;
  p.meta = meta ? static_cast<const int32_t*>(meta->data) : nullptr;
  p.lda = 2 * va.sr;
  p.a_gs = 2 * va.sg;
  p.ldb = 2 * vb.sr;
  p.b_gs = 2 * vb.sg;
  p.ldd = vd.sr;
  p.d_gs = d_f32 ? 2 * vd.sg : vd.sg;  // (the kernels step d in BF16-sized units)
  p.M = (int32_t)M;
  p.N = (int32_t)N;
  p.k_bytes = (int32_t)(2 * K);
  p.G = (int32_t)G;
  if (G == 0 || M == 0 || N == 0) return ok();
  if (K == 0) return fail(DG_UNSUPPORTED, "%s: K = 0 is not supported", fname);
  return check_launch(dgmi::launch_bf16_gemm(p, mode, stream), fname);
}

}  // namespace

extern "C" {

const char* dg_last_error(void) { return g_err.c_str(); }

int dgmi_init(void) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DG_LAUNCH_FAILED, "dgmi_init: no HIP device: %s", hipGetErrorString(e));
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return fail(DG_LAUNCH_FAILED, "dgmi_init: %s", hipGetErrorString(e));
  if (std::string(prop.gcnArchName).rfind("gfx950", 0) != 0)
    return fail(DG_UNSUPPORTED, "dgmi_init: device %d is %s, this library is built for gfx950", dev, prop.gcnArchName);
  return ok();
}

int fp8_gemm_nt(const dg_tensor* a, const dg_tensor* b, const dg_tensor* sfa, const dg_tensor* sfb,
                const dg_tensor* c, const dg_tensor* d, hipStream_t stream) {
  return fp8_gemm_common(dgmi::MODE_DENSE, a, b, sfa, sfb, c, d, nullptr, 0, stream, "fp8_gemm_nt");
}

// The other three layouts: a descriptor given in its stored shape ([K, M]
// for A, [K, N] for B, row-major) is viewed as its transpose and handed to
// the common path, which takes the view as MN-major.
namespace {
int transposed(const dg_tensor* t, const char* name, const char* fname, dg_tensor* out) {
  if (t == nullptr) return fail(DG_INVALID_ARG, "%s: %s descriptor is NULL", fname, name);
  if (t->ndim != 2) return fail(DG_INVALID_ARG, "%s: %s must be 2-D", fname, name);
  *out = *t;
  out->shape[0] = t->shape[1];
  out->shape[1] = t->shape[0];
  out->stride[0] = t->stride[1];
  out->stride[1] = t->stride[0];
  if (t->shape[1] > 1 && t->stride[1] != 1)
    return fail(DG_INVALID_ARG, "%s: %s must be row-major (innermost stride 1)", fname, name);
  return DG_OK;
}
}  // namespace

int fp8_gemm_nn(const dg_tensor* a, const dg_tensor* b, const dg_tensor* sfa, const dg_tensor* sfb,
                const dg_tensor* c, const dg_tensor* d, hipStream_t stream) {
  dg_tensor bt;
  DG_TRY(transposed(b, "b", "fp8_gemm_nn", &bt));
  return fp8_gemm_common(dgmi::MODE_DENSE, a, &bt, sfa, sfb, c, d, nullptr, 0, stream, "fp8_gemm_nn");
}

int fp8_gemm_tn(const dg_tensor* a, const dg_tensor* b, const dg_tensor* sfa, const dg_tensor* sfb,
                const dg_tensor* c, const dg_tensor* d, hipStream_t stream) {
  dg_tensor at, bt;
  DG_TRY(transposed(a, "a", "fp8_gemm_tn", &at));
  DG_TRY(transposed(b, "b", "fp8_gemm_tn", &bt));
  return fp8_gemm_common(dgmi::MODE_DENSE, &at, &bt, sfa, sfb, c, d, nullptr, 0, stream, "fp8_gemm_tn");
}

int fp8_gemm_tt(const dg_tensor* a, const dg_tensor* b, const dg_tensor* sfa, const dg_tensor* sfb,
                const dg_tensor* c, const dg_tensor* d, hipStream_t stream) {
  dg_tensor at;
  DG_TRY(transposed(a, "a", "fp8_gemm_tt", &at));
  return fp8_gemm_common(dgmi::MODE_DENSE, &at, b, sfa, sfb, c, d, nullptr, 0, stream, "fp8_gemm_tt");
}

int fp8_gemm_nt_fp8_out(const dg_tensor* a, const dg_tensor* b, const dg_tensor* sfa, const dg_tensor* sfb,
                        const dg_tensor* c, const dg_tensor* q, const dg_tensor* sfq, int use_ue8m0,
                        hipStream_t stream) {
  if (q == nullptr || sfq == nullptr) return fail(DG_INVALID_ARG, "fp8_gemm_nt_fp8_out: q and sfq must not be NULL");
  return fp8_gemm_common(dgmi::MODE_DENSE, a, b, sfa, sfb, c, nullptr, nullptr, 0, stream, "fp8_gemm_nt_fp8_out", q,
                         sfq, use_ue8m0);
}

int m_grouped_fp8_gemm_nt_contiguous(const dg_tensor* a, const dg_tensor* b, const dg_tensor* sfa,
                                     const dg_tensor* sfb, const dg_tensor* d, const dg_tensor* grouped_layout,
                                     hipStream_t stream) {
  if (grouped_layout == nullptr) return fail(DG_INVALID_ARG, "m_grouped_fp8_gemm_nt_contiguous: grouped_layout is NULL");
  return fp8_gemm_common(dgmi::MODE_CONTIG, a, b, sfa, sfb, nullptr, d, grouped_layout, 0, stream,
                         "m_grouped_fp8_gemm_nt_contiguous");
}

int m_grouped_fp8_gemm_nt_masked(const dg_tensor* a, const dg_tensor* b, const dg_tensor* sfa, const dg_tensor* sfb,
                                 const dg_tensor* d, const dg_tensor* masked_m, int64_t max_m_per_group,
                                 hipStream_t stream) {
  if (masked_m == nullptr) return fail(DG_INVALID_ARG, "m_grouped_fp8_gemm_nt_masked: masked_m is NULL");
  return fp8_gemm_common(dgmi::MODE_MASKED, a, b, sfa, sfb, nullptr, d, masked_m, max_m_per_group, stream,
                         "m_grouped_fp8_gemm_nt_masked");
}

int m_grouped_fp8_gemm_nt_contiguous_acc(const dg_tensor* a, const dg_tensor* b, const dg_tensor* sfa,
                                         const dg_tensor* sfb, const dg_tensor* c, const dg_tensor* d,
                                         const dg_tensor* grouped_layout, hipStream_t stream) {
  if (grouped_layout == nullptr)
    return fail(DG_INVALID_ARG, "m_grouped_fp8_gemm_nt_contiguous_acc: grouped_layout is NULL");
  return fp8_gemm_common(dgmi::MODE_CONTIG, a, b, sfa, sfb, c, d, grouped_layout, 0, stream,
                         "m_grouped_fp8_gemm_nt_contiguous_acc");
}

int m_grouped_fp8_gemm_nt_masked_acc(const dg_tensor* a, const dg_tensor* b, const dg_tensor* sfa,
                                     const dg_tensor* sfb, const dg_tensor* c, const dg_tensor* d,
                                     const dg_tensor* masked_m, int64_t max_m_per_group, hipStream_t stream) {
  if (masked_m == nullptr) return fail(DG_INVALID_ARG, "m_grouped_fp8_gemm_nt_masked_acc: masked_m is NULL");
  return fp8_gemm_common(dgmi::MODE_MASKED, a, b, sfa, sfb, c, d, masked_m, max_m_per_group, stream,
                         "m_grouped_fp8_gemm_nt_masked_acc");
}

int bf16_gemm_nt(const dg_tensor* a, const dg_tensor* b, const dg_tensor* c, const dg_tensor* d, hipStream_t stream) {
  return bf16_gemm_common(dgmi::MODE_DENSE, a, b, c, d, nullptr, 0, stream, "bf16_gemm_nt");
}

int m_grouped_bf16_gemm_nt_contiguous(const dg_tensor* a, const dg_tensor* b, const dg_tensor* d,
                                      const dg_tensor* grouped_layout, hipStream_t stream) {
  if (grouped_layout == nullptr) return fail(DG_INVALID_ARG, "m_grouped_bf16_gemm_nt_contiguous: grouped_layout is NULL");
  return bf16_gemm_common(dgmi::MODE_CONTIG, a, b, nullptr, d, grouped_layout, 0, stream,
                          "m_grouped_bf16_gemm_nt_contiguous");
}

int m_grouped_bf16_gemm_nt_masked(const dg_tensor* a, const dg_tensor* b, const dg_tensor* d,
                                  const dg_tensor* masked_m, int64_t max_m_per_group, hipStream_t stream) {
  if (masked_m == nullptr) return fail(DG_INVALID_ARG, "m_grouped_bf16_gemm_nt_masked: masked_m is NULL");
  return bf16_gemm_common(dgmi::MODE_MASKED, a, b, nullptr, d, masked_m, max_m_per_group, stream,
                          "m_grouped_bf16_gemm_nt_masked");
}

int m_grouped_bf16_gemm_nt_contiguous_acc(const dg_tensor* a, const dg_tensor* b, const dg_tensor* c,
                                          const dg_tensor* d, const dg_tensor* grouped_layout, hipStream_t stream) {
  if (grouped_layout == nullptr)
    return fail(DG_INVALID_ARG, "m_grouped_bf16_gemm_nt_contiguous_acc: grouped_layout is NULL");
  return bf16_gemm_common(dgmi::MODE_CONTIG, a, b, c, d, grouped_layout, 0, stream,
                          "m_grouped_bf16_gemm_nt_contiguous_acc");
}

int m_grouped_bf16_gemm_nt_masked_acc(const dg_tensor* a, const dg_tensor* b, const dg_tensor* c, const dg_tensor* d,
                                      const dg_tensor* masked_m, int64_t max_m_per_group, hipStream_t stream) {
  if (masked_m == nullptr) return fail(DG_INVALID_ARG, "m_grouped_bf16_gemm_nt_masked_acc: masked_m is NULL");
  return bf16_gemm_common(dgmi::MODE_MASKED, a, b, c, d, masked_m, max_m_per_group, stream,
                          "m_grouped_bf16_gemm_nt_masked_acc");
}

int per_token_cast_to_fp8(const dg_tensor* x, const dg_tensor* q, const dg_tensor* sf, int use_ue8m0,
                          hipStream_t stream) {
  return quant_common(x, q, sf, use_ue8m0, stream, false, "per_token_cast_to_fp8");
}

int per_block_cast_to_fp8(const dg_tensor* x, const dg_tensor* q, const dg_tensor* sf, int use_ue8m0,
                          hipStream_t stream) {
  return quant_common(x, q, sf, use_ue8m0, stream, true, "per_block_cast_to_fp8");
}

int pack_ue8m0_to_int(const dg_tensor* x, const dg_tensor* out, int32_t* invalid_count, hipStream_t stream) {
  const char* fname = "pack_ue8m0_to_int";
  DG_TRY(check_basic(x, "x", true));
  DG_TRY(check_basic(out, "out", true));
  DG_TRY(check_dtype(x, "x", DG_F32));
  DG_TRY(check_dtype(out, "out", DG_I32));
  if (x->ndim != out->ndim || x->ndim > 3) return fail(DG_INVALID_ARG, "%s: x and out must have the same rank (1..3)", fname);
  for (int i = 0; i + 1 < x->ndim; ++i)
    if (x->shape[i] != out->shape[i]) return fail(DG_INVALID_ARG, "%s: leading shapes of x and out differ", fname);
  const int64_t n = x->shape[x->ndim - 1];
  const int64_t nw = (n + 3) / 4;
  if (out->shape[out->ndim - 1] != nw)
    return fail(DG_INVALID_ARG, "%s: out has %lld words per row, expected ceil(%lld/4) = %lld", fname,
                (long long)out->shape[out->ndim - 1], (long long)n, (long long)nw);
  if (!aligned(x->data, 4) || !aligned(out->data, 4)) return fail(DG_INVALID_ARG, "%s: x and out must be 4-byte aligned", fname);
  DG_TRY(check_no_alias(out, "out", x, "x"));
  dgmi::PackArgs p = {};
  p.x = static_cast<const float*>(x->data);
  p.out = static_cast<int32_t*>(out->data);
  p.n = (int32_t)n;
  p.nw = (int32_t)nw;
  p.invalid = invalid_count;
  if (x->ndim == 1) {
    p.G = 1; p.R = 1; p.sx_g = p.sx_r = 0; p.so_g = p.so_r = 0;
  } else if (x->ndim == 2) {
    p.G = 1; p.R = (int32_t)x->shape[0]; p.sx_g = 0; p.sx_r = x->stride[0]; p.so_g = 0; p.so_r = out->stride[0];
  } else {
    p.G = (int32_t)x->shape[0]; p.R = (int32_t)x->shape[1];
    p.sx_g = x->stride[0]; p.sx_r = x->stride[1]; p.so_g = out->stride[0]; p.so_r = out->stride[1];
  }
  if (p.G == 0 || p.R == 0 || nw == 0) return ok();
  return check_launch(dgmi::launch_pack_ue8m0(p, stream), fname);
}

int moe_dispatch_masked_fp8(const dg_tensor* x, const dg_tensor* topk_idx, const dg_tensor* a, const dg_tensor* sfa,
                            const dg_tensor* masked_m, const dg_tensor* slot, const dg_tensor* src, int use_ue8m0,
                            hipStream_t stream) {
  const char* fname = "moe_dispatch_masked_fp8";
  DG_TRY(check_basic(x, "x", true));
  DG_TRY(check_basic(topk_idx, "topk_idx", true));
  DG_TRY(check_basic(a, "a", true));
  DG_TRY(check_basic(sfa, "sfa", false));
  DG_TRY(check_basic(masked_m, "masked_m", true));
  DG_TRY(check_basic(slot, "slot", true));
  DG_TRY(check_basic(src, "src", true));
  if (x->dtype != DG_F32 && x->dtype != DG_BF16) return fail(DG_INVALID_ARG, "%s: x must be F32 or BF16", fname);
  DG_TRY(check_dtype(topk_idx, "topk_idx", DG_I32));
  DG_TRY(check_dtype(a, "a", DG_E4M3));
  DG_TRY(check_dtype(sfa, "sfa", DG_F32));
  DG_TRY(check_dtype(masked_m, "masked_m", DG_I32));
  DG_TRY(check_dtype(slot, "slot", DG_I32));
  DG_TRY(check_dtype(src, "src", DG_I32));
  if (x->ndim != 2 || topk_idx->ndim != 2 || a->ndim != 3 || sfa->ndim != 3 || masked_m->ndim != 1 ||
      slot->ndim != 2 || src->ndim != 2)
    return fail(DG_INVALID_ARG, "%s: x [T, K], topk_idx [T, k], a [G, max_m, K], sfa [G, max_m, K/128], "
                "masked_m [G], slot [T, k], src [G, max_m]", fname);
  const int64_t T = x->shape[0], K = x->shape[1], k = topk_idx->shape[1];
  const int64_t G = a->shape[0], max_m = a->shape[1];
  if (topk_idx->shape[0] != T) return fail(DG_INVALID_ARG, "%s: topk_idx must have T = %lld rows", fname, (long long)T);
  if (a->shape[2] != K) return fail(DG_INVALID_ARG, "%s: a must be [G, max_m, K = %lld]", fname, (long long)K);
  if (sfa->shape[0] != G || sfa->shape[1] != max_m || sfa->shape[2] != (K + 127) / 128)
    return fail(DG_INVALID_ARG, "%s: sfa must be [G, max_m, ceil(K/128)] = [%lld, %lld, %lld]", fname, (long long)G,
                (long long)max_m, (long long)((K + 127) / 128));
  if (masked_m->shape[0] != G) return fail(DG_INVALID_ARG, "%s: masked_m must be [G = %lld]", fname, (long long)G);
  if (slot->shape[0] != T || slot->shape[1] != k)
    return fail(DG_INVALID_ARG, "%s: slot must have the shape of topk_idx", fname);
  if (src->shape[0] != G || src->shape[1] != max_m)
    return fail(DG_INVALID_ARG, "%s: src must be [G, max_m] = [%lld, %lld]", fname, (long long)G, (long long)max_m);
  // the routing tables are read and written as flat arrays
  if ((T > 1 && topk_idx->stride[0] != k) || (T > 1 && slot->stride[0] != k) || (G > 1 && src->stride[0] != max_m))
    return fail(DG_INVALID_ARG, "%s: topk_idx, slot and src must be contiguous", fname);
  if (G * max_m > INT32_MAX || T * k > INT32_MAX)
    return fail(DG_UNSUPPORTED, "%s: G * max_m and T * k must fit in int32", fname);
  const int xe = elem_size(x->dtype);
  if (!aligned(x->data, 16) || (T > 1 && (x->stride[0] * xe) % 16))
    return fail(DG_INVALID_ARG, "%s: x needs a 16-byte aligned base and row stride", fname);
  if (!aligned(a->data, 4) || (max_m > 1 && a->stride[1] % 4) || (G > 1 && a->stride[0] % 4))
    return fail(DG_INVALID_ARG, "%s: a needs a 4-byte aligned base and row/group strides", fname);
  if (!aligned(sfa->data, 4)) return fail(DG_INVALID_ARG, "%s: sfa must be 4-byte aligned", fname);
  const dg_tensor* outs[] = {a, sfa, masked_m, slot, src};
  const char* onames[] = {"a", "sfa", "masked_m", "slot", "src"};
  for (int i = 0; i < 5; ++i) {
    DG_TRY(check_no_alias(outs[i], onames[i], x, "x"));
    DG_TRY(check_no_alias(outs[i], onames[i], topk_idx, "topk_idx"));
    for (int j = i + 1; j < 5; ++j) DG_TRY(check_no_alias(outs[i], onames[i], outs[j], onames[j]));
  }
  if (G == 0) return ok();
  dgmi::MoeRouteArgs r = {};
  r.topk = static_cast<const int32_t*>(topk_idx->data);
  r.T = (int32_t)T;
  r.k = (int32_t)k;
  r.G = (int32_t)G;
  r.max_m = (int32_t)max_m;
  r.vec = aligned(topk_idx->data, 16) ? 1 : 0;
  r.masked_m = static_cast<int32_t*>(masked_m->data);
  r.slot = static_cast<int32_t*>(slot->data);
  r.src = static_cast<int32_t*>(src->data);
  hipError_t e = dgmi::launch_moe_route(r, stream);
  if (e != hipSuccess || max_m == 0 || K == 0 || T == 0 || k == 0) return check_launch(e, fname);
  // the per-token cast of each token, stored into every row its slots name
  dgmi::QuantScatterArgs q = {};
  q.x = x->data;
  q.x_bf16 = x->dtype == DG_BF16;
  q.sx_g = 0;
  q.sx_r = x->stride[0];
  q.q = static_cast<uint8_t*>(a->data);
  q.sq_g = a->stride[0];
  q.sq_r = a->stride[1];
  q.sf = static_cast<float*>(sfa->data);
  q.ssf_g = sfa->stride[0];
  q.ssf_r = sfa->stride[1];
  q.ssf_k = sfa->stride[2];
  q.G = 1;
  q.R = (int32_t)T;
  q.K = (int32_t)K;
  q.ue8m0 = use_ue8m0 ? 1 : 0;
  q.slot = r.slot;
  q.k = (int32_t)k;
  q.max_m = (int32_t)max_m;
  q.rows = (int32_t)(G * max_m);
  q.flat = (q.sq_g == max_m * q.sq_r && q.ssf_g == max_m * q.ssf_r) ? 1 : 0;
  q.qvec = (aligned(a->data, 16) && q.sq_r % 16 == 0 && q.sq_g % 16 == 0) ? 1 : 0;
  return check_launch(dgmi::launch_per_token_scatter(q, stream), fname);
}

int moe_dispatch_contiguous_fp8(const dg_tensor* x, const dg_tensor* topk_idx, const dg_tensor* a,
                                const dg_tensor* sfa, const dg_tensor* grouped_layout, const dg_tensor* counts,
                                const dg_tensor* slot, int32_t align, int use_ue8m0, hipStream_t stream) {
  const char* fname = "moe_dispatch_contiguous_fp8";
  if (align != 128 && align != 256) return fail(DG_INVALID_ARG, "%s: align must be 128 or 256 (got %d)", fname, align);
  DG_TRY(check_basic(x, "x", true));
  DG_TRY(check_basic(topk_idx, "topk_idx", true));
  DG_TRY(check_basic(a, "a", true));
  DG_TRY(check_basic(sfa, "sfa", false));
  DG_TRY(check_basic(grouped_layout, "grouped_layout", true));
  DG_TRY(check_basic(counts, "counts", true));
  DG_TRY(check_basic(slot, "slot", true));
  if (x->dtype != DG_F32 && x->dtype != DG_BF16) return fail(DG_INVALID_ARG, "%s: x must be F32 or BF16", fname);
  DG_TRY(check_dtype(topk_idx, "topk_idx", DG_I32));
  DG_TRY(check_dtype(a, "a", DG_E4M3));
  DG_TRY(check_dtype(sfa, "sfa", DG_F32));
  DG_TRY(check_dtype(grouped_layout, "grouped_layout", DG_I32));
  DG_TRY(check_dtype(counts, "counts", DG_I32));
  DG_TRY(check_dtype(slot, "slot", DG_I32));
  if (x->ndim != 2 || topk_idx->ndim != 2 || a->ndim != 2 || sfa->ndim != 2 || grouped_layout->ndim != 1 ||
      counts->ndim != 1 || slot->ndim != 2)
    return fail(DG_INVALID_ARG, "%s: x [T, K], topk_idx [T, k], a [Mcap, K], sfa [Mcap, K/128], "
                "grouped_layout [Mcap/128], counts [G], slot [T, k]", fname);
  const int64_t T = x->shape[0], K = x->shape[1], k = topk_idx->shape[1];
  const int64_t Mcap = a->shape[0], G = counts->shape[0];
  if (topk_idx->shape[0] != T) return fail(DG_INVALID_ARG, "%s: topk_idx must have T = %lld rows", fname, (long long)T);
  if (a->shape[1] != K) return fail(DG_INVALID_ARG, "%s: a must be [Mcap, K = %lld]", fname, (long long)K);
  if (Mcap % 128 != 0) return fail(DG_INVALID_ARG, "%s: Mcap = %lld is not a multiple of 128", fname, (long long)Mcap);
  if (sfa->shape[0] != Mcap || sfa->shape[1] != (K + 127) / 128)
    return fail(DG_INVALID_ARG, "%s: sfa must be [Mcap, ceil(K/128)] = [%lld, %lld]", fname, (long long)Mcap,
                (long long)((K + 127) / 128));
  if (grouped_layout->shape[0] != Mcap / 128)
    return fail(DG_INVALID_ARG, "%s: grouped_layout must be [Mcap/128 = %lld]", fname, (long long)(Mcap / 128));
  if (slot->shape[0] != T || slot->shape[1] != k)
    return fail(DG_INVALID_ARG, "%s: slot must have the shape of topk_idx", fname);
  if ((T > 1 && topk_idx->stride[0] != k) || (T > 1 && slot->stride[0] != k))
    return fail(DG_INVALID_ARG, "%s: topk_idx and slot must be contiguous", fname);
  if (Mcap > INT32_MAX || T * k > INT32_MAX)
    return fail(DG_UNSUPPORTED, "%s: Mcap and T * k must fit in int32", fname);
  const int xe = elem_size(x->dtype);
  if (!aligned(x->data, 16) || (T > 1 && (x->stride[0] * xe) % 16))
    return fail(DG_INVALID_ARG, "%s: x needs a 16-byte aligned base and row stride", fname);
  if (!aligned(a->data, 4) || (Mcap > 1 && a->stride[0] % 4))
    return fail(DG_INVALID_ARG, "%s: a needs a 4-byte aligned base and row stride", fname);
  if (!aligned(sfa->data, 4)) return fail(DG_INVALID_ARG, "%s: sfa must be 4-byte aligned", fname);
  const dg_tensor* outs[] = {a, sfa, grouped_layout, counts, slot};
  const char* onames[] = {"a", "sfa", "grouped_layout", "counts", "slot"};
  for (int i = 0; i < 5; ++i) {
    DG_TRY(check_no_alias(outs[i], onames[i], x, "x"));
    DG_TRY(check_no_alias(outs[i], onames[i], topk_idx, "topk_idx"));
    for (int j = i + 1; j < 5; ++j) DG_TRY(check_no_alias(outs[i], onames[i], outs[j], onames[j]));
  }
  if (Mcap == 0 && G == 0) return ok();
  dgmi::MoeRouteArgs r = {};
  r.topk = static_cast<const int32_t*>(topk_idx->data);
  r.T = (int32_t)T;
  r.k = (int32_t)k;
  r.G = (int32_t)G;
  r.vec = aligned(topk_idx->data, 16) ? 1 : 0;
  r.slot = static_cast<int32_t*>(slot->data);
  r.counts = static_cast<int32_t*>(counts->data);
  r.layout = static_cast<int32_t*>(grouped_layout->data);
  r.mcap = Mcap;
  r.align = align;
  hipError_t e = dgmi::launch_moe_route_contiguous(r, stream);
  if (e != hipSuccess || Mcap == 0 || K == 0 || T == 0 || k == 0) return check_launch(e, fname);
  // the per-token cast of each token, stored into every row its slots name
  dgmi::QuantScatterArgs q = {};
  q.x = x->data;
  q.x_bf16 = x->dtype == DG_BF16;
  q.sx_g = 0;
  q.sx_r = x->stride[0];
  q.q = static_cast<uint8_t*>(a->data);
  q.sq_g = 0;
  q.sq_r = a->stride[0];
  q.sf = static_cast<float*>(sfa->data);
  q.ssf_g = 0;
  q.ssf_r = sfa->stride[0];
  q.ssf_k = sfa->stride[1];
  q.G = 1;
  q.R = (int32_t)T;
  q.K = (int32_t)K;
  q.ue8m0 = use_ue8m0 ? 1 : 0;
  q.slot = r.slot;
  q.k = (int32_t)k;
  q.max_m = (int32_t)Mcap;
  q.rows = (int32_t)Mcap;
  q.flat = 1;  // a slot is a row of a and sfa
  q.qvec = (aligned(a->data, 16) && q.sq_r % 16 == 0) ? 1 : 0;
  return check_launch(dgmi::launch_per_token_scatter(q, stream), fname);
}

int moe_combine(const dg_tensor* d, const dg_tensor* slot, const dg_tensor* topk_weights, const dg_tensor* y,
                hipStream_t stream) {
  const char* fname = "moe_combine";
  DG_TRY(check_basic(d, "d", true));
  DG_TRY(check_basic(slot, "slot", true));
  DG_TRY(check_basic(topk_weights, "topk_weights", true));
  DG_TRY(check_basic(y, "y", true));
  DG_TRY(check_dtype(d, "d", DG_BF16));
  DG_TRY(check_dtype(slot, "slot", DG_I32));
  DG_TRY(check_dtype(topk_weights, "topk_weights", DG_F32));
  DG_TRY(check_dtype(y, "y", DG_BF16));
  if (d->ndim != 3 || slot->ndim != 2 || topk_weights->ndim != 2 || y->ndim != 2)
    return fail(DG_INVALID_ARG, "%s: d [G, max_m, N], slot [T, k], topk_weights [T, k], y [T, N]", fname);
  const int64_t G = d->shape[0], max_m = d->shape[1], N = d->shape[2], T = slot->shape[0], k = slot->shape[1];
  if (topk_weights->shape[0] != T || topk_weights->shape[1] != k)
    return fail(DG_INVALID_ARG, "%s: topk_weights must have the shape of slot", fname);
  if (y->shape[0] != T || y->shape[1] != N)
    return fail(DG_INVALID_ARG, "%s: y must be [T, N] = [%lld, %lld]", fname, (long long)T, (long long)N);
  if ((T > 1 && slot->stride[0] != k) || (T > 1 && topk_weights->stride[0] != k))
    return fail(DG_INVALID_ARG, "%s: slot and topk_weights must be contiguous", fname);
  if (G * max_m > INT32_MAX) return fail(DG_UNSUPPORTED, "%s: G * max_m must fit in int32", fname);
  if (!aligned(d->data, 2) || !aligned(y->data, 2)) return fail(DG_INVALID_ARG, "%s: d and y must be 2-byte aligned", fname);
  DG_TRY(check_no_alias(y, "y", d, "d"));
  DG_TRY(check_no_alias(y, "y", slot, "slot"));
  DG_TRY(check_no_alias(y, "y", topk_weights, "topk_weights"));
  dgmi::MoeCombineArgs p = {};
  p.d = static_cast<const uint16_t*>(d->data);
  p.sd_g = d->stride[0];
  p.sd_r = d->stride[1];
  p.G = (int32_t)G;
  p.max_m = (int32_t)max_m;
  p.N = (int32_t)N;
  p.slot = static_cast<const int32_t*>(slot->data);
  p.w = static_cast<const float*>(topk_weights->data);
  p.T = (int32_t)T;
  p.k = (int32_t)k;
  p.y = static_cast<uint16_t*>(y->data);
  p.sy = y->stride[0];
  p.vec = (aligned(d->data, 16) && (max_m <= 1 || d->stride[1] % 8 == 0) && (G <= 1 || d->stride[0] % 8 == 0)) ? 1 : 0;
  p.y_vec = (aligned(y->data, 16) && (T <= 1 || y->stride[0] % 8 == 0)) ? 1 : 0;
  if (T == 0 || N == 0) return ok();
  return check_launch(dgmi::launch_moe_combine(p, stream), fname);
}

int dg_query_config(int32_t kind, int64_t G, int64_t M, int64_t N, int64_t K, dg_config* out) {
  if (out == nullptr) return fail(DG_INVALID_ARG, "dg_query_config: out is NULL");
  if (G < 0 || M < 0 || N < 0 || K < 0) return fail(DG_INVALID_ARG, "dg_query_config: negative size");
  dgmi::GemmPlan c;
  int mode;
  if (kind == DG_KIND_BF16_MASKED || kind == DG_KIND_BF16_DENSE || kind == DG_KIND_BF16_CONTIGUOUS) {
    mode = kind == DG_KIND_BF16_DENSE ? dgmi::MODE_DENSE
                                      : (kind == DG_KIND_BF16_CONTIGUOUS ? dgmi::MODE_CONTIG : dgmi::MODE_MASKED);
    c = dgmi::bf16_gemm_plan(mode, G, M, N, K);
  } else if (kind >= DG_KIND_DENSE && kind <= DG_KIND_MASKED) {
    mode = kind == DG_KIND_DENSE ? dgmi::MODE_DENSE : (kind == DG_KIND_CONTIGUOUS ? dgmi::MODE_CONTIG : dgmi::MODE_MASKED);
    c = dgmi::fp8_gemm_plan(mode, G, M, N, K, dgmi::SF_F32);
  } else if (kind == DG_KIND_DENSE_FP8_OUT || kind == DG_KIND_DENSE_FP8_OUT_ROWB) {
    mode = dgmi::MODE_DENSE;
    c = dgmi::fp8_out_gemm_plan(M, N, dgmi::SF_F32 | (kind == DG_KIND_DENSE_FP8_OUT_ROWB ? dgmi::SF_ROWB : 0));
  } else if (kind == DG_KIND_DENSE_MN) {
    mode = dgmi::MODE_DENSE;
    c = dgmi::fp8_mn_gemm_plan();
  } else if (kind >= DG_KIND_DENSE_ROWB && kind <= DG_KIND_MASKED_ROWB) {
    mode = kind == DG_KIND_DENSE_ROWB ? dgmi::MODE_DENSE
                                      : (kind == DG_KIND_CONTIGUOUS_ROWB ? dgmi::MODE_CONTIG : dgmi::MODE_MASKED);
    c = dgmi::fp8_gemm_plan(mode, G, M, N, K, dgmi::SF_F32 | dgmi::SF_ROWB);
  } else {
    return fail(DG_INVALID_ARG, "dg_query_config: unknown kind %d", kind);
  }
  out->block_m = c.cfg[0].bm;
  out->block_n = c.cfg[0].bn;
  out->threads = c.cfg[0].threads;
  out->grid = dgmi::plan_grid(c, 0, mode, G, M, N);
  out->lds_bytes = dgmi::plan_lds(c, 0, mode);
  out->n_split = c.parts == 2 ? c.n_split : N;
  out->block_n2 = c.parts == 2 ? c.cfg[1].bn : 0;
  out->grid2 = dgmi::plan_grid(c, 1, mode, G, M, N);
  out->lds_bytes2 = dgmi::plan_lds(c, 1, mode);
  return ok();
}

}  // extern "C"
