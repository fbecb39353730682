"""ctypes binding of libdgmi (include/dgmi.h).

Argument marshalling only: every function below builds dg_tensor
descriptors from torch tensors (device memory owned by the caller), passes
the current HIP stream, and calls the C entry point of the same name.  All
computation happens in the library's HIP kernels; there is no fallback.  A
missing or unloadable library raises at once.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdgmi.so")

DG_F32, DG_BF16, DG_E4M3, DG_I32 = 0, 1, 2, 3
DG_OK, DG_INVALID_ARG, DG_UNSUPPORTED, DG_LAUNCH_FAILED = 0, 1, 2, 3
DG_KIND_DENSE, DG_KIND_CONTIGUOUS, DG_KIND_MASKED = 0, 1, 2
DG_KIND_BF16_MASKED, DG_KIND_BF16_DENSE, DG_KIND_BF16_CONTIGUOUS = 3, 4, 5
DG_KIND_DENSE_ROWB, DG_KIND_CONTIGUOUS_ROWB, DG_KIND_MASKED_ROWB = 6, 7, 8  # FP8, one B scale per row of B
DG_KIND_DENSE_FP8_OUT = 9  # fp8_gemm_nt_fp8_out
DG_KIND_DENSE_MN = 10  # fp8_gemm_nn / _tn / _tt
DG_KIND_DENSE_FP8_OUT_ROWB = 11  # fp8_gemm_nt_fp8_out, one B scale per row

ENTRY_POINTS = (
    "dg_last_error",
    "dgmi_init",
    "fp8_gemm_nt",
    "fp8_gemm_nt_fp8_out",
    "fp8_gemm_nn",
    "fp8_gemm_tn",
    "fp8_gemm_tt",
    "m_grouped_fp8_gemm_nt_contiguous",
    "m_grouped_fp8_gemm_nt_masked",
    "m_grouped_fp8_gemm_nt_contiguous_acc",
    "m_grouped_fp8_gemm_nt_masked_acc",
    "m_grouped_bf16_gemm_nt_masked",
    "bf16_gemm_nt",
    "m_grouped_bf16_gemm_nt_contiguous",
    "m_grouped_bf16_gemm_nt_contiguous_acc",
    "m_grouped_bf16_gemm_nt_masked_acc",
    "per_token_cast_to_fp8",
    "per_block_cast_to_fp8",
    "pack_ue8m0_to_int",
    "moe_dispatch_masked_fp8",
    "moe_dispatch_contiguous_fp8",
    "moe_combine",
    "dg_query_config",
)


class DgTensor(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("ndim", ctypes.c_int32),
        ("shape", ctypes.c_int64 * 4),
        ("stride", ctypes.c_int64 * 4),
    ]


class DgConfig(ctypes.Structure):
    _fields_ = [
        ("block_m", ctypes.c_int32),
        ("block_n", ctypes.c_int32),
        ("threads", ctypes.c_int32),
        ("grid", ctypes.c_int64),
        ("lds_bytes", ctypes.c_int32),
        ("n_split", ctypes.c_int64),
        ("block_n2", ctypes.c_int32),
        ("grid2", ctypes.c_int64),
        ("lds_bytes2", ctypes.c_int32),
    ]


class DgmiError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"[dgmi status {code}] {message}")
        self.code = code


_LIB = None


def load_library(path=None):
    """Open libdgmi.so (built in-tree by moe_grouped_gemm_x128_amd.build)."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libdgmi.so not found at {p}: build it with `python -m moe_grouped_gemm_x128_amd.build`")
    lib = ctypes.CDLL(p)
    T = ctypes.POINTER(DgTensor)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    sig = {
        "dg_last_error": ([], ctypes.c_char_p),
        "dgmi_init": ([], ctypes.c_int),
        "fp8_gemm_nt": ([T, T, T, T, T, T, vp], ctypes.c_int),
        "fp8_gemm_nt_fp8_out": ([T, T, T, T, T, T, T, ctypes.c_int, vp], ctypes.c_int),
        "fp8_gemm_nn": ([T, T, T, T, T, T, vp], ctypes.c_int),
        "fp8_gemm_tn": ([T, T, T, T, T, T, vp], ctypes.c_int),
        "fp8_gemm_tt": ([T, T, T, T, T, T, vp], ctypes.c_int),
        "m_grouped_fp8_gemm_nt_contiguous": ([T, T, T, T, T, T, vp], ctypes.c_int),
        "m_grouped_fp8_gemm_nt_masked": ([T, T, T, T, T, T, i64, vp], ctypes.c_int),
        "m_grouped_fp8_gemm_nt_contiguous_acc": ([T, T, T, T, T, T, T, vp], ctypes.c_int),
        "m_grouped_fp8_gemm_nt_masked_acc": ([T, T, T, T, T, T, T, i64, vp], ctypes.c_int),
        "m_grouped_bf16_gemm_nt_contiguous_acc": ([T, T, T, T, T, vp], ctypes.c_int),
        "m_grouped_bf16_gemm_nt_masked_acc": ([T, T, T, T, T, i64, vp], ctypes.c_int),
        "m_grouped_bf16_gemm_nt_masked": ([T, T, T, T, i64, vp], ctypes.c_int),
        "bf16_gemm_nt": ([T, T, T, T, vp], ctypes.c_int),
        "m_grouped_bf16_gemm_nt_contiguous": ([T, T, T, T, vp], ctypes.c_int),
        "per_token_cast_to_fp8": ([T, T, T, ctypes.c_int, vp], ctypes.c_int),
        "per_block_cast_to_fp8": ([T, T, T, ctypes.c_int, vp], ctypes.c_int),
        "pack_ue8m0_to_int": ([T, T, vp, vp], ctypes.c_int),
        "moe_dispatch_masked_fp8": ([T, T, T, T, T, T, T, ctypes.c_int, vp], ctypes.c_int),
        "moe_dispatch_contiguous_fp8": ([T, T, T, T, T, T, T, i32, ctypes.c_int, vp], ctypes.c_int),
        "moe_combine": ([T, T, T, T, vp], ctypes.c_int),
        "dg_query_config": ([i32, i64, i64, i64, i64, ctypes.POINTER(DgConfig)], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    if path is None:
        _LIB = lib
    return lib


def _dtype_code(t):
    import torch

    m = {
        torch.float32: DG_F32,
        torch.bfloat16: DG_BF16,
        torch.uint8: DG_E4M3,
        torch.int32: DG_I32,
    }
    f8 = getattr(torch, "float8_e4m3fn", None)
    if f8 is not None:
        m[f8] = DG_E4M3
    if t.dtype not in m:
        raise TypeError(f"unsupported tensor dtype {t.dtype}")
    return m[t.dtype]


def describe(t, dtype=None):
    """dg_tensor for a torch tensor (None -> NULL descriptor)."""
    if t is None:
        return None
    if t.dim() < 1 or t.dim() > 4:
        raise ValueError("dg_tensor supports 1 to 4 dims")
    d = DgTensor()
    d.data = t.data_ptr() or None
    d.dtype = _dtype_code(t) if dtype is None else dtype
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _ref(d):
    return ctypes.byref(d) if d is not None else None


def _stream(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(rc):
    if rc != DG_OK:
        raise DgmiError(rc, load_library().dg_last_error().decode())


def last_error():
    return load_library().dg_last_error().decode()


def dgmi_init():
    _check(load_library().dgmi_init())


def fp8_gemm_nt(a, b, sfa, sfb, c, d, stream=None):
    """d = c + a . b^T with block scales; c is None or a BF16/F32 [M, N] tensor (may be d)."""
    lib = load_library()
    _check(lib.fp8_gemm_nt(_ref(describe(a)), _ref(describe(b)), _ref(describe(sfa)), _ref(describe(sfb)),
                           _ref(describe(c)), _ref(describe(d)), _stream(stream)))
    return d


def _fp8_gemm_layout(name, a, b, sfa, sfb, c, d, stream):
    lib = load_library()
    _check(getattr(lib, name)(_ref(describe(a)), _ref(describe(b)), _ref(describe(sfa)), _ref(describe(sfb)),
                              _ref(describe(c)), _ref(describe(d)), _stream(stream)))
    return d


def fp8_gemm_nn(a, b, sfa, sfb, c, d, stream=None):
    """d = c + a . b with a [M, K] (K contiguous) and b [K, N] (N contiguous), FP8."""
    return _fp8_gemm_layout("fp8_gemm_nn", a, b, sfa, sfb, c, d, stream)


def fp8_gemm_tn(a, b, sfa, sfb, c, d, stream=None):
    """d = c + a^T . b with a [K, M] (M contiguous) and b [K, N], FP8."""
    return _fp8_gemm_layout("fp8_gemm_tn", a, b, sfa, sfb, c, d, stream)


def fp8_gemm_tt(a, b, sfa, sfb, c, d, stream=None):
    """d = c + a^T . b^T with a [K, M] (M contiguous) and b [N, K] (K contiguous), FP8."""
    return _fp8_gemm_layout("fp8_gemm_tt", a, b, sfa, sfb, c, d, stream)


def fp8_gemm_nt_fp8_out(a, b, sfa, sfb, c, q, sfq, use_ue8m0=False, stream=None):
    """(q, sfq) = per-token FP8 cast of the BF16 D = c + a . b^T, in one kernel."""
    lib = load_library()
    _check(lib.fp8_gemm_nt_fp8_out(_ref(describe(a)), _ref(describe(b)), _ref(describe(sfa)), _ref(describe(sfb)),
                                   _ref(describe(c)), _ref(describe(q)), _ref(describe(sfq)), int(bool(use_ue8m0)),
                                   _stream(stream)))
    return q, sfq


def m_grouped_fp8_gemm_nt_contiguous(a, b, sfa, sfb, d, grouped_layout, stream=None, c=None):
    """Contiguous grouped GEMM; with c (BF16/F32, d's shape, may be d) the
    accumulate form d = c + a . b^T (m_grouped_fp8_gemm_nt_contiguous_acc)."""
    lib = load_library()
    if c is not None:
        _check(lib.m_grouped_fp8_gemm_nt_contiguous_acc(_ref(describe(a)), _ref(describe(b)), _ref(describe(sfa)),
                                                        _ref(describe(sfb)), _ref(describe(c)), _ref(describe(d)),
                                                        _ref(describe(grouped_layout)), _stream(stream)))
        return d
    _check(lib.m_grouped_fp8_gemm_nt_contiguous(_ref(describe(a)), _ref(describe(b)), _ref(describe(sfa)),
                                                _ref(describe(sfb)), _ref(describe(d)),
                                                _ref(describe(grouped_layout)), _stream(stream)))
    return d


def m_grouped_fp8_gemm_nt_masked(a, b, sfa, sfb, d, masked_m, max_m_per_group, stream=None, c=None):
    """Masked grouped GEMM; with c (BF16/F32, d's shape, may be d) the
    accumulate form d = c + a . b^T (m_grouped_fp8_gemm_nt_masked_acc)."""
    lib = load_library()
    if c is not None:
        _check(lib.m_grouped_fp8_gemm_nt_masked_acc(_ref(describe(a)), _ref(describe(b)), _ref(describe(sfa)),
                                                    _ref(describe(sfb)), _ref(describe(c)), _ref(describe(d)),
                                                    _ref(describe(masked_m)), int(max_m_per_group), _stream(stream)))
        return d
    _check(lib.m_grouped_fp8_gemm_nt_masked(_ref(describe(a)), _ref(describe(b)), _ref(describe(sfa)),
                                            _ref(describe(sfb)), _ref(describe(d)), _ref(describe(masked_m)),
                                            int(max_m_per_group), _stream(stream)))
    return d


def m_grouped_bf16_gemm_nt_masked(a, b, d, masked_m, max_m_per_group, stream=None, c=None):
    """Masked grouped BF16 GEMM; with c (BF16/F32, d's shape, may be d) the
    accumulate form d = c + a . b^T (m_grouped_bf16_gemm_nt_masked_acc)."""
    lib = load_library()
    if c is not None:
        _check(lib.m_grouped_bf16_gemm_nt_masked_acc(_ref(describe(a)), _ref(describe(b)), _ref(describe(c)),
                                                     _ref(describe(d)), _ref(describe(masked_m)), int(max_m_per_group),
                                                     _stream(stream)))
        return d
    _check(lib.m_grouped_bf16_gemm_nt_masked(_ref(describe(a)), _ref(describe(b)), _ref(describe(d)),
                                             _ref(describe(masked_m)), int(max_m_per_group), _stream(stream)))
    return d


def bf16_gemm_nt(a, b, c, d, stream=None):
    """d = c + a . b^T in BF16 (FP32 accumulation); c is None or a BF16/F32 [M, N] tensor (may be d)."""
    lib = load_library()
    _check(lib.bf16_gemm_nt(_ref(describe(a)), _ref(describe(b)), _ref(describe(c)), _ref(describe(d)),
                            _stream(stream)))
    return d


def m_grouped_bf16_gemm_nt_contiguous(a, b, d, grouped_layout, stream=None, c=None):
    """Contiguous grouped BF16 GEMM; with c (BF16/F32, d's shape, may be d)
    the accumulate form d = c + a . b^T (m_grouped_bf16_gemm_nt_contiguous_acc)."""
    lib = load_library()
    if c is not None:
        _check(lib.m_grouped_bf16_gemm_nt_contiguous_acc(_ref(describe(a)), _ref(describe(b)), _ref(describe(c)),
                                                         _ref(describe(d)), _ref(describe(grouped_layout)),
                                                         _stream(stream)))
        return d
    _check(lib.m_grouped_bf16_gemm_nt_contiguous(_ref(describe(a)), _ref(describe(b)), _ref(describe(d)),
                                                 _ref(describe(grouped_layout)), _stream(stream)))
    return d


def per_token_cast_to_fp8(x, q, sf, use_ue8m0=False, stream=None):
    lib = load_library()
    _check(lib.per_token_cast_to_fp8(_ref(describe(x)), _ref(describe(q)), _ref(describe(sf)),
                                     int(bool(use_ue8m0)), _stream(stream)))
    return q, sf


def per_block_cast_to_fp8(x, q, sf, use_ue8m0=False, stream=None):
    lib = load_library()
    _check(lib.per_block_cast_to_fp8(_ref(describe(x)), _ref(describe(q)), _ref(describe(sf)),
                                     int(bool(use_ue8m0)), _stream(stream)))
    return q, sf


def pack_ue8m0_to_int(x, out, invalid_count=None, stream=None):
    """Pack FP32 power-of-two scales into int32 words of four UE8M0 bytes.
    invalid_count: optional int32 device tensor (1 element) that receives the
    number of non-UE8M0 inputs, added on the device."""
    lib = load_library()
    cnt = ctypes.c_void_p(invalid_count.data_ptr()) if invalid_count is not None else None
    _check(lib.pack_ue8m0_to_int(_ref(describe(x)), _ref(describe(out)), cnt, _stream(stream)))
    return out


def moe_dispatch_masked_fp8(x, topk_idx, a, sfa, masked_m, slot, src, use_ue8m0=False, stream=None):
    """Route (token, choice) pairs into the expert buffers a / sfa (masked
    layout) with the per-token FP8 cast; fills masked_m, slot and src."""
    lib = load_library()
    _check(lib.moe_dispatch_masked_fp8(_ref(describe(x)), _ref(describe(topk_idx)), _ref(describe(a)),
                                       _ref(describe(sfa)), _ref(describe(masked_m)), _ref(describe(slot)),
                                       _ref(describe(src)), int(bool(use_ue8m0)), _stream(stream)))
    return a, sfa, masked_m, slot, src


def moe_dispatch_contiguous_fp8(x, topk_idx, a, sfa, grouped_layout, counts, slot, align=128, use_ue8m0=False,
                                stream=None):
    """Route (token, choice) pairs into the contiguous layout (a region of
    whole `align`-row granules per expert, align 128 or 256) with the
    per-token FP8 cast; fills grouped_layout, counts and slot."""
    lib = load_library()
    _check(lib.moe_dispatch_contiguous_fp8(_ref(describe(x)), _ref(describe(topk_idx)), _ref(describe(a)),
                                           _ref(describe(sfa)), _ref(describe(grouped_layout)), _ref(describe(counts)),
                                           _ref(describe(slot)), int(align), int(bool(use_ue8m0)), _stream(stream)))
    return a, sfa, grouped_layout, counts, slot


def moe_combine(d, slot, topk_weights, y, stream=None):
    """y[t] = sum_j topk_weights[t, j] * d[slot[t, j]] (BF16 out)."""
    lib = load_library()
    _check(lib.moe_combine(_ref(describe(d)), _ref(describe(slot)), _ref(describe(topk_weights)), _ref(describe(y)),
                           _stream(stream)))
    return y


def query_config(kind, G, M, N, K):
    cfg = DgConfig()
    _check(load_library().dg_query_config(int(kind), int(G), int(M), int(N), int(K), ctypes.byref(cfg)))
    return dict(block_m=cfg.block_m, block_n=cfg.block_n, threads=cfg.threads, grid=cfg.grid, lds_bytes=cfg.lds_bytes,
                n_split=cfg.n_split, block_n2=cfg.block_n2, grid2=cfg.grid2, lds_bytes2=cfg.lds_bytes2)
