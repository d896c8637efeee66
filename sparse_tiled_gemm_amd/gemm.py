"""Python binding of libstgemm.so (include/gemm.h).  Argument marshalling only:
every step of the computation runs in the library's HIP kernels.  Device
buffers are passed as torch tensors (their data pointers) or raw integer
addresses; PyTorch provides memory and streams only.

The functions carry the C names: gemm_validate_desc, gemm_plan,
gemm_plan_destroy, gemm_plan_describe, gemm_run, gemm_sparse24_sizes,
gemm_sparse24_compress, gemm_sparse24_compress_noalloc, gemm_sparse24_run, gemm_mx_run, gemm_w4a16_run, gemm_status_string,
gemm_last_error.  Non-OK statuses raise GemmError (except
gemm_validate_desc, which returns the status).
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libstgemm.so")

# gemm_status_t
GEMM_OK = 0
GEMM_ERR_NULL_POINTER = 1
GEMM_ERR_INVALID_VALUE = 2
GEMM_ERR_UNSUPPORTED = 3
GEMM_ERR_MISALIGNED = 4
GEMM_ERR_NOT_SPARSE24 = 5
GEMM_ERR_DEVICE = 6
GEMM_ERR_HIP = 7

# gemm_dtype_t
DTYPES = {"f16": 1, "bf16": 2, "e4m3": 3, "e5m2": 4, "s8": 5, "f32": 6, "s32": 7,
          "e2m3": 8, "e3m2": 9, "e2m1": 10, "u4": 11, "u8": 12}
ROW_MAJOR, COL_MAJOR = 0, 1
ACT_NONE, ACT_RELU = 0, 1
# gemm_algo_t
ALGO = {"auto": 0, "tiled": 1, "generic": 2, "skinny": 3, "tiled128": 4, "tiled256": 5}

ELEM_BYTES = {"f16": 2, "bf16": 2, "e4m3": 1, "e5m2": 1, "s8": 1, "u8": 1, "f32": 4, "s32": 4}


class GemmError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s: %s" % (_status_name(status), message))
        self.status = status


class gemm_desc_t(ctypes.Structure):
    _fields_ = [
        ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
        ("a_type", ctypes.c_int32), ("b_type", ctypes.c_int32),
        ("c_type", ctypes.c_int32), ("d_type", ctypes.c_int32),
        ("a_layout", ctypes.c_int32), ("b_layout", ctypes.c_int32),
        ("lda", ctypes.c_int64), ("ldb", ctypes.c_int64),
        ("ldc", ctypes.c_int64), ("ldd", ctypes.c_int64),
        ("alpha", ctypes.c_float),
        ("has_c", ctypes.c_int32), ("has_bias", ctypes.c_int32), ("act", ctypes.c_int32),
        ("sparse_a", ctypes.c_int32), ("algo", ctypes.c_int32),
        ("block_scale", ctypes.c_int32), ("saturate", ctypes.c_int32),
    ]


_lib = None


def load():
    """Load libstgemm.so; raises if it has not been built (no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libstgemm.so is not built (%s); run "
                           "`python -m sparse_tiled_gemm_amd.build`" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    st = ctypes.c_int
    dp = ctypes.POINTER(gemm_desc_t)
    sig = {
        "gemm_validate_desc": (st, [dp]),
        "gemm_plan": (st, [dp, ctypes.POINTER(vp)]),
        "gemm_plan_destroy": (st, [vp]),
        "gemm_plan_describe": (st, [vp, ctypes.c_char_p, ctypes.c_size_t]),
        "gemm_run": (st, [vp, vp, vp, vp, vp, vp, vp]),
        "gemm_mx_run": (st, [vp, vp, vp, vp, vp, vp, vp, vp, vp]),
        "gemm_w4a16_run": (st, [vp, vp, vp, vp, vp, vp, vp, vp, vp]),
        "gemm_sparse24_sizes": (st, [i64, i64, i32, ctypes.POINTER(ctypes.c_size_t),
                                     ctypes.POINTER(ctypes.c_size_t)]),
        "gemm_sparse24_compress": (st, [i64, i64, i32, vp, vp, vp, vp]),
        "gemm_sparse24_compress_noalloc": (st, [i64, i64, i32, vp, vp, vp, vp]),
        "gemm_sparse24_run": (st, [vp, vp, vp, vp, vp, vp, vp, vp]),
        "gemm_diag_mfma_loop": (st, [i32, i32, i64, vp, vp]),
        "gemm_status_string": (ctypes.c_char_p, [st]),
        "gemm_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _status_name(s):
    try:
        return load().gemm_status_string(s).decode()
    except Exception:
        return "status %d" % s


def gemm_status_string(status):
    return load().gemm_status_string(status).decode()


def gemm_last_error():
    return load().gemm_last_error().decode()


def _check(status):
    if status != GEMM_OK:
        raise GemmError(status, gemm_last_error())


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_desc(M, N, K, a_type, b_type, d_type, *, c_type=None, has_c=True, has_bias=False,
              alpha=1.0, act="none", a_layout="row", b_layout="col", lda=0, ldb=0, ldc=0,
              ldd=0, sparse_a=False, algo="auto", block_scale=0, saturate=False):
    """Build a gemm_desc_t from readable arguments (type names as in DTYPES)."""
    integer = a_type in ("s8", "u8") and d_type == "s32"
    if c_type is None:
        c_type = "s32" if integer else "f32"
    d = gemm_desc_t()
    d.M, d.N, d.K = M, N, K
    d.a_type, d.b_type = DTYPES[a_type], DTYPES[b_type]
    d.c_type, d.d_type = DTYPES[c_type], DTYPES[d_type]
    d.a_layout = ROW_MAJOR if a_layout == "row" else COL_MAJOR
    d.b_layout = ROW_MAJOR if b_layout == "row" else COL_MAJOR
    d.lda, d.ldb, d.ldc, d.ldd = lda, ldb, ldc, ldd
    d.alpha = alpha
    d.has_c, d.has_bias = int(bool(has_c)), int(bool(has_bias))
    d.act = ACT_RELU if act == "relu" else ACT_NONE
    d.sparse_a = int(bool(sparse_a))
    d.algo = ALGO[algo] if isinstance(algo, str) else int(algo)
    d.block_scale = int(block_scale)
    d.saturate = int(bool(saturate))
    return d


def gemm_validate_desc(desc):
    """Returns the status code (GEMM_OK or an error); never raises."""
    return load().gemm_validate_desc(ctypes.byref(desc) if desc is not None else None)


class Plan:
    """Owns a gemm_plan_t*; released by gemm_plan_destroy / close()."""

    def __init__(self, handle, desc):
        self.handle = handle
        self.desc = desc

    def close(self):
        if self.handle:
            load().gemm_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def name(self):
        return gemm_plan_describe(self)


def gemm_plan(desc):
    L = load()
    h = ctypes.c_void_p()
    _check(L.gemm_plan(ctypes.byref(desc), ctypes.byref(h)))
    return Plan(h.value, desc)


def gemm_plan_destroy(plan):
    plan.close()


def gemm_plan_describe(plan):
    buf = ctypes.create_string_buffer(128)
    _check(load().gemm_plan_describe(plan.handle, buf, len(buf)))
    return buf.value.decode()


def gemm_run(plan, A, B, C, bias, D, stream=None):
    _check(load().gemm_run(plan.handle, _ptr(A), _ptr(B), _ptr(C), _ptr(bias), _ptr(D),
                           _stream(stream)))


def gemm_sparse24_sizes(M, K, a_type="f16"):
    vb, mb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().gemm_sparse24_sizes(M, K, DTYPES[a_type], ctypes.byref(vb), ctypes.byref(mb)))
    return vb.value, mb.value


def gemm_sparse24_compress(M, K, a_type, A, values, meta, stream=None):
    _check(load().gemm_sparse24_compress(M, K, DTYPES[a_type], _ptr(A), _ptr(values), _ptr(meta),
                                         _stream(stream)))


def gemm_sparse24_compress_noalloc(M, K, a_type, A, values, meta, stream=None):
    _check(load().gemm_sparse24_compress_noalloc(M, K, DTYPES[a_type], _ptr(A), _ptr(values),
                                                 _ptr(meta), _stream(stream)))


def gemm_sparse24_run(plan, values, meta, B, C, bias, D, stream=None):
    _check(load().gemm_sparse24_run(plan.handle, _ptr(values), _ptr(meta), _ptr(B), _ptr(C),
                                    _ptr(bias), _ptr(D), _stream(stream)))


def gemm_mx_run(plan, A, scale_a, B, scale_b, C, bias, D, stream=None):
    _check(load().gemm_mx_run(plan.handle, _ptr(A), _ptr(scale_a), _ptr(B), _ptr(scale_b),
                              _ptr(C), _ptr(bias), _ptr(D), _stream(stream)))


def gemm_w4a16_run(plan, A, B, scales, zeros, C, bias, D, stream=None):
    _check(load().gemm_w4a16_run(plan.handle, _ptr(A), _ptr(B), _ptr(scales), _ptr(zeros),
                                 _ptr(C), _ptr(bias), _ptr(D), _stream(stream)))


def gemm_diag_mfma_loop(kind, blocks, iters, out, stream=None):
    """Diagnostic MFMA-only loop (include/gemm_diag.h); kind 0 bf16, 1 fp8,
    2 int8 (32x32 forms), 3..5 the same types' 16x16 forms; out: a device
    float tensor of blocks * 512 elements."""
    _check(load().gemm_diag_mfma_loop(kind, blocks, iters, _ptr(out), _stream(stream)))
