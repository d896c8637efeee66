"""ctypes wrapper over the CPU oracle (liboracle.so).  TEST INFRASTRUCTURE ONLY.

Arrays are numpy arrays holding raw element bits:
  f16, bf16 -> uint16    e4m3, e5m2 -> uint8    s8 -> int8    u8 -> uint8
  f32 -> float32         s32 -> int32
The library is built from oracle.c on first use when it is missing.
"""
import ctypes
import os

import numpy as np

from . import build as _build

TYPES = {"f16": 0, "bf16": 1, "e4m3": 2, "e5m2": 3, "s8": 4, "f32": 5, "s32": 6,
         "e2m3": 7, "e3m2": 8, "e2m1": 9, "e8m0": 10, "u8": 11}
INT_IN = ("s8", "u8")
# bits per element of the MX element formats (6- and 4-bit ones are stored packed)
MX_BITS = {"e4m3": 8, "e5m2": 8, "e2m3": 6, "e3m2": 6, "e2m1": 4}
STORAGE = {
    "f16": np.uint16, "bf16": np.uint16, "e4m3": np.uint8, "e5m2": np.uint8,
    "s8": np.int8, "u8": np.uint8, "f32": np.float32, "s32": np.int32,
}

_lib = None


class _Desc(ctypes.Structure):
    _fields_ = [
        ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
        ("a_type", ctypes.c_int), ("b_type", ctypes.c_int),
        ("c_type", ctypes.c_int), ("d_type", ctypes.c_int),
        ("a_col_major", ctypes.c_int), ("b_col_major", ctypes.c_int),
        ("lda", ctypes.c_int64), ("ldb", ctypes.c_int64),
        ("ldc", ctypes.c_int64), ("ldd", ctypes.c_int64),
        ("alpha", ctypes.c_float),
        ("has_c", ctypes.c_int), ("has_bias", ctypes.c_int), ("relu", ctypes.c_int),
        ("saturate", ctypes.c_int),
    ]


def lib():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        vp, i64, dp = ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p
        L.oracle_decode.restype = ctypes.c_double
        L.oracle_decode.argtypes = [ctypes.c_int, vp, i64]
        L.oracle_encode.restype = ctypes.c_int
        L.oracle_encode.argtypes = [ctypes.c_int, ctypes.c_double, vp, i64]
        L.oracle_decode_array.restype = None
        L.oracle_decode_array.argtypes = [ctypes.c_int, vp, i64, dp]
        L.oracle_encode_array.restype = ctypes.c_int
        L.oracle_encode_array.argtypes = [ctypes.c_int, dp, i64, vp]
        L.oracle_gemm.restype = ctypes.c_int
        L.oracle_gemm.argtypes = [ctypes.POINTER(_Desc), vp, vp, vp, vp, vp, dp, dp]
        L.oracle_gemm_entries.restype = ctypes.c_int
        L.oracle_gemm_entries.argtypes = [ctypes.POINTER(_Desc), vp, vp, vp, vp, i64, vp, vp,
                                          vp, dp, dp]
        L.oracle_epilogue_f32.restype = ctypes.c_int
        L.oracle_epilogue_f32.argtypes = [i64, i64, vp, ctypes.c_float, vp, ctypes.c_int,
                                          ctypes.c_int, vp]
        L.oracle_sparse24_compress.restype = ctypes.c_int64
        L.oracle_sparse24_compress.argtypes = [ctypes.c_int, i64, i64, vp, vp, vp]
        L.oracle_sparse24_decompress.restype = ctypes.c_int
        L.oracle_sparse24_decompress.argtypes = [ctypes.c_int, i64, i64, vp, vp, vp]
        L.oracle_mx_gemm.restype = ctypes.c_int
        L.oracle_mx_gemm.argtypes = [ctypes.POINTER(_Desc), vp, vp, vp, vp, vp, vp, vp, dp, dp]
        L.oracle_mx_gemm_entries.restype = ctypes.c_int
        L.oracle_mx_gemm_entries.argtypes = [ctypes.POINTER(_Desc), vp, vp, vp, vp, vp, vp, i64,
                                             vp, vp, vp, dp, dp]
        L.oracle_w4a16_dequant.restype = ctypes.c_int
        L.oracle_w4a16_dequant.argtypes = [ctypes.c_int, i64, i64, i64, vp, i64, vp, vp, vp]
        L.oracle_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads():
    return lib().oracle_num_threads()


def decode(type_name, bits):
    """Decode a raw array of the given type to float64, element by element."""
    bits = np.ascontiguousarray(bits, dtype=STORAGE[type_name])
    flat = bits.reshape(-1)
    out = np.empty(flat.size, dtype=np.float64)
    lib().oracle_decode_array(TYPES[type_name], _ptr(flat), flat.size, _ptr(out))
    return out.reshape(bits.shape)


def encode(type_name, values):
    """RNE-encode float64 values (integers for s32) to raw bits of type_name."""
    values = np.ascontiguousarray(values, dtype=np.float64)
    flat = values.reshape(-1)
    out = np.empty(flat.size, dtype=STORAGE[type_name])
    if lib().oracle_encode_array(TYPES[type_name], _ptr(flat), flat.size, _ptr(out)) != 0:
        raise ValueError("oracle cannot encode %s" % type_name)
    return out.reshape(values.shape)


def _desc(M, N, K, a_type, b_type, c_type, d_type, a_col_major, b_col_major,
          lda, ldb, ldc, ldd, alpha, has_c, has_bias, relu, saturate=False):
    return _Desc(M, N, K, TYPES[a_type], TYPES[b_type], TYPES[c_type], TYPES[d_type],
                 int(a_col_major), int(b_col_major), lda, ldb, ldc, ldd,
                 float(alpha), int(has_c), int(has_bias), int(relu), int(saturate))


def _lds(M, N, K, a_col_major, b_col_major):
    lda = M if a_col_major else K
    ldb = K if b_col_major else N
    return lda, ldb, N, N


def gemm(A, B, C, bias, M, N, K, a_type, b_type, d_type, *, a_col_major=False,
         b_col_major=True, alpha=1.0, relu=False, want_y=True, want_s=True, saturate=False,
         c_type=None):
    """Full oracle GEMM on packed operands.

    A is [M,K] row-major (or [K,M] when a_col_major), B is stored [N,K] when
    b_col_major (else [K,N]), C and D are [M,N] row-major.  Returns
    (D_bits, Y, S): the encoded output, the fp64 pre-cast result and the
    error scale sum_k |a b| + |c|.  saturate: an int32 output clamps the exact
    acc + C to the int32 range instead of wrapping.
    """
    integer = a_type in INT_IN and d_type == "s32"
    c_type = c_type or ("s32" if integer else "f32")
    lda, ldb, ldc, ldd = _lds(M, N, K, a_col_major, b_col_major)
    g = _desc(M, N, K, a_type, b_type, c_type, d_type, a_col_major, b_col_major,
              lda, ldb, ldc, ldd, alpha, C is not None, bias is not None, relu, saturate)
    A = np.ascontiguousarray(A, dtype=STORAGE[a_type])
    B = np.ascontiguousarray(B, dtype=STORAGE[b_type])
    if C is not None:
        C = np.ascontiguousarray(C, dtype=STORAGE[c_type])
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
    D = np.zeros((M, N), dtype=STORAGE[d_type])
    Y = np.empty((M, N), dtype=np.float64) if want_y else None
    S = np.empty((M, N), dtype=np.float64) if want_s else None
    rc = lib().oracle_gemm(ctypes.byref(g), _ptr(A), _ptr(B), _ptr(C), _ptr(bias), _ptr(D),
                           _ptr(Y), _ptr(S))
    if rc != 0:
        raise ValueError("oracle_gemm rejected the problem")
    return D, Y, S


def gemm_entries(A, B, C, bias, M, N, K, a_type, b_type, d_type, rows, cols, *,
                 a_col_major=False, b_col_major=True, alpha=1.0, relu=False, saturate=False,
                 c_type=None):
    """The oracle definition at chosen (rows[i], cols[i]) only: (D_bits, Y, S)."""
    integer = a_type in INT_IN and d_type == "s32"
    c_type = c_type or ("s32" if integer else "f32")
    lda, ldb, ldc, ldd = _lds(M, N, K, a_col_major, b_col_major)
    g = _desc(M, N, K, a_type, b_type, c_type, d_type, a_col_major, b_col_major,
              lda, ldb, ldc, ldd, alpha, C is not None, bias is not None, relu, saturate)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    n = rows.size
    D = np.zeros(n, dtype=STORAGE[d_type])
    Y = np.empty(n, dtype=np.float64)
    S = np.empty(n, dtype=np.float64)
    rc = lib().oracle_gemm_entries(ctypes.byref(g), _ptr(A), _ptr(B), _ptr(C), _ptr(bias), n,
                                   _ptr(rows), _ptr(cols), _ptr(D), _ptr(Y), _ptr(S))
    if rc != 0:
        raise ValueError("oracle_gemm_entries rejected the problem")
    return D, Y, S


def epilogue_f32(T, alpha, bias, relu, d_type):
    """fp32-semantics epilogue of a given fp32 [M,N] tile (see oracle.h)."""
    T = np.ascontiguousarray(T, dtype=np.float32)
    M, N = T.shape
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
    D = np.zeros((M, N), dtype=STORAGE[d_type])
    rc = lib().oracle_epilogue_f32(M, N, _ptr(T), float(alpha), _ptr(bias), int(relu),
                                   TYPES[d_type], _ptr(D))
    if rc != 0:
        raise ValueError("oracle_epilogue_f32 rejected the output type")
    return D


class NotSparse24(ValueError):
    pass


SPARSE24_TYPES = ("f16", "bf16", "e4m3", "e5m2", "s8", "u8")


def sparse24_compress(A, type_name="f16"):
    """[M,K] raw bits of type_name -> (values [M,K/2] same storage,
    meta [M,ceil(K/32)] uint32)."""
    if type_name not in SPARSE24_TYPES:
        raise ValueError("no 2:4 form for %s" % type_name)
    A = np.ascontiguousarray(A, dtype=STORAGE[type_name])
    M, K = A.shape
    if K % 4:
        raise ValueError("K must be a multiple of 4")
    values = np.zeros((M, K // 2), dtype=A.dtype)
    meta = np.zeros((M, (K + 31) // 32), dtype=np.uint32)
    rc = lib().oracle_sparse24_compress(TYPES[type_name], M, K, _ptr(A), _ptr(values), _ptr(meta))
    if rc > 0:
        raise NotSparse24("row %d has a group with more than two non-zeros" % (rc - 1))
    if rc < 0:
        raise ValueError("bad shape")
    return values, meta


def sparse24_decompress(values, meta, M, K, type_name="f16"):
    if type_name not in SPARSE24_TYPES:
        raise ValueError("no 2:4 form for %s" % type_name)
    values = np.ascontiguousarray(values, dtype=STORAGE[type_name])
    meta = np.ascontiguousarray(meta, dtype=np.uint32)
    A = np.zeros((M, K), dtype=values.dtype)
    rc = lib().oracle_sparse24_decompress(TYPES[type_name], M, K, _ptr(values), _ptr(meta),
                                          _ptr(A))
    if rc != 0:
        raise ValueError("metadata not ascending or bad shape")
    return A


# ---------------------------------------------------------------- MX

def decode_packed(type_name, packed, n):
    """First n elements of a packed row-major byte array of an MX element
    format (or e8m0 scales), decoded to float64."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8).reshape(-1)
    need = (n * MX_BITS.get(type_name, 8) + 7) // 8
    if packed.size < need:
        raise ValueError("packed array too short")
    out = np.empty(n, dtype=np.float64)
    lib().oracle_decode_array(TYPES[type_name], _ptr(packed), n, _ptr(out))
    return out


def _mx_args(A, SA, B, SB, C, bias, M, N, K, a_type, b_type, d_type, alpha, relu):
    g = _desc(M, N, K, a_type, b_type, "f32", d_type, False, True, K, K, N, N, alpha,
              C is not None, bias is not None, relu)
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    SA = np.ascontiguousarray(SA, dtype=np.uint8)
    SB = np.ascontiguousarray(SB, dtype=np.uint8)
    if A.size * 8 < M * K * MX_BITS[a_type] or B.size * 8 < N * K * MX_BITS[b_type]:
        raise ValueError("A or B shorter than M*K / N*K packed elements")
    if SA.size < M * (K // 32) or SB.size < N * (K // 32):
        raise ValueError("scales shorter than M*K/32 / N*K/32")
    if C is not None:
        C = np.ascontiguousarray(C, dtype=np.float32)
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
    return g, A, SA, B, SB, C, bias


def mx_gemm(A, SA, B, SB, C, bias, M, N, K, a_type, b_type, d_type, *, alpha=1.0, relu=False,
            want_y=True, want_s=True):
    """Block-scaled GEMM on packed operands: A [M, K] row-major and B stored
    [N, K] (column-major K x N), each as bytes of packed elements; SA [M, K/32],
    SB [N, K/32] E8M0 codes.  Returns (D_bits, Y, S) as gemm() does."""
    g, A, SA, B, SB, C, bias = _mx_args(A, SA, B, SB, C, bias, M, N, K, a_type, b_type, d_type,
                                        alpha, relu)
    D = np.zeros((M, N), dtype=STORAGE[d_type])
    Y = np.empty((M, N), dtype=np.float64) if want_y else None
    S = np.empty((M, N), dtype=np.float64) if want_s else None
    rc = lib().oracle_mx_gemm(ctypes.byref(g), _ptr(A), _ptr(SA), _ptr(B), _ptr(SB), _ptr(C),
                              _ptr(bias), _ptr(D), _ptr(Y), _ptr(S))
    if rc != 0:
        raise ValueError("oracle_mx_gemm rejected the problem")
    return D, Y, S


def mx_gemm_entries(A, SA, B, SB, C, bias, M, N, K, a_type, b_type, d_type, rows, cols, *,
                    alpha=1.0, relu=False):
    g, A, SA, B, SB, C, bias = _mx_args(A, SA, B, SB, C, bias, M, N, K, a_type, b_type, d_type,
                                        alpha, relu)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    n = rows.size
    D = np.zeros(n, dtype=STORAGE[d_type])
    Y = np.empty(n, dtype=np.float64)
    S = np.empty(n, dtype=np.float64)
    rc = lib().oracle_mx_gemm_entries(ctypes.byref(g), _ptr(A), _ptr(SA), _ptr(B), _ptr(SB),
                                      _ptr(C), _ptr(bias), n, _ptr(rows), _ptr(cols), _ptr(D),
                                      _ptr(Y), _ptr(S))
    if rc != 0:
        raise ValueError("oracle_mx_gemm_entries rejected the problem")
    return D, Y, S


# ---------------------------------------------------------------- W4A16

def w4a16_dequant(Bq, scales, zeros, N, K, gs, w_type):
    """[N, K/2] packed u4 codes + [N, K/gs] scales (w_type bits) + [N, K/gs]
    u8 zero points (or None: 8) -> [N, K] w_type bits (see oracle.h)."""
    Bq = np.ascontiguousarray(Bq, dtype=np.uint8).reshape(N, -1)
    scales = np.ascontiguousarray(scales, dtype=STORAGE[w_type])
    if zeros is not None:
        zeros = np.ascontiguousarray(zeros, dtype=np.uint8)
    W = np.zeros((N, K), dtype=STORAGE[w_type])
    rc = lib().oracle_w4a16_dequant(TYPES[w_type], N, K, gs, _ptr(Bq), Bq.shape[1],
                                    _ptr(scales), _ptr(zeros), _ptr(W))
    if rc != 0:
        raise ValueError("oracle_w4a16_dequant rejected the arguments")
    return W
