"""Helpers for the GPU tests: move raw-bit numpy arrays to device tensors and
run the library through its C ABI (sparse_tiled_gemm_amd.gemm)."""
import sys

import numpy as np
import torch

from sparse_tiled_gemm_amd import gemm as G

_VIEW = {1: np.uint8, 2: np.int16, 4: np.int32, 8: np.int64}
OUT_NP = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16, "s32": np.int32,
          "e4m3": np.uint8, "e5m2": np.uint8}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a):
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(_VIEW[a.itemsize]).copy()).cuda()


def to_host(t, np_dtype):
    return t.cpu().numpy().view(np_dtype)


def empty_out(M, N, d_type, ldd=0):
    ld = ldd or N
    eb = G.ELEM_BYTES[d_type]
    return torch.empty(max(M * ld, 1) * eb, dtype=torch.uint8, device="cuda")


def gpu_gemm(A, B, C, bias, M, N, K, a_type, b_type, d_type, *, alpha=1.0, relu=False,
             a_col=False, b_col=True, algo="auto", lda=0, ldb=0, ldc=0, ldd=0,
             a_dev=None, b_dev=None, c_dev=None, out=None, saturate=False):
    """Run D = epilogue(A*B + C) on the GPU; returns (D bits [M,N], plan name)."""
    desc = G.make_desc(M, N, K, a_type, b_type, d_type, has_c=C is not None or c_dev is not None,
                       has_bias=bias is not None, alpha=alpha, act="relu" if relu else "none",
                       a_layout="col" if a_col else "row", b_layout="col" if b_col else "row",
                       lda=lda, ldb=ldb, ldc=ldc, ldd=ldd, algo=algo, saturate=saturate)
    plan = G.gemm_plan(desc)
    tA = a_dev if a_dev is not None else to_dev(A)
    tB = b_dev if b_dev is not None else to_dev(B)
    tC = c_dev if c_dev is not None else (to_dev(C) if C is not None else None)
    tb = to_dev(bias) if bias is not None else None
    D = out if out is not None else empty_out(M, N, d_type, ldd)
    G.gemm_run(plan, tA, tB, tC, tb, D)
    torch.cuda.synchronize()
    ld = ldd or N
    h = D.cpu().numpy().view(OUT_NP[d_type])
    return h[: M * ld].reshape(M, ld)[:, :N].copy(), plan.name


def gpu_compress(A_logical, a_type="f16"):
    M, K = A_logical.shape
    vb, mb = G.gemm_sparse24_sizes(M, K, a_type)
    tA = to_dev(A_logical)
    vals = torch.empty(max(vb, 16), dtype=torch.uint8, device="cuda")
    meta = torch.empty(max(mb, 16), dtype=torch.uint8, device="cuda")
    G.gemm_sparse24_compress(M, K, a_type, tA, vals, meta)
    torch.cuda.synchronize()
    return vals, meta, vb, mb


def gpu_sparse_gemm(vals, meta, B, C, M, N, K, d_type="f32", *, algo="auto", bias=None,
                    alpha=1.0, relu=False, b_col=True, a_type="f16", b_type=None,
                    saturate=False):
    desc = G.make_desc(M, N, K, a_type, b_type or a_type, d_type, has_c=C is not None,
                       has_bias=bias is not None, alpha=alpha, act="relu" if relu else "none",
                       b_layout="col" if b_col else "row", sparse_a=True, algo=algo,
                       saturate=saturate)
    plan = G.gemm_plan(desc)
    tB = to_dev(B)
    tC = to_dev(C) if C is not None else None
    tb = to_dev(bias) if bias is not None else None
    D = empty_out(M, N, d_type)
    G.gemm_sparse24_run(plan, vals, meta, tB, tC, tb, D)
    torch.cuda.synchronize()
    return D.cpu().numpy().view(OUT_NP[d_type]).reshape(M, N).copy(), plan.name
