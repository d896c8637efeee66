"""Exact reference arithmetic for pinning the oracle: operand values decoded
with numpy/torch's own conversions (not the oracle's decoders), sums formed
in Python's exact rationals, and an exact RNE rounding of a rational to fp32."""
from fractions import Fraction

import numpy as np
import torch

_TORCH = {"bf16": torch.bfloat16, "e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


def lib_decode(type_name, bits):
    bits = np.ascontiguousarray(bits)
    if type_name == "f16":
        return bits.view(np.float16).astype(np.float64)
    if type_name in ("s8", "s32"):
        return bits.astype(np.float64)
    if type_name == "f32":
        return bits.astype(np.float64)
    t = torch.from_numpy(bits.view(np.int16) if type_name == "bf16" else bits)
    return t.view(_TORCH[type_name]).to(torch.float32).numpy().astype(np.float64)


def logical_a(A, type_name, M, K, col_major):
    v = lib_decode(type_name, A)
    return v.reshape(K, M).T if col_major else v.reshape(M, K)


def logical_b(B, type_name, K, N, col_major):
    """Logical K x N matrix from B stored [N,K] (col_major) or [K,N]."""
    v = lib_decode(type_name, B)
    return v.reshape(N, K).T if col_major else v.reshape(K, N)


def exact_gemm(a, b, c=None):
    """Exact sum_k a[m,k] b[k,n] (+ c[m,n]) and sum_k |a b| + |c| as Fractions."""
    M, K = a.shape
    N = b.shape[1]
    fa = [[Fraction(float(x)) for x in row] for row in a]
    fb = [[Fraction(float(b[k, n])) for k in range(K)] for n in range(N)]
    out = [[None] * N for _ in range(M)]
    sab = [[None] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            s = Fraction(0)
            t = Fraction(0)
            for k in range(K):
                p = fa[m][k] * fb[n][k]
                s += p
                t += abs(p)
            if c is not None:
                cv = Fraction(float(c[m, n]))
                s += cv
                t += abs(cv)
            out[m][n] = s
            sab[m][n] = t
    return out, sab


def round_f32(x):
    """Exact round-to-nearest-even of a Fraction to fp32 (finite range)."""
    f = np.float32(float(x))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]

    def key(c):
        d = abs(Fraction(float(c)) - x)
        odd = int(np.array([c], np.float32).view(np.uint32)[0] & 1)
        return (d, odd)

    return min(cands, key=key)
