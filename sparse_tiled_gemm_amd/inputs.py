"""Seeded synthetic inputs for the GEMM workloads.

This module only draws random numbers and stores them in the operand formats,
using numpy's and torch's own conversions (numpy float16; torch bfloat16 and
float8).  It holds none of the GEMM arithmetic and is shared by the CPU checks
and the GPU runs so both read identical bytes.

Arrays are returned as numpy arrays of raw element bits:
  f16, bf16 -> uint16, e4m3, e5m2 -> uint8, s8 -> int8, f32 -> float32,
  s32 -> int32.
Operand layouts: A is [M,K] row-major, B is stored [N,K] (column-major K x N),
C and D are [M,N] row-major, bias is [N] fp32.

Seeds are 1000*workload + tensor (A=1, B=2, C=3, bias=4, sparsity pattern=5).
For the 2:4 workloads the A seed draws the kept values.
"""
import numpy as np
import torch

E4M3_MAX = 448.0
E5M2_MAX = 57344.0


def _rng(workload, tensor):
    return np.random.default_rng(1000 * workload + tensor)


def to_f16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def to_bf16(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def to_e4m3(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def to_e5m2(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e5m2)
    return t.view(torch.uint8).numpy()


def f16_values(bits):
    """float64 view of fp16 bits (numpy's own conversion; used by generators)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


class Problem(dict):
    """Operands plus the call description: keys M, N, K, a_type, b_type, d_type,
    A, B, C (or None), bias (or None), alpha, relu, and for the 2:4 workload
    A_logical (the dense fp16 matrix the compressor receives)."""

    @property
    def flops(self):
        return 2.0 * self["M"] * self["N"] * self["K"]


def dense_f16(M=128, N=128, K=128, workload=1):
    """fp16 A, B uniform[-1,1]; C fp32 uniform[-1,1]; fp32 out, no epilogue."""
    A = to_f16(_rng(workload, 1).uniform(-1.0, 1.0, size=(M, K)))
    B = to_f16(_rng(workload, 2).uniform(-1.0, 1.0, size=(N, K)))
    C = _rng(workload, 3).uniform(-1.0, 1.0, size=(M, N)).astype(np.float32)
    return Problem(M=M, N=N, K=K, a_type="f16", b_type="f16", d_type="f32", A=A, B=B, C=C,
                   bias=None, alpha=1.0, relu=False)


def dense_bf16(M=8192, N=8192, K=8192, workload=2, d_type="bf16"):
    """bf16 A, B normal(0,1)/sqrt(K); C fp32 zeros (a real buffer); bf16 out."""
    s = 1.0 / np.sqrt(K)
    A = to_bf16(_rng(workload, 1).standard_normal(size=(M, K), dtype=np.float32) * s)
    B = to_bf16(_rng(workload, 2).standard_normal(size=(N, K), dtype=np.float32) * s)
    C = np.zeros((M, N), dtype=np.float32)
    return Problem(M=M, N=N, K=K, a_type="bf16", b_type="bf16", d_type=d_type, A=A, B=B, C=C,
                   bias=None, alpha=1.0, relu=False)


def dense_s8(M=8192, N=8192, K=8192, workload=3):
    """s8 A, B uniform integers in [-128,127]; C s32 uniform in [-2^20, 2^20]."""
    A = _rng(workload, 1).integers(-128, 128, size=(M, K), dtype=np.int8)
    B = _rng(workload, 2).integers(-128, 128, size=(N, K), dtype=np.int8)
    C = _rng(workload, 3).integers(-(1 << 20), (1 << 20) + 1, size=(M, N), dtype=np.int32)
    return Problem(M=M, N=N, K=K, a_type="s8", b_type="s8", d_type="s32", A=A, B=B, C=C,
                   bias=None, alpha=1.0, relu=False)


def dense_fp8(M=8192, N=8192, K=8192, workload=4):
    """A normal(0,1) scaled by sA = 448/amax(A), clamped and rounded to E4M3;
    B likewise with sB = 57344/amax(B) to E5M2; no C; alpha = fp32(1/(sA*sB));
    bias fp32 normal(0,1) [N]; out = relu(alpha*acc + bias[n]) as fp16."""
    a = _rng(workload, 1).standard_normal(size=(M, K), dtype=np.float32).astype(np.float64)
    b = _rng(workload, 2).standard_normal(size=(N, K), dtype=np.float32).astype(np.float64)
    sA = E4M3_MAX / np.abs(a).max()
    sB = E5M2_MAX / np.abs(b).max()
    A = to_e4m3(np.clip(a * sA, -E4M3_MAX, E4M3_MAX))
    B = to_e5m2(np.clip(b * sB, -E5M2_MAX, E5M2_MAX))
    bias = _rng(workload, 4).standard_normal(size=(N,)).astype(np.float32)
    alpha = float(np.float32(1.0 / (sA * sB)))
    return Problem(M=M, N=N, K=K, a_type="e4m3", b_type="e5m2", d_type="f16", A=A, B=B, C=None,
                   bias=bias, alpha=alpha, relu=True)


_PAIRS = np.array([(0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3)], dtype=np.int64)
# bits that must be non-zero for an element to count as a non-zero
_NZ_MASK = {"f16": 0x7FFF, "bf16": 0x7FFF, "e4m3": 0x7F, "e5m2": 0x7F, "s8": 0xFF}


def _scatter_24(M, K, workload, draw_kept, a_type):
    """Logical [M,K] A with exactly two non-zeros in every 4 consecutive K
    positions (one of the 6 position pairs, uniformly; seed tensor 5).
    draw_kept(rng, n) returns n raw-bit values of a_type; exact zeros are
    redrawn, so the non-zero positions are exactly the drawn pattern."""
    if K % 4:
        raise ValueError("K must be a multiple of 4")
    G = K // 4
    choice = _rng(workload, 5).integers(0, 6, size=(M, G))
    pos = _PAIRS[choice]  # [M, G, 2], ascending
    vr = _rng(workload, 1)
    vals = draw_kept(vr, M * G * 2).reshape(M, G, 2)
    mask = _NZ_MASK[a_type]
    zero = (vals.view(np.uint16 if vals.itemsize == 2 else np.uint8) & mask) == 0
    while zero.any():
        vals[zero] = draw_kept(vr, int(zero.sum()))
        zero = (vals.view(np.uint16 if vals.itemsize == 2 else np.uint8) & mask) == 0
    A = np.zeros((M, G, 4), dtype=vals.dtype)
    rows = np.arange(M)[:, None]
    grps = np.arange(G)[None, :]
    A[rows, grps, pos[..., 0]] = vals[..., 0]
    A[rows, grps, pos[..., 1]] = vals[..., 1]
    return A.reshape(M, K)


def sparse24_f16(M=8192, N=8192, K=8192, workload=5):
    """Logical fp16 A with exactly two non-zeros in every 4 consecutive K
    positions (one of the 6 position pairs, uniformly), non-zero values
    uniform[-1,1] with exact zeros redrawn; B fp16 uniform[-1,1]; C fp32
    uniform[-1,1]; fp32 out.  A_logical is what the compressor receives."""
    A = _scatter_24(M, K, workload, lambda r, n: to_f16(r.uniform(-1.0, 1.0, size=n)), "f16")
    B = to_f16(_rng(workload, 2).uniform(-1.0, 1.0, size=(N, K)))
    C = _rng(workload, 3).uniform(-1.0, 1.0, size=(M, N)).astype(np.float32)
    return Problem(M=M, N=N, K=K, a_type="f16", b_type="f16", d_type="f32", A=None, B=B, C=C,
                   bias=None, alpha=1.0, relu=False, A_logical=A)


def sparse24_bf16(M=8192, N=8192, K=8192, workload=6, d_type="bf16"):
    """The bf16 workload with A pruned 2:4: kept values normal(0,1)*sqrt(2/K)
    (the same row variance as a dense normal(0,1)/sqrt(K) row), B
    normal(0,1)/sqrt(K), C fp32 uniform[-1,1]; bf16 out."""
    s = np.sqrt(2.0 / K) if K else 1.0
    A = _scatter_24(M, K, workload,
                    lambda r, n: to_bf16(r.standard_normal(size=n, dtype=np.float32) * s), "bf16")
    B = to_bf16(_rng(workload, 2).standard_normal(size=(N, K), dtype=np.float32) /
                np.sqrt(max(K, 1)))
    C = _rng(workload, 3).uniform(-1.0, 1.0, size=(M, N)).astype(np.float32)
    return Problem(M=M, N=N, K=K, a_type="bf16", b_type="bf16", d_type=d_type, A=None, B=B, C=C,
                   bias=None, alpha=1.0, relu=False, A_logical=A)


def sparse24_s8(M=8192, N=8192, K=8192, workload=7):
    """s8 A pruned 2:4 with kept values uniform in [-128,127] minus 0, B
    uniform in [-128,127]; C s32 uniform in [-2^20, 2^20]; s32 out."""
    A = _scatter_24(M, K, workload, lambda r, n: r.integers(-128, 128, size=n, dtype=np.int8), "s8")
    B = _rng(workload, 2).integers(-128, 128, size=(N, K), dtype=np.int8)
    C = _rng(workload, 3).integers(-(1 << 20), (1 << 20) + 1, size=(M, N), dtype=np.int32)
    return Problem(M=M, N=N, K=K, a_type="s8", b_type="s8", d_type="s32", A=None, B=B, C=C,
                   bias=None, alpha=1.0, relu=False, A_logical=A)


def sparse24_fp8(M=8192, N=8192, K=8192, workload=8, a_type="e4m3", b_type="e5m2"):
    """The fp8 workload with A pruned 2:4: kept values normal(0,1) scaled by
    sA = max/amax and rounded to a_type, B normal(0,1) scaled likewise to
    b_type; no C; alpha = fp32(1/(sA*sB)); bias fp32 normal(0,1) [N];
    out = relu(alpha*acc + bias[n]) as fp16."""
    mx = {"e4m3": E4M3_MAX, "e5m2": E5M2_MAX}
    enc = {"e4m3": to_e4m3, "e5m2": to_e5m2}
    st = {}

    def draw(r, n):
        # sA is fixed by the first draw (all kept values); redraws of exact
        # zeros reuse it
        x = r.standard_normal(size=n, dtype=np.float32).astype(np.float64)
        if "sA" not in st:
            st["sA"] = mx[a_type] / max(np.abs(x).max(), 1e-30) if x.size else 1.0
        return enc[a_type](np.clip(x * st["sA"], -mx[a_type], mx[a_type]))

    A = _scatter_24(M, K, workload, draw, a_type)
    sA = st.get("sA", 1.0)
    b = _rng(workload, 2).standard_normal(size=(N, K), dtype=np.float32).astype(np.float64)
    sB = mx[b_type] / max(np.abs(b).max(), 1e-30) if b.size else 1.0
    B = enc[b_type](np.clip(b * sB, -mx[b_type], mx[b_type]))
    bias = _rng(workload, 4).standard_normal(size=(N,)).astype(np.float32)
    alpha = float(np.float32(1.0 / (sA * sB)))
    return Problem(M=M, N=N, K=K, a_type=a_type, b_type=b_type, d_type="f16", A=None, B=B,
                   C=None, bias=bias, alpha=alpha, relu=True, A_logical=A)


def sparse24(a_type, M, N, K, **kw):
    """The 2:4 problem of the given A type (f16, bf16, s8, e4m3, e5m2)."""
    if a_type == "f16":
        return sparse24_f16(M, N, K, **kw)
    if a_type == "bf16":
        return sparse24_bf16(M, N, K, **kw)
    if a_type == "s8":
        return sparse24_s8(M, N, K, **kw)
    if a_type in ("e4m3", "e5m2"):
        return sparse24_fp8(M, N, K, a_type=a_type, **kw)
    raise ValueError(a_type)


# ---------------------------------------------------------------- MX block-scaled

# OCP MX element formats: exponent bits, fraction bits, bias, and the exponent
# of the largest normal value (the emax of the MX quantisation recipe)
_MX_FMT = {"e4m3": (4, 3, 7, 8), "e5m2": (5, 2, 15, 15), "e2m3": (2, 3, 1, 2),
           "e3m2": (3, 2, 3, 4), "e2m1": (2, 1, 1, 2)}
MX_BITS = {"e4m3": 8, "e5m2": 8, "e2m3": 6, "e3m2": 6, "e2m1": 4}


def _mx_grid(fmt):
    """Non-negative finite values of an MX element format and their codes,
    ascending (E4M3 without its NaN code, E5M2 without inf/NaN)."""
    eb, fb, bias, _ = _MX_FMT[fmt]
    vals, codes = [], []
    for c in range(1 << (eb + fb)):
        e, f = c >> fb, c & ((1 << fb) - 1)
        if fmt == "e4m3" and c == 0x7F:
            continue
        if fmt == "e5m2" and e == 31:
            continue
        v = f * 2.0 ** (1 - bias - fb) if e == 0 else (1 + f / 2.0 ** fb) * 2.0 ** (e - bias)
        vals.append(v)
        codes.append(c)
    order = np.argsort(vals)
    return np.array(vals)[order], np.array(codes)[order]


def mx_encode(x, fmt):
    """Round to nearest (ties to the even code), saturating at the largest
    finite value; returns codes (sign in the top bit of the format)."""
    v, c = _mx_grid(fmt)
    a = np.minimum(np.abs(np.asarray(x, dtype=np.float64)), v[-1])
    i = np.clip(np.searchsorted(v, a), 1, len(v) - 1)
    lo, hi = v[i - 1], v[i]
    pick_hi = (a - lo > hi - a) | ((a - lo == hi - a) & (c[i] % 2 == 0))
    code = np.where(pick_hi, c[i], c[i - 1])
    sign = (np.signbit(x) & (code != 0)).astype(np.int64) << (MX_BITS[fmt] - 1)
    return (code | sign).astype(np.uint8)


def mx_quantize(x, fmt):
    """The MX recipe along the last axis: per block of 32, shared exponent
    floor(log2(amax)) - emax (E8M0 code = that + 127, clamped to 0..254),
    elements = x / 2^shared rounded to the format.  Returns (codes, scales)."""
    x = np.asarray(x, dtype=np.float64)
    rows, K = x.shape
    xb = x.reshape(rows, K // 32, 32)
    amax = np.abs(xb).max(-1)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))), -127.0)
    shared = np.clip(e - _MX_FMT[fmt][3], -127, 127)
    codes = mx_encode(xb / np.ldexp(1.0, shared.astype(np.int64))[..., None], fmt)
    return codes.reshape(rows, K), (shared + 127).astype(np.uint8)


def mx_pack(codes, fmt):
    """Pack [rows, K] codes along each row: 8-bit one per byte, E2M1 two per
    byte (even element in the low nibble), 6-bit as a little-endian bit
    string (element i in bits 6i .. 6i+5)."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows, K = codes.shape
    b = MX_BITS[fmt]
    if b == 8:
        return codes.copy()
    if b == 4:
        c = codes.reshape(rows, K // 2, 2).astype(np.uint8)
        return (c[..., 0] | (c[..., 1] << 4)).astype(np.uint8)
    c = codes.reshape(rows, K // 4, 4).astype(np.uint32)
    w = c[..., 0] | (c[..., 1] << 6) | (c[..., 2] << 12) | (c[..., 3] << 18)  # 24 bits
    out = np.stack([w & 0xFF, (w >> 8) & 0xFF, (w >> 16) & 0xFF], axis=-1)
    return out.reshape(rows, K // 4 * 3).astype(np.uint8)


def mx_problem(M=8192, N=8192, K=8192, a_type="e4m3", b_type="e4m3", workload=9,
               d_type="bf16"):
    """A and B normal(0,1), each MX-quantised to its format per block of 32 K
    (B along K of each column, i.e. rows of its stored [N, K] form); no C,
    alpha 1, no bias, d_type out.  A, B are packed bytes; SA [M, K/32] and SB
    [N, K/32] E8M0 codes."""
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    a = _rng(workload, 1).standard_normal(size=(M, K), dtype=np.float32)
    b = _rng(workload, 2).standard_normal(size=(N, K), dtype=np.float32)
    ca, SA = mx_quantize(a, a_type)
    cb, SB = mx_quantize(b, b_type)
    return Problem(M=M, N=N, K=K, a_type=a_type, b_type=b_type, d_type=d_type,
                   A=mx_pack(ca, a_type), B=mx_pack(cb, b_type), SA=SA, SB=SB, C=None,
                   bias=None, alpha=1.0, relu=False, mx=True)


# ---------------------------------------------------------------- W4A16

def w4_pack(q):
    """[N, K] codes 0..15 -> [N, K/2] bytes, element k in bits 4(k%2) .. of byte k/2."""
    q = np.asarray(q, dtype=np.uint8)
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)


def w4a16_problem(M=8192, N=8192, K=8192, a_type="bf16", gs=128, workload=12, zeros=True):
    """Activations A normal(0,1) in a_type; weights normal(0, 1/K) quantised
    asymmetrically per group of gs K: s = (max - min) / 15 rounded to a_type,
    z = round(-min / s) in 0..15 (or 8 when zeros is False), q = clamp(round(w
    / s) + z, 0, 15); B = packed codes [N, K/2]; no C, no bias, a_type out."""
    enc = to_f16 if a_type == "f16" else to_bf16
    dec = (lambda b: np.asarray(b, np.uint16).view(np.float16).astype(np.float64)) \
        if a_type == "f16" else \
        (lambda b: (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    A = enc(_rng(workload, 1).standard_normal(size=(M, K), dtype=np.float32))
    w = _rng(workload, 2).standard_normal(size=(N, K), dtype=np.float32).astype(np.float64)
    w /= np.sqrt(K)
    wg = w.reshape(N, K // gs, gs)
    lo = np.minimum(wg.min(-1), 0.0)
    hi = np.maximum(wg.max(-1), 0.0)
    if zeros:
        S = enc(np.maximum(hi - lo, 1e-8) / 15.0)
        s = dec(S)
        Z = np.clip(np.round(-lo / s), 0, 15).astype(np.uint8)
    else:
        S = enc(np.maximum(np.maximum(hi, -lo), 1e-8) / 7.0)
        s = dec(S)
        Z = None
    z = Z.astype(np.float64) if zeros else 8.0
    q = np.clip(np.round(wg / s[..., None]) + (z[..., None] if zeros else z), 0, 15)
    B = w4_pack(q.reshape(N, K).astype(np.uint8))
    return Problem(M=M, N=N, K=K, a_type=a_type, b_type="u4", d_type=a_type, A=A, B=B,
                   scales=S, zeros=Z, gs=gs, C=None, bias=None, alpha=1.0, relu=False, w4=True)


WORKLOADS = {
    "f16_128": lambda: dense_f16(128, 128, 128),
    "bf16_8192": lambda: dense_bf16(8192, 8192, 8192),
    "bf16_skinny_16x8192x8192": lambda: dense_bf16(16, 8192, 8192),
    "s8_8192": lambda: dense_s8(8192, 8192, 8192),
    "fp8_8192": lambda: dense_fp8(8192, 8192, 8192),
    "sparse24_f16_8192": lambda: sparse24_f16(8192, 8192, 8192),
    "sparse24_bf16_8192": lambda: sparse24_bf16(8192, 8192, 8192),
    "sparse24_s8_8192": lambda: sparse24_s8(8192, 8192, 8192),
    "sparse24_fp8_8192": lambda: sparse24_fp8(8192, 8192, 8192),
    "mxfp8_8192": lambda: mx_problem(8192, 8192, 8192, "e4m3", "e4m3", 9),
    "mxfp6_8192": lambda: mx_problem(8192, 8192, 8192, "e2m3", "e2m3", 10),
    "w4a16_bf16_8192": lambda: w4a16_problem(8192, 8192, 8192, "bf16", 128, 12),
    "w4a16_bf16_16x8192x8192": lambda: w4a16_problem(16, 8192, 8192, "bf16", 128, 13),
    "mxfp4_8192": lambda: mx_problem(8192, 8192, 8192, "e2m1", "e2m1", 11),
}
