"""Pins for the oracle GEMM D = A*B + C and its epilogue, against things other
than the oracle itself: exact rational brute force (one 16x8x16 tile, odd tiny
shapes, all layouts and input types), closed forms (identity, all-ones,
int8 extremes at K = 8192, modulo-2^32 wrap) and hand-built epilogue cases.

The definition pinned is the GEMM element equation of "NVIDIA MMA", section
"From FMA to MMA to GEMM", followed by the scale/bias/activation/cast epilogue
of its section "Input / accumulate / output"; the 16x8x16 tile is the
m16n8k16 tile of its section "PTX types" (2048 multiply-adds)."""
import zlib
from fractions import Fraction

import numpy as np
import pytest
import torch

from exact import exact_gemm, lib_decode, logical_a, logical_b, round_f32
from sparse_tiled_gemm_amd import inputs

EPS = 2.0 ** -53


def _rand_bits(type_name, shape, rng, scale=1.0):
    if type_name == "s8":
        return rng.integers(-128, 128, size=shape, dtype=np.int8)
    x = rng.uniform(-scale, scale, size=shape)
    return {"f16": inputs.to_f16, "bf16": inputs.to_bf16, "e4m3": inputs.to_e4m3,
            "e5m2": inputs.to_e5m2}[type_name](x)


def _int_valued_bits(type_name, shape, rng):
    x = rng.integers(-3, 4, size=shape).astype(np.float64)
    if type_name == "s8":
        return x.astype(np.int8)
    return {"f16": inputs.to_f16, "bf16": inputs.to_bf16, "e4m3": inputs.to_e4m3,
            "e5m2": inputs.to_e5m2}[type_name](x)


def test_single_16x8x16_tile_exact_rational(orc):
    """One m16n8k16 tile: 16*8*16 = 2048 products, brute force in exact
    rationals.  fp64 sum of 16 exact products + C: |Y - exact| <= 17*2^-53*S."""
    rng = np.random.default_rng(1)
    M, N, K = 16, 8, 16
    A = _rand_bits("f16", (M, K), rng)
    B = _rand_bits("f16", (N, K), rng)
    C = rng.uniform(-1, 1, size=(M, N)).astype(np.float32)
    D, Y, S = orc.gemm(A, B, C, None, M, N, K, "f16", "f16", "f32")
    ex, sab = exact_gemm(logical_a(A, "f16", M, K, False), logical_b(B, "f16", K, N, True), C)
    assert sum(1 for _ in range(M) for _ in range(N)) * K == 2048
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(Y[m, n]) - ex[m][n]) <= Fraction(17 * EPS) * sab[m][n]
            assert abs(float(S[m, n]) - float(sab[m][n])) <= 17 * EPS * float(sab[m][n])
            # fp32 output is the RNE rounding of Y
            assert D[m, n] == np.float32(Y[m, n])


def test_single_tile_integer_valued_is_exact(orc):
    rng = np.random.default_rng(2)
    M, N, K = 16, 8, 16
    A = _int_valued_bits("f16", (M, K), rng)
    B = _int_valued_bits("f16", (N, K), rng)
    C = rng.integers(-100, 100, size=(M, N)).astype(np.float32)
    D, Y, S = orc.gemm(A, B, C, None, M, N, K, "f16", "f16", "f32")
    ex, _ = exact_gemm(logical_a(A, "f16", M, K, False), logical_b(B, "f16", K, N, True), C)
    assert np.array_equal(Y, np.array([[float(v) for v in r] for r in ex]))
    assert np.array_equal(D, Y.astype(np.float32))


TYPE_PAIRS = [("f16", "f16"), ("bf16", "bf16"), ("e4m3", "e5m2"), ("e5m2", "e4m3"),
              ("e4m3", "e4m3"), ("s8", "s8")]


@pytest.mark.parametrize("a_type,b_type", TYPE_PAIRS)
@pytest.mark.parametrize("a_col,b_col", [(False, True), (False, False), (True, True), (True, False)])
@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 5, 7), (17, 9, 20)])
def test_tiny_shapes_all_layouts(orc, a_type, b_type, a_col, b_col, shape):
    M, N, K = shape
    rng = np.random.default_rng(zlib.crc32(repr((a_type, b_type, a_col, b_col, shape)).encode()))
    A = _rand_bits(a_type, (K, M) if a_col else (M, K), rng)
    B = _rand_bits(b_type, (N, K) if b_col else (K, N), rng)
    integer = a_type == "s8"
    if integer:
        C = rng.integers(-1000, 1000, size=(M, N)).astype(np.int32)
        d_type = "s32"
    else:
        C = rng.uniform(-1, 1, size=(M, N)).astype(np.float32)
        d_type = "f32"
    D, Y, S = orc.gemm(A, B, C, None, M, N, K, a_type, b_type, d_type,
                       a_col_major=a_col, b_col_major=b_col)
    a = logical_a(A, a_type, M, K, a_col)
    b = logical_b(B, b_type, K, N, b_col)
    ex, sab = exact_gemm(a, b, C)
    for m in range(M):
        for n in range(N):
            if integer:
                assert Y[m, n] == float(ex[m][n]) and D[m, n] == int(ex[m][n])
            else:
                err = abs(Fraction(Y[m, n]) - ex[m][n])
                assert err <= Fraction((K + 1) * EPS) * sab[m][n]


@pytest.mark.parametrize("a_type,b_type,one_a,one_b", [
    ("f16", "f16", 0x3C00, 0x3C00), ("bf16", "bf16", 0x3F80, 0x3F80),
    ("e4m3", "e5m2", 0x38, 0x3C), ("s8", "s8", 1, 1)])
def test_identity_gives_b_plus_c(orc, a_type, b_type, one_a, one_b):
    """A = I (M = K): D[m,n] = B[m,n] + C[m,n] exactly (fp8 1.0 = 0x38 / 0x3C)."""
    rng = np.random.default_rng(3)
    M = K = 48
    N = 40
    st = orc.STORAGE
    A = np.zeros((M, K), dtype=st[a_type])
    A[np.arange(M), np.arange(M)] = one_a
    B = _rand_bits(b_type, (N, K), rng)
    integer = a_type == "s8"
    C = (rng.integers(-1000, 1000, size=(M, N)).astype(np.int32) if integer
         else rng.uniform(-1, 1, size=(M, N)).astype(np.float32))
    D, Y, _ = orc.gemm(A, B, C, None, M, N, K, a_type, b_type, "s32" if integer else "f32")
    bl = logical_b(B, b_type, K, N, True)  # [K,N], here K == M
    expect = bl + C.astype(np.float64)
    assert np.array_equal(Y, expect)
    if integer:
        assert np.array_equal(D, expect.astype(np.int64).astype(np.int32))
    else:
        assert np.array_equal(D, expect.astype(np.float32))


@pytest.mark.parametrize("a_type,one", [("f16", 0x3C00), ("bf16", 0x3F80), ("e4m3", 0x38),
                                        ("e5m2", 0x3C), ("s8", 1)])
def test_all_ones_gives_k_plus_c(orc, a_type, one):
    M, N, K = 33, 65, 300
    st = orc.STORAGE
    A = np.full((M, K), one, dtype=st[a_type])
    B = np.full((N, K), one, dtype=st[a_type])
    rng = np.random.default_rng(4)
    integer = a_type == "s8"
    C = (rng.integers(-1000, 1000, size=(M, N)).astype(np.int32) if integer
         else rng.integers(-1000, 1000, size=(M, N)).astype(np.float32))
    D, Y, S = orc.gemm(A, B, C, None, M, N, K, a_type, a_type, "s32" if integer else "f32")
    assert np.array_equal(Y, K + C.astype(np.float64))
    assert np.array_equal(S, K + np.abs(C.astype(np.float64)))


def test_int8_extremes_no_overflow_at_k8192(orc):
    """-128*-128 summed over K = 8192 is 2^27 (plus C <= 2^20): far inside
    int32, the analogue of the page's INT4 7*7 = 49 overflow remark."""
    M, N, K = 4, 4, 8192
    A = np.full((M, K), -128, np.int8)
    B = np.full((N, K), -128, np.int8)
    C = np.array([[-(1 << 20), 0, 1 << 20, 7]] * M, dtype=np.int32)
    D, Y, _ = orc.gemm(A, B, C, None, M, N, K, "s8", "s8", "s32")
    assert np.array_equal(D, (16384 * K + C.astype(np.int64)).astype(np.int32))
    assert 16384 * K + (1 << 20) < 2 ** 31
    B2 = np.full((N, K), 127, np.int8)
    D2, _, _ = orc.gemm(A, B2, C, None, M, N, K, "s8", "s8", "s32")
    assert np.array_equal(D2, (-16256 * K + C.astype(np.int64)).astype(np.int32))


def test_int_overflow_wraps_modulo_2_32(orc):
    """Integer MMA without saturation wraps modulo 2^32 ("NVIDIA MMA", section
    "Ampere: FP16/BF16 and integer MMA baseline")."""
    K = 140000
    A = np.full((1, K), 127, np.int8)
    B = np.full((2, K), 127, np.int8)
    B[1, :] = -128
    C = np.array([[5, -5]], np.int32)
    D, Y, _ = orc.gemm(A, B, C, None, 1, 2, K, "s8", "s8", "s32")
    exact = [127 * 127 * K + 5, -127 * 128 * K - 5]
    wrapped = [((v + 2 ** 31) % 2 ** 32) - 2 ** 31 for v in exact]
    assert D.tolist() == [wrapped] and exact[0] > 2 ** 31
    assert wrapped == [-2036907291, 2019127291]
    assert Y.tolist() == [[float(w) for w in wrapped]]


def test_epilogue_scale_bias_relu_cast(orc):
    """Hand-built epilogue: acc from an integer GEMM, then alpha, bias[n],
    relu and an RNE cast, in the order scale -> bias -> activation -> cast."""
    M, N, K = 2, 4, 3
    A = inputs.to_f16(np.array([[1, 2, 3], [-1, 0, 2]], np.float64))
    B = inputs.to_f16(np.array([[1, 1, 1], [0, 1, 0], [2, 0, -1], [1, -1, 1]], np.float64))
    C = np.array([[0.5, 0, 0, 0], [0, 0, 0, -0.25]], np.float32)
    bias = np.array([1.0, -3.0, 0.125, 0.0], np.float32)
    alpha = 0.5
    # acc rows: [6, 2, -1, 2], [1, 0, -4, 1]
    acc = np.array([[6, 2, -1, 2], [1, 0, -4, 1]], np.float64)
    y = alpha * (acc + C) + bias
    z = np.where(y > 0, y, 0.0)
    for d_type, cast in [("f32", lambda v: v.astype(np.float32)),
                         ("f16", lambda v: v.astype(np.float16).view(np.uint16)),
                         ("bf16", lambda v: inputs.to_bf16(v))]:
        D, Y, _ = orc.gemm(A, B, C, bias, M, N, K, "f16", "f16", d_type, alpha=alpha, relu=True)
        assert np.array_equal(Y, z)
        assert np.array_equal(D, cast(z))
    # relu maps negatives (and -0) to +0
    D, Y, _ = orc.gemm(A, B, C, bias, M, N, K, "f16", "f16", "f32", alpha=alpha, relu=True)
    assert not np.signbit(D).any()
    D, Y, _ = orc.gemm(A, B, C, bias, M, N, K, "f16", "f16", "f32", alpha=alpha, relu=False)
    assert np.array_equal(Y, y)


def test_bf16_cast_is_single_rne_from_fp64(orc):
    """A sum whose fp64 value sits just above a bf16 tie must round up, which
    a cast through fp32 would get wrong (double rounding)."""
    # 1 + 2^-8 is a bf16 tie (bf16 ulp at 1 is 2^-7); add 2^-40
    M, N, K = 1, 1, 3
    A = inputs.to_f16(np.array([[1.0, 2.0 ** -8, 2.0 ** -20]]))
    B = inputs.to_f16(np.array([[1.0, 1.0, 2.0 ** -20]]))
    D, Y, _ = orc.gemm(A, B, None, None, M, N, K, "f16", "f16", "bf16")
    assert Y[0, 0] == 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert D[0, 0] == 0x3F81  # 1 + 2^-7: rounded up, not to the even 1.0


def test_entries_match_full(orc):
    p = inputs.dense_fp8(M=40, N=50, K=96)
    D, Y, S = orc.gemm(p["A"], p["B"], None, p["bias"], 40, 50, 96, "e4m3", "e5m2", "f16",
                       alpha=p["alpha"], relu=True)
    rng = np.random.default_rng(5)
    rows = rng.integers(0, 40, 300)
    cols = rng.integers(0, 50, 300)
    De, Ye, Se = orc.gemm_entries(p["A"], p["B"], None, p["bias"], 40, 50, 96, "e4m3", "e5m2",
                                  "f16", rows, cols, alpha=p["alpha"], relu=True)
    assert np.array_equal(De, D[rows, cols])
    assert np.array_equal(Ye, Y[rows, cols]) and np.array_equal(Se, S[rows, cols])


def _py_int_dot(A, B, m, n, K, a_col, b_col):
    """sum_k A[m,k] B[k,n] in Python integers (no numpy arithmetic)."""
    s = 0
    for k in range(K):
        a = int(A[k, m]) if a_col else int(A[m, k])
        b = int(B[n, k]) if b_col else int(B[k, n])
        s += a * b
    return s


def _wrap32(x):
    return (x + 2 ** 31) % 2 ** 32 - 2 ** 31


@pytest.mark.parametrize("a_col,b_col", [(False, True), (True, False)])
@pytest.mark.parametrize("mode", ["wrap", "saturate", "bf16", "f32_epi"])
def test_entries_s8_match_full_and_integer_sums(orc, a_col, b_col, mode):
    """The integer branch of gemm_entries (the checker of every sampled s8
    entry at full size): equal to the full oracle in D, Y and S, and to sums
    of Python integers, for s32 outputs (wrapping or saturating, the Ampere
    section's .satfinite-or-wrap rule of "NVIDIA MMA") and for the int8 ->
    float epilogue.  C near the int32 bounds makes a fifth of the entries
    leave the int32 range."""
    rng = np.random.default_rng(11)
    M, N, K = 23, 37, 320
    A = rng.integers(-128, 128, size=(K, M) if a_col else (M, K), dtype=np.int8)
    B = rng.integers(-128, 128, size=(N, K) if b_col else (K, N), dtype=np.int8)
    kw = dict(a_col_major=a_col, b_col_major=b_col)
    if mode in ("wrap", "saturate"):
        C = rng.integers(-2 ** 31, 2 ** 31, size=(M, N), dtype=np.int64)
        near = np.sign(C) * (2 ** 31 - 1 - rng.integers(0, 2 ** 15, (M, N)))
        C = np.where(rng.random((M, N)) < 0.5, near, C).astype(np.int32)
        d_type, bias, alpha, relu = "s32", None, 1.0, False
        kw["saturate"] = mode == "saturate"
    else:
        C = rng.uniform(-1e5, 1e5, size=(M, N)).astype(np.float32)
        d_type = "bf16" if mode == "bf16" else "f32"
        bias = rng.uniform(-1e3, 1e3, size=N).astype(np.float32)
        alpha, relu = 0.75, True
    D, Y, S = orc.gemm(A, B, C, bias, M, N, K, "s8", "s8", d_type, alpha=alpha, relu=relu, **kw)
    rows = np.concatenate([np.arange(M), rng.integers(0, M, 200)])
    cols = np.concatenate([np.arange(M) % N, rng.integers(0, N, 200)])
    De, Ye, Se = orc.gemm_entries(A, B, C, bias, M, N, K, "s8", "s8", d_type, rows, cols,
                                  alpha=alpha, relu=relu, **kw)
    assert np.array_equal(De, D[rows, cols])
    assert np.array_equal(Ye, Y[rows, cols]) and np.array_equal(Se, S[rows, cols])
    n_out = 0
    for i, (m, n) in enumerate(zip(rows, cols)):
        acc = _py_int_dot(A, B, m, n, K, a_col, b_col)
        sabs = sum(abs((int(A[k, m]) if a_col else int(A[m, k])) *
                       (int(B[n, k]) if b_col else int(B[k, n]))) for k in range(K))
        c = int(C[m, n]) if d_type == "s32" else Fraction(float(C[m, n]))
        assert Se[i] == float(sabs + abs(c))
        if d_type == "s32":
            t = acc + c
            n_out += not (-2 ** 31 <= t < 2 ** 31)
            want = max(-2 ** 31, min(2 ** 31 - 1, t)) if mode == "saturate" else _wrap32(t)
            assert int(De[i]) == want
        else:
            # the int32 sum (exact here) through the fp64 epilogue
            y = Fraction(alpha) * (acc + c) + Fraction(float(bias[n]))
            y = max(y, Fraction(0))
            assert Ye[i] == float(y)
    if d_type == "s32":
        assert n_out > len(rows) // 10  # the wrap / clamp is exercised


def test_entries_s8_wrap_closed_form(orc):
    """A = B = -128 everywhere: every sum is 16384 K.  At K = 131072 that is
    2^31, which wraps to -2^31 (saturates to 2^31 - 1); one K group less
    (K = 131068) stays 2^31 - 65536, in range."""
    for K, wrap, sat in [(131072, -2 ** 31, 2 ** 31 - 1), (131068, 2 ** 31 - 65536, 2 ** 31 - 65536)]:
        A = np.full((2, K), -128, np.int8)
        B = np.full((3, K), -128, np.int8)
        rows, cols = np.array([0, 1, 1]), np.array([2, 0, 1])
        for saturate, want in [(False, wrap), (True, sat)]:
            D, Y, S = orc.gemm_entries(A, B, None, None, 2, 3, K, "s8", "s8", "s32", rows, cols,
                                       saturate=saturate)
            assert (D == want).all() and (Y == want).all()
            assert (S == 16384.0 * K).all()


@pytest.mark.parametrize("d_type", ["f32", "f16", "bf16"])
def test_epilogue_f32_is_exactly_rounded(orc, d_type):
    """The fp32-semantics epilogue: fmaf(alpha, t, bias) is one RNE rounding of
    the exact alpha*t + bias; relu; then the library's RNE cast."""
    rng = np.random.default_rng(6)
    M, N = 7, 33
    T = (rng.standard_normal((M, N)) * 3).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32)
    alpha = np.float32(0.3)
    D = orc.epilogue_f32(T, float(alpha), bias, True, d_type)
    for m in range(M):
        for n in range(N):
            y = round_f32(Fraction(float(alpha)) * Fraction(float(T[m, n])) +
                          Fraction(float(bias[n])))
            z = y if y > 0 else np.float32(0.0)
            if d_type == "f32":
                ref = np.float32(z)
                assert D[m, n].view(np.uint32) == ref.view(np.uint32)
            elif d_type == "f16":
                assert D[m, n] == np.float16(z).view(np.uint16)
            else:
                ref = torch.tensor([z], dtype=torch.float32).to(torch.bfloat16)
                assert D[m, n] == ref.view(torch.int16).numpy().view(np.uint16)[0]
    # without bias the scale is a plain fp32 product
    D2 = orc.epilogue_f32(T, float(alpha), None, False, "f32")
    assert np.array_equal(D2, alpha * T)


def test_rejects_unsupported(orc):
    A = np.zeros((2, 2), np.int8)
    with pytest.raises(ValueError):
        orc.gemm(A, A, None, None, 2, 2, 2, "s8", "s8", "s32", alpha=2.0)
    with pytest.raises(ValueError):
        orc.gemm(A, np.zeros((2, 2), np.uint16), None, None, 2, 2, 2, "s8", "f16", "f32")
