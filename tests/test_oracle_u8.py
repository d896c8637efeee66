"""Pins for the oracle's unsigned 8-bit inputs.

The INT8 rows of the instruction tables on "NVIDIA MMA" (section "Ampere:
FP16/BF16 and integer MMA baseline", and its sparse INT8 row) let each of A
and B be signed or unsigned 8-bit integers, accumulating in INT32 with
wrap-around unless saturation is asked for.  Pinned here against things that
do not use the oracle: sums written out by hand, sums of Python integers,
the 255 * 255 * K boundary of the int32 range, and the 2:4 worked example of
the section "Dense and 2:4 structured sparse multiplication" with u8 values
(where 0x80 is 128, a non-zero)."""
import zlib

import numpy as np
import pytest

PAIRS = [("u8", "s8"), ("s8", "u8"), ("u8", "u8")]


def _bits(t, shape, rng):
    if t == "u8":
        return rng.integers(0, 256, size=shape, dtype=np.uint8)
    return rng.integers(-128, 128, size=shape, dtype=np.int8)


def test_u8_decodes_every_code(orc):
    codes = np.arange(256, dtype=np.uint8)
    assert np.array_equal(orc.decode("u8", codes), np.arange(256, dtype=np.float64))


def test_hand_worked_sums(orc):
    # u8 x s8: 255*-128 + 0*127 + 128*-1 + 1*100 = -32640 - 128 + 100 = -32668, + C 5
    A = np.array([[255, 0, 128, 1]], np.uint8)
    B = np.array([[-128, 127, -1, 100]], np.int8)  # stored N x K
    C = np.array([[5]], np.int32)
    D, Y, S = orc.gemm(A, B, C, None, 1, 1, 4, "u8", "s8", "s32")
    assert D[0, 0] == -32663 and Y[0, 0] == -32663
    assert S[0, 0] == 32640 + 0 + 128 + 100 + 5
    # s8 x u8, the same four products
    D, _, _ = orc.gemm(B, A, C, None, 1, 1, 4, "s8", "u8", "s32")
    assert D[0, 0] == -32663
    # u8 x u8: 255*255 + 255*2 + 1*3 + 0*200 = 65025 + 510 + 3 = 65538
    A = np.array([[255, 255, 1, 0]], np.uint8)
    B = np.array([[255, 2, 3, 200]], np.uint8)
    D, _, _ = orc.gemm(A, B, None, None, 1, 1, 4, "u8", "u8", "s32")
    assert D[0, 0] == 65538
    # 0x80 is 128 as u8 and -128 as s8
    A = np.array([[0x80]], np.uint8)
    B = np.array([[0x80]], np.uint8)
    assert orc.gemm(A, B, None, None, 1, 1, 1, "u8", "u8", "s32")[0][0, 0] == 16384
    assert orc.gemm(A, B.view(np.int8), None, None, 1, 1, 1, "u8", "s8", "s32")[0][0, 0] == -16384


@pytest.mark.parametrize("a_type,b_type", PAIRS)
@pytest.mark.parametrize("a_col,b_col", [(False, True), (False, False), (True, True), (True, False)])
@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 5, 7), (17, 9, 20)])
def test_python_int_brute_force(orc, a_type, b_type, a_col, b_col, shape):
    M, N, K = shape
    rng = np.random.default_rng(zlib.crc32(repr((a_type, b_type, a_col, b_col, shape)).encode()))
    A = _bits(a_type, (K, M) if a_col else (M, K), rng)
    B = _bits(b_type, (N, K) if b_col else (K, N), rng)
    C = rng.integers(-1000, 1000, size=(M, N)).astype(np.int32)
    D, Y, S = orc.gemm(A, B, C, None, M, N, K, a_type, b_type, "s32",
                       a_col_major=a_col, b_col_major=b_col)
    for m in range(M):
        for n in range(N):
            s, sa = 0, 0
            for k in range(K):
                a = int(A[k, m] if a_col else A[m, k])
                b = int(B[n, k] if b_col else B[k, n])
                s += a * b
                sa += abs(a * b)
            assert int(D[m, n]) == s + int(C[m, n]) and Y[m, n] == s + int(C[m, n])
            assert S[m, n] == sa + abs(int(C[m, n]))


def _wrap32(x):
    return (x + 2 ** 31) % 2 ** 32 - 2 ** 31


def test_u8_u8_int32_range_boundary(orc):
    """255 * 255 = 65025 per product: K = 33025 gives 2147450625, still below
    2^31; one more K (33026) gives 2147515650, which wraps (or, saturating,
    clamps to 2^31 - 1)."""
    for K, fits in [(33025, True), (33026, False)]:
        A = np.full((1, K), 255, np.uint8)
        B = np.full((2, K), 255, np.uint8)
        exact = 65025 * K
        assert (exact < 2 ** 31) == fits
        D, Y, _ = orc.gemm(A, B, None, None, 1, 2, K, "u8", "u8", "s32")
        assert (D == _wrap32(exact)).all() and (Y == _wrap32(exact)).all()
        D, _, _ = orc.gemm(A, B, None, None, 1, 2, K, "u8", "u8", "s32", saturate=True)
        assert (D == min(exact, 2 ** 31 - 1)).all()
    # the most negative u8 x s8 sum: 255 * -128 per product
    K = 65794  # 32640 * 65794 = 2147516160 > 2^31
    A = np.full((1, K), 255, np.uint8)
    B = np.full((1, K), -128, np.int8)
    D, _, _ = orc.gemm(A, B, None, None, 1, 1, K, "u8", "s8", "s32")
    assert D[0, 0] == _wrap32(-32640 * K) and -32640 * K < -2 ** 31


@pytest.mark.parametrize("a_type,b_type", PAIRS)
def test_float_epilogue_of_unsigned_sums(orc, a_type, b_type):
    """The int8 -> float epilogue applies to u8 inputs the same way: the
    int32 sum (exact here), then C, scale, bias, relu in fp64 and one cast."""
    rng = np.random.default_rng(3)
    M, N, K = 5, 6, 40
    A = _bits(a_type, (M, K), rng)
    B = _bits(b_type, (N, K), rng)
    C = rng.uniform(-1e4, 1e4, (M, N)).astype(np.float32)
    bias = rng.uniform(-1e3, 1e3, N).astype(np.float32)
    D, Y, _ = orc.gemm(A, B, C, bias, M, N, K, a_type, b_type, "f32", alpha=0.25, relu=True)
    for m in range(M):
        for n in range(N):
            s = sum(int(A[m, k]) * int(B[n, k]) for k in range(K))
            y = 0.25 * (s + float(C[m, n])) + float(bias[n])
            assert Y[m, n] == max(y, 0.0)
            assert D[m, n] == np.float32(Y[m, n])


def test_u8_rejects_float_pairing(orc):
    A = np.zeros((2, 2), np.uint8)
    with pytest.raises(ValueError):
        orc.gemm(A, np.zeros((2, 2), np.uint16), None, None, 2, 2, 2, "u8", "f16", "f32")


def test_sparse24_u8_worked_example_and_zero(orc):
    """[7, 0, 0, 200] -> values [7, 200], positions [0, 3] (nibble 0xC); the
    u8 code 0x80 (= 128) is a non-zero, unlike for a float format."""
    A = np.array([[7, 0, 0, 200, 0, 0x80, 0, 0]], np.uint8)
    vals, meta = orc.sparse24_compress(A, "u8")
    # second group: 0x80 at position 1 kept, position 0 (the lowest free one)
    # fills the pair, in ascending order
    assert vals.tolist() == [[7, 200, 0, 0x80]]
    assert int(meta[0, 0]) == 0xC | ((0 | (1 << 2)) << 4)
    assert np.array_equal(orc.sparse24_decompress(vals, meta, 1, 8, "u8"), A)
    with pytest.raises(orc.NotSparse24):
        orc.sparse24_compress(np.array([[1, 2, 3, 0]], np.uint8), "u8")


@pytest.mark.parametrize("b_type", ["s8", "u8"])
def test_sparse24_u8_product_equals_dense(orc, b_type):
    """The 2:4 path multiplies the decompressed A: with u8 A it equals the
    dense oracle on the logical A, and a Python-integer sum."""
    rng = np.random.default_rng(9)
    M, N, K = 6, 7, 64
    A = rng.integers(1, 256, size=(M, K), dtype=np.uint8)
    for g in range(K // 4):
        drop = rng.choice(4, 2, replace=False)
        A[:, 4 * g + drop] = 0
    vals, meta = orc.sparse24_compress(A, "u8")
    Al = orc.sparse24_decompress(vals, meta, M, K, "u8")
    assert np.array_equal(Al, A)
    B = _bits(b_type, (N, K), rng)
    D, _, _ = orc.gemm(Al, B, None, None, M, N, K, "u8", b_type, "s32")
    for m in range(M):
        for n in range(N):
            assert D[m, n] == sum(int(A[m, k]) * int(B[n, k]) for k in range(K))
