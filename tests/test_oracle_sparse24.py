"""Pins for the oracle's 2:4 compressor/decompressor and its sparse path.

The format is "NVIDIA MMA", section "Dense and 2:4 structured sparse
multiplication": along K every 4 consecutive positions of A keep 2 values plus
their positions; only A is compressed.  The ordered-metadata remark of the
section "Ampere: FP16/BF16 and integer MMA baseline" requires ascending
positions.  The nibble packing (i0 | i1 << 2, 8 groups per little-endian u32)
is this library's reading; the pages fix no bit layout."""
import itertools
import os

import numpy as np
import pytest

from sparse_tiled_gemm_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sparse24_worked_example.txt")


def _read_golden():
    rows = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            rows[key.strip()] = val.split()
    return rows


def test_worked_example_from_the_page(orc):
    g = _read_golden()
    subst = {"a0": 1.5, "a3": -2.25, "0": 0.0}
    logical = np.array([[subst[t] for t in g["logical"]]])
    A = inputs.to_f16(logical)
    values, meta = orc.sparse24_compress(A)
    assert inputs.f16_values(values).tolist() == [[subst[t] for t in g["values"]]]
    pos = [int(t) for t in g["positions"]]
    nib = int(meta[0, 0]) & 0xF
    assert [nib & 3, nib >> 2] == pos
    assert nib == 0xC  # positions 0 and 3 in this library's packing
    assert np.array_equal(orc.sparse24_decompress(values, meta, 1, 4), A)


def test_every_zero_pattern_of_a_group(orc):
    """All 16 zero/non-zero patterns of one group of 4."""
    for mask in range(16):
        nz = [i for i in range(4) if mask >> i & 1]
        logical = np.array([[float(i + 1) if i in nz else 0.0 for i in range(4)]])
        A = inputs.to_f16(logical)
        if len(nz) > 2:
            with pytest.raises(orc.NotSparse24):
                orc.sparse24_compress(A)
            continue
        values, meta = orc.sparse24_compress(A)
        nib = int(meta[0, 0])
        i0, i1 = nib & 3, nib >> 2
        assert i0 < i1 and meta[0, 0] < 16
        kept = sorted(set(nz) | set([p for p in range(4) if p not in nz][:2 - len(nz)]))
        assert [i0, i1] == kept  # non-zeros first, then the lowest free positions
        assert np.array_equal(orc.sparse24_decompress(values, meta, 1, 4), A)


def test_negative_zero_counts_as_zero_and_nan_as_nonzero(orc):
    A = np.array([[0x8000, 0x3C00, 0x8000, 0x4000]], np.uint16)  # -0, 1, -0, 2
    values, meta = orc.sparse24_compress(A)
    assert int(meta[0, 0]) == (1 | 3 << 2)
    A2 = np.array([[0x7E00, 0x3C00, 0x0000, 0x4000]], np.uint16)  # NaN, 1, 0, 2
    with pytest.raises(orc.NotSparse24):
        orc.sparse24_compress(A2)


@pytest.mark.parametrize("M,K", [(1, 4), (3, 36), (17, 128), (64, 1000)])
def test_round_trip_and_ascending(orc, M, K):
    p = inputs.sparse24_f16(M=M, N=8, K=K)
    A = p["A_logical"]
    values, meta = orc.sparse24_compress(A)
    assert values.shape == (M, K // 2) and meta.shape == (M, (K + 31) // 32)
    assert np.array_equal(orc.sparse24_decompress(values, meta, M, K), A)
    G = K // 4
    for m in range(M):
        for g in range(G):
            nib = (int(meta[m, g // 8]) >> (4 * (g % 8))) & 0xF
            assert (nib & 3) < (nib >> 2)
        # nibbles past the last group are zero
        if G % 8:
            assert int(meta[m, -1]) >> (4 * (G % 8)) == 0
    # the generator draws no exact zero among kept values, so the positions
    # are exactly the generator's non-zero positions
    nz = (A.reshape(M, G, 4) & 0x7FFF) != 0
    assert (nz.sum(-1) == 2).all()


def test_decompress_rejects_non_ascending(orc):
    values = np.zeros((1, 2), np.uint16)
    for nib in [0x0, 0x5, 0xF, 0x3, 0x6]:  # (0,0) (1,1) (3,3) (3,0) (2,1)
        with pytest.raises(ValueError):
            orc.sparse24_decompress(values, np.array([[nib]], np.uint32), 1, 4)


def test_sparse_gemm_equals_dense_gemm_on_logical_a(orc):
    """Zeros add exactly 0 in fp64, so GEMM on decompress(compress(A)) equals
    GEMM on A bit for bit."""
    M, N, K = 24, 40, 72
    p = inputs.sparse24_f16(M=M, N=N, K=K)
    values, meta = orc.sparse24_compress(p["A_logical"])
    A2 = orc.sparse24_decompress(values, meta, M, K)
    D1, Y1, S1 = orc.gemm(p["A_logical"], p["B"], p["C"], None, M, N, K, "f16", "f16", "f32")
    D2, Y2, S2 = orc.gemm(A2, p["B"], p["C"], None, M, N, K, "f16", "f16", "f32")
    assert np.array_equal(Y1, Y2) and np.array_equal(D1, D2) and np.array_equal(S1, S2)


def test_generator_pattern_is_uniform_over_the_six_pairs():
    p = inputs.sparse24_f16(M=256, N=1, K=256)
    nz = (p["A_logical"].reshape(256, 64, 4) & 0x7FFF) != 0
    codes = nz[..., 0] * 1 + nz[..., 1] * 2 + nz[..., 2] * 4 + nz[..., 3] * 8
    counts = np.bincount(codes.reshape(-1), minlength=16)
    pairs = [a | b for a, b in itertools.combinations([1, 2, 4, 8], 2)]
    assert counts[pairs].sum() == 256 * 64
    assert (np.abs(counts[pairs] / (256 * 64) - 1 / 6) < 0.02).all()


# ---------------------------------------------------------------- other types
# The sparse rows of the instruction tables on "NVIDIA MMA" (sections
# "Ampere: FP16/BF16 and integer MMA baseline" and "Ada: mma.sync adds FP8")
# apply the same 2:4 format to BF16, INT8 and FP8 E4M3/E5M2 A.  Encodings
# here come from numpy / torch conversions, not from the oracle.

def _enc(t, x):
    x = np.asarray(x, dtype=np.float64)
    if t == "s8":
        return x.astype(np.int8)
    return {"f16": inputs.to_f16, "bf16": inputs.to_bf16, "e4m3": inputs.to_e4m3,
            "e5m2": inputs.to_e5m2}[t](x)


# a0, a3 of the worked example: values every format holds exactly
_A0A3 = {"f16": (1.5, -2.25), "bf16": (1.5, -2.25), "e4m3": (1.5, -2.25), "e5m2": (1.5, -3.0),
         "s8": (3, -7)}
TYPES = ["f16", "bf16", "e4m3", "e5m2", "s8"]


@pytest.mark.parametrize("t", TYPES)
def test_worked_example_every_type(orc, t):
    a0, a3 = _A0A3[t]
    A = _enc(t, [[a0, 0, 0, a3]])
    values, meta = orc.sparse24_compress(A, t)
    assert values.dtype == A.dtype and values.shape == (1, 2)
    assert values.tolist() == _enc(t, [[a0, a3]]).tolist()
    assert int(meta[0, 0]) == 0xC  # positions 0 and 3
    assert np.array_equal(orc.sparse24_decompress(values, meta, 1, 4, t), A)


@pytest.mark.parametrize("t", TYPES)
def test_every_zero_pattern_every_type(orc, t):
    for mask in range(16):
        nz = [i for i in range(4) if mask >> i & 1]
        A = _enc(t, [[float(i + 1) if i in nz else 0.0 for i in range(4)]])
        if len(nz) > 2:
            with pytest.raises(orc.NotSparse24):
                orc.sparse24_compress(A, t)
            continue
        values, meta = orc.sparse24_compress(A, t)
        nib = int(meta[0, 0])
        kept = sorted(set(nz) | set([p for p in range(4) if p not in nz][:2 - len(nz)]))
        assert [nib & 3, nib >> 2] == kept
        assert np.array_equal(orc.sparse24_decompress(values, meta, 1, 4, t), A)


def test_zero_codes_of_the_8_bit_formats(orc):
    # fp8: 0x80 is -0, a zero; 0x7F (E4M3 NaN) and 0x7C (E5M2 +inf) are not
    for t in ("e4m3", "e5m2"):
        A = np.array([[0x80, 0x38, 0x80, 0x40]], np.uint8)
        _, meta = orc.sparse24_compress(A, t)
        assert int(meta[0, 0]) == (1 | 3 << 2)
    with pytest.raises(orc.NotSparse24):
        orc.sparse24_compress(np.array([[0x7F, 0x38, 0x00, 0x40]], np.uint8), "e4m3")
    with pytest.raises(orc.NotSparse24):
        orc.sparse24_compress(np.array([[0x7C, 0x3C, 0x00, 0x40]], np.uint8), "e5m2")
    # s8: 0x80 is -128, a non-zero
    A = np.array([[-128, 0, 0, 7]], np.int8)
    values, meta = orc.sparse24_compress(A, "s8")
    assert int(meta[0, 0]) == (0 | 3 << 2) and values.tolist() == [[-128, 7]]
    with pytest.raises(orc.NotSparse24):
        orc.sparse24_compress(np.array([[-128, 5, -128, 0]], np.int8), "s8")


@pytest.mark.parametrize("t", ["bf16", "e4m3", "e5m2", "s8"])
@pytest.mark.parametrize("M,K", [(1, 4), (5, 68), (33, 256)])
def test_round_trip_every_type(orc, t, M, K):
    p = inputs.sparse24(t, M, 8, K)
    A = p["A_logical"]
    values, meta = orc.sparse24_compress(A, t)
    assert values.shape == (M, K // 2) and values.dtype == A.dtype
    assert np.array_equal(orc.sparse24_decompress(values, meta, M, K, t), A)
    # exactly the generator's pattern: two non-zeros per group, ascending
    mask = 0x7FFF if A.itemsize == 2 else (0xFF if t == "s8" else 0x7F)
    nz = (A.view(np.uint16 if A.itemsize == 2 else np.uint8).reshape(M, K // 4, 4) & mask) != 0
    assert (nz.sum(-1) == 2).all()
    G = K // 4
    for m in range(M):
        for g in range(G):
            nib = (int(meta[m, g // 8]) >> (4 * (g % 8))) & 0xF
            where = np.nonzero(nz[m, g])[0].tolist()
            assert [nib & 3, nib >> 2] == where


@pytest.mark.parametrize("t", ["bf16", "e4m3", "e5m2", "s8"])
def test_sparse_gemm_equals_dense_gemm_every_type(orc, t):
    M, N, K = 20, 24, 72
    p = inputs.sparse24(t, M, N, K)
    values, meta = orc.sparse24_compress(p["A_logical"], t)
    A2 = orc.sparse24_decompress(values, meta, M, K, t)
    args = dict(alpha=p["alpha"], relu=p["relu"])
    D1, Y1, S1 = orc.gemm(p["A_logical"], p["B"], p["C"], p["bias"], M, N, K, p["a_type"],
                          p["b_type"], p["d_type"], **args)
    D2, Y2, S2 = orc.gemm(A2, p["B"], p["C"], p["bias"], M, N, K, p["a_type"], p["b_type"],
                          p["d_type"], **args)
    assert np.array_equal(Y1, Y2) and np.array_equal(D1, D2) and np.array_equal(S1, S2)


def test_s8_sparse_product_by_hand(orc):
    """A 1 x 8 by 8 x 1 2:4 product summed by hand in Python integers."""
    A = np.array([[0, 5, 0, -3, -128, 0, 0, 127]], np.int8)
    B = np.array([[1, 2, 3, 4, 5, 6, 7, 8]], np.int8)  # stored [N, K]
    values, meta = orc.sparse24_compress(A, "s8")
    assert values.tolist() == [[5, -3, -128, 127]]
    assert int(meta[0, 0]) == (1 | 3 << 2) | ((0 | 3 << 2) << 4)
    D, _, _ = orc.gemm(orc.sparse24_decompress(values, meta, 1, 8, "s8"), B,
                       np.array([[10]], np.int32), None, 1, 1, 8, "s8", "s8", "s32")
    assert int(D[0, 0]) == 5 * 2 - 3 * 4 - 128 * 5 + 127 * 8 + 10
