"""Pins for the oracle's element codecs: every code of each 8/16-bit input
format against numpy/torch's own conversions and against closed-form values,
and the round-to-nearest-even output casts against library conversions and
the round-half-even bit method."""
import numpy as np
import pytest
import torch

from sparse_tiled_gemm_amd import inputs


def _torch_decode(bits, dtype):
    t = torch.from_numpy(np.ascontiguousarray(bits))
    return t.view(dtype).to(torch.float32).numpy().astype(np.float64)


def test_f16_decode_all_codes(orc):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.decode("f16", bits)
    ref = bits.view(np.float16).astype(np.float64)
    assert np.array_equal(got, ref, equal_nan=True)


def test_bf16_decode_all_codes(orc):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.decode("bf16", bits)
    ref = _torch_decode(bits.view(np.int16), torch.bfloat16)
    assert np.array_equal(got, ref, equal_nan=True)


@pytest.mark.parametrize("name,tdtype", [("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)])
def test_fp8_decode_all_codes(orc, name, tdtype):
    bits = np.arange(256, dtype=np.uint16).astype(np.uint8)
    got = orc.decode(name, bits)
    ref = _torch_decode(bits, tdtype)
    assert np.array_equal(got, ref, equal_nan=True)


def test_fp8_closed_forms(orc):
    e4 = lambda b: float(orc.decode("e4m3", np.array([b], np.uint8))[0])
    e5 = lambda b: float(orc.decode("e5m2", np.array([b], np.uint8))[0])
    # OCP E4M3: max normal S.1111.110 = 1.75 * 2^8, one = 0.0111.000, smallest subnormal 2^-9
    assert e4(0x7E) == 448.0 and e4(0xFE) == -448.0
    assert e4(0x38) == 1.0 and e4(0x01) == 2.0 ** -9 and e4(0x08) == 2.0 ** -6
    assert np.isnan(e4(0x7F)) and np.isnan(e4(0xFF))
    assert e4(0x80) == 0.0 and np.signbit(e4(0x80))
    # OCP E5M2: max normal 1.75 * 2^15, one = 0.01111.00, smallest subnormal 2^-16, inf 0x7C
    assert e5(0x7B) == 57344.0 and e5(0x3C) == 1.0 and e5(0x01) == 2.0 ** -16
    assert e5(0x7C) == np.inf and e5(0xFC) == -np.inf and np.isnan(e5(0x7D))


def _f16_grid_samples(rng):
    """Doubles that exercise f16 rounding: random values over the whole
    range, exact midpoints between neighbours (ties), subnormals, overflow."""
    h = np.arange(0, 0x7C00, dtype=np.uint16)
    v = h.view(np.float16).astype(np.float64)
    mids = (v[:-1] + v[1:]) / 2.0  # exact in fp64
    near = np.concatenate([np.nextafter(mids, 0), np.nextafter(mids, 1e9)])
    rnd = rng.uniform(-70000, 70000, size=200000)
    small = rng.uniform(-2 ** -13, 2 ** -13, size=100000)
    edge = np.array([65504.0, 65519.99, 65520.0, 65536.0, 1e9, 2 ** -25, 2 ** -25 * 1.0000001,
                     3 * 2 ** -26, 0.0, -0.0, np.inf, -np.inf])
    x = np.concatenate([v, mids, near, rnd, small, edge])
    return np.concatenate([x, -x])


def test_f16_encode_matches_numpy(orc):
    x = _f16_grid_samples(np.random.default_rng(11))
    got = orc.encode("f16", x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def _bf16_rne_bits(f32):
    """Round-half-even of fp32 bit patterns to their upper 16 bits
    (the classic integer method); NaNs excluded by the caller."""
    u = f32.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def test_bf16_encode_matches_bit_method_and_torch(orc):
    rng = np.random.default_rng(12)
    u = rng.integers(0, 1 << 32, size=3_000_000, dtype=np.uint64).astype(np.uint32)
    # all tie cases and their neighbours around a sweep of exponents
    hi = rng.integers(0, 1 << 16, size=200000, dtype=np.uint32) << 16
    ties = np.concatenate([hi | 0x8000, hi | 0x7FFF, hi | 0x8001])
    u = np.concatenate([u, ties, np.array([0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0x00000001,
                                           0x00008000, 0x00018000, 0x80008000], np.uint32)])
    f = u.view(np.float32)
    f = f[~np.isnan(f)]
    got = orc.encode("bf16", f.astype(np.float64))
    assert np.array_equal(got, _bf16_rne_bits(f))
    ref_t = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref_t)


def test_f32_encode_matches_numpy(orc):
    rng = np.random.default_rng(13)
    x = np.concatenate([rng.standard_normal(500000) * 10.0 ** rng.integers(-40, 40, 500000),
                        np.array([3.4028235677973366e38, 3.4028235e38 * 1.0000001, 1e-46, 0.0])])
    x = np.concatenate([x, -x])
    got = orc.encode("f32", x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_s32_encode_wraps(orc):
    x = np.array([0, 1, -1, 2 ** 31 - 1, 2 ** 31, -2 ** 31, -2 ** 31 - 1, 2 ** 32 + 5], np.float64)
    got = orc.encode("s32", x)
    assert got.tolist() == [0, 1, -1, 2 ** 31 - 1, -2 ** 31, -2 ** 31, 2 ** 31 - 1, 5]


# ---------------------------------------------------------------- fp8 outputs
# FP8 outputs round to nearest even and saturate at the largest finite value
# (E4M3 has no infinity; the reading is the satfinite conversion).  Within
# range the result must equal torch's own conversion.

@pytest.mark.parametrize("t,maxv", [("e4m3", 448.0), ("e5m2", 57344.0)])
def test_fp8_output_encode_against_torch_and_saturation(orc, t, maxv):
    rng = np.random.default_rng(8)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 1.0, 30.0, maxv / 4)])
    x = x[np.abs(x) <= maxv]
    ours = orc.encode(t, x)
    tt = torch.float8_e4m3fn if t == "e4m3" else torch.float8_e5m2
    ref = torch.from_numpy(x.astype(np.float32)).to(tt).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    # beyond the range: +-max, also past the rounding boundary and at infinity
    big = np.array([maxv * 1.01, maxv * 3, 1e30, np.inf, -maxv * 1.5, -np.inf])
    dec = orc.decode(t, orc.encode(t, big))
    assert dec.tolist() == [maxv, maxv, maxv, maxv, -maxv, -maxv]
    assert orc.encode(t, np.array([np.nan]))[0] == 0x7F


def test_s8_float_output_is_the_wrapped_int32_sum(orc):
    """int8 -> float: the int32 accumulator (wrapping modulo 2^32) as a value,
    then C and the float epilogue."""
    M, N, K = 2, 3, 70000  # 127*127*70000 > 2^31: the sum wraps
    A = np.full((M, K), 127, np.int8)
    B = np.full((N, K), 127, np.int8)
    C = np.full((M, N), 0.5, np.float32)
    D, Y, S = orc.gemm(A, B, C, None, M, N, K, "s8", "s8", "f32")
    wrapped = ((127 * 127 * K + 2 ** 31) % 2 ** 32) - 2 ** 31
    assert np.all(Y == wrapped + 0.5)
    D2, Y2, _ = orc.gemm(A[:, :8], B[:, :8], None, None, M, N, 8, "s8", "s8", "bf16", alpha=0.25)
    assert np.all(Y2 == 127 * 127 * 8 * 0.25)


def test_s32_saturation_clamps_the_exact_sum(orc):
    """The saturating int32 output ("NVIDIA MMA", section "Ampere: FP16/BF16
    and integer MMA baseline": integer MMA saturates to the INT32 bounds with
    .satfinite, else wraps): D = clamp(sum_k a b + c, -2^31, 2^31 - 1), the
    expected values worked out by hand.  Row 0: 4 * (127 * 127) = 64516 on top
    of c = 2^31 - 10000 -> clamps to 2^31 - 1 (wrapping gives
    -2^31 + 54516).  Row 1: 4 * (-128 * 127) = -65024 below c = -2^31 + 5 ->
    clamps to -2^31 (wraps to 2^31 - 65019).  Row 2: in range, identical to
    wrapping."""
    A = np.array([[127] * 4, [-128] * 4, [3, -2, 1, 0]], dtype=np.int8)
    B = np.array([[127, 127, 127, 127]], dtype=np.int8)  # N x K (column-major)
    C = np.array([[2**31 - 10000], [-(2**31) + 5], [7]], dtype=np.int32)
    D, _, _ = orc.gemm(A, B, C, None, 3, 1, 4, "s8", "s8", "s32", saturate=True)
    assert D[:, 0].tolist() == [2**31 - 1, -(2**31), 3 * 127 - 2 * 127 + 127 + 7]
    W, _, _ = orc.gemm(A, B, C, None, 3, 1, 4, "s8", "s8", "s32")
    assert W[:, 0].tolist() == [-(2**31) + 54516, 2**31 - 65019, 3 * 127 - 2 * 127 + 127 + 7]
    with pytest.raises(ValueError):  # saturation is an int32-output option
        orc.gemm(A.astype(np.int8), B, C.astype(np.float32), None, 3, 1, 4, "s8", "s8", "f32",
                 saturate=True)


@pytest.mark.parametrize("ct", ["f16", "bf16"])
def test_16bit_c_is_its_exact_widening(orc, ct):
    """A 16-bit C enters as its exact value: the result equals the fp32-C
    result on the widened values (every f16 / bf16 value is an fp32 value)."""
    rng = np.random.default_rng(8)
    M, N, K = 5, 7, 16
    A = inputs.to_bf16(rng.standard_normal((M, K)))
    B = inputs.to_bf16(rng.standard_normal((N, K)))
    conv = inputs.to_f16 if ct == "f16" else inputs.to_bf16
    C16 = conv(rng.uniform(-3, 3, (M, N)) * 2.0 ** rng.integers(-20, 10, (M, N)))
    C32 = orc.decode(ct, C16).astype(np.float32).reshape(M, N)
    D16, Y16, _ = orc.gemm(A, B, C16, None, M, N, K, "bf16", "bf16", "f32", c_type=ct)
    D32, Y32, _ = orc.gemm(A, B, C32, None, M, N, K, "bf16", "bf16", "f32")
    assert np.array_equal(D16.view(np.uint32), D32.view(np.uint32))
    assert np.array_equal(Y16, Y32)
