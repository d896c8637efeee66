"""Pins for the oracle's MX block-scaled GEMM and its narrow formats.

"NVIDIA MMA", section "Blackwell: FP4/FP6 and block-scaled MMA": the
block-scaled product is D = C + sum_g (A_g S_A,g)(B_g S_B,g), each scale
applied to its K block's partial sum; the "MXFP4 and NVFP4" table gives
UE8M0 scales over 32 K elements.  The element formats (E2M1, E2M3, E3M2,
and the fp8 ones) and UE8M0 are the OCP Microscaling formats the page names;
the values below are that specification's, not the oracle's own tables."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from sparse_tiled_gemm_amd import inputs


def _codes_values(orc, fmt, n):
    codes = np.arange(n, dtype=np.uint8)
    return orc.decode_packed(fmt, inputs.mx_pack(codes.reshape(1, -1), fmt), n)


def test_e2m1_every_code(orc):
    v = _codes_values(orc, "e2m1", 16)
    pos = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert v[:8].tolist() == pos
    assert v[8:].tolist() == [-x for x in pos]


@pytest.mark.parametrize("fmt,vmax,min_normal,min_sub", [("e2m3", 7.5, 1.0, 0.125),
                                                          ("e3m2", 28.0, 0.25, 0.0625)])
def test_fp6_formats(orc, fmt, vmax, min_normal, min_sub):
    v = _codes_values(orc, fmt, 64)
    pos, neg = v[:32], v[32:]
    assert pos[0] == 0.0 and neg[0] == 0.0 and np.array_equal(neg, -pos)
    assert np.all(np.diff(pos) > 0)                 # codes order the values
    assert pos[-1] == vmax and pos[1] == min_sub
    fb = 3 if fmt == "e2m3" else 2
    assert pos[1 << fb] == min_normal               # first normal code
    assert np.all(np.mod(pos / min_sub, 1) == 0)   # all on the subnormal grid
    # constant spacing within each binade: 2^fb values per binade
    for e in range(1, 1 << (5 - fb)):
        seg = pos[e << fb:(e + 1) << fb]
        assert len(set(np.diff(seg).tolist())) <= 1


def test_e8m0_against_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.decode_packed("e8m0", codes, 256)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255])


def test_packing_reading(orc):
    # E2M1: two per byte, the even element in the low nibble
    assert orc.decode_packed("e2m1", np.array([0x21, 0x9F], np.uint8), 4).tolist() == \
        [0.5, 1.0, -6.0, -0.5]
    # 6-bit: little-endian bit string, element i in bits 6i .. 6i+5
    w = 1 | (2 << 6) | (3 << 12) | (63 << 18)
    b = np.array([w & 0xFF, (w >> 8) & 0xFF, w >> 16], np.uint8)
    assert orc.decode_packed("e2m3", b, 4).tolist() == [0.125, 0.25, 0.375, -7.5]
    assert np.array_equal(inputs.mx_pack(np.array([[1, 2, 3, 63]]), "e2m3")[0], b)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2", "e2m3", "e3m2", "e2m1"])
def test_generator_encoder_rounds_to_nearest(orc, fmt):
    """The generator's encoder against the oracle's decoder: every value
    lands on the nearest representable one (two separate implementations)."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal(4000) * {"e4m3": 100, "e5m2": 5000, "e2m3": 3, "e3m2": 10,
                                     "e2m1": 2}[fmt]
    codes = inputs.mx_encode(x, fmt)
    got = orc.decode_packed(fmt, inputs.mx_pack(codes.reshape(1, -1), fmt), x.size)
    n = 1 << inputs.MX_BITS[fmt]
    allv = orc.decode_packed(fmt, inputs.mx_pack(np.arange(n, dtype=np.uint8).reshape(1, -1), fmt),
                             n)
    allv = allv[np.isfinite(allv)]
    vmax = np.abs(allv).max()
    clipped = np.clip(x, -vmax, vmax)
    best = np.abs(clipped[:, None] - allv[None, :]).min(1)
    assert np.array_equal(np.abs(got - clipped), best)


def _problem(a_type, b_type, M, N, K, seed):
    return inputs.mx_problem(M, N, K, a_type, b_type, workload=seed, d_type="f32")


def test_unit_scales_equal_the_plain_gemm(orc):
    M, N, K = 12, 20, 128
    p = _problem("e4m3", "e4m3", M, N, K, 30)
    ones_a = np.full_like(p["SA"], 127)
    ones_b = np.full_like(p["SB"], 127)
    C = np.random.default_rng(2).uniform(-1, 1, (M, N)).astype(np.float32)
    D1, Y1, S1 = orc.mx_gemm(p["A"], ones_a, p["B"], ones_b, C, None, M, N, K, "e4m3", "e4m3",
                             "f32")
    D2, Y2, S2 = orc.gemm(p["A"], p["B"], C, None, M, N, K, "e4m3", "e4m3", "f32")
    assert np.array_equal(Y1, Y2) and np.array_equal(S1, S2) and np.array_equal(D1, D2)


def test_brute_force_fractions_fp4_x_fp6(orc):
    """Exact rational sum from the generator's own value tables."""
    M, N, K = 2, 3, 64
    rng = np.random.default_rng(5)
    ca = rng.integers(0, 16, (M, K)).astype(np.uint8)
    cb = rng.integers(0, 64, (N, K)).astype(np.uint8)
    SA = rng.integers(120, 135, (M, K // 32)).astype(np.uint8)
    SB = rng.integers(120, 135, (N, K // 32)).astype(np.uint8)
    _, Y, _ = orc.mx_gemm(inputs.mx_pack(ca, "e2m1"), SA, inputs.mx_pack(cb, "e2m3"), SB, None,
                          None, M, N, K, "e2m1", "e2m3", "f32")

    def table(fmt):
        v, c = inputs._mx_grid(fmt)
        t = {}
        sbit = 1 << (inputs.MX_BITS[fmt] - 1)
        for val, code in zip(v, c):
            t[int(code)] = Fraction(val)
            t[int(code) | sbit] = -Fraction(val)
        return t
    ta, tb = table("e2m1"), table("e2m3")
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for g in range(K // 32):
                part = sum(ta[int(ca[m, k])] * tb[int(cb[n, k])] for k in range(32 * g, 32 * g + 32))
                tot += part * Fraction(2) ** (int(SA[m, g]) - 127) * Fraction(2) ** (int(SB[n, g]) - 127)
            assert Y[m, n] == float(tot)


def test_a_scale_acts_on_its_block_only(orc):
    """Raising SA[m, g] by one adds exactly block g's contribution to row m."""
    M, N, K = 4, 6, 128
    p = _problem("e2m1", "e4m3", M, N, K, 31)
    args = ("e2m1", "e4m3", "f32")
    _, Y, _ = orc.mx_gemm(p["A"], p["SA"], p["B"], p["SB"], None, None, M, N, K, *args)
    m, g = 2, 1
    SA2 = p["SA"].copy()
    SA2[m, g] += 1
    _, Y2, _ = orc.mx_gemm(p["A"], SA2, p["B"], p["SB"], None, None, M, N, K, *args)
    # block g alone: zero every other block of A (code 0 is +0)
    codes = np.zeros((M, K), np.uint8)
    unpacked = np.stack([p["A"] & 0xF, p["A"] >> 4], -1).reshape(M, K)
    codes[:, 32 * g:32 * g + 32] = unpacked[:, 32 * g:32 * g + 32]
    _, Yg, _ = orc.mx_gemm(inputs.mx_pack(codes, "e2m1"), p["SA"], p["B"], p["SB"], None, None,
                           M, N, K, *args)
    assert np.array_equal(np.delete(Y2, m, 0), np.delete(Y, m, 0))
    assert np.allclose(Y2[m] - Y[m], Yg[m], rtol=0, atol=1e-12 * np.abs(Y).max())
    assert np.any(Yg[m] != 0)


def test_nan_scale_gives_nan_row(orc):
    M, N, K = 3, 4, 64
    p = _problem("e4m3", "e5m2", M, N, K, 32)
    SA = p["SA"].copy()
    SA[1, 0] = 0xFF
    _, Y, _ = orc.mx_gemm(p["A"], SA, p["B"], p["SB"], None, None, M, N, K, "e4m3", "e5m2", "f32")
    assert np.isnan(Y[1]).all() and np.isfinite(Y[[0, 2]]).all()


def test_generator_recipe(orc):
    """Each block's largest element lands in the format's top binade (the MX
    shared-exponent rule) and the scales reproduce the data to the format's
    precision."""
    M, K = 64, 256
    p = inputs.mx_problem(M, 8, K, "e2m1", "e2m1", workload=33)
    vals = orc.decode_packed("e2m1", p["A"], M * K).reshape(M, K // 32, 32)
    amax = np.abs(vals).max(-1)
    assert np.all((amax >= 4.0) | (amax == 6.0))  # E2M1 top binade: 4 and 6
    x = np.random.default_rng(1000 * 33 + 1).standard_normal((M, K), dtype=np.float32)
    sc = orc.decode_packed("e8m0", p["SA"], M * K // 32).reshape(M, K // 32)
    rec = vals * sc[..., None]
    err = np.abs(rec.reshape(M, K) - x) / np.repeat(sc, 32, axis=1)
    # in units of the scale: half the top binade's spacing (1) below 6, and
    # saturation to 6 for block maxima in [6, 8) (the recipe's known clipping)
    assert err.max() < 2.0
    small = np.abs(x) / np.repeat(sc, 32, axis=1) < 6
    assert err[small].max() <= 1.0


def test_entries_match_full(orc):
    M, N, K = 16, 24, 96
    p = _problem("e3m2", "e2m3", M, N, K, 34)
    C = np.random.default_rng(3).uniform(-1, 1, (M, N)).astype(np.float32)
    bias = np.random.default_rng(4).standard_normal(N).astype(np.float32)
    D, Y, S = orc.mx_gemm(p["A"], p["SA"], p["B"], p["SB"], C, bias, M, N, K, "e3m2", "e2m3",
                          "f16", alpha=0.5, relu=True)
    rows = np.array([0, 5, 15, 7]); cols = np.array([0, 23, 4, 11])
    De, Ye, Se = orc.mx_gemm_entries(p["A"], p["SA"], p["B"], p["SB"], C, bias, M, N, K, "e3m2",
                                     "e2m3", "f16", rows, cols, alpha=0.5, relu=True)
    assert np.array_equal(De, D[rows, cols]) and np.array_equal(Ye, Y[rows, cols])
