"""Pins for the oracle's W4A16 weight dequantisation.

"NVIDIA MMA", section "How quantisation configurations map to MMA": W4A16
is INT4 weight-only, run as an FP16 x FP16 or BF16 x BF16 MMA on a weight
tile dequantised first; the page leaves the scale / zero-point / packing
contract to the kernel.  Reading: unsigned codes q, per-group zero point z
and scale s, w = RNE((q - z) s) in the activation type; codes two per byte
along K, the even element in the low nibble."""
import numpy as np
import pytest
import torch

from sparse_tiled_gemm_amd import inputs


def _enc(t, x):
    return inputs.to_f16(x) if t == "f16" else inputs.to_bf16(x)


@pytest.mark.parametrize("t", ["f16", "bf16"])
def test_unit_scale_gives_the_signed_codes(orc, t):
    N, K, gs = 2, 32, 32
    q = np.tile(np.arange(16, dtype=np.uint8), (N, 2))
    W = orc.w4a16_dequant(inputs.w4_pack(q), _enc(t, np.ones((N, 1))), None, N, K, gs, t)
    vals = W.view(np.float16).astype(np.float64) if t == "f16" else \
        (W.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(vals, q.astype(np.float64) - 8)


def test_packing_reading(orc):
    Bq = np.array([[0x21, 0xF0]], np.uint8)  # codes 1, 2, 0, 15
    W = orc.w4a16_dequant(Bq, _enc("f16", [[1.0]]), np.array([[0]], np.uint8), 1, 4, 4, "f16")
    assert W.view(np.float16).tolist() == [[1.0, 2.0, 0.0, 15.0]]


@pytest.mark.parametrize("t", ["f16", "bf16"])
def test_rounding_against_numpy_and_torch(orc, t):
    """(q - z) s is exact in fp64 and fp32; the cast is numpy's (fp16) or
    torch's (bf16) round-to-nearest-even conversion."""
    rng = np.random.default_rng(3)
    N, K, gs = 16, 256, 64
    q = rng.integers(0, 16, (N, K)).astype(np.uint8)
    z = rng.integers(0, 16, (N, K // gs)).astype(np.uint8)
    S = _enc(t, rng.standard_normal((N, K // gs)) * 0.37)
    W = orc.w4a16_dequant(inputs.w4_pack(q), S, z, N, K, gs, t)
    if t == "f16":
        s = S.view(np.float16).astype(np.float64)
        ref = ((q.astype(np.float64) - np.repeat(z, gs, 1)) * np.repeat(s, gs, 1)).astype(np.float16)
        assert np.array_equal(W, ref.view(np.uint16))
    else:
        s = torch.from_numpy(S.view(np.int16)).view(torch.bfloat16).float().numpy()
        prod = (q.astype(np.float32) - np.repeat(z, gs, 1).astype(np.float32)) * np.repeat(s, gs, 1)
        ref = torch.from_numpy(prod).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(W, ref)


def test_groups_are_independent(orc):
    rng = np.random.default_rng(4)
    N, K, gs = 4, 512, 128
    q = rng.integers(0, 16, (N, K)).astype(np.uint8)
    S = _enc("bf16", rng.uniform(0.5, 2.0, (N, K // gs)))
    z = rng.integers(0, 16, (N, K // gs)).astype(np.uint8)
    W1 = orc.w4a16_dequant(inputs.w4_pack(q), S, z, N, K, gs, "bf16")
    S2 = S.copy()
    S2[2, 1] = _enc("bf16", [3.0])[0]
    W2 = orc.w4a16_dequant(inputs.w4_pack(q), S2, z, N, K, gs, "bf16")
    diff = W1 != W2
    assert not diff[:, :gs].any() and not diff[:, 2 * gs:].any()
    assert not np.delete(diff, 2, 0).any()
    assert diff[2, gs:2 * gs].sum() == np.count_nonzero(q[2, gs:2 * gs] != z[2, 1])


def test_generator_reconstructs_the_weights(orc):
    """The quantised weights stay within half a step of the drawn ones."""
    N, K, gs = 32, 256, 128
    p = inputs.w4a16_problem(8, N, K, "f16", gs, workload=50)
    W = orc.w4a16_dequant(p["B"], p["scales"], p["zeros"], N, K, gs, "f16").view(np.float16)
    w = np.random.default_rng(1000 * 50 + 2).standard_normal((N, K), dtype=np.float32) / np.sqrt(K)
    s = np.repeat(p["scales"].view(np.float16).astype(np.float64), gs, 1)
    assert np.all(np.abs(W.astype(np.float64) - w) <= 0.5 * s + 2.0 ** -10 * np.abs(w) + 1e-7)
