"""GPU parity of the unsigned 8-bit pairs (u8 x s8, s8 x u8, u8 x u8) against
the oracle, bit-exact on int32 outputs.

The INT8 rows of the instruction tables on "NVIDIA MMA" (section "Ampere:
FP16/BF16 and integer MMA baseline", and its sparse INT8 row) take A and B
signed or unsigned.  gfx950's int8 matrix instructions are signed only: the
kernels feed an unsigned operand as x - 128 and add the offset terms from
row and column sums afterwards, so every case here is compared exactly:
dense kernel families (K-major tiled, generic for the other layouts),
ragged tails, K not a multiple of the instruction's K, int32 wrap-around,
saturation at its K limit, the dequantising float epilogue, and the 2:4
kernels (the 8-wave kernel takes an unsigned B; an unsigned A runs the
generic 2:4 kernel)."""
import zlib

import numpy as np
import pytest

from checks import check
from gpu_util import gpu_compress, gpu_gemm, gpu_sparse_gemm, say
from sparse_tiled_gemm_amd import gemm as G
from sparse_tiled_gemm_amd import inputs

pytestmark = pytest.mark.gpu

PAIRS = [("u8", "s8"), ("s8", "u8"), ("u8", "u8")]
IDS = ["x".join(p) for p in PAIRS]


def _ints(t, shape, rng):
    if t == "u8":
        return rng.integers(0, 256, size=shape, dtype=np.uint8)
    return rng.integers(-128, 128, size=shape, dtype=np.int8)


def _problem(a_type, b_type, M, N, K, a_col=False, b_col=True, tag=""):
    rng = np.random.default_rng(zlib.crc32(repr((a_type, b_type, M, N, K, a_col, b_col,
                                                 tag)).encode()))
    A = _ints(a_type, (K, M) if a_col else (M, K), rng)
    B = _ints(b_type, (N, K) if b_col else (K, N), rng)
    C = rng.integers(-(1 << 20), (1 << 20) + 1, size=(M, N), dtype=np.int32)
    return A, B, C


def _exact(orc, A, B, C, M, N, K, a_type, b_type, algo, expect=None, a_col=False, b_col=True,
           **kw):
    say("u8 case", a_type, b_type, (M, N, K), algo, a_col, b_col, kw)
    D, name = gpu_gemm(A, B, C, None, M, N, K, a_type, b_type, "s32", algo=algo, a_col=a_col,
                       b_col=b_col, **kw)
    if expect:
        assert name.startswith(expect), name
    Dr, _, _ = orc.gemm(A, B, C, None, M, N, K, a_type, b_type, "s32", a_col_major=a_col,
                        b_col_major=b_col, saturate=kw.get("saturate", False))
    bad = int((D != Dr).sum())
    say("  ", name, "mismatches", bad)
    assert bad == 0, name
    return D, name


@pytest.mark.parametrize("pair", PAIRS, ids=IDS)
@pytest.mark.parametrize("algo,shape", [("tiled256", (600, 520, 256)),
                                        ("tiled128", (300, 260, 192)),
                                        ("tiled128", (260, 136, 1088)),
                                        ("generic", (129, 257, 96)),
                                        ("generic", (17, 9, 20))])
def test_u8_dense_parity(orc, pair, algo, shape):
    M, N, K = shape
    A, B, C = _problem(*pair, M, N, K)
    _exact(orc, A, B, C, M, N, K, *pair, algo, expect=algo)


@pytest.mark.parametrize("pair", PAIRS, ids=IDS)
@pytest.mark.parametrize("shape", [(600, 520, 256), (256, 256, 64), (300, 700, 448)])
def test_u8_dense_256_w8t(orc, monkeypatch, pair, shape):
    """The 256 x 256 8-wave kernel int8 runs (the only 256 x 256 variant
    built for unsigned operands)."""
    monkeypatch.setenv("STGEMM_FORCE_KERNEL", "tiled256w8t")
    M, N, K = shape
    A, B, C = _problem(*pair, M, N, K, tag="w8t")
    _exact(orc, A, B, C, M, N, K, *pair, "auto", expect="tiled256w8t")


@pytest.mark.parametrize("pair", PAIRS, ids=IDS)
@pytest.mark.parametrize("a_col,b_col", [(True, True), (False, False), (True, False)])
def test_u8_other_layouts_run_generic(orc, pair, a_col, b_col):
    M, N, K = 200, 136, 320
    A, B, C = _problem(*pair, M, N, K, a_col=a_col, b_col=b_col)
    _exact(orc, A, B, C, M, N, K, *pair, "auto", expect="generic", a_col=a_col, b_col=b_col)


@pytest.mark.parametrize("pair", PAIRS, ids=IDS)
@pytest.mark.parametrize("M", [1, 16])
def test_u8_small_m(orc, pair, M):
    """Small M: the automatic choice skips the (signed-only) small-M kernel."""
    N, K = 300, 1024
    A, B, C = _problem(*pair, M, N, K)
    _, name = _exact(orc, A, B, C, M, N, K, *pair, "auto")
    assert not name.startswith("skinny"), name


@pytest.mark.parametrize("algo", ["tiled128", "generic"])
def test_u8_wraps_modulo_2_32(orc, algo):
    """255 * 255 * K passes 2^31 at K = 33026: the int32 result wraps."""
    M, N, K = 64, 64, 33280
    A = np.full((M, K), 255, np.uint8)
    B = np.full((N, K), 255, np.uint8)
    B[1::2, ::3] = 7
    C = np.zeros((M, N), np.int32)
    D, _ = _exact(orc, A, B, C, M, N, K, "u8", "u8", algo, expect=algo)
    assert 255 * 255 * K > 2 ** 31 and D[0, 0] == 255 * 255 * K - 2 ** 32


@pytest.mark.parametrize("pair,K", [(("u8", "u8"), 33024), (("u8", "s8"), 65792),
                                    (("s8", "u8"), 65792)], ids=IDS)
@pytest.mark.parametrize("algo", ["tiled128", "generic"])
def test_u8_saturate_at_limit(orc, pair, K, algo):
    """Saturation at the largest K the library accepts for the pair: extreme
    values with C pushing the sums past both ends of the int32 range."""
    M, N = 64, 64
    rng = np.random.default_rng(K)
    hi = {"u8": 255, "s8": -128}
    A = np.full((M, K), hi[pair[0]], dtype=np.uint8 if pair[0] == "u8" else np.int8)
    B = np.full((N, K), hi[pair[1]], dtype=np.uint8 if pair[1] == "u8" else np.int8)
    B[::2, : K // 2] = 0
    C = rng.integers(-(2 ** 31), 2 ** 31, size=(M, N), dtype=np.int64).astype(np.int32)
    C[0, 0], C[0, 1], C[1, 0] = 2 ** 31 - 1, -(2 ** 31), 2 ** 31 - 1
    D, _ = _exact(orc, A, B, C, M, N, K, *pair, algo, expect=algo, saturate=True)
    assert (D == 2 ** 31 - 1).any() or (D == -(2 ** 31)).any()
    d = G.make_desc(M, N, K + 4, pair[0], pair[1], "s32", has_c=True, saturate=True)
    with pytest.raises(G.GemmError) as e:
        G.gemm_plan(d)
    assert e.value.status == G.GEMM_ERR_UNSUPPORTED


@pytest.mark.parametrize("pair", PAIRS, ids=IDS)
@pytest.mark.parametrize("algo", ["tiled256", "generic"])
@pytest.mark.parametrize("d_type", ["f32", "bf16"])
def test_u8_dequantising_epilogue(orc, pair, algo, d_type):
    """int32 sum -> fp32 (round to nearest even) -> alpha, bias, relu, cast."""
    M, N, K = 520, 264, 512
    A, B, _ = _problem(*pair, M, N, K, tag="deq")
    rng = np.random.default_rng(3)
    C = rng.uniform(-1, 1, size=(M, N)).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32)
    alpha = 1.0 / 4096
    D, name = gpu_gemm(A, B, C, bias, M, N, K, *pair, d_type, algo=algo, alpha=alpha, relu=True)
    assert name.startswith(algo), name
    Dr, Y, S = orc.gemm(A, B, C, bias, M, N, K, *pair, d_type, alpha=alpha, relu=True)
    r = check(D, d_type, Dr, Y, S, "s8", alpha)
    say("  ", name, d_type, r)
    assert r.ok, r
    if d_type == "f32":  # the epilogue's fp32 arithmetic, bit for bit
        T, _ = gpu_gemm(A, B, None, None, M, N, K, *pair, "s32", algo=algo)
        ref = orc.epilogue_f32(T.astype(np.float32) + C, alpha, bias, True, "f32")
        assert np.array_equal(D.view(np.uint32), ref.view(np.uint32))


# ---------------------------------------------------------------- 2:4 A


def _sparse_problem(a_type, b_type, M, N, K):
    rng = np.random.default_rng(zlib.crc32(repr(("sp", a_type, b_type, M, N, K)).encode()))
    G4 = K // 4
    pairs = np.array([(0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3)])
    pos = pairs[rng.integers(0, 6, size=(M, G4))]
    lo = 1 if a_type == "u8" else -128
    vals = rng.integers(lo, 256 if a_type == "u8" else 128, size=(M, G4, 2))
    vals[vals == 0] = 1
    A = np.zeros((M, G4, 4), np.int64)
    r, g = np.arange(M)[:, None], np.arange(G4)[None, :]
    A[r, g, pos[..., 0]] = vals[..., 0]
    A[r, g, pos[..., 1]] = vals[..., 1]
    A = A.reshape(M, K).astype(np.uint8 if a_type == "u8" else np.int8)
    B = _ints(b_type, (N, K), rng)
    C = rng.integers(-(1 << 20), (1 << 20) + 1, size=(M, N), dtype=np.int32)
    return A, B, C


@pytest.mark.parametrize("M,K", [(1, 4), (130, 200), (64, 4100)])
def test_u8_compress_matches_oracle(orc, M, K):
    """u8 zeros are 0 only (0x80 is 128)."""
    A, _, _ = _sparse_problem("u8", "s8", M, 4, K)
    A.reshape(M, K // 4, 4)[:, ::3, :][A.reshape(M, K // 4, 4)[:, ::3, :] != 0] = 0x80
    vals, meta, vb, mb = gpu_compress(A, "u8")
    rv, rm = orc.sparse24_compress(A, "u8")
    assert np.array_equal(vals.cpu().numpy()[:vb].reshape(rv.shape), rv.view(np.uint8))
    assert np.array_equal(meta.cpu().numpy()[:mb].view(np.uint32).reshape(rm.shape), rm)


_SPARSE_CASES = [
    (("u8", "s8"), "sparse24_generic", [(129, 257, 96), (17, 9, 20), (300, 264, 512)]),
    (("u8", "u8"), "sparse24_generic", [(129, 257, 96), (300, 264, 512)]),
    (("s8", "u8"), "sparse24_dma8", [(600, 520, 256), (300, 700, 768), (40, 1000, 1280)]),
    (("s8", "u8"), "sparse24_generic", [(129, 257, 96), (17, 9, 20)]),
]


@pytest.mark.parametrize("pair,family,shapes", _SPARSE_CASES,
                         ids=["x".join(c[0]) + "-" + c[1] for c in _SPARSE_CASES])
def test_u8_sparse_parity(orc, pair, family, shapes):
    for M, N, K in shapes:
        A, B, C = _sparse_problem(*pair, M, N, K)
        say("u8 sparse", pair, family, (M, N, K))
        vals, meta, _, _ = gpu_compress(A, pair[0])
        D, name = gpu_sparse_gemm(vals, meta, B, C, M, N, K, "s32", a_type=pair[0],
                                  b_type=pair[1])
        assert name.startswith(family), name
        Dr, _, _ = orc.gemm(A, B, C, None, M, N, K, *pair, "s32")
        bad = int((D != Dr).sum())
        say("  ", name, "mismatches", bad)
        assert bad == 0


@pytest.mark.parametrize("pair", PAIRS, ids=IDS)
def test_u8_sparse_plan(pair):
    """Unsigned A: the generic 2:4 kernel at any K; unsigned B: the 8-wave
    kernel where it applies (K % 256 == 0), else the generic one (the 4-wave
    kernel is not built for unsigned operands)."""
    for K in [256, 384, 192]:
        plan = G.gemm_plan(G.make_desc(512, 512, K, *pair, "s32", sparse_a=True))
        fam = "sparse24_dma8" if pair[0] == "s8" and K % 256 == 0 else "sparse24_generic"
        assert plan.name.startswith(fam), (pair, K, plan.name)


def test_u8_sparse_float_epilogue(orc):
    M, N, K = 384, 320, 512
    A, B, _ = _sparse_problem("s8", "u8", M, N, K)
    rng = np.random.default_rng(8)
    bias = rng.standard_normal(N).astype(np.float32)
    vals, meta, _, _ = gpu_compress(A, "s8")
    D, name = gpu_sparse_gemm(vals, meta, B, None, M, N, K, "bf16", bias=bias, alpha=1.0 / 2048,
                              relu=True, a_type="s8", b_type="u8")
    assert name.startswith("sparse24_dma8"), name
    Dr, Y, S = orc.gemm(A, B, None, bias, M, N, K, "s8", "u8", "bf16", alpha=1.0 / 2048,
                        relu=True)
    r = check(D, "bf16", Dr, Y, S, "s8", 1.0 / 2048)
    say("  ", name, r)
    assert r.ok, r
