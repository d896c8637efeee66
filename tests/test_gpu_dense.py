"""GPU parity of the dense kernels against the oracle, element by element,
at sizes the oracle finishes in seconds that span several workgroup tiles
with ragged M/N tails, for every input-type pair and kernel family, plus
epilogue, layout, stride, alignment and degenerate-shape cases."""
import zlib

import numpy as np
import pytest
import torch

from checks import check
from gpu_util import gpu_gemm, say, to_dev, empty_out
from sparse_tiled_gemm_amd import gemm as G
from sparse_tiled_gemm_amd import inputs

pytestmark = pytest.mark.gpu

CONV = {"f16": inputs.to_f16, "bf16": inputs.to_bf16, "e4m3": inputs.to_e4m3,
        "e5m2": inputs.to_e5m2}
PAIRS = [("f16", "f16"), ("bf16", "bf16"), ("e4m3", "e5m2"), ("e5m2", "e4m3"),
         ("e4m3", "e4m3"), ("e5m2", "e5m2"), ("s8", "s8")]


def make(a_type, b_type, M, N, K, seed, a_col=False, b_col=True, c=True, bias=False):
    rng = np.random.default_rng(seed)
    ashape = (K, M) if a_col else (M, K)
    bshape = (N, K) if b_col else (K, N)
    if a_type == "s8":
        A = rng.integers(-128, 128, size=ashape, dtype=np.int8)
        B = rng.integers(-128, 128, size=bshape, dtype=np.int8)
        C = rng.integers(-(1 << 20), (1 << 20) + 1, size=(M, N), dtype=np.int32) if c else None
        return A, B, C, None
    sa = 16.0 if a_type.startswith("e") else 1.0
    A = CONV[a_type](rng.standard_normal(ashape) * sa)
    B = CONV[b_type](rng.standard_normal(bshape) * sa)
    C = rng.uniform(-1, 1, size=(M, N)).astype(np.float32) if c else None
    bv = rng.standard_normal(N).astype(np.float32) if bias else None
    return A, B, C, bv


def compare(orc, A, B, C, bias, M, N, K, a_type, b_type, d_type, algo, expect_kernel=None,
            **kw):
    say("case", a_type, b_type, d_type, (M, N, K), algo, kw.get("alpha", 1.0),
        kw.get("relu", False), kw.get("a_col", False), kw.get("b_col", True))
    D, name = gpu_gemm(A, B, C, bias, M, N, K, a_type, b_type, d_type, algo=algo, **kw)
    if expect_kernel:
        assert name.startswith(expect_kernel), name
    okw = dict(a_col_major=kw.get("a_col", False), b_col_major=kw.get("b_col", True),
               alpha=kw.get("alpha", 1.0), relu=kw.get("relu", False))
    Dr, Y, S = orc.gemm(A, B, C, bias, M, N, K, a_type, b_type, d_type, **okw)
    r = check(D, d_type, Dr, Y, S, a_type, kw.get("alpha", 1.0))
    say("  ", name, r)
    assert r.ok, r
    return D, name


@pytest.mark.parametrize("a_type,b_type", PAIRS)
@pytest.mark.parametrize("algo,shape", [("tiled256", (600, 520, 256)),
                                        ("tiled128", (300, 260, 192)),
                                        ("generic", (129, 257, 96)),
                                        ("generic", (17, 9, 20))])
def test_dense_parity(orc, a_type, b_type, algo, shape):
    M, N, K = shape
    A, B, C, _ = make(a_type, b_type, M, N, K, seed=zlib.crc32(repr((a_type, b_type, shape)).encode()))
    d_type = "s32" if a_type == "s8" else "f32"
    compare(orc, A, B, C, None, M, N, K, a_type, b_type, d_type, algo, expect_kernel=algo)


@pytest.mark.parametrize("family", ["tiled256", "tiled256w8", "tiled256w8t"])
@pytest.mark.parametrize("a_type,b_type", PAIRS)
@pytest.mark.parametrize("shape", [(600, 520, 256), (256, 256, 64), (300, 700, 448)])
def test_dense_parity_256_variants(orc, monkeypatch, family, a_type, b_type, shape):
    """Every 256 x 256 kernel variant, each selected through the
    STGEMM_FORCE_KERNEL tuning override (the automatic choice takes one of
    them per operand type)."""
    monkeypatch.setenv("STGEMM_FORCE_KERNEL", family)
    M, N, K = shape
    A, B, C, _ = make(a_type, b_type, M, N, K, seed=zlib.crc32(repr((family, a_type, shape)).encode()))
    d_type = "s32" if a_type == "s8" else "f32"
    compare(orc, A, B, C, None, M, N, K, a_type, b_type, d_type, "auto", expect_kernel=family)


# the rolling-fragment kernels (k_tiled16): 16-bit and int8 inputs on the
# 16x16 forms, fp8 on the 32x32x64 form; K-contiguous
K16_FAMILIES = ["tiled256w8k16", "tiled256w8tk16"]
K16_PAIRS = [("f16", "f16"), ("bf16", "bf16"), ("s8", "s8"), ("e4m3", "e5m2"), ("e5m2", "e4m3"),
             ("e4m3", "e4m3"), ("e5m2", "e5m2")]


@pytest.mark.parametrize("family", K16_FAMILIES)
@pytest.mark.parametrize("a_type,b_type", K16_PAIRS)
@pytest.mark.parametrize("shape", [(600, 520, 256), (256, 256, 64), (300, 700, 448),
                                   (1000, 777, 576), (17, 300, 128)])
def test_dense_parity_k16(orc, monkeypatch, family, a_type, b_type, shape):
    """Both arrangements of the 16x16-form kernel (forced), ragged M and N,
    K from one tile up."""
    monkeypatch.setenv("STGEMM_FORCE_KERNEL", family)
    M, N, K = shape
    A, B, C, _ = make(a_type, b_type, M, N, K, seed=zlib.crc32(repr((family, a_type, shape)).encode()))
    d_type = "s32" if a_type == "s8" else "f32"
    compare(orc, A, B, C, None, M, N, K, a_type, b_type, d_type, "auto", expect_kernel=family)


@pytest.mark.parametrize("family", K16_FAMILIES)
@pytest.mark.parametrize("a_type,b_type,d_type", [("bf16", "bf16", "bf16"), ("f16", "f16", "f16"),
                                                  ("bf16", "bf16", "f16"),
                                                  ("e4m3", "e5m2", "f16")])
def test_epilogue_bit_exact_k16(orc, monkeypatch, family, a_type, b_type, d_type):
    """The fused epilogue of the rolling-fragment kernels against the
    oracle's fp32 epilogue on the same kernel's fp32 output, bit for bit."""
    monkeypatch.setenv("STGEMM_FORCE_KERNEL", family)
    M, N, K = 384, 320, 256
    A, B, C, bias = make(a_type, b_type, M, N, K, seed=12, bias=True)
    alpha = 0.3 if not a_type.startswith("e") else 0.3 / 256.0
    T, n1 = gpu_gemm(A, B, C, None, M, N, K, a_type, b_type, "f32")
    D, n2 = gpu_gemm(A, B, C, bias, M, N, K, a_type, b_type, d_type, alpha=alpha, relu=True)
    assert n1.startswith(family) and n2.startswith(family), (n1, n2)
    ref = orc.epilogue_f32(T, alpha, bias, True, d_type)
    mism = int((D != ref).sum())
    say("epilogue", family, a_type, d_type, "mismatches", mism)
    assert mism == 0


def test_k16_is_the_automatic_choice():
    """K-contiguous f16 / bf16 / s8 / fp8 at 256 x 256 scale take the
    rolling-fragment kernel; MN-major and unsigned operands keep theirs."""
    def name(t, d, **kw):
        return G.gemm_plan(G.make_desc(8192, 8192, 8192, t, t, d, **kw)).name
    assert name("bf16", "bf16") == "tiled256w8tk16_bf16"
    assert name("f16", "f32") == "tiled256w8tk16_f16"
    assert name("s8", "s32") == "tiled256w8tk16_s8"
    assert name("bf16", "bf16", a_layout="col") == "tiled256w8_bf16_acol"
    assert name("s8", "s32", b_layout="row") == "tiled256w8t_s8_brow"
    assert name("u8", "s32").startswith("tiled256w8t")
    fp8 = G.make_desc(8192, 8192, 8192, "e4m3", "e5m2", "f16")
    assert G.gemm_plan(fp8).name == "tiled256w8k16_e4m3xe5m2"
    fp8mn = G.make_desc(8192, 8192, 8192, "e4m3", "e5m2", "f16", a_layout="col")
    assert G.gemm_plan(fp8mn).name.startswith("tiled256_")


@pytest.mark.parametrize("a_type,b_type", PAIRS)
@pytest.mark.parametrize("shape", [(16, 1024, 2048), (1, 300, 512), (7, 96, 1024), (16, 33, 256),
                                   (12, 8192, 768)])
def test_skinny_parity(orc, a_type, b_type, shape):
    """Small-M kernel: M <= 16, K split over the workgroup's waves."""
    M, N, K = shape
    A, B, C, _ = make(a_type, b_type, M, N, K, seed=zlib.crc32(repr(("skinny", a_type, shape)).encode()))
    d_type = "s32" if a_type == "s8" else "f32"
    compare(orc, A, B, C, None, M, N, K, a_type, b_type, d_type, "skinny", expect_kernel="skinny")


@pytest.mark.parametrize("a_type,b_type,d_type", [("bf16", "bf16", "bf16"), ("e4m3", "e5m2", "f16"),
                                                  ("f16", "f16", "f16")])
def test_skinny_epilogue(orc, a_type, b_type, d_type):
    M, N, K = 16, 520, 1024
    A, B, C, bias = make(a_type, b_type, M, N, K, seed=23, bias=True)
    alpha = 0.5 if not a_type.startswith("e") else 1.0 / 512
    compare(orc, A, B, C, bias, M, N, K, a_type, b_type, d_type, "skinny", expect_kernel="skinny",
            alpha=alpha, relu=True)
    T, _ = gpu_gemm(A, B, C, None, M, N, K, a_type, b_type, "f32", algo="skinny")
    D, _ = gpu_gemm(A, B, C, bias, M, N, K, a_type, b_type, d_type, algo="skinny", alpha=alpha,
                    relu=True)
    assert (D != orc.epilogue_f32(T, alpha, bias, True, d_type)).sum() == 0


def test_skinny_is_chosen_for_small_m():
    assert G.gemm_plan(G.make_desc(16, 8192, 8192, "bf16", "bf16", "bf16")).name == "skinny_bf16"
    assert G.gemm_plan(G.make_desc(17, 8192, 8192, "bf16", "bf16", "bf16")).name != "skinny_bf16"


@pytest.mark.parametrize("family", ["tiled256w8"])
@pytest.mark.parametrize("d_type", ["f16", "bf16"])
def test_forced_family_epilogue(orc, monkeypatch, family, d_type):
    monkeypatch.setenv("STGEMM_FORCE_KERNEL", family)
    M, N, K = 520, 390, 320
    A, B, C, bias = make("e4m3", "e5m2", M, N, K, seed=17, bias=True)
    compare(orc, A, B, C, bias, M, N, K, "e4m3", "e5m2", d_type, "auto", expect_kernel=family,
            alpha=1.0 / 512, relu=True)


@pytest.mark.parametrize("a_type,b_type", [("bf16", "bf16"), ("f16", "f16"), ("e4m3", "e5m2")])
@pytest.mark.parametrize("d_type", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("algo", ["tiled128", "generic"])
@pytest.mark.parametrize("epi", [dict(), dict(alpha=0.75), dict(bias=True, relu=True),
                                 dict(alpha=-1.5, bias=True, c=False)])
def test_epilogue_variants(orc, a_type, b_type, d_type, algo, epi):
    M, N, K = 200, 136, 128
    A, B, C, bias = make(a_type, b_type, M, N, K, seed=7, c=epi.get("c", True),
                         bias=epi.get("bias", False))
    if a_type.startswith("e"):
        # keep fp16 outputs in range for fp8 inputs of magnitude ~16
        epi = dict(epi)
        epi["alpha"] = epi.get("alpha", 1.0) / 256.0
    compare(orc, A, B, C, bias, M, N, K, a_type, b_type, d_type, algo, expect_kernel=algo,
            alpha=epi.get("alpha", 1.0), relu=epi.get("relu", False))


@pytest.mark.parametrize("algo", ["tiled256", "tiled128", "generic", "tiled256w8", "tiled256w8t"])
@pytest.mark.parametrize("a_type,b_type,d_type", [("bf16", "bf16", "bf16"), ("f16", "f16", "f16"),
                                                  ("e4m3", "e5m2", "f16"),
                                                  ("e4m3", "e5m2", "bf16")])
def test_epilogue_bit_exact(orc, monkeypatch, algo, a_type, b_type, d_type):
    """The fused epilogue equals the oracle's fp32 epilogue applied to the
    same kernel's fp32 accumulator output, bit for bit (same plan family, so
    the same summation order)."""
    if algo.startswith("tiled256") and algo != "tiled256":
        monkeypatch.setenv("STGEMM_FORCE_KERNEL", algo)
        algo = "tiled256"
    M, N, K = 384, 320, 256
    A, B, C, bias = make(a_type, b_type, M, N, K, seed=11, bias=True)
    alpha = 0.3 if not a_type.startswith("e") else 0.3 / 256.0
    T, n1 = gpu_gemm(A, B, C, None, M, N, K, a_type, b_type, "f32", algo=algo)
    D, n2 = gpu_gemm(A, B, C, bias, M, N, K, a_type, b_type, d_type, algo=algo, alpha=alpha,
                     relu=True)
    assert n1 == n2 and n1.startswith(algo), (n1, n2)
    ref = orc.epilogue_f32(T, alpha, bias, True, d_type)
    mism = int((D != ref).sum())
    say("epilogue", algo, a_type, d_type, "mismatches", mism)
    assert mism == 0


@pytest.mark.parametrize("a_type,b_type", [("f16", "f16"), ("bf16", "bf16"), ("e4m3", "e5m2"),
                                           ("s8", "s8")])
@pytest.mark.parametrize("a_col,b_col", [(False, False), (True, True), (True, False)])
def test_other_layouts(orc, a_type, b_type, a_col, b_col):
    M, N, K = 70, 90, 100
    A, B, C, _ = make(a_type, b_type, M, N, K, seed=3, a_col=a_col, b_col=b_col)
    d_type = "s32" if a_type == "s8" else "f32"
    compare(orc, A, B, C, None, M, N, K, a_type, b_type, d_type, "auto", expect_kernel="generic",
            a_col=a_col, b_col=b_col)


@pytest.mark.parametrize("a_type,b_type", [("bf16", "bf16"), ("s8", "s8"), ("e4m3", "e5m2")])
@pytest.mark.parametrize("shape", [(1, 1, 1), (1, 4096, 64), (64, 1, 64), (5, 7, 1000),
                                   (256, 256, 100), (33, 65, 4)])
def test_edge_shapes(orc, a_type, b_type, shape):
    M, N, K = shape
    A, B, C, _ = make(a_type, b_type, M, N, K, seed=5)
    d_type = "s32" if a_type == "s8" else "f32"
    compare(orc, A, B, C, None, M, N, K, a_type, b_type, d_type, "auto")


@pytest.mark.parametrize("a_type", ["bf16", "s8"])
def test_k_zero_gives_epilogue_of_c(orc, a_type):
    M, N = 40, 24
    A, B, C, _ = make(a_type, a_type, M, N, 1, seed=9)
    d_type = "s32" if a_type == "s8" else "f32"
    D, _ = gpu_gemm(A[:, :0], B[:, :0], C, None, M, N, 0, a_type, a_type, d_type)
    assert np.array_equal(D, C)


def test_padded_leading_dimensions(orc, monkeypatch):
    M, N, K = 300, 200, 256
    lda, ldb, ldc, ldd = K + 64, K + 32, N + 8, N + 24
    rng = np.random.default_rng(21)
    Ap = inputs.to_bf16(rng.standard_normal((M, lda)))
    Bp = inputs.to_bf16(rng.standard_normal((N, ldb)))
    Cp = rng.uniform(-1, 1, (M, ldc)).astype(np.float32)
    Dr, Y, S = orc.gemm(np.ascontiguousarray(Ap[:, :K]), np.ascontiguousarray(Bp[:, :K]),
                        np.ascontiguousarray(Cp[:, :N]), None, M, N, K, "bf16", "bf16", "bf16")
    for algo in ["tiled128", "tiled256", "generic", "tiled256w8", "tiled256w8t",
                 "tiled256w8k16", "tiled256w8tk16"]:
        say("padded", algo)
        monkeypatch.delenv("STGEMM_FORCE_KERNEL", raising=False)
        if algo.startswith("tiled256") and algo != "tiled256":
            monkeypatch.setenv("STGEMM_FORCE_KERNEL", algo)
        D, name = gpu_gemm(Ap, Bp, Cp, None, M, N, K, "bf16", "bf16", "bf16",
                           algo="tiled256" if algo.startswith("tiled256") else algo,
                           lda=lda, ldb=ldb, ldc=ldc, ldd=ldd)
        assert name.startswith(algo)
        r = check(D, "bf16", Dr, Y, S, "bf16")
        assert r.ok, r


def test_misaligned_operands_fall_back(orc):
    """A and B offset by one element: the tiled plan falls back to the
    generic kernel at run time and the result is still right."""
    M, N, K = 256, 192, 128
    A, B, C, _ = make("bf16", "bf16", M, N, K, seed=4)
    tA = to_dev(np.concatenate([np.zeros(1, np.uint16), A.reshape(-1)]))
    tB = to_dev(np.concatenate([np.zeros(1, np.uint16), B.reshape(-1)]))
    desc = G.make_desc(M, N, K, "bf16", "bf16", "f32", algo="tiled128")
    plan = G.gemm_plan(desc)
    D = empty_out(M, N, "f32")
    G.gemm_run(plan, tA.data_ptr() + 2, tB.data_ptr() + 2, to_dev(C), None, D)
    torch.cuda.synchronize()
    D = D.cpu().numpy().view(np.float32).reshape(M, N)
    Dr, Y, S = orc.gemm(A, B, C, None, M, N, K, "bf16", "bf16", "f32")
    assert check(D, "f32", Dr, Y, S, "bf16").ok


def test_in_place_accumulate_d_equals_c(orc):
    M, N, K = 256, 256, 128
    A, B, C, _ = make("f16", "f16", M, N, K, seed=6)
    tC = to_dev(C)
    D, _ = gpu_gemm(A, B, None, None, M, N, K, "f16", "f16", "f32", c_dev=tC, out=tC)
    Dr, Y, S = orc.gemm(A, B, C, None, M, N, K, "f16", "f16", "f32")
    assert check(D, "f32", Dr, Y, S, "f16").ok


def test_overlapping_d_is_rejected():
    """D may be C itself (same element size and leading dimension); any other
    overlap of D with C, A, B or bias is refused before a launch."""
    M, N, K = 64, 64, 64
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    base = buf.data_ptr()

    def run(d_type, D, C=None, A=None, B=None, bias=None, ldc=0):
        desc = G.make_desc(M, N, K, "bf16", "bf16", d_type, has_c=C is not None,
                           has_bias=bias is not None, ldc=ldc)
        plan = G.gemm_plan(desc)
        try:
            G.gemm_run(plan, A or base + 600000, B or base + 700000, C, bias, D)
            torch.cuda.synchronize()
            return G.GEMM_OK
        except G.GemmError as e:
            return e.status

    assert run("f32", base, C=base) == G.GEMM_OK                      # in place
    assert run("bf16", base, C=base) == G.GEMM_ERR_UNSUPPORTED        # narrower D over C
    assert run("f32", base, C=base, ldc=N + 4) == G.GEMM_ERR_UNSUPPORTED  # other pitch
    assert run("f32", base + 256, C=base) == G.GEMM_ERR_UNSUPPORTED   # shifted
    assert run("f32", base, A=base + 1024) == G.GEMM_ERR_UNSUPPORTED  # D over A
    assert run("f32", base, B=base + 4096) == G.GEMM_ERR_UNSUPPORTED  # D over B
    assert run("f32", base, bias=base + 64) == G.GEMM_ERR_UNSUPPORTED  # D over bias
    assert run("f32", base, C=base + M * N * 4) == G.GEMM_OK          # adjacent, disjoint


@pytest.mark.parametrize("algo", ["tiled128", "generic"])
def test_int32_wraps_modulo_2_32(orc, algo):
    """127*127 summed over K = 140032 exceeds 2^31: the int32 result wraps."""
    M, N, K = 64, 64, 140032
    A = np.full((M, K), 127, np.int8)
    B = np.full((N, K), 127, np.int8)
    B[1::2] = -128
    C = np.zeros((M, N), np.int32)
    D, name = gpu_gemm(A, B, C, None, M, N, K, "s8", "s8", "s32", algo=algo)
    Dr, _, _ = orc.gemm(A, B, C, None, M, N, K, "s8", "s8", "s32")
    assert np.array_equal(D, Dr)
    assert 127 * 127 * K > 2 ** 31 and D[0, 0] == 127 * 127 * K - 2 ** 32


def test_plan_does_not_depend_on_epilogue():
    names = set()
    for d_type in ["f32", "f16", "bf16"]:
        for bias, relu in [(False, False), (True, True)]:
            d = G.make_desc(8192, 8192, 8192, "bf16", "bf16", d_type, has_bias=bias,
                            act="relu" if relu else "none")
            names.add(G.gemm_plan(d).name)
    assert len(names) == 1, names
