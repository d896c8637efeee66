"""GPU parity of the 2:4 path: the compressor's bytes against the oracle's
compressor (bit-exact), its rejection of groups with more than two
non-zeros, and sparse GEMM results against the oracle's dense GEMM on the
logical A."""
import numpy as np
import pytest
import torch

from checks import check
from gpu_util import gpu_compress, gpu_sparse_gemm, say, to_dev
from sparse_tiled_gemm_amd import gemm as G
from sparse_tiled_gemm_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K", [(1, 4), (3, 36), (130, 200), (257, 1024), (64, 4100)])
def test_compress_matches_oracle(orc, M, K):
    p = inputs.sparse24_f16(M=M, N=4, K=K)
    say("compress", M, K)
    vals, meta, vb, mb = gpu_compress(p["A_logical"])
    rv, rm = orc.sparse24_compress(p["A_logical"])
    assert np.array_equal(vals.cpu().numpy()[:vb].view(np.uint16).reshape(rv.shape), rv)
    assert np.array_equal(meta.cpu().numpy()[:mb].view(np.uint32).reshape(rm.shape), rm)


def test_compress_fewer_than_two_nonzeros(orc):
    rng = np.random.default_rng(2)
    M, K = 64, 256
    p = inputs.sparse24_f16(M=M, N=4, K=K)
    A = p["A_logical"].copy()
    # zero out one or both kept values in a third of the groups; write -0 in some
    g = A.reshape(M, K // 4, 4)
    kill = rng.random((M, K // 4, 4)) < 0.3
    g[kill & (g != 0)] = 0
    g[(rng.random(g.shape) < 0.1) & (g == 0)] = 0x8000
    A = g.reshape(M, K)
    vals, meta, vb, mb = gpu_compress(A)
    rv, rm = orc.sparse24_compress(A)
    assert np.array_equal(vals.cpu().numpy()[:vb].view(np.uint16).reshape(rv.shape), rv)
    assert np.array_equal(meta.cpu().numpy()[:mb].view(np.uint32).reshape(rm.shape), rm)


def test_compress_rejects_three_nonzeros():
    p = inputs.sparse24_f16(M=32, N=4, K=64)
    A = p["A_logical"].copy()
    A[17, 8:12] = inputs.to_f16(np.array([1.0, 2.0, 3.0, 0.0]))
    with pytest.raises(G.GemmError) as e:
        gpu_compress(A)
    assert e.value.status == G.GEMM_ERR_NOT_SPARSE24
    assert "17" in str(e.value)


@pytest.mark.parametrize("algo,shape", [("tiled", (600, 520, 256)), ("tiled", (256, 256, 64)),
                                        ("generic", (129, 257, 96)), ("generic", (17, 9, 20)),
                                        ("auto", (100, 100, 100))])
def test_sparse_parity(orc, algo, shape):
    M, N, K = shape
    p = inputs.sparse24_f16(M=M, N=N, K=K)
    say("sparse", algo, shape)
    vals, meta, _, _ = gpu_compress(p["A_logical"])
    D, name = gpu_sparse_gemm(vals, meta, p["B"], p["C"], M, N, K, algo=algo)
    say("  ", name)
    if algo != "auto":
        tiled = "sparse24_dma8" if K % 256 == 0 else "sparse24_tiled"
        assert name.startswith({"tiled": tiled, "generic": "sparse24_generic"}[algo]), name
    Dr, Y, S = orc.gemm(p["A_logical"], p["B"], p["C"], None, M, N, K, "f16", "f16", "f32")
    r = check(D, "f32", Dr, Y, S, "f16")
    say("  ", r)
    assert r.ok, r


@pytest.mark.parametrize("algo", ["tiled", "generic"])
@pytest.mark.parametrize("d_type", ["bf16", "f16"])
def test_sparse_epilogue(orc, algo, d_type):
    M, N, K = 300, 264, 128
    p = inputs.sparse24_f16(M=M, N=N, K=K)
    bias = np.random.default_rng(3).standard_normal(N).astype(np.float32)
    vals, meta, _, _ = gpu_compress(p["A_logical"])
    D, name = gpu_sparse_gemm(vals, meta, p["B"], p["C"], M, N, K, d_type, algo=algo, bias=bias,
                              alpha=0.5, relu=True)
    Dr, Y, S = orc.gemm(p["A_logical"], p["B"], p["C"], bias, M, N, K, "f16", "f16", d_type,
                        alpha=0.5, relu=True)
    r = check(D, d_type, Dr, Y, S, "f16", 0.5)
    assert r.ok, r


def test_sparse_row_major_b(orc):
    M, N, K = 96, 80, 64
    p = inputs.sparse24_f16(M=M, N=N, K=K)
    Brow = np.ascontiguousarray(p["B"].T)  # [K, N]
    vals, meta, _, _ = gpu_compress(p["A_logical"])
    D, name = gpu_sparse_gemm(vals, meta, Brow, p["C"], M, N, K, b_col=False)
    assert name.startswith("sparse24_generic")
    Dr, Y, S = orc.gemm(p["A_logical"], Brow, p["C"], None, M, N, K, "f16", "f16", "f32",
                        b_col_major=False)
    assert check(D, "f32", Dr, Y, S, "f16").ok


@pytest.mark.parametrize("family,shape", [
    ("sparse24_tiled", (600, 520, 256)), ("sparse24_tiled", (256, 256, 64)),
    ("sparse24_tiled", (300, 700, 448)), ("sparse24_tiled", (40, 1000, 192)),
    # the 8-wave kernel takes K in multiples of 256: one metadata group, odd
    # and even group counts, group counts that do and do not divide the
    # workgroup's K rotation
    ("sparse24_dma8", (600, 520, 256)), ("sparse24_dma8", (256, 256, 512)),
    ("sparse24_dma8", (300, 700, 768)), ("sparse24_dma8", (512, 264, 1024)),
    ("sparse24_dma8", (40, 1000, 1280)), ("sparse24_dma8", (2100, 300, 2304))])
def test_sparse_parity_variants(orc, monkeypatch, family, shape):
    """Each 256 x 256 SMFMAC kernel (selected through the STGEMM_FORCE_KERNEL
    tuning override): ragged M and N, one and several K tiles."""
    monkeypatch.setenv("STGEMM_FORCE_KERNEL", family)
    M, N, K = shape
    p = inputs.sparse24_f16(M=M, N=N, K=K)
    say("sparse", family, shape)
    vals, meta, _, _ = gpu_compress(p["A_logical"])
    D, name = gpu_sparse_gemm(vals, meta, p["B"], p["C"], M, N, K, algo="auto")
    assert name.startswith(family), name
    Dr, Y, S = orc.gemm(p["A_logical"], p["B"], p["C"], None, M, N, K, "f16", "f16", "f32")
    r = check(D, "f32", Dr, Y, S, "f16")
    say("  ", r)
    assert r.ok, r


@pytest.mark.parametrize("family", ["sparse24_tiled", "sparse24_dma8"])
@pytest.mark.parametrize("d_type", ["bf16", "f16"])
def test_sparse_epilogue_bit_exact(orc, monkeypatch, family, d_type):
    """The fused epilogue of the SMFMAC kernels equals the oracle's fp32
    epilogue applied to the same kernel's fp32 output, bit for bit."""
    monkeypatch.setenv("STGEMM_FORCE_KERNEL", family)
    M, N, K = 384, 320, 256
    p = inputs.sparse24_f16(M=M, N=N, K=K)
    bias = np.random.default_rng(4).standard_normal(N).astype(np.float32)
    vals, meta, _, _ = gpu_compress(p["A_logical"])
    T, n1 = gpu_sparse_gemm(vals, meta, p["B"], p["C"], M, N, K, "f32", algo="auto")
    D, n2 = gpu_sparse_gemm(vals, meta, p["B"], p["C"], M, N, K, d_type, algo="auto", bias=bias,
                            alpha=0.3, relu=True)
    assert n1.startswith(family) and n2.startswith(family), (n1, n2)
    ref = orc.epilogue_f32(T, 0.3, bias, True, d_type)
    mism = int((D != ref).sum())
    say("sparse epilogue", family, d_type, "mismatches", mism)
    assert mism == 0


def test_sparse_dma8_needs_whole_metadata_groups():
    """K not a multiple of 256 goes to the 4-wave SMFMAC kernel."""
    for K, name in [(256, "sparse24_dma8"), (512, "sparse24_dma8"), (192, "sparse24_tiled"),
                    (320, "sparse24_tiled")]:
        plan = G.gemm_plan(G.make_desc(512, 512, K, "f16", "f16", "f32", sparse_a=True))
        assert plan.name.startswith(name), (K, plan.name)


# ---------------------------------------------------------------- bf16, s8, fp8 A
# The same 2:4 format for the other types with a sparse form (the sparse
# BF16, INT8 and FP8 rows of the instruction tables on "NVIDIA MMA").

TYPES = ["bf16", "s8", "e4m3", "e5m2"]
PAIRS = [("bf16", "bf16"), ("s8", "s8"), ("e4m3", "e5m2"), ("e4m3", "e4m3"), ("e5m2", "e4m3"),
         ("e5m2", "e5m2")]


def _problem(a_type, b_type, M, N, K):
    if a_type in ("e4m3", "e5m2"):
        return inputs.sparse24_fp8(M, N, K, a_type=a_type, b_type=b_type)
    return inputs.sparse24(a_type, M, N, K)


def _gpu_vs_oracle(orc, p, vals, meta, d_type=None, alpha=None, bias=True, relu=None,
                   b_col=True):
    M, N, K = p["M"], p["N"], p["K"]
    d_type = d_type or p["d_type"]
    alpha = p["alpha"] if alpha is None else alpha
    relu = p["relu"] if relu is None else relu
    bias = p["bias"] if bias else None
    B = p["B"] if b_col else np.ascontiguousarray(p["B"].T)
    D, name = gpu_sparse_gemm(vals, meta, B, p["C"], M, N, K, d_type, bias=bias, alpha=alpha,
                              relu=relu, b_col=b_col, a_type=p["a_type"], b_type=p["b_type"])
    Dr, Y, S = orc.gemm(p["A_logical"], B, p["C"], bias, M, N, K, p["a_type"], p["b_type"],
                        d_type, alpha=alpha, relu=relu, b_col_major=b_col)
    return check(D, d_type, Dr, Y, S, p["a_type"], alpha), name


def _host_bytes(t, n, dtype):
    return t.cpu().numpy()[:n].view(dtype)


@pytest.mark.parametrize("t", TYPES)
@pytest.mark.parametrize("M,K", [(1, 4), (3, 36), (130, 200), (257, 1024), (64, 4100)])
def test_compress_matches_oracle_types(orc, t, M, K):
    p = inputs.sparse24(t, M, 4, K)
    say("compress", t, M, K)
    vals, meta, vb, mb = gpu_compress(p["A_logical"], t)
    rv, rm = orc.sparse24_compress(p["A_logical"], t)
    assert np.array_equal(_host_bytes(vals, vb, rv.dtype).reshape(rv.shape), rv)
    assert np.array_equal(_host_bytes(meta, mb, np.uint32).reshape(rm.shape), rm)


@pytest.mark.parametrize("t", ["s8", "e4m3", "e5m2"])
def test_compress_8_bit_zero_codes(orc, t):
    """Groups with fewer than two non-zeros; 0x80 is -0 (a zero) in fp8 and
    -128 (a non-zero) in s8."""
    rng = np.random.default_rng(6)
    M, K = 64, 256
    A = inputs.sparse24(t, M, 4, K)["A_logical"].copy()
    g = A.view(np.uint8).reshape(M, K // 4, 4)
    g[(rng.random(g.shape) < 0.3) & (g != 0)] = 0
    if t == "s8":
        g[(rng.random(g.shape) < 0.2) & (g != 0)] = 0x80
    else:
        g[(rng.random(g.shape) < 0.2) & (g == 0)] = 0x80
    A = g.reshape(M, K).view(A.dtype)
    vals, meta, vb, mb = gpu_compress(A, t)
    rv, rm = orc.sparse24_compress(A, t)
    assert np.array_equal(_host_bytes(vals, vb, rv.dtype).reshape(rv.shape), rv)
    assert np.array_equal(_host_bytes(meta, mb, np.uint32).reshape(rm.shape), rm)


@pytest.mark.parametrize("t", ["bf16", "s8"])
def test_compress_rejects_three_nonzeros_types(t):
    A = inputs.sparse24(t, 32, 4, 64)["A_logical"].copy()
    A[21, 8:12] = (inputs.to_bf16(np.array([1.0, 2.0, 3.0, 0.0])) if t == "bf16"
                   else np.array([1, 2, 3, 0], np.int8))
    with pytest.raises(G.GemmError) as e:
        gpu_compress(A, t)
    assert e.value.status == G.GEMM_ERR_NOT_SPARSE24
    assert "21" in str(e.value)


# family -> shapes: ragged M and N, one and several K tiles (a K tile is 64
# logical K of a 16-bit type, 128 of an 8-bit type; the 8-wave kernel takes K
# in multiples of 256, the 4-wave kernel in whole tiles)
_FAMILY_SHAPES = {
    "sparse24_dma8": [(600, 520, 256), (300, 700, 768), (40, 1000, 1280)],
    "sparse24_tiled": [(600, 520, 384), (256, 256, 128), (130, 300, 640)],
    "sparse24_generic": [(129, 257, 96), (17, 9, 20)],
}


@pytest.mark.parametrize("pair", PAIRS, ids=["x".join(p) for p in PAIRS])
@pytest.mark.parametrize("family", list(_FAMILY_SHAPES))
def test_sparse_parity_types(orc, monkeypatch, pair, family):
    """Every kernel family for every type pair, with each workload's own
    epilogue (C for bf16 and s8; alpha, bias and relu into fp16 for fp8)."""
    monkeypatch.setenv("STGEMM_FORCE_KERNEL", family)
    for M, N, K in _FAMILY_SHAPES[family]:
        p = _problem(pair[0], pair[1], M, N, K)
        say("sparse", pair, family, (M, N, K))
        vals, meta, _, _ = gpu_compress(p["A_logical"], pair[0])
        r, name = _gpu_vs_oracle(orc, p, vals, meta)
        say("  ", name, r)
        assert name.startswith(family), name
        assert r.ok, r


@pytest.mark.parametrize("pair", [("bf16", "bf16"), ("e4m3", "e5m2"), ("e5m2", "e5m2")],
                         ids=["bf16", "e4m3xe5m2", "e5m2xe5m2"])
@pytest.mark.parametrize("family", ["sparse24_dma8", "sparse24_tiled"])
def test_sparse_parity_types_f32_out(orc, monkeypatch, pair, family):
    """fp32 output without an epilogue: the accumulator itself."""
    monkeypatch.setenv("STGEMM_FORCE_KERNEL", family)
    M, N, K = 520, 264, 1024
    p = _problem(pair[0], pair[1], M, N, K)
    vals, meta, _, _ = gpu_compress(p["A_logical"], pair[0])
    r, name = _gpu_vs_oracle(orc, p, vals, meta, d_type="f32", alpha=1.0, bias=False, relu=False)
    say("  ", name, r)
    assert name.startswith(family) and r.ok, (name, r)


@pytest.mark.parametrize("pair", [("bf16", "bf16"), ("e4m3", "e5m2")], ids=["bf16", "fp8"])
@pytest.mark.parametrize("family", ["sparse24_dma8", "sparse24_tiled"])
@pytest.mark.parametrize("d_type", ["bf16", "f16"])
def test_sparse_epilogue_bit_exact_types(orc, monkeypatch, pair, family, d_type):
    monkeypatch.setenv("STGEMM_FORCE_KERNEL", family)
    M, N, K = 384, 320, 512
    p = _problem(pair[0], pair[1], M, N, K)
    bias = np.random.default_rng(4).standard_normal(N).astype(np.float32)
    vals, meta, _, _ = gpu_compress(p["A_logical"], pair[0])
    kw = dict(a_type=pair[0], b_type=pair[1])
    T, n1 = gpu_sparse_gemm(vals, meta, p["B"], p["C"], M, N, K, "f32", **kw)
    D, n2 = gpu_sparse_gemm(vals, meta, p["B"], p["C"], M, N, K, d_type, bias=bias, alpha=0.3,
                            relu=True, **kw)
    assert n1.startswith(family) and n2.startswith(family), (n1, n2)
    ref = orc.epilogue_f32(T, 0.3, bias, True, d_type)
    mism = int((D != ref).sum())
    say("  ", n2, d_type, "mismatches:", mism)
    assert mism == 0


@pytest.mark.parametrize("t", ["s8", "e4m3"])
def test_sparse_row_major_b_and_misaligned_values_types(orc, t):
    """Row-major B runs the generic kernel; values not 16-byte aligned make a
    tiled plan fall back to it at run time."""
    M, N, K = 96, 80, 256
    p = _problem(t, "e5m2" if t == "e4m3" else t, M, N, K)
    vals, meta, vb, _ = gpu_compress(p["A_logical"], t)
    r, name = _gpu_vs_oracle(orc, p, vals, meta, b_col=False)
    assert name.startswith("sparse24_generic") and r.ok, (name, r)
    shifted = torch.zeros(vb + 32, dtype=torch.uint8, device="cuda")
    shifted[2:2 + vb] = vals[:vb]
    r, name = _gpu_vs_oracle(orc, p, shifted[2:], meta)
    assert name.startswith("sparse24_dma8") and r.ok, (name, r)


@pytest.mark.parametrize("t", ["s8", "e4m3"])
def test_sparse_dma8_needs_whole_metadata_groups_types(monkeypatch, t):
    """The 8-wave kernel takes K in multiples of 256 for 8-bit types too; the
    4-wave kernel takes whole 128-wide tiles; other K run the generic kernel."""
    b = "e5m2" if t == "e4m3" else t
    d = "s32" if t == "s8" else "f32"
    for K, fam in [(256, "sparse24_dma8"), (384, "sparse24_tiled"), (192, "sparse24_generic")]:
        plan = G.gemm_plan(G.make_desc(512, 512, K, t, b, d, sparse_a=True))
        assert plan.name.startswith(fam), (K, plan.name)
    monkeypatch.setenv("STGEMM_FORCE_KERNEL", "sparse24_dma8")
    plan = G.gemm_plan(G.make_desc(512, 512, 384, t, b, d, sparse_a=True))
    assert not plan.name.startswith("sparse24_dma8")
