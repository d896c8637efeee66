"""GPU parity of the MX block-scaled path ("NVIDIA MMA", section "Blackwell:
FP4/FP6 and block-scaled MMA"): every pair of element formats through the
generic kernel, the tiled kernel for pairs of one width, the 6-bit pairs
through the expansion to 8-bit codes and the tiled kernel, ragged shapes,
padded rows, the run-time fallbacks, and the fused epilogue bit for bit -
all against the oracle's block-scaled GEMM on the same packed bytes."""
import numpy as np
import pytest
import torch

from checks import check
from gpu_util import OUT_NP, empty_out, say, to_dev
from sparse_tiled_gemm_amd import gemm as G
from sparse_tiled_gemm_amd import inputs

pytestmark = pytest.mark.gpu

FMTS = ["e4m3", "e5m2", "e2m3", "e3m2", "e2m1"]
TILED_PAIRS = [("e4m3", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e4m3"), ("e5m2", "e5m2"),
               ("e2m1", "e2m1")]
# pairs with a 6-bit operand and a 6- or 8-bit partner
TILED6_PAIRS = [("e2m3", "e2m3"), ("e3m2", "e3m2"), ("e2m3", "e3m2"), ("e3m2", "e2m3"),
                ("e2m3", "e4m3"), ("e5m2", "e3m2")]


def _problem(a, b, M, N, K, seed=40):
    return inputs.mx_problem(M, N, K, a, b, workload=seed, d_type="f32")


def _extras(M, N, seed):
    rng = np.random.default_rng(seed)
    C = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32)
    return C, bias


def gpu_mx(p, d_type="f32", C=None, bias=None, alpha=1.0, relu=False, algo="auto", lda=0,
           ldb=0, A=None, B=None, a_dev=None):
    M, N, K = p["M"], p["N"], p["K"]
    desc = G.make_desc(M, N, K, p["a_type"], p["b_type"], d_type, has_c=C is not None,
                       has_bias=bias is not None, alpha=alpha, act="relu" if relu else "none",
                       lda=lda, ldb=ldb, algo=algo, block_scale=32)
    plan = G.gemm_plan(desc)
    tA = a_dev if a_dev is not None else to_dev(p["A"] if A is None else A)
    tB = to_dev(p["B"] if B is None else B)
    tSA, tSB = to_dev(p["SA"]), to_dev(p["SB"])
    tC = to_dev(C) if C is not None else None
    tb = to_dev(bias) if bias is not None else None
    D = empty_out(M, N, d_type)
    G.gemm_mx_run(plan, tA, tSA, tB, tSB, tC, tb, D)
    torch.cuda.synchronize()
    return D.cpu().numpy().view(OUT_NP[d_type]).reshape(M, N).copy(), plan.name


def _vs_oracle(orc, p, D, d_type="f32", C=None, bias=None, alpha=1.0, relu=False):
    M, N, K = p["M"], p["N"], p["K"]
    Dr, Y, S = orc.mx_gemm(p["A"], p["SA"], p["B"], p["SB"], C, bias, M, N, K, p["a_type"],
                           p["b_type"], d_type, alpha=alpha, relu=relu)
    return check(D, d_type, Dr, Y, S, p["a_type"], alpha)


@pytest.mark.parametrize("a", FMTS)
def test_mx_generic_every_pair(orc, a):
    """All 25 format pairs; K = 96 leaves the last instruction half empty."""
    for b in FMTS:
        for (M, N, K) in [(67, 45, 96), (33, 70, 256)]:
            p = _problem(a, b, M, N, K)
            C, _ = _extras(M, N, 1)
            say("mx generic", a, b, (M, N, K))
            D, name = gpu_mx(p, C=C, algo="generic")
            assert name.startswith("mx_generic"), name
            r = _vs_oracle(orc, p, D, C=C)
            say("  ", r)
            assert r.ok, (a, b, r)


@pytest.mark.parametrize("pair", TILED_PAIRS, ids=["x".join(q) for q in TILED_PAIRS])
def test_mx_tiled(orc, pair):
    for (M, N, K) in [(600, 520, 512), (256, 256, 1024), (130, 300, 1536), (17, 700, 512)]:
        p = _problem(pair[0], pair[1], M, N, K, seed=41)
        C, _ = _extras(M, N, 2)
        say("mx tiled", pair, (M, N, K))
        D, name = gpu_mx(p, C=C)
        assert name.startswith("mx_tiled"), name
        r = _vs_oracle(orc, p, D, C=C)
        say("  ", r)
        assert r.ok, r


@pytest.mark.parametrize("pair", TILED6_PAIRS, ids=["x".join(q) for q in TILED6_PAIRS])
def test_mx_tiled6(orc, pair):
    """Every 6-bit code (subnormals, both zeros, the largest) reaches the
    product: uniform codes rather than quantised normals."""
    for (M, N, K) in [(600, 520, 512), (130, 300, 1536), (17, 700, 512)]:
        p = _problem(pair[0], pair[1], M, N, K, seed=45)
        rng = np.random.default_rng(M + N)
        for side, rows in (("A", M), ("B", N)):
            f = p[side.lower() + "_type"]
            if inputs.MX_BITS[f] == 6:
                p[side] = inputs.mx_pack(rng.integers(0, 64, (rows, K)), f)
        C, _ = _extras(M, N, 5)
        say("mx tiled6", pair, (M, N, K))
        D, name = gpu_mx(p, C=C)
        assert name.startswith("mx_tiled6"), name
        r = _vs_oracle(orc, p, D, C=C)
        say("  ", r)
        assert r.ok, r


def test_mx_tiled6_repeated_calls(orc):
    """Back-to-back calls of different sizes on one stream reuse the
    expansion's temporaries; each result stays right."""
    outs = []
    for (M, N, K, seed) in [(512, 512, 2048, 46), (300, 200, 512, 47), (512, 512, 2048, 48)]:
        p = _problem("e3m2", "e2m3", M, N, K, seed=seed)
        M, N, K = p["M"], p["N"], p["K"]
        desc = G.make_desc(M, N, K, "e3m2", "e2m3", "f32", has_c=False, block_scale=32)
        plan = G.gemm_plan(desc)
        D = empty_out(M, N, "f32")
        G.gemm_mx_run(plan, to_dev(p["A"]), to_dev(p["SA"]), to_dev(p["B"]), to_dev(p["SB"]),
                      None, None, D)
        outs.append((p, D, plan.name))
    torch.cuda.synchronize()
    for p, D, name in outs:
        assert name.startswith("mx_tiled6"), name
        r = _vs_oracle(orc, p, D.cpu().numpy().view(np.float32).reshape(p["M"], p["N"]))
        assert r.ok, r


@pytest.mark.parametrize("pair", [("e4m3", "e4m3"), ("e2m1", "e2m1"), ("e2m3", "e3m2")],
                         ids=["mxfp8", "mxfp4", "mxfp6"])
@pytest.mark.parametrize("d_type", ["bf16", "f16"])
def test_mx_epilogue(orc, pair, d_type):
    """The fused epilogue bit for bit against the oracle's fp32 epilogue on
    the same kernel's fp32 output, and the cast result against the oracle."""
    M, N, K = 384, 320, 1024
    p = _problem(pair[0], pair[1], M, N, K, seed=42)
    C, bias = _extras(M, N, 3)
    T, n1 = gpu_mx(p, "f32", C=C)
    D, n2 = gpu_mx(p, d_type, C=C, bias=bias, alpha=0.3, relu=True)
    assert n1 == n2
    ref = orc.epilogue_f32(T, 0.3, bias, True, d_type)
    assert int((D != ref).sum()) == 0
    r = _vs_oracle(orc, p, D, d_type, C=C, bias=bias, alpha=0.3, relu=True)
    assert r.ok, r


def _pad_rows(packed, extra_bytes):
    rows = packed.shape[0]
    return np.concatenate([packed, np.zeros((rows, extra_bytes), np.uint8)], axis=1)


@pytest.mark.parametrize("fmt,pad_elems", [("e2m1", 32), ("e4m3", 16), ("e2m3", 4),
                                           ("e2m3", 16), ("e2m3", 32), ("e3m2", 8)])
def test_mx_padded_rows(orc, fmt, pad_elems):
    M, N, K = 200, 150, 512
    p = _problem(fmt, fmt, M, N, K, seed=43)
    bits = inputs.MX_BITS[fmt]
    A = _pad_rows(p["A"], pad_elems * bits // 8)
    B = _pad_rows(p["B"], pad_elems * bits // 8)
    D, name = gpu_mx(p, lda=K + pad_elems, ldb=K + pad_elems, A=A, B=B)
    say("  padded", fmt, name)
    if bits == 6:   # the expansion reads 4-byte words: rows of a multiple of 4 bytes
        want = "mx_tiled6" if pad_elems * bits % 32 == 0 else "mx_generic"
    else:
        want = "mx_tiled" if pad_elems * bits % 128 == 0 else "mx_generic"
    assert name.startswith(want), name
    r = _vs_oracle(orc, p, D)
    assert r.ok, r


@pytest.mark.parametrize("pair,off", [(("e4m3", "e5m2"), 8), (("e2m3", "e3m2"), 2),
                                      (("e4m3", "e3m2"), 4), (("e2m3", "e3m2"), 4),
                                      (("e2m3", "e3m2"), 8)])
def test_mx_misaligned_a_falls_back(orc, pair, off):
    """A off the alignment the tiled path reads it with (16 bytes for 8-bit
    codes, 4 for packed 6-bit ones): the run takes the generic kernel.  A
    6-bit pair 4- but not 8-byte aligned takes the 8-bit code expansion
    instead of the padded regrouping; 8-byte aligned, the regrouping."""
    M, N, K = 160, 96, 512
    p = _problem(pair[0], pair[1], M, N, K, seed=44)
    buf = torch.zeros(p["A"].size + 64, dtype=torch.uint8, device="cuda")
    buf[off:off + p["A"].size] = to_dev(p["A"]).view(-1)
    D, name = gpu_mx(p, a_dev=buf[off:])
    assert name.startswith("mx_tiled")  # the plan; the run used the generic kernel
    r = _vs_oracle(orc, p, D)
    assert r.ok, r


def test_mx_plan_choice():
    def name(a, b, K):
        return G.gemm_plan(G.make_desc(512, 512, K, a, b, "f32", has_c=False,
                                       block_scale=32)).name
    assert name("e4m3", "e5m2", 512).startswith("mx_tiled")
    assert name("e2m1", "e2m1", 1024).startswith("mx_tiled")
    assert name("e4m3", "e4m3", 96).startswith("mx_generic")    # K % 512
    assert name("e2m1", "e2m1", 256).startswith("mx_generic")
    assert name("e2m1", "e4m3", 512).startswith("mx_generic")   # two widths
    assert name("e2m3", "e2m3", 512).startswith("mx_tiled6")
    assert name("e3m2", "e4m3", 1024).startswith("mx_tiled6")
    assert name("e5m2", "e2m3", 512).startswith("mx_tiled6")
    assert name("e2m3", "e2m1", 512).startswith("mx_generic")   # 6-bit with 4-bit
    assert name("e2m3", "e3m2", 256).startswith("mx_generic")   # K % 512
    with pytest.raises(G.GemmError):
        G.gemm_plan(G.make_desc(512, 512, 96, "e4m3", "e4m3", "f32", has_c=False,
                                block_scale=32, algo="tiled"))


def test_mx_run_rejects_plain_plans():
    plan = G.gemm_plan(G.make_desc(64, 64, 64, "e4m3", "e4m3", "f32", has_c=False))
    t = torch.zeros(64 * 64 * 4, dtype=torch.uint8, device="cuda")
    with pytest.raises(G.GemmError):
        G.gemm_mx_run(plan, t, t, t, t, None, None, t)
    mx = G.gemm_plan(G.make_desc(64, 64, 64, "e4m3", "e4m3", "f32", has_c=False,
                                 block_scale=32))
    with pytest.raises(G.GemmError):
        G.gemm_run(mx, t, t, None, None, t)
    with pytest.raises(G.GemmError) as e:
        G.gemm_mx_run(mx, t, None, t, t, None, None, t)
    assert e.value.status == G.GEMM_ERR_NULL_POINTER
