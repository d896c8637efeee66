"""GPU parity of the W4A16 path ("NVIDIA MMA", section "How quantisation
configurations map to MMA": INT4 weights dequantised to FP16 / BF16 in the
main loop, then a float MMA): the tiled and generic kernels against the
oracle's dequantisation followed by its dense GEMM, several group sizes,
with and without zero points, the fused epilogue bit for bit, the
misaligned fallback and the plan choice."""
import numpy as np
import pytest
import torch

from checks import check
from gpu_util import OUT_NP, empty_out, say, to_dev
from sparse_tiled_gemm_amd import gemm as G
from sparse_tiled_gemm_amd import inputs

pytestmark = pytest.mark.gpu


def gpu_w4(p, d_type=None, C=None, bias=None, alpha=1.0, relu=False, algo="auto", b_dev=None,
           zeros=True):
    M, N, K = p["M"], p["N"], p["K"]
    d_type = d_type or p["d_type"]
    desc = G.make_desc(M, N, K, p["a_type"], "u4", d_type, has_c=C is not None,
                       has_bias=bias is not None, alpha=alpha, act="relu" if relu else "none",
                       algo=algo, block_scale=p["gs"])
    plan = G.gemm_plan(desc)
    tA = to_dev(p["A"])
    tB = b_dev if b_dev is not None else to_dev(p["B"])
    tS = to_dev(p["scales"])
    tZ = to_dev(p["zeros"]) if (zeros and p["zeros"] is not None) else None
    tC = to_dev(C) if C is not None else None
    tb = to_dev(bias) if bias is not None else None
    D = empty_out(M, N, d_type)
    G.gemm_w4a16_run(plan, tA, tB, tS, tZ, tC, tb, D)
    torch.cuda.synchronize()
    return D.cpu().numpy().view(OUT_NP[d_type]).reshape(M, N).copy(), plan.name


def _vs_oracle(orc, p, D, d_type=None, C=None, bias=None, alpha=1.0, relu=False):
    M, N, K = p["M"], p["N"], p["K"]
    d_type = d_type or p["d_type"]
    W = orc.w4a16_dequant(p["B"], p["scales"], p["zeros"], N, K, p["gs"], p["a_type"])
    Dr, Y, S = orc.gemm(p["A"], W, C, bias, M, N, K, p["a_type"], p["a_type"], d_type,
                        alpha=alpha, relu=relu)
    return check(D, d_type, Dr, Y, S, p["a_type"], alpha)


def _C(M, N, seed=1):
    return np.random.default_rng(seed).uniform(-1, 1, (M, N)).astype(np.float32)


# the 4-wave kernel on the 32x32 forms and the 16x16-form kernel, each
# forced through the tuning override
W4_TILED = ["w4_tiled", "w4_tiled16"]


@pytest.mark.parametrize("family", W4_TILED)
@pytest.mark.parametrize("a_type", ["bf16", "f16"])
@pytest.mark.parametrize("gs", [32, 64, 128])
def test_w4_tiled(orc, monkeypatch, family, a_type, gs):
    monkeypatch.setenv("STGEMM_FORCE_KERNEL", family)
    for (M, N, K) in [(600, 520, 512), (256, 256, 128), (130, 300, 1024), (17, 700, 256)]:
        p = inputs.w4a16_problem(M, N, K, a_type, gs, workload=60)
        C = _C(M, N)
        say("w4 tiled", family, a_type, gs, (M, N, K))
        D, name = gpu_w4(p, "f32", C=C)
        assert name.startswith(family + "_"), name
        r = _vs_oracle(orc, p, D, "f32", C=C)
        say("  ", r)
        assert r.ok, r


@pytest.mark.parametrize("a_type", ["bf16", "f16"])
def test_w4_generic(orc, a_type):
    for (M, N, K, gs) in [(129, 257, 96, 32), (17, 9, 64, 64), (70, 33, 256, 128)]:
        p = inputs.w4a16_problem(M, N, K, a_type, gs, workload=61)
        C = _C(M, N, 2)
        D, name = gpu_w4(p, "f32", C=C, algo="generic")
        assert name.startswith("w4_generic"), name
        r = _vs_oracle(orc, p, D, "f32", C=C)
        say("  generic", (M, N, K, gs), r)
        assert r.ok, r


@pytest.mark.parametrize("a_type", ["bf16", "f16"])
@pytest.mark.parametrize("gs", [32, 128])
def test_w4_skinny(orc, a_type, gs):
    """M <= 16: the skinny kernel, codes streamed and dequantised in registers."""
    for (M, N, K) in [(1, 700, 1024), (5, 96, 2048), (16, 8192, 1024), (16, 130, 4096)]:
        p = inputs.w4a16_problem(M, N, K, a_type, gs, workload=65)
        C = _C(M, N, 5)
        D, name = gpu_w4(p, "f32", C=C)
        assert name.startswith("w4_skinny"), name
        r = _vs_oracle(orc, p, D, "f32", C=C)
        say("  skinny", a_type, gs, (M, N, K), r)
        assert r.ok, r
    p = inputs.w4a16_problem(16, 512, 1024, a_type, gs, workload=66, zeros=False)
    D, name = gpu_w4(p, a_type)
    assert name.startswith("w4_skinny") and _vs_oracle(orc, p, D, a_type).ok


@pytest.mark.parametrize("algo", ["auto", "generic", "w4_tiled16"])
def test_w4_without_zero_points(orc, monkeypatch, algo):
    if algo == "w4_tiled16":
        monkeypatch.setenv("STGEMM_FORCE_KERNEL", algo)
        algo = "auto"
    M, N, K = 300, 264, 512
    p = inputs.w4a16_problem(M, N, K, "bf16", 128, workload=62, zeros=False)
    assert p["zeros"] is None
    D, name = gpu_w4(p, "bf16", algo=algo)
    r = _vs_oracle(orc, p, D, "bf16")
    assert r.ok, r


@pytest.mark.parametrize("family", W4_TILED)
@pytest.mark.parametrize("a_type", ["bf16", "f16"])
@pytest.mark.parametrize("d_type", ["bf16", "f16"])
def test_w4_epilogue_bit_exact(orc, monkeypatch, family, a_type, d_type):
    monkeypatch.setenv("STGEMM_FORCE_KERNEL", family)
    M, N, K = 384, 320, 512
    p = inputs.w4a16_problem(M, N, K, a_type, 64, workload=63)
    C = _C(M, N, 3)
    bias = np.random.default_rng(4).standard_normal(N).astype(np.float32)
    T, n1 = gpu_w4(p, "f32", C=C)
    D, n2 = gpu_w4(p, d_type, C=C, bias=bias, alpha=0.3, relu=True)
    assert n1 == n2 and n1.startswith(family + "_")
    ref = orc.epilogue_f32(T, 0.3, bias, True, d_type)
    assert int((D != ref).sum()) == 0
    r = _vs_oracle(orc, p, D, d_type, C=C, bias=bias, alpha=0.3, relu=True)
    assert r.ok, r


def test_w4_misaligned_b_falls_back(orc):
    M, N, K = 160, 96, 256
    p = inputs.w4a16_problem(M, N, K, "bf16", 128, workload=64)
    buf = torch.zeros(p["B"].size + 64, dtype=torch.uint8, device="cuda")
    buf[8:8 + p["B"].size] = to_dev(p["B"]).view(-1)
    D, name = gpu_w4(p, "f32", b_dev=buf[8:])
    assert name.startswith("w4_tiled")  # the plan; the run used the generic kernel
    r = _vs_oracle(orc, p, D, "f32")
    assert r.ok, r


def test_w4_plan_choice_and_errors():
    def plan(K, gs, **kw):
        return G.gemm_plan(G.make_desc(512, 512, K, "bf16", "u4", "bf16", has_c=False,
                                       block_scale=gs, **kw))
    assert plan(512, 128).name.startswith("w4_tiled")
    assert G.gemm_plan(G.make_desc(16, 512, 512, "bf16", "u4", "bf16", has_c=False,
                                   block_scale=128)).name.startswith("w4_skinny")
    assert G.gemm_plan(G.make_desc(16, 512, 480, "bf16", "u4", "bf16", has_c=False,
                                   block_scale=32)).name.startswith("w4_tiled")  # K % 128
    assert plan(512, 128, lda=520).name.startswith("w4_tiled")     # 1040-byte A rows
    assert plan(512, 128, lda=516).name.startswith("w4_generic")   # A rows not 16-byte
    assert plan(512, 128, ldb=520).name.startswith("w4_generic")   # code rows of 260 bytes
    with pytest.raises(G.GemmError):
        plan(512, 48)
    t = torch.zeros(512 * 512 * 4, dtype=torch.uint8, device="cuda")
    pl = plan(512, 128)
    with pytest.raises(G.GemmError):
        G.gemm_run(pl, t, t, None, None, t)
    with pytest.raises(G.GemmError) as e:
        G.gemm_w4a16_run(pl, t, t, None, None, None, None, t)
    assert e.value.status == G.GEMM_ERR_NULL_POINTER
