"""GPU parity of the saturating int32 output (descriptor flag `saturate`):
D = clamp(sum_k a b + C, -2^31, 2^31 - 1), bit for bit against the oracle,
for every kernel family that produces int32 outputs (dense tiled, 128 x 128,
generic, skinny, MN-major; 2:4 direct-copy and generic), on both epilogue
paths (vector and scalar C access), with C placed near both int32 bounds so
that part of the outputs saturate and part do not; and the wrapping default
on the same inputs."""
import numpy as np
import pytest
import torch

from gpu_util import gpu_compress, gpu_gemm, gpu_sparse_gemm, say, to_dev
from sparse_tiled_gemm_amd import gemm as G
from sparse_tiled_gemm_amd import inputs

pytestmark = pytest.mark.gpu

I32_MAX, I32_MIN = 2**31 - 1, -(2**31)


def _c_near_bounds(M, N, seed):
    """C: a third near +2^31, a third near -2^31, a third small."""
    rng = np.random.default_rng(seed)
    r = rng.integers(0, 100000, size=(M, N), dtype=np.int64)
    pick = rng.integers(0, 3, size=(M, N))
    C = np.where(pick == 0, I32_MAX - r, np.where(pick == 1, I32_MIN + r, r - 50000))
    return C.astype(np.int32)


def _check(orc, D, A, B, C, M, N, K, saturate, a_col=False, b_col=True):
    Dr, _, _ = orc.gemm(A, B, C, None, M, N, K, "s8", "s8", "s32", a_col_major=a_col,
                        b_col_major=b_col, saturate=saturate)
    bad = int((D != Dr).sum())
    sat = int(((Dr == I32_MAX) | (Dr == I32_MIN)).sum())
    say("  saturate" if saturate else "  wrap", "mismatches", bad, "clamped outputs", sat)
    assert bad == 0
    if saturate:
        assert sat > M * N // 10, sat  # the case exercises the clamp
    return sat


@pytest.mark.parametrize("fam,shape", [("tiled256w8t", (520, 300, 256)),
                                       ("tiled128", (200, 136, 128)),
                                       ("generic", (70, 90, 100)),
                                       ("skinny", (16, 264, 512)),
                                       ("tiled256w8tk16", (520, 300, 256)),
                                       ("tiled256w8k16", (300, 520, 192))],
                         ids=["tiled256w8t", "tiled128", "generic", "skinny", "tiled256w8tk16",
                              "tiled256w8k16"])
@pytest.mark.parametrize("saturate", [True, False], ids=["sat", "wrap"])
def test_dense_s32_saturation(orc, monkeypatch, fam, shape, saturate):
    monkeypatch.setenv("STGEMM_FORCE_KERNEL", fam)
    M, N, K = shape
    p = inputs.dense_s8(M, N, K)
    C = _c_near_bounds(M, N, seed=M)
    desc = G.make_desc(M, N, K, "s8", "s8", "s32", saturate=saturate)
    plan = G.gemm_plan(desc)
    assert plan.name.startswith(fam), plan.name
    D = torch.empty(M * N, dtype=torch.int32, device="cuda")
    G.gemm_run(plan, to_dev(p["A"]), to_dev(p["B"]), to_dev(C), None, D)
    torch.cuda.synchronize()
    say("dense", plan.name, shape)
    _check(orc, D.cpu().numpy().reshape(M, N), p["A"], p["B"], C, M, N, K, saturate)


def test_scalar_epilogue_path_saturates(orc, monkeypatch):
    """ldc = N + 1 rules out the vector epilogue: the per-element store path."""
    monkeypatch.setenv("STGEMM_FORCE_KERNEL", "tiled256w8t")
    M, N, K = 264, 260, 128
    p = inputs.dense_s8(M, N, K)
    C = _c_near_bounds(M, N, seed=3)
    Cp = np.zeros((M, N + 1), dtype=np.int32)
    Cp[:, :N] = C
    D, name = gpu_gemm(p["A"], p["B"], None, None, M, N, K, "s8", "s8", "s32", ldc=N + 1,
                       c_dev=to_dev(Cp), saturate=True)
    say("scalar path", name)
    _check(orc, D, p["A"], p["B"], C, M, N, K, True)


def test_mn_major_saturates(orc):
    """A column-major, B row-major int8 on the tiled kernel."""
    M, N, K = 512, 272, 256
    p = inputs.dense_s8(M, N, K)
    At, Bt = np.ascontiguousarray(p["A"].T), np.ascontiguousarray(p["B"].T)
    C = _c_near_bounds(M, N, seed=5)
    D, name = gpu_gemm(At, Bt, C, None, M, N, K, "s8", "s8", "s32", a_col=True, b_col=False,
                       saturate=True)
    say("mn", name)
    assert name.endswith("_acol_brow"), name
    _check(orc, D, At, Bt, C, M, N, K, True, a_col=True, b_col=False)


@pytest.mark.parametrize("algo", ["tiled", "generic"])
def test_sparse_s8_saturation(orc, algo):
    M, N, K = 300, 264, 512
    p = inputs.sparse24("s8", M, N, K)
    C = _c_near_bounds(M, N, seed=7)
    vals, meta, _, _ = gpu_compress(p["A_logical"], "s8")
    D, name = gpu_sparse_gemm(vals, meta, p["B"], C, M, N, K, "s32", algo=algo, a_type="s8",
                              saturate=True)
    say("sparse", name)
    _check(orc, D, p["A_logical"], p["B"], C, M, N, K, True)


def test_saturate_validation():
    def plan(**kw):
        return G.gemm_plan(G.make_desc(256, 256, kw.pop("K", 256), "s8", "s8",
                                       kw.pop("d", "s32"), **kw))
    assert plan(saturate=True).name.startswith("tiled")
    with pytest.raises(G.GemmError):  # float outputs do not saturate
        plan(d="bf16", saturate=True)
    with pytest.raises(G.GemmError):  # the int32 sum itself could overflow
        plan(K=131072, saturate=True)
    assert plan(K=131072 - 64, saturate=True) is not None
