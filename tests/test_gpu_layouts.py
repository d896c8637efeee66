"""GPU parity of the MN-major operand layouts on the LDS-tiled kernels: A
column-major (M contiguous) and / or B row-major (N contiguous), 16-bit
types, whose tiles are kept in LDS in memory order and read with the
transposing LDS load.  Against the oracle element by element at sizes that
span several tiles with ragged M/N tails, with padded leading dimensions,
at the full 8192^3 size on sampled entries, and bit for bit against the
K-major kernel on the same values (same K order inside every MFMA)."""
import numpy as np
import pytest
import torch

from checks import check
from gpu_util import OUT_NP, gpu_gemm, say, to_dev
from sparse_tiled_gemm_amd import gemm as G
from sparse_tiled_gemm_amd import inputs

pytestmark = pytest.mark.gpu

CONV = {"f16": inputs.to_f16, "bf16": inputs.to_bf16}
# (a column-major, b column-major): the three layouts with an MN-major operand
MN_LAYOUTS = [(True, True), (False, False), (True, False)]
SUFFIX = {(True, True): "_acol", (False, False): "_brow", (True, False): "_acol_brow"}


def _make(t, M, N, K, a_col, b_col, seed):
    rng = np.random.default_rng(seed)
    A = CONV[t](rng.standard_normal((K, M) if a_col else (M, K)))
    B = CONV[t](rng.standard_normal((N, K) if b_col else (K, N)))
    C = rng.uniform(-1, 1, size=(M, N)).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32)
    return A, B, C, bias


def _oracle_check(orc, D, A, B, C, bias, M, N, K, t, d_type, a_col, b_col, alpha, relu):
    Dr, Y, S = orc.gemm(A, B, C, bias, M, N, K, t, t, d_type, a_col_major=a_col,
                        b_col_major=b_col, alpha=alpha, relu=relu)
    r = check(D, d_type, Dr, Y, S, t, alpha)
    say("  ", r)
    assert r.ok, r


@pytest.mark.parametrize("t", ["f16", "bf16"])
@pytest.mark.parametrize("a_col,b_col", MN_LAYOUTS, ids=["acol", "brow", "acol_brow"])
@pytest.mark.parametrize("fam,shape", [("tiled256w8", (600, 520, 256)),
                                       ("tiled128", (264, 200, 192))],
                         ids=["tiled256w8", "tiled128"])
def test_mn_tiled(orc, monkeypatch, t, a_col, b_col, fam, shape):
    monkeypatch.setenv("STGEMM_FORCE_KERNEL", fam)
    M, N, K = shape
    A, B, C, bias = _make(t, M, N, K, a_col, b_col, seed=M + N)
    relu = t == "bf16"
    D, name = gpu_gemm(A, B, C, bias, M, N, K, t, t, t, alpha=0.75, relu=relu, a_col=a_col,
                       b_col=b_col)
    say("mn", name, t, shape)
    assert name.startswith(fam) and name.endswith(SUFFIX[(a_col, b_col)]), name
    _oracle_check(orc, D, A, B, C, bias, M, N, K, t, t, a_col, b_col, 0.75, relu)


@pytest.mark.parametrize("a_col,b_col", MN_LAYOUTS, ids=["acol", "brow", "acol_brow"])
def test_mn_padded_leading_dims(orc, a_col, b_col):
    """lda / ldb beyond the packed extent (the pad holds NaN, never read into
    a kept output), M and N tails of 8, K of 3 tiles."""
    t, M, N, K = "bf16", 264, 392, 96
    A, B, C, _ = _make(t, M, N, K, a_col, b_col, seed=5)
    lda = (M if a_col else K) + 24
    ldb = (K if b_col else N) + 40
    Ap = np.full((A.shape[0], lda), 0x7FC0, dtype=A.dtype)
    Ap[:, : A.shape[1]] = A
    Bp = np.full((B.shape[0], ldb), 0x7FC0, dtype=B.dtype)
    Bp[:, : B.shape[1]] = B
    D, name = gpu_gemm(A, B, C, None, M, N, K, t, t, "f32", a_col=a_col, b_col=b_col,
                       lda=lda, ldb=ldb, a_dev=to_dev(Ap), b_dev=to_dev(Bp))
    say("mn padded", name, lda, ldb)
    assert name.startswith("tiled") and name.endswith(SUFFIX[(a_col, b_col)]), name
    _oracle_check(orc, D, A, B, C, None, M, N, K, t, "f32", a_col, b_col, 1.0, False)


@pytest.mark.parametrize("a_col,b_col", MN_LAYOUTS, ids=["acol", "brow", "acol_brow"])
def test_mn_matches_k_major_bitwise(a_col, b_col):
    """Same values, MN-major vs K-major storage, same tile family: every MFMA
    sees the same K order, so the outputs are identical bit for bit."""
    t, M, N, K = "f16", 512, 768, 320
    A, B, C, bias = _make(t, M, N, K, False, True, seed=11)
    At = np.ascontiguousarray(A.T) if a_col else A
    Bt = B if b_col else np.ascontiguousarray(B.T)
    for fam in ("tiled256w8", "tiled128"):
        ref, n0 = gpu_gemm(A, B, C, bias, M, N, K, t, t, "f32", algo="tiled256"
                           if fam == "tiled256w8" else "tiled128")
        D, n1 = gpu_gemm(At, Bt, C, bias, M, N, K, t, t, "f32", a_col=a_col, b_col=b_col,
                         algo="tiled256" if fam == "tiled256w8" else "tiled128")
        say("bitwise", n0, n1)
        assert n0.startswith(fam) and n1.startswith(fam), (n0, n1)
        assert np.array_equal(D.view(np.uint32), ref.view(np.uint32)), int((D != ref).sum())


def test_mn_plan_choices(monkeypatch):
    """Which layouts reach the tiled kernels: 16-bit only, M (N) in whole
    16-byte chunks; everything else stays on the generic kernel."""
    def name(M, N, K, t, d, **kw):
        return G.gemm_plan(G.make_desc(M, N, K, t, t, d, has_c=False, **kw)).name
    assert name(8192, 8192, 8192, "bf16", "bf16", a_layout="col") == "tiled256w8_bf16_acol"
    assert name(8192, 8192, 8192, "f16", "f16", b_layout="row") == "tiled256w8_f16_brow"
    assert name(512, 512, 512, "bf16", "bf16", a_layout="col",
                b_layout="row") == "tiled128_bf16_acol_brow"
    # 16 rows: no skinny kernel for MN-major A
    assert name(16, 4096, 4096, "bf16", "bf16", a_layout="col").startswith("tiled128")
    assert name(100, 512, 512, "bf16", "bf16", a_layout="col").startswith("generic")  # M % 8
    assert name(512, 100, 512, "bf16", "bf16", b_layout="row").startswith("generic")  # N % 8
    assert name(512, 512, 80, "bf16", "bf16", b_layout="row").startswith("generic")  # K % 32
    assert name(512, 512, 512, "e4m3", "f32", b_layout="row").startswith("generic")
    assert name(512, 512, 512, "s8", "s32", a_layout="col").startswith("generic")
    # tuning families that do not take MN-major operands are not forced
    monkeypatch.setenv("STGEMM_FORCE_KERNEL", "pingpong4")
    assert name(512, 512, 512, "bf16", "bf16", b_layout="row").startswith("tiled128")


NS = 4096


@pytest.mark.parametrize("a_col,b_col", [(True, False)], ids=["acol_brow"])
def test_mn_full_size_bf16(orc, a_col, b_col):
    """The bf16 8192^3 workload (C, bf16 out) with both operands MN-major:
    sampled entries (random positions, a whole row and a whole column)
    against the oracle, and every output against the K-major kernel."""
    p = inputs.dense_bf16(8192, 8192, 8192)
    M, N, K = p["M"], p["N"], p["K"]
    A, B = p["A"], p["B"]  # [M,K], [N,K]
    At, Bt = np.ascontiguousarray(A.T), np.ascontiguousarray(B.T)
    outs = {}
    for lay, (a, b, ac, bc) in {"k": (A, B, False, True), "mn": (At, Bt, a_col, b_col)}.items():
        desc = G.make_desc(M, N, K, "bf16", "bf16", p["d_type"], has_c=True,
                           a_layout="col" if ac else "row", b_layout="col" if bc else "row")
        plan = G.gemm_plan(desc)
        D = torch.empty(M * N * 2, dtype=torch.uint8, device="cuda")
        G.gemm_run(plan, to_dev(a), to_dev(b), to_dev(p["C"]), None, D)
        torch.cuda.synchronize()
        outs[lay] = D.cpu().numpy().view(OUT_NP[p["d_type"]]).reshape(M, N)
        say("  ran", plan.name)
        del D
    rng = np.random.default_rng(1)
    rows = np.concatenate([rng.integers(0, M, NS), np.full(N, M - 1), np.arange(M)])
    cols = np.concatenate([rng.integers(0, N, NS), np.arange(N), np.full(M, N // 2)])
    Dr, Y, S = orc.gemm_entries(At, Bt, p["C"], None, M, N, K, "bf16", "bf16", p["d_type"],
                                rows, cols, a_col_major=a_col, b_col_major=b_col)
    r = check(outs["mn"][rows, cols], p["d_type"], Dr, Y, S, "bf16", 1.0)
    say("  sampled", r)
    assert r.ok, r
    assert np.array_equal(outs["mn"], outs["k"])
