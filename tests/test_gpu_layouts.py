"""GPU parity of the MN-major operand layouts on the LDS-tiled kernels: A
column-major (M contiguous) and / or B row-major (N contiguous), 16-bit,
fp8 and int8 types, whose tiles are kept in LDS in memory order and read
with the transposing LDS loads.  Against the oracle element by element at sizes that
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

CONV = {"f16": inputs.to_f16, "bf16": inputs.to_bf16, "e4m3": inputs.to_e4m3,
        "e5m2": inputs.to_e5m2}
# (a column-major, b column-major): the three layouts with an MN-major operand
MN_LAYOUTS = [(True, True), (False, False), (True, False)]
SUFFIX = {(True, True): "_acol", (False, False): "_brow", (True, False): "_acol_brow"}


def _make(t, M, N, K, a_col, b_col, seed, tb=None):
    tb = tb or t
    rng = np.random.default_rng(seed)
    ash, bsh = (K, M) if a_col else (M, K), (N, K) if b_col else (K, N)
    if t == "s8":
        A = rng.integers(-128, 128, size=ash, dtype=np.int8)
        B = rng.integers(-128, 128, size=bsh, dtype=np.int8)
    else:
        sc = 16.0 if t.startswith("e") else 1.0
        A = CONV[t](rng.standard_normal(ash) * sc)
        B = CONV[tb](rng.standard_normal(bsh) * sc)
    C = rng.uniform(-1, 1, size=(M, N)).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32)
    return A, B, C, bias


def _oracle_check(orc, D, A, B, C, bias, M, N, K, t, d_type, a_col, b_col, alpha, relu, tb=None):
    Dr, Y, S = orc.gemm(A, B, C, bias, M, N, K, t, tb or t, d_type, a_col_major=a_col,
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


# 8-bit: (a type, b type, d type, 256 x 256 family); fp8 pairs may differ
EIGHT = [("e4m3", "e5m2", "f16", "tiled256"), ("e5m2", "e4m3", "bf16", "tiled256"),
         ("e4m3", "e4m3", "f32", "tiled256"), ("e5m2", "e5m2", "e4m3", "tiled256"),
         ("s8", "s8", "s32", "tiled256w8t"), ("s8", "s8", "bf16", "tiled256w8t")]


@pytest.mark.parametrize("ta,tb,d_type,fam256", EIGHT,
                         ids=["%s_%s_%s" % e[:3] for e in EIGHT])
@pytest.mark.parametrize("a_col,b_col", MN_LAYOUTS, ids=["acol", "brow", "acol_brow"])
@pytest.mark.parametrize("big", [True, False], ids=["256", "128"])
def test_mn_tiled_8bit(orc, monkeypatch, ta, tb, d_type, fam256, a_col, b_col, big):
    """fp8 (any pairing) and int8 MN-major operands, transposing 8-bit reads;
    M, N multiples of 16 with ragged tails, K of several 64-byte tiles."""
    fam = fam256 if big else "tiled128"
    monkeypatch.setenv("STGEMM_FORCE_KERNEL", fam)
    M, N, K = (528, 400, 320) if big else (272, 208, 192)
    A, B, C, bias = _make(ta, M, N, K, a_col, b_col, seed=M + K, tb=tb)
    if ta == "s8" and d_type == "s32":
        C = np.random.default_rng(3).integers(-(1 << 20), 1 << 20, size=(M, N), dtype=np.int32)
        bias, alpha, relu = None, 1.0, False
    else:
        alpha, relu = (1.0 / 512 if ta == "s8" else 1.0 / 256), True
    D, name = gpu_gemm(A, B, C, bias, M, N, K, ta, tb, d_type, alpha=alpha, relu=relu,
                       a_col=a_col, b_col=b_col)
    say("mn8", name, ta, tb, d_type, (M, N, K))
    assert name.startswith(fam) and name.endswith(SUFFIX[(a_col, b_col)]), name
    _oracle_check(orc, D, A, B, C, bias, M, N, K, ta, d_type, a_col, b_col, alpha, relu, tb=tb)


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


@pytest.mark.parametrize("t,fam256", [("f16", "tiled256w8"), ("e4m3", "tiled256"),
                                      ("s8", "tiled256w8t")], ids=["f16", "e4m3", "s8"])
@pytest.mark.parametrize("a_col,b_col", MN_LAYOUTS, ids=["acol", "brow", "acol_brow"])
def test_mn_matches_k_major_bitwise(t, fam256, a_col, b_col):
    """Same values, MN-major vs K-major storage, same tile family: every MFMA
    sees the same K order, so the outputs are identical bit for bit."""
    M, N, K = 512, 768, 320
    A, B, C, bias = _make(t, M, N, K, False, True, seed=11)
    if t == "s8":
        C, bias = None, None
    d_type = "s32" if t == "s8" else "f32"
    At = np.ascontiguousarray(A.T) if a_col else A
    Bt = B if b_col else np.ascontiguousarray(B.T)
    for fam in (fam256, "tiled128"):
        algo = "tiled256" if fam == fam256 else "tiled128"
        ref, n0 = gpu_gemm(A, B, C, bias, M, N, K, t, t, d_type, algo=algo)
        D, n1 = gpu_gemm(At, Bt, C, bias, M, N, K, t, t, d_type, a_col=a_col, b_col=b_col,
                         algo=algo)
        say("bitwise", n0, n1)
        assert n0.startswith(fam) and n1.startswith(fam), (n0, n1)
        assert np.array_equal(D.view(np.uint32), ref.view(np.uint32)), int((D != ref).sum())


def test_mn_plan_choices(monkeypatch):
    """Which layouts reach the tiled kernels: M (N) in whole 16-byte chunks,
    K in whole 64-byte tiles; everything else stays on the generic kernel."""
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
    assert name(8192, 8192, 8192, "e4m3", "f16", b_layout="row") == "tiled256_e4m3xe4m3_brow"
    assert name(8192, 8192, 8192, "s8", "s32", a_layout="col") == "tiled256w8t_s8_acol"
    assert name(520, 512, 512, "s8", "s32", a_layout="col").startswith("generic")  # M % 16
    assert name(512, 512, 96, "e4m3", "f32", b_layout="row").startswith("generic")  # K % 64
    # a 256 x 256 arrangement other than the type's own does not take
    # MN-major operands: forcing it is ignored
    monkeypatch.setenv("STGEMM_FORCE_KERNEL", "tiled256w8t")
    assert name(8192, 8192, 8192, "bf16", "bf16", b_layout="row") == "tiled256w8_bf16_brow"


NS = 4096


@pytest.mark.parametrize("wl", ["bf16", "fp8", "s8"])
def test_mn_full_size(orc, wl):
    """The 8192^3 workloads (bf16 with C -> bf16; e4m3 x e5m2 -> relu(alpha
    acc + bias) f16; s8 with C -> s32) with both operands MN-major: sampled
    entries (random positions, a whole row and a whole column) against the
    oracle, and every output against the K-major kernel."""
    p = {"bf16": inputs.dense_bf16, "fp8": inputs.dense_fp8, "s8": inputs.dense_s8}[wl](
        8192, 8192, 8192)
    M, N, K = p["M"], p["N"], p["K"]
    A, B = p["A"], p["B"]  # [M,K], [N,K]
    At, Bt = np.ascontiguousarray(A.T), np.ascontiguousarray(B.T)
    eb = G.ELEM_BYTES[p["d_type"]]
    outs = {}
    for lay, (a, b, ac, bc) in {"k": (A, B, False, True), "mn": (At, Bt, True, False)}.items():
        desc = G.make_desc(M, N, K, p["a_type"], p["b_type"], p["d_type"],
                           has_c=p["C"] is not None, has_bias=p["bias"] is not None,
                           alpha=p["alpha"], act="relu" if p["relu"] else "none",
                           a_layout="col" if ac else "row", b_layout="col" if bc else "row")
        plan = G.gemm_plan(desc)
        D = torch.empty(M * N * eb, dtype=torch.uint8, device="cuda")
        G.gemm_run(plan, to_dev(a), to_dev(b), to_dev(p["C"]) if p["C"] is not None else None,
                   to_dev(p["bias"]) if p["bias"] is not None else None, D)
        torch.cuda.synchronize()
        outs[lay] = D.cpu().numpy().view(OUT_NP[p["d_type"]]).reshape(M, N)
        say("  ran", plan.name)
        if lay == "mn":
            assert plan.name.endswith("_acol_brow"), plan.name
        del D
    rng = np.random.default_rng(1)
    rows = np.concatenate([rng.integers(0, M, NS), np.full(N, M - 1), np.arange(M)])
    cols = np.concatenate([rng.integers(0, N, NS), np.arange(N), np.full(M, N // 2)])
    Dr, Y, S = orc.gemm_entries(At, Bt, p["C"], p["bias"], M, N, K, p["a_type"], p["b_type"],
                                p["d_type"], rows, cols, a_col_major=True, b_col_major=False,
                                alpha=p["alpha"], relu=p["relu"])
    r = check(outs["mn"][rows, cols], p["d_type"], Dr, Y, S, p["a_type"], p["alpha"])
    say("  sampled", r)
    assert r.ok, r
    assert np.array_equal(outs["mn"], outs["k"])
