"""Parity at the workloads' full sizes, through the plan bench.py times.

The dense bf16, int8 and fp8 workloads, every 2:4 workload and W4A16 are
compared with the full oracle element by element over all M x N outputs
(int32 bit-exact; fp32 within the normalised bound; 16-bit and FP8 outputs
within one ulp of the oracle's correctly rounded value or the accumulation
bound, the count of elements that needed the second clause reported).  The
MX workloads are checked on a sample of entries (random positions plus a
whole row and a whole column, each computed by the oracle on its own) and
by their column sums over every output.  The 2:4 compressor's output is
compared byte for byte with the oracle's over the whole matrix, and the
fp8 workloads' fused epilogue is pinned bit for bit against the oracle's
fp32 epilogue applied to the same kernel's fp32 accumulator output."""
import numpy as np
import pytest
import torch

from checks import TOL, check, check_rows, ulp16
from exact import lib_decode
from gpu_util import OUT_NP, say, to_dev
from sparse_tiled_gemm_amd import gemm as G
from sparse_tiled_gemm_amd import inputs

pytestmark = pytest.mark.gpu

NS = 4096  # random sampled entries per workload


def _run(p, d_type=None, alpha=None, bias=True, relu=None, sparse_dev=None):
    M, N, K = p["M"], p["N"], p["K"]
    d_type = d_type or p["d_type"]
    use_bias = bias and p["bias"] is not None
    desc = G.make_desc(M, N, K, p["a_type"], p["b_type"], d_type, has_c=p["C"] is not None,
                       has_bias=use_bias, alpha=p["alpha"] if alpha is None else alpha,
                       act="relu" if (p["relu"] if relu is None else relu) else "none",
                       sparse_a=sparse_dev is not None)
    plan = G.gemm_plan(desc)
    tB = to_dev(p["B"])
    tC = to_dev(p["C"]) if p["C"] is not None else None
    tb = to_dev(p["bias"]) if use_bias else None
    D = torch.empty(M * N * G.ELEM_BYTES[d_type], dtype=torch.uint8, device="cuda")
    if sparse_dev is not None:
        G.gemm_sparse24_run(plan, sparse_dev[0], sparse_dev[1], tB, tC, tb, D)
    else:
        G.gemm_run(plan, to_dev(p["A"]), tB, tC, tb, D)
    torch.cuda.synchronize()
    out = D.cpu().numpy().view(OUT_NP[d_type]).reshape(M, N)
    say("  ran", plan.name, d_type)
    return out, plan.name


def _samples(M, N, seed):
    rng = np.random.default_rng(seed)
    r = rng.integers(0, M, NS)
    c = rng.integers(0, N, NS)
    rr = np.concatenate([r, np.full(N, M - 1), np.arange(M)])
    cc = np.concatenate([c, np.arange(N), np.full(M, N // 2)])
    return rr, cc


def _check_samples(orc, p, D, a_logical=None, seed=0):
    M, N, K = p["M"], p["N"], p["K"]
    rows, cols = _samples(M, N, seed)
    A = p["A"] if a_logical is None else a_logical
    Dr, Y, S = orc.gemm_entries(A, p["B"], p["C"], p["bias"], M, N, K, p["a_type"], p["b_type"],
                                p["d_type"], rows, cols, alpha=p["alpha"], relu=p["relu"])
    r = check(D[rows, cols], p["d_type"], Dr, Y, S, p["a_type"], p["alpha"])
    say("  sampled", r)
    assert r.ok, r


def _check_full(orc, p, D, a_logical=None):
    """Every output against the full oracle run on the same operands."""
    M, N, K = p["M"], p["N"], p["K"]
    A = p["A"] if a_logical is None else a_logical
    integer = p["d_type"] == "s32"
    Dr, Y, S = orc.gemm(A, p["B"], p["C"], p["bias"], M, N, K, p["a_type"], p["b_type"],
                        p["d_type"], alpha=p["alpha"], relu=p["relu"], want_y=not integer,
                        want_s=not integer)
    r = check_rows(D, p["d_type"], Dr, Y, S, p["a_type"], p["alpha"])
    say("  all %d outputs vs the full oracle:" % (M * N), r)
    assert r.ok and r.n == M * N, r


def test_full_f16_128(orc):
    say("workload f16 128^3 (full oracle)")
    p = inputs.dense_f16(128, 128, 128)
    D, name = _run(p)
    Dr, Y, S = orc.gemm(p["A"], p["B"], p["C"], None, 128, 128, 128, "f16", "f16", "f32")
    r = check(D, "f32", Dr, Y, S, "f16")
    say("  ", name, r)
    assert r.ok, r


def test_full_bf16_8192(orc):
    say("workload bf16 8192^3 -> bf16")
    p = inputs.dense_bf16(8192, 8192, 8192)
    D, name = _run(p)
    assert name.startswith("tiled256")
    _check_full(orc, p, D)


def test_full_bf16_skinny(orc):
    say("workload bf16 16x8192x8192 -> bf16 (full oracle)")
    p = inputs.dense_bf16(16, 8192, 8192)
    D, name = _run(p)
    assert name.startswith("skinny")
    Dr, Y, S = orc.gemm(p["A"], p["B"], p["C"], None, 16, 8192, 8192, "bf16", "bf16", "bf16")
    r = check(D, "bf16", Dr, Y, S, "bf16")
    say("  ", r)
    assert r.ok, r


def test_full_s8_8192(orc):
    say("workload s8 8192^3 -> s32")
    p = inputs.dense_s8(8192, 8192, 8192)
    D, name = _run(p)
    _check_full(orc, p, D)
    # exact column sums modulo 2^32
    colA = p["A"].astype(np.int64).sum(axis=0)                 # [K]
    ref = p["B"].astype(np.int64) @ colA + p["C"].astype(np.int64).sum(axis=0)
    got = D.astype(np.int64).sum(axis=0)
    assert np.array_equal(np.mod(got, 2 ** 32), np.mod(ref, 2 ** 32))
    say("  column sums exact")


def test_full_fp8_8192(orc):
    say("workload fp8 e4m3 x e5m2 8192^3 -> relu(alpha acc + bias) f16")
    p = inputs.dense_fp8(8192, 8192, 8192)
    D, name = _run(p)
    _check_full(orc, p, D)
    # the fused epilogue, bit for bit, against the same kernel's fp32 output
    T, name32 = _run(p, d_type="f32", alpha=1.0, bias=False, relu=False)
    assert name32.split("_")[0] == name.split("_")[0]
    ref = orc.epilogue_f32(T, p["alpha"], p["bias"], True, "f16")
    mism = int((D != ref).sum())
    say("  fused epilogue mismatches:", mism)
    assert mism == 0


def test_full_sparse24_8192(orc):
    say("workload 2:4 f16 8192^3 -> f32")
    p = inputs.sparse24_f16(8192, 8192, 8192)
    M, K = 8192, 8192
    vb, mb = G.gemm_sparse24_sizes(M, K)
    vals = torch.empty(vb, dtype=torch.uint8, device="cuda")
    meta = torch.empty(mb, dtype=torch.uint8, device="cuda")
    G.gemm_sparse24_compress(M, K, "f16", to_dev(p["A_logical"]), vals, meta)
    rv, rm = orc.sparse24_compress(p["A_logical"])
    assert np.array_equal(vals.cpu().numpy().view(np.uint16).reshape(rv.shape), rv)
    assert np.array_equal(meta.cpu().numpy().view(np.uint32).reshape(rm.shape), rm)
    say("  compressor bytes identical to the oracle's")
    D, name = _run(p, sparse_dev=(vals, meta))
    assert name.startswith("sparse24_dma8")
    pd = dict(p)
    pd["A"] = p["A_logical"]
    _check_full(orc, pd, D, a_logical=p["A_logical"])


@pytest.mark.parametrize("t", ["bf16", "s8", "e4m3"])
def test_full_sparse24_types_8192(orc, t):
    """2:4 A of the other types at 8192^3 through the plan the 8-wave SMFMAC
    kernel serves: bf16 -> bf16 with C, s8 -> s32 with C, e4m3 x e5m2 ->
    relu(alpha acc + bias) as fp16."""
    say("workload 2:4", t, "8192^3")
    p = inputs.sparse24(t, 8192, 8192, 8192)
    M, K = 8192, 8192
    vb, mb = G.gemm_sparse24_sizes(M, K, t)
    vals = torch.empty(vb, dtype=torch.uint8, device="cuda")
    meta = torch.empty(mb, dtype=torch.uint8, device="cuda")
    G.gemm_sparse24_compress(M, K, t, to_dev(p["A_logical"]), vals, meta)
    rv, rm = orc.sparse24_compress(p["A_logical"], t)
    assert np.array_equal(vals.cpu().numpy().view(rv.dtype).reshape(rv.shape), rv)
    assert np.array_equal(meta.cpu().numpy().view(np.uint32).reshape(rm.shape), rm)
    say("  compressor bytes identical to the oracle's")
    D, name = _run(p, sparse_dev=(vals, meta))
    assert name.startswith("sparse24_dma8")
    pd = dict(p)
    pd["A"] = p["A_logical"]
    _check_full(orc, pd, D, a_logical=p["A_logical"])
    if t == "s8":
        colA = p["A_logical"].astype(np.int64).sum(axis=0)
        ref = p["B"].astype(np.int64) @ colA + p["C"].astype(np.int64).sum(axis=0)
        got = D.astype(np.int64).sum(axis=0)
        assert np.array_equal(np.mod(got, 2 ** 32), np.mod(ref, 2 ** 32))
        say("  column sums exact")
    elif t != "bf16":
        T, name32 = _run(p, d_type="f32", alpha=1.0, bias=False, relu=False,
                         sparse_dev=(vals, meta))
        assert name32.startswith("sparse24_dma8")
        ref = orc.epilogue_f32(T, p["alpha"], p["bias"], True, "f16")
        mism = int((D != ref).sum())
        say("  fused epilogue mismatches:", mism)
        assert mism == 0


@pytest.mark.parametrize("name,a,seed", [("mxfp8", "e4m3", 9), ("mxfp4", "e2m1", 11),
                                         ("mxfp6", "e2m3", 10)])
def test_full_mx_8192(orc, name, a, seed):
    """MX block-scaled GEMM at 8192^3 -> bf16 through the plan bench.py times
    (the tiled kernel; for MXFP6 after the expansion to 8-bit codes):
    sampled entries against the oracle, and column sums over every output."""
    say("workload", name, "8192^3 -> bf16")
    M = N = K = 8192
    p = inputs.mx_problem(M, N, K, a, a, seed)
    desc = G.make_desc(M, N, K, a, a, "bf16", has_c=False, block_scale=32)
    plan = G.gemm_plan(desc)
    D = torch.empty(M * N * 2, dtype=torch.uint8, device="cuda")
    G.gemm_mx_run(plan, to_dev(p["A"]), to_dev(p["SA"]), to_dev(p["B"]), to_dev(p["SB"]), None,
                  None, D)
    torch.cuda.synchronize()
    D = D.cpu().numpy().view(np.uint16).reshape(M, N)
    say("  ran", plan.name)
    assert plan.name.startswith("mx_tiled6" if a == "e2m3" else "mx_tiled")
    rows, cols = _samples(M, N, seed)
    Dr, Y, S = orc.mx_gemm_entries(p["A"], p["SA"], p["B"], p["SB"], None, None, M, N, K, a, a,
                                   "bf16", rows, cols)
    r = check(D[rows, cols], "bf16", Dr, Y, S, a)
    say("  sampled", r)
    assert r.ok, r
    # column sums: sum_m D[m,n] = sum_k b'[k,n] sum_m a'[m,k], a', b' the scaled values
    sa = np.repeat(orc.decode_packed("e8m0", p["SA"], M * K // 32).reshape(M, K // 32), 32, 1)
    A = orc.decode_packed(a, p["A"], M * K).reshape(M, K) * sa
    del sa
    sb = np.repeat(orc.decode_packed("e8m0", p["SB"], N * K // 32).reshape(N, K // 32), 32, 1)
    B = orc.decode_packed(a, p["B"], N * K).reshape(N, K) * sb
    del sb
    ref = B @ A.sum(axis=0)
    sabs = np.abs(B) @ np.abs(A).sum(axis=0)
    del A, B
    d = lib_decode("bf16", D)
    got = d.sum(axis=0)
    bound = TOL[a] * sabs + ulp16(d, "bf16").sum(axis=0) * 2
    say("  column sums: max |diff|/bound = %.3g" % float((np.abs(got - ref) / bound).max()))
    assert (np.abs(got - ref) <= bound).all()


def test_full_w4a16_8192(orc):
    """W4A16 at 8192^3 (bf16 activations, groups of 128, bf16 out) through the
    plan bench.py times: sampled entries against the oracle's dequantisation
    plus dense GEMM, and column sums over every output."""
    say("workload W4A16 bf16 8192^3 -> bf16")
    M = N = K = 8192
    p = inputs.w4a16_problem(M, N, K, "bf16", 128, 12)
    desc = G.make_desc(M, N, K, "bf16", "u4", "bf16", has_c=False, block_scale=128)
    plan = G.gemm_plan(desc)
    D = torch.empty(M * N * 2, dtype=torch.uint8, device="cuda")
    G.gemm_w4a16_run(plan, to_dev(p["A"]), to_dev(p["B"]), to_dev(p["scales"]),
                     to_dev(p["zeros"]), None, None, D)
    torch.cuda.synchronize()
    D = D.cpu().numpy().view(np.uint16).reshape(M, N)
    say("  ran", plan.name)
    assert plan.name.startswith("w4_tiled")
    W = orc.w4a16_dequant(p["B"], p["scales"], p["zeros"], N, K, 128, "bf16")
    q = dict(p)
    q["B"], q["b_type"] = W, "bf16"
    _check_full(orc, q, D)
