"""GPU parity of the output signatures beyond the basic ones: FP8 (E4M3 /
E5M2) outputs of every kernel family (round to nearest even, saturating),
and the int8 -> float epilogue (s8 inputs, int32 sum, float output) -
against the oracle, and each fused epilogue bit for bit against the
oracle's fp32 epilogue applied to the same kernel's fp32 output."""
import numpy as np
import pytest
import torch

from checks import check
from gpu_util import gpu_compress, gpu_gemm, gpu_sparse_gemm, say, to_dev
from sparse_tiled_gemm_amd import gemm as G
from sparse_tiled_gemm_amd import inputs

pytestmark = pytest.mark.gpu

FP8 = ["e4m3", "e5m2"]


def _bias(N, seed=7):
    return np.random.default_rng(seed).standard_normal(N).astype(np.float32)


def _dense(a_type, M, N, K):
    if a_type == "bf16":
        return inputs.dense_bf16(M, N, K, d_type="f32")
    if a_type == "f16":
        return inputs.dense_f16(M, N, K)
    if a_type == "s8":
        return inputs.dense_s8(M, N, K)
    return inputs.dense_fp8(M, N, K)


def _fused_vs_f32(orc, run, d_type, alpha, bias, relu):
    """run(d_type, alpha, bias, relu) -> D bits; the fused result must equal the
    oracle's fp32 epilogue on the same kernel's fp32 output."""
    T = run("f32", 1.0, None, False)
    D = run(d_type, alpha, bias, relu)
    ref = orc.epilogue_f32(T, alpha, bias, relu, d_type)
    return int((D != ref).sum())


# (family forced, a_type, shape): the float kernels with an fp8 output
DENSE_FAMILIES = [("tiled256w8", "bf16", (300, 520, 256)), ("tiled256", "e4m3", (384, 264, 512)),
                  ("tiled256w8tk16", "bf16", (300, 520, 256)),
                  ("tiled256w8k16", "f16", (264, 300, 192)),
                  ("tiled128", "f16", (130, 200, 128)), ("generic", "bf16", (67, 45, 96)),
                  ("skinny", "bf16", (16, 300, 1024))]


@pytest.mark.parametrize("fam,a_type,shape", DENSE_FAMILIES, ids=[f[0] for f in DENSE_FAMILIES])
@pytest.mark.parametrize("d_type", FP8)
def test_dense_fp8_output(orc, monkeypatch, fam, a_type, shape, d_type):
    monkeypatch.setenv("STGEMM_FORCE_KERNEL", fam)
    M, N, K = shape
    p = _dense(a_type, M, N, K)
    bias = _bias(N)
    # scale results toward the fp8 range: 30 (e4m3) / 2000 (e5m2) times the
    # unit-variance sums, so some outputs saturate
    alpha = 30.0 if d_type == "e4m3" else 2000.0
    if a_type == "e4m3":
        alpha *= p["alpha"]

    def run(dt, al, bi, relu):
        D, name = gpu_gemm(p["A"], p["B"], p["C"], bi, M, N, K, p["a_type"], p["b_type"], dt,
                           alpha=al, relu=relu)
        assert name.startswith(fam), name
        return D
    D = run(d_type, alpha, bias, True)
    Dr, Y, S = orc.gemm(p["A"], p["B"], p["C"], bias, M, N, K, p["a_type"], p["b_type"], d_type,
                        alpha=alpha, relu=True)
    r = check(D, d_type, Dr, Y, S, p["a_type"], alpha)
    say(fam, d_type, r, "saturated:", int((np.abs(Y) >= (448 if d_type == "e4m3" else 57344)).sum()))
    assert r.ok, r
    assert _fused_vs_f32(orc, run, d_type, alpha, bias, True) == 0


S8_FAMILIES = [("tiled256w8t", (300, 520, 256)), ("tiled128", (130, 200, 128)),
               ("tiled256w8tk16", (300, 520, 256)), ("tiled256w8k16", (264, 300, 192)),
               ("generic", (67, 45, 96)), ("skinny", (16, 300, 1024))]


@pytest.mark.parametrize("fam,shape", S8_FAMILIES, ids=[f[0] for f in S8_FAMILIES])
@pytest.mark.parametrize("d_type", ["f32", "bf16", "f16", "e4m3"])
def test_s8_dequant_epilogue(orc, monkeypatch, fam, shape, d_type):
    """s8 x s8 -> int32 sum -> float output with C (fp32), alpha, bias, relu."""
    monkeypatch.setenv("STGEMM_FORCE_KERNEL", fam)
    M, N, K = shape
    p = inputs.dense_s8(M, N, K)
    C = np.random.default_rng(9).uniform(-1e4, 1e4, (M, N)).astype(np.float32)
    bias = _bias(N) * 100
    alpha = 1.0 / 4096 if d_type == "e4m3" else 1.0 / 512

    def run(dt, al, bi, relu):
        D, name = gpu_gemm(p["A"], p["B"], C, bi, M, N, K, "s8", "s8", dt, alpha=al, relu=relu)
        assert name.startswith(fam), name
        return D
    D = run(d_type, alpha, bias, True)
    Dr, Y, S = orc.gemm(p["A"], p["B"], C, bias, M, N, K, "s8", "s8", d_type, alpha=alpha,
                        relu=True)
    r = check(D, d_type, Dr, Y, S, "s8", alpha)
    say(fam, d_type, r)
    assert r.ok, r
    if d_type != "f32":
        assert _fused_vs_f32(orc, run, d_type, alpha, bias, True) == 0


@pytest.mark.parametrize("t", ["f16", "s8"])
def test_sparse_outputs(orc, t):
    """2:4 kernels (8-wave and generic): f16 A -> e4m3, s8 A -> bf16."""
    M, N, K = 300, 264, 512
    p = inputs.sparse24(t, M, N, K)
    d_type = "e4m3" if t == "f16" else "bf16"
    C = p["C"].astype(np.float32) if t == "f16" else \
        np.random.default_rng(5).uniform(-1e4, 1e4, (M, N)).astype(np.float32)
    alpha = 30.0 if t == "f16" else 1.0 / 512
    vals, meta, _, _ = gpu_compress(p["A_logical"], t)
    for algo in ("tiled", "generic"):
        D, name = gpu_sparse_gemm(vals, meta, p["B"], C, M, N, K, d_type, algo=algo, alpha=alpha,
                                  a_type=t)
        Dr, Y, S = orc.gemm(p["A_logical"], p["B"], C, None, M, N, K, t, t, d_type, alpha=alpha)
        r = check(D, d_type, Dr, Y, S, t, alpha)
        say("sparse", t, algo, name, r)
        assert r.ok, r


def test_mx_and_w4_fp8_outputs(orc):
    """The MX tiled kernel and the W4A16 tiled / skinny kernels with an E4M3 output."""
    M, N, K = 256, 256, 512
    p = inputs.mx_problem(M, N, K, "e4m3", "e4m3", workload=70, d_type="f32")
    desc = G.make_desc(M, N, K, "e4m3", "e4m3", "e4m3", has_c=False, alpha=4.0, block_scale=32)
    plan = G.gemm_plan(desc)
    D = torch.empty(M * N, dtype=torch.uint8, device="cuda")
    G.gemm_mx_run(plan, to_dev(p["A"]), to_dev(p["SA"]), to_dev(p["B"]), to_dev(p["SB"]), None,
                  None, D)
    torch.cuda.synchronize()
    Dr, Y, S = orc.mx_gemm(p["A"], p["SA"], p["B"], p["SB"], None, None, M, N, K, "e4m3", "e4m3",
                           "e4m3", alpha=4.0)
    r = check(D.cpu().numpy().reshape(M, N), "e4m3", Dr, Y, S, "e4m3", 4.0)
    assert plan.name.startswith("mx_tiled") and r.ok, (plan.name, r)
    for Mw in (256, 16):
        q = inputs.w4a16_problem(Mw, N, K, "bf16", 128, workload=71)
        desc = G.make_desc(Mw, N, K, "bf16", "u4", "e5m2", has_c=False, alpha=100.0,
                           block_scale=128)
        plan = G.gemm_plan(desc)
        D = torch.empty(Mw * N, dtype=torch.uint8, device="cuda")
        G.gemm_w4a16_run(plan, to_dev(q["A"]), to_dev(q["B"]), to_dev(q["scales"]),
                         to_dev(q["zeros"]), None, None, D)
        torch.cuda.synchronize()
        W = orc.w4a16_dequant(q["B"], q["scales"], q["zeros"], N, K, 128, "bf16")
        Dr, Y, S = orc.gemm(q["A"], W, None, None, Mw, N, K, "bf16", "bf16", "e5m2", alpha=100.0)
        r = check(D.cpu().numpy().reshape(Mw, N), "e5m2", Dr, Y, S, "bf16", 100.0)
        say("w4", plan.name, r)
        assert r.ok, r


@pytest.mark.parametrize("fam,shape", [("tiled256w8", (256, 256, 128)), ("skinny", (16, 256, 256)),
                                       ("generic", (40, 72, 64))],
                         ids=["tiled256w8", "skinny", "generic"])
@pytest.mark.parametrize("d_type", FP8)
@pytest.mark.parametrize("relu", [False, True])
def test_fp8_output_specials(orc, monkeypatch, fam, shape, d_type, relu):
    """NaN, infinities and values around the largest finite value reach the FP8
    cast through C: NaN -> 0x7F (relu maps it to +0), +-inf and finite values
    beyond the maximum -> +-max, the rest rounded to nearest even - bit for bit
    against the oracle's fp32 epilogue of the same kernel's fp32 output."""
    monkeypatch.setenv("STGEMM_FORCE_KERNEL", fam)
    M, N, K = shape
    p = _dense("bf16", M, N, K)
    mx = 448.0 if d_type == "e4m3" else 57344.0
    specials = np.array([np.nan, np.inf, -np.inf, 1e30, -1e30, mx, -mx, mx * 1.03, mx * 1.07,
                         -mx * 1.07, mx * 0.97, 2.0 ** -12, -(2.0 ** -18), 0.0], np.float32)
    rng = np.random.default_rng(13)
    C = p["C"].astype(np.float32).copy()
    flat = C.reshape(-1)
    pos = rng.choice(flat.size, size=4 * specials.size, replace=False)
    flat[pos] = np.tile(specials, 4)

    def run(dt, al, bi, rl):
        D, name = gpu_gemm(p["A"], p["B"], C, bi, M, N, K, "bf16", "bf16", dt, alpha=al, relu=rl)
        assert name.startswith(fam), name
        return D
    T = run("f32", 1.0, None, False)
    D = run(d_type, 1.0, None, relu)
    ref = orc.epilogue_f32(T, 1.0, None, relu, d_type)
    bad = int((D != ref).sum())
    nan_pos = pos[np.isnan(np.tile(specials, 4))]
    want_nan = 0 if relu else 0x7F
    assert np.all(D.reshape(-1)[nan_pos] == want_nan), D.reshape(-1)[nan_pos]
    assert bad == 0, bad


# 16-bit C ("NVIDIA MMA", section "Input / accumulate / output": the C type is
# a separate choice): C given as fp16 or bf16, widened exactly to fp32 and
# then the same epilogue
C16_FAMILIES = [("tiled256w8", "bf16", (300, 264, 256)), ("tiled128", "f16", (130, 200, 128)),
                ("generic", "bf16", (67, 45, 96)), ("skinny", "f16", (16, 300, 1024)),
                ("tiled256", "e4m3", (264, 300, 256)), ("tiled256w8t", "s8", (264, 300, 256)),
                ("tiled256w8tk16", "bf16", (300, 264, 256)), ("tiled256w8tk16", "s8", (264, 300, 256)),
                ("tiled256w8k16", "f16", (264, 300, 128))]


@pytest.mark.parametrize("fam,a_type,shape", C16_FAMILIES, ids=[f[0] + "_" + f[1] for f in C16_FAMILIES])
@pytest.mark.parametrize("c_type", ["f16", "bf16"])
def test_16bit_c(orc, monkeypatch, fam, a_type, shape, c_type):
    monkeypatch.setenv("STGEMM_FORCE_KERNEL", fam)
    M, N, K = shape
    p = _dense(a_type, M, N, K)
    rng = np.random.default_rng(21)
    conv = inputs.to_f16 if c_type == "f16" else inputs.to_bf16
    C = conv(rng.uniform(-4, 4, size=(M, N)))
    d_type = "bf16" if a_type != "f16" else "f32"
    alpha = (1.0 / 512 if a_type == "s8" else (p["alpha"] if a_type == "e4m3" else 1.0))
    bias = _bias(N)
    desc = G.make_desc(M, N, K, p["a_type"], p["b_type"], d_type, c_type=c_type, has_c=True,
                       has_bias=True, alpha=alpha, act="relu")
    plan = G.gemm_plan(desc)
    assert plan.name.startswith(fam), plan.name
    D = torch.empty(M * N * G.ELEM_BYTES[d_type], dtype=torch.uint8, device="cuda")
    G.gemm_run(plan, to_dev(p["A"]), to_dev(p["B"]), to_dev(C), to_dev(bias), D)
    torch.cuda.synchronize()
    out = D.cpu().numpy().view({"bf16": np.uint16, "f32": np.float32}[d_type]).reshape(M, N)
    Dr, Y, S = orc.gemm(p["A"], p["B"], C, bias, M, N, K, p["a_type"], p["b_type"], d_type,
                        alpha=alpha, relu=True, c_type=c_type)
    r = check(out, d_type, Dr, Y, S, p["a_type"], alpha)
    say("c16", plan.name, c_type, r)
    assert r.ok, r


@pytest.mark.parametrize("c_type", ["f16", "bf16"])
def test_16bit_c_sparse_and_w4(orc, c_type):
    """2:4 (direct-copy kernel) and W4A16 (tiled and skinny) with a 16-bit C."""
    conv = inputs.to_f16 if c_type == "f16" else inputs.to_bf16
    M, N, K = 300, 264, 512
    p = inputs.sparse24("f16", M, N, K)
    C = conv(np.random.default_rng(4).uniform(-2, 2, size=(M, N)))
    vals, meta, _, _ = gpu_compress(p["A_logical"], "f16")
    desc = G.make_desc(M, N, K, "f16", "f16", "f32", c_type=c_type, has_c=True, sparse_a=True)
    plan = G.gemm_plan(desc)
    D = torch.empty(M * N * 4, dtype=torch.uint8, device="cuda")
    G.gemm_sparse24_run(plan, vals, meta, to_dev(p["B"]), to_dev(C), None, D)
    torch.cuda.synchronize()
    Dr, Y, S = orc.gemm(p["A_logical"], p["B"], C, None, M, N, K, "f16", "f16", "f32",
                        c_type=c_type)
    r = check(D.cpu().numpy().view(np.float32).reshape(M, N), "f32", Dr, Y, S, "f16", 1.0)
    say("c16 sparse", plan.name, r)
    assert r.ok, r
    for Mw in (256, 16):
        q = inputs.w4a16_problem(Mw, N, K, "bf16", 128, workload=72)
        Cw = conv(np.random.default_rng(6).uniform(-1, 1, size=(Mw, N)))
        desc = G.make_desc(Mw, N, K, "bf16", "u4", "bf16", c_type=c_type, has_c=True,
                           block_scale=128)
        plan = G.gemm_plan(desc)
        D = torch.empty(Mw * N * 2, dtype=torch.uint8, device="cuda")
        G.gemm_w4a16_run(plan, to_dev(q["A"]), to_dev(q["B"]), to_dev(q["scales"]),
                         to_dev(q["zeros"]), to_dev(Cw), None, D)
        torch.cuda.synchronize()
        W = orc.w4a16_dequant(q["B"], q["scales"], q["zeros"], N, K, 128, "bf16")
        Dr, Y, S = orc.gemm(q["A"], W, Cw, None, Mw, N, K, "bf16", "bf16", "bf16", c_type=c_type)
        r = check(D.cpu().numpy().view(np.uint16).reshape(Mw, N), "bf16", Dr, Y, S, "bf16", 1.0)
        say("c16 w4", plan.name, r)
        assert r.ok, r


def test_16bit_c_validation():
    with pytest.raises(G.GemmError):  # int32 outputs take an int32 C
        G.gemm_plan(G.make_desc(256, 256, 256, "s8", "s8", "s32", c_type="f16"))
    with pytest.raises(G.GemmError):  # block-scaled GEMM keeps an fp32 C
        G.gemm_plan(G.make_desc(256, 256, 512, "e4m3", "e4m3", "bf16", c_type="bf16",
                                block_scale=32))


@pytest.mark.parametrize("c_type", ["f16", "bf16"])
@pytest.mark.parametrize("ldc_pad,c_shift", [(0, 0), (4, 0), (2, 0), (0, 1)],
                         ids=["packed", "ldc+4", "ldc+2", "misaligned"])
def test_16bit_c_bit_exact(orc, c_type, ldc_pad, c_shift):
    """A 16-bit C through the 256 x 256 kernel's epilogue, bit for bit: D =
    the fp32 epilogue of (the kernel's own fp32 accumulator + C widened).
    8-byte-aligned C rows take the vector path (4 C elements per lane in one
    load); an odd pitch or a C not 8-byte aligned takes the element path."""
    M, N, K = 520, 392, 256
    p = _dense("bf16", M, N, K)
    conv = inputs.to_f16 if c_type == "f16" else inputs.to_bf16
    ldc = N + ldc_pad
    C = conv(np.random.default_rng(31).uniform(-8, 8, size=(M, ldc)))
    bias = _bias(N)
    tA, tB = to_dev(p["A"]), to_dev(p["B"])
    # the fp32 accumulator, no C
    dT = G.make_desc(M, N, K, "bf16", "bf16", "f32", has_c=False, algo="tiled256")
    T = torch.empty(M * N * 4, dtype=torch.uint8, device="cuda")
    G.gemm_run(G.gemm_plan(dT), tA, tB, None, None, T)
    buf = torch.zeros(M * ldc * 2 + 16, dtype=torch.uint8, device="cuda")
    off = 2 * c_shift
    buf[off:off + M * ldc * 2] = to_dev(C.reshape(-1).view(np.uint8))
    for d_type in ["bf16", "f32"]:
        desc = G.make_desc(M, N, K, "bf16", "bf16", d_type, c_type=c_type, has_c=True, ldc=ldc,
                           has_bias=True, alpha=0.75, act="relu", algo="tiled256")
        plan = G.gemm_plan(desc)
        D = torch.empty(M * N * G.ELEM_BYTES[d_type], dtype=torch.uint8, device="cuda")
        G.gemm_run(plan, tA, tB, buf[off:], to_dev(bias), D)
        torch.cuda.synchronize()
        Tc = (T.cpu().numpy().view(np.float32).reshape(M, N) +
              orc.decode(c_type, C[:, :N]).astype(np.float32))
        ref = orc.epilogue_f32(Tc, 0.75, bias, True, d_type)
        out = D.cpu().numpy().view(ref.dtype).reshape(M, N)
        mism = int((out.view(np.uint32 if d_type == "f32" else np.uint16) !=
                    ref.view(np.uint32 if d_type == "f32" else np.uint16)).sum())
        say("c16 exact", plan.name, c_type, d_type, ldc_pad, c_shift, "mismatches", mism)
        assert mism == 0
