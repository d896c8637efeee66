"""CPU-side checks of the C ABI: the library loads, exports every function
declared in include/gemm.h, and gemm_validate_desc (a pure host function)
maps bad descriptors to the documented status codes.  No GPU needed."""
import ctypes
import os
import re

import pytest

from sparse_tiled_gemm_amd import gemm as G

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "gemm.h")


def _declared_functions():
    names = set()
    inc = os.path.dirname(HEADER)
    for h in sorted(os.listdir(inc)):
        text = open(os.path.join(inc, h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(gemm_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_function():
    L = G.load()
    names = _declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert "gemm_sparse24_run" in names and "gemm_plan" in names
    assert "gemm_diag_mfma_loop" in names and "gemm_sparse24_compress_noalloc" in names


def test_status_strings():
    for code, name in [(0, "GEMM_OK"), (3, "GEMM_ERR_UNSUPPORTED"), (5, "GEMM_ERR_NOT_SPARSE24")]:
        assert G.gemm_status_string(code) == name


def _ok(**kw):
    base = dict(M=64, N=64, K=64, a_type="bf16", b_type="bf16", d_type="bf16")
    base.update(kw)
    return G.make_desc(**base)


@pytest.mark.parametrize("desc,status", [
    (dict(), G.GEMM_OK),
    (dict(a_type="f16", b_type="f16", d_type="f32"), G.GEMM_OK),
    (dict(a_type="e4m3", b_type="e5m2", d_type="f16", has_c=False, has_bias=True, alpha=0.5,
          act="relu"), G.GEMM_OK),
    (dict(a_type="s8", b_type="s8", d_type="s32"), G.GEMM_OK),
    (dict(M=-1), G.GEMM_ERR_INVALID_VALUE),
    (dict(K=-5), G.GEMM_ERR_INVALID_VALUE),
    (dict(lda=10), G.GEMM_ERR_INVALID_VALUE),          # row-major A needs lda >= K
    (dict(ldb=3), G.GEMM_ERR_INVALID_VALUE),
    (dict(ldd=63), G.GEMM_ERR_INVALID_VALUE),
    (dict(a_type="s8", b_type="f16", d_type="f32"), G.GEMM_ERR_UNSUPPORTED),
    (dict(a_type="f16", b_type="bf16", d_type="f32"), G.GEMM_ERR_UNSUPPORTED),
    (dict(a_type="f16", b_type="e4m3", d_type="f32"), G.GEMM_ERR_UNSUPPORTED),
    (dict(a_type="s8", b_type="s8", d_type="s32", alpha=2.0), G.GEMM_ERR_UNSUPPORTED),
    (dict(a_type="s8", b_type="s8", d_type="s32", has_bias=True), G.GEMM_ERR_UNSUPPORTED),
    (dict(a_type="s8", b_type="s8", d_type="s32", act="relu"), G.GEMM_ERR_UNSUPPORTED),
    (dict(a_type="s8", b_type="s8", d_type="f32"), G.GEMM_OK),          # int8 -> float
    (dict(a_type="s8", b_type="s8", d_type="e4m3", alpha=0.5, act="relu"), G.GEMM_OK),
    (dict(a_type="s8", b_type="s8", d_type="bf16", c_type="s32"), G.GEMM_ERR_UNSUPPORTED),
    # unsigned 8-bit A and / or B (with s8 or u8 only); saturation's K limit
    # is K * max|a| * max|b| < 2^31
    (dict(a_type="u8", b_type="s8", d_type="s32"), G.GEMM_OK),
    (dict(a_type="s8", b_type="u8", d_type="s32"), G.GEMM_OK),
    (dict(a_type="u8", b_type="u8", d_type="s32"), G.GEMM_OK),
    (dict(a_type="u8", b_type="u8", d_type="bf16", alpha=0.25, act="relu"), G.GEMM_OK),
    (dict(a_type="u8", b_type="bf16", d_type="f32"), G.GEMM_ERR_UNSUPPORTED),
    (dict(a_type="e4m3", b_type="u8", d_type="f32"), G.GEMM_ERR_UNSUPPORTED),
    (dict(a_type="u8", b_type="u8", d_type="s32", alpha=2.0), G.GEMM_ERR_UNSUPPORTED),
    (dict(a_type="u8", b_type="u8", d_type="s32", saturate=True, K=33024), G.GEMM_OK),
    (dict(a_type="u8", b_type="u8", d_type="s32", saturate=True, K=33028),
     G.GEMM_ERR_UNSUPPORTED),
    (dict(a_type="u8", b_type="s8", d_type="s32", saturate=True, K=65792), G.GEMM_OK),
    (dict(a_type="s8", b_type="u8", d_type="s32", saturate=True, K=65796),
     G.GEMM_ERR_UNSUPPORTED),
    (dict(a_type="s8", b_type="s8", d_type="s32", saturate=True, K=131068), G.GEMM_OK),
    (dict(a_type="s8", b_type="s8", d_type="s32", saturate=True, K=131072),
     G.GEMM_ERR_UNSUPPORTED),
    (dict(sparse_a=True, a_type="u8", b_type="s8", d_type="s32"), G.GEMM_OK),
    (dict(sparse_a=True, a_type="s8", b_type="u8", d_type="f32"), G.GEMM_OK),
    (dict(sparse_a=True, a_type="u8", b_type="u8", d_type="s32"), G.GEMM_OK),
    (dict(a_type="u8", b_type="u8", block_scale=32), G.GEMM_ERR_UNSUPPORTED),
    (dict(a_type="bf16", b_type="bf16", d_type="e5m2"), G.GEMM_OK),      # fp8 output
    (dict(a_type="e4m3", b_type="e5m2", d_type="e4m3", has_c=False), G.GEMM_OK),
    (dict(d_type="s32"), G.GEMM_ERR_UNSUPPORTED),
    (dict(d_type="e2m1"), G.GEMM_ERR_UNSUPPORTED),
    (dict(c_type="s32"), G.GEMM_ERR_UNSUPPORTED),
    (dict(c_type="bf16"), G.GEMM_OK),
    (dict(c_type="f16"), G.GEMM_OK),
    (dict(sparse_a=True), G.GEMM_OK),                  # 2:4 bf16
    (dict(sparse_a=True, a_type="s8", b_type="s8", d_type="s32"), G.GEMM_OK),
    (dict(sparse_a=True, a_type="e4m3", b_type="e5m2", d_type="f16"), G.GEMM_OK),
    (dict(sparse_a=True, a_type="e5m2", b_type="e5m2", d_type="f32"), G.GEMM_OK),
    (dict(sparse_a=True, a_type="f16", b_type="bf16", d_type="f32"), G.GEMM_ERR_UNSUPPORTED),
    (dict(sparse_a=True, a_type="s8", b_type="s8", d_type="f32"), G.GEMM_OK),
    (dict(sparse_a=True, a_type="f16", b_type="f16", K=66), G.GEMM_ERR_UNSUPPORTED),
    (dict(sparse_a=True, a_type="f16", b_type="f16", a_layout="col"), G.GEMM_ERR_UNSUPPORTED),
    (dict(sparse_a=True, a_type="f16", b_type="f16", d_type="f32"), G.GEMM_OK),
    # MX block-scaled
    (dict(a_type="e4m3", b_type="e4m3", block_scale=32), G.GEMM_OK),
    (dict(a_type="e2m1", b_type="e5m2", d_type="f16", block_scale=32, has_bias=True,
          act="relu"), G.GEMM_OK),
    (dict(a_type="e2m3", b_type="e3m2", d_type="f32", block_scale=32), G.GEMM_OK),
    (dict(a_type="e2m1", b_type="e2m1", block_scale=16), G.GEMM_ERR_INVALID_VALUE),
    (dict(a_type="e2m1", b_type="e2m1"), G.GEMM_ERR_UNSUPPORTED),      # fp4 needs scales
    (dict(a_type="bf16", b_type="bf16", block_scale=32), G.GEMM_ERR_UNSUPPORTED),
    (dict(a_type="e4m3", b_type="e4m3", block_scale=32, K=48), G.GEMM_ERR_UNSUPPORTED),
    (dict(a_type="e4m3", b_type="e4m3", block_scale=32, a_layout="col"), G.GEMM_ERR_UNSUPPORTED),
    (dict(a_type="e4m3", b_type="e4m3", block_scale=32, sparse_a=True), G.GEMM_ERR_UNSUPPORTED),
    (dict(a_type="e4m3", b_type="e4m3", block_scale=32, d_type="s32"), G.GEMM_ERR_UNSUPPORTED),
    (dict(a_type="e2m1", b_type="e2m1", block_scale=32, lda=65), G.GEMM_ERR_UNSUPPORTED),
    (dict(a_type="e2m3", b_type="e2m3", block_scale=32, lda=66), G.GEMM_ERR_UNSUPPORTED),
    (dict(a_type="e2m3", b_type="e2m3", block_scale=32, lda=68), G.GEMM_OK),
    # W4A16 (block_scale = the weight group size)
    (dict(a_type="bf16", b_type="u4", block_scale=64), G.GEMM_OK),
    (dict(a_type="f16", b_type="u4", d_type="f32", block_scale=32, has_bias=True), G.GEMM_OK),
    (dict(a_type="bf16", b_type="u4", block_scale=0), G.GEMM_ERR_UNSUPPORTED),
    (dict(a_type="bf16", b_type="u4", block_scale=48), G.GEMM_ERR_UNSUPPORTED),
    (dict(a_type="bf16", b_type="u4", block_scale=128), G.GEMM_ERR_UNSUPPORTED),  # K = 64
    (dict(a_type="e4m3", b_type="u4", block_scale=32), G.GEMM_ERR_UNSUPPORTED),
    (dict(a_type="bf16", b_type="u4", block_scale=32, b_layout="row"), G.GEMM_ERR_UNSUPPORTED),
    (dict(a_type="bf16", b_type="u4", block_scale=32, ldb=65), G.GEMM_ERR_UNSUPPORTED),
    (dict(a_type="bf16", b_type="bf16", block_scale=64), G.GEMM_ERR_INVALID_VALUE),
])
def test_validate_desc(desc, status):
    assert G.gemm_validate_desc(_ok(**desc)) == status, G.gemm_last_error()


def test_validate_bad_enums_and_null():
    d = _ok()
    d.a_type = 99
    assert G.gemm_validate_desc(d) == G.GEMM_ERR_INVALID_VALUE
    d = _ok()
    d.act = 7
    assert G.gemm_validate_desc(d) == G.GEMM_ERR_INVALID_VALUE
    d = _ok()
    d.algo = 42
    assert G.gemm_validate_desc(d) == G.GEMM_ERR_INVALID_VALUE
    assert G.gemm_validate_desc(None) == G.GEMM_ERR_NULL_POINTER
    assert "NULL" in G.gemm_last_error()


def test_sparse24_sizes():
    vb, mb = G.gemm_sparse24_sizes(8192, 8192)
    assert vb == 8192 * 4096 * 2 and mb == 8192 * 256 * 4
    vb, mb = G.gemm_sparse24_sizes(3, 36)
    assert vb == 3 * 18 * 2 and mb == 3 * 2 * 4
    with pytest.raises(G.GemmError) as e:
        G.gemm_sparse24_sizes(4, 6)
    assert e.value.status == G.GEMM_ERR_UNSUPPORTED
    # values are elements of A's type; the metadata does not depend on it
    assert G.gemm_sparse24_sizes(4, 8, "bf16") == (4 * 4 * 2, 4 * 4)
    for t in ("s8", "u8", "e4m3", "e5m2"):
        assert G.gemm_sparse24_sizes(4, 40, t) == (4 * 20, 4 * 2 * 4)
    with pytest.raises(G.GemmError) as e:
        G.gemm_sparse24_sizes(4, 8, "f32")
    assert e.value.status == G.GEMM_ERR_UNSUPPORTED


def test_run_rejects_null_plan_without_gpu():
    L = G.load()
    assert L.gemm_run(None, None, None, None, None, None, None) == G.GEMM_ERR_NULL_POINTER
    assert L.gemm_plan(None, ctypes.byref(ctypes.c_void_p())) == G.GEMM_ERR_NULL_POINTER
