"""The allocation-free compressor entry point, gemm_sparse24_compress_noalloc,
against gemm_sparse24_compress (which allocates its flag per call): the same
values and metadata bytes, and the same status, on calls in a row - the
later ones smaller, of other types, and one that fails (a group with three
non-zeros) followed by one that must succeed, which shows the shared device
flag is cleared at the start of every call."""
import numpy as np
import pytest
import torch

from gpu_util import say, to_dev
from sparse_tiled_gemm_amd import gemm as G
from sparse_tiled_gemm_amd import inputs

pytestmark = pytest.mark.gpu


def _both(A, t):
    """Compress A (raw bits [M,K]) with both entry points; returns the
    statuses and the output bytes of each."""
    M, K = A.shape
    vb, mb = G.gemm_sparse24_sizes(M, K, t)
    tA = to_dev(A)
    outs = []
    for fn in (G.gemm_sparse24_compress, G.gemm_sparse24_compress_noalloc):
        vals = torch.full((max(vb, 16),), 0xA5, dtype=torch.uint8, device="cuda")
        meta = torch.full((max(mb, 16),), 0x5A, dtype=torch.uint8, device="cuda")
        status, msg = G.GEMM_OK, ""
        try:
            fn(M, K, t, tA, vals, meta)
        except G.GemmError as e:
            status, msg = e.status, str(e)
        torch.cuda.synchronize()
        outs.append((status, msg, vals[:vb].cpu().numpy(), meta[:mb].cpu().numpy()))
    return outs


@pytest.mark.parametrize("first,second", [
    (("f16", 512, 1024), ("f16", 96, 160)),
    (("bf16", 384, 512), ("s8", 64, 96)),
    (("e4m3", 1024, 2048), ("e5m2", 8, 32)),
])
def test_noalloc_matches_compress_two_calls(orc, first, second):
    for t, M, K in (first, second):
        say("noalloc compress", t, M, K)
        p = inputs.sparse24(t, M, 64, K)
        (s0, _, v0, m0), (s1, _, v1, m1) = _both(p["A_logical"], t)
        assert s0 == G.GEMM_OK and s1 == G.GEMM_OK
        assert np.array_equal(v0, v1) and np.array_equal(m0, m1)
        # and both are the oracle's bytes
        rv, rm = orc.sparse24_compress(p["A_logical"], t)
        assert np.array_equal(v1.view(rv.dtype).reshape(rv.shape), rv)
        assert np.array_equal(m1.view(np.uint32).reshape(rm.shape), rm)


def test_noalloc_error_then_success():
    """A failing call leaves the flag set on the device; the next call,
    smaller and valid, must still succeed."""
    p = inputs.sparse24("f16", 256, 64, 512)
    bad = p["A_logical"].copy()
    row = 77
    g = np.flatnonzero(bad[row, 0:4] == 0)[0]  # a zero of group 0 made non-zero
    bad[row, g] = 0x3C00  # 1.0
    say("noalloc compress with a 3-non-zero group in row", row)
    (s0, msg0, _, _), (s1, msg1, _, _) = _both(bad, "f16")
    assert s0 == G.GEMM_ERR_NOT_SPARSE24 and s1 == G.GEMM_ERR_NOT_SPARSE24
    assert ("row: %d" % row) in msg0 and ("row: %d" % row) in msg1
    q = inputs.sparse24("f16", 128, 64, 256)
    say("noalloc compress after the failure, smaller input")
    (s0, _, v0, m0), (s1, _, v1, m1) = _both(q["A_logical"], "f16")
    assert s0 == G.GEMM_OK and s1 == G.GEMM_OK
    assert np.array_equal(v0, v1) and np.array_equal(m0, m1)


def test_noalloc_argument_errors():
    vals = torch.empty(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(G.GemmError) as e:
        G.gemm_sparse24_compress_noalloc(4, 6, "f16", vals, vals, vals)  # K % 4 != 0
    assert e.value.status == G.GEMM_ERR_UNSUPPORTED
    with pytest.raises(G.GemmError) as e:
        G.gemm_sparse24_compress_noalloc(4, 8, "f16", None, vals, vals)
    assert e.value.status == G.GEMM_ERR_NULL_POINTER
    # nothing to do: OK without touching the device
    G.gemm_sparse24_compress_noalloc(0, 8, "f16", None, None, None)
