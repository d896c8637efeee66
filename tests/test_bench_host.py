"""Host-side logic of bench.py (no GPU): the one-GPU contract, the
algorithmic byte counts the roofline uses, and the rule that the measured
HBM traffic is reported only when the counters were taken on the current
kernel sources."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from sparse_tiled_gemm_amd import inputs  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_algorithmic_bytes_dense_and_sparse():
    M, N, K = 64, 96, 128
    p = inputs.dense_bf16(M, N, K)  # bf16 A, B; fp32 C; bf16 D; no bias
    assert bench.algorithmic_bytes(p) == M * K * 2 + N * K * 2 + M * N * 4 + M * N * 2
    q = inputs.sparse24_f16(M, N, K)  # values M x K/2 fp16 + one u32 per 32 K
    want = M * (K // 2) * 2 + M * (K // 32) * 4 + N * K * 2 + M * N * 4 + M * N * 4
    assert bench.algorithmic_bytes(q, sparse=True) == want


def test_traffic_only_for_current_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    # the hash is taken over ROOT's kernel sources: give the temporary root a copy
    src = tmp_path / "sparse_tiled_gemm_amd" / "csrc"
    src.mkdir(parents=True)
    (src / "k.hip").write_text("kernel one")
    h = bench.kernel_source_hash()
    (prof / "traffic_w.json").write_text(json.dumps(
        {"kernel_source_hash": h, "fetch_bytes_scaled": 10, "write_bytes_scaled": 5}))
    assert bench.measured_traffic("w") == 15
    (src / "k.hip").write_text("kernel two")  # sources changed since the counters
    assert bench.measured_traffic("w") is None
    assert bench.measured_traffic("absent") is None

