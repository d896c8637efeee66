"""The library's host layer (descriptor validation, kernel planning, argument
and overlap checks of every entry point: csrc/gemm_api.cpp) built with g++
under AddressSanitizer and UndefinedBehaviorSanitizer, with the HIP runtime
and the kernel launchers replaced by stubs (tests/host_sanitize/driver.cpp),
and driven through fixed cases and a seeded fuzz of extreme descriptors.
CPU only: no GPU code is built or run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_tiled_gemm_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_host_layer_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_driver")
    cmd = ["g++", "-std=c++20", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-o", exe, os.path.join(ROOT, "tests", "host_sanitize", "driver.cpp"),
           os.path.join(CSRC, "gemm_api.cpp")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe, "300000"], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "ok" in r.stdout and "runtime error" not in r.stderr
