"""Compile the HIP library libstgemm.so in-tree for gfx950.

Each source is compiled on its own (in parallel) with hipcc, then linked.
Run `python -m sparse_tiled_gemm_amd.build [-v] [--asm] [--incremental]`;
--asm also keeps the gfx950 assembly under _build/ for inspection;
--incremental recompiles only the sources whose object file is older than the
source or a header (build() called without it compiles everything).
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libstgemm.so")
SOURCES = ["gemm_api.cpp", "kernels_dense.hip", "kernels_sparse.hip", "kernels_mx.hip",
           "kernels_w4.hip", "kernels_mn.hip", "kernels_diag.hip", "kernels_k16.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC", "-ffp-contract=off",
    "-Wall", "-Wno-unused-function",
    # packed fp32 instructions stay out of generated code (they are not used
    # deliberately anywhere here); the host pass warns it does not know the
    # feature, which is harmless
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src, asm, verbose):
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC] + FLAGS + ["-x", "hip", "-c", path, "-o", obj]
    if asm:
        cmd += ["-save-temps=obj"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, msgs))
    if verbose and msgs.strip():
        print(msgs)
    return obj


def _stale(src):
    """True when src's object is missing or older than src or any header."""
    obj = os.path.join(BUILD, src + ".o")
    if not os.path.exists(obj):
        return True
    deps = [os.path.join(CSRC, src)] + [os.path.join(CSRC, f) for f in os.listdir(CSRC)
                                        if f.endswith((".hpp", ".h"))]
    deps += [os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE)]
    t = os.path.getmtime(obj)
    return any(os.path.getmtime(d) > t for d in deps)


def build(verbose=False, asm=False, incremental=False):
    """Compile every source (incremental=True: only those whose object is
    older than the source or a header) and link libstgemm.so."""
    os.makedirs(BUILD, exist_ok=True)
    todo = [s for s in SOURCES if not incremental or asm or _stale(s)]
    if todo:
        with concurrent.futures.ThreadPoolExecutor(max_workers=len(todo)) as ex:
            list(ex.map(lambda s: _compile(s, asm, verbose), todo))
    objs = [os.path.join(BUILD, s + ".o") for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, asm="--asm" in sys.argv,
                incremental="--incremental" in sys.argv))
