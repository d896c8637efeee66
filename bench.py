#!/usr/bin/env python3
"""Throughput of the gfx950 GEMM library on its synthetic workloads.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-extras] [--no-cpu-baseline] [--ceiling]

One step is one call of the library (gemm_run, or gemm_sparse24_run for the
2:4 workload) over the workload's operands, which are resident in device
memory before the timed region starts.  The headline workload is the dense
bf16 GEMM at M = N = K = 8192 (bf16 out); its TFLOPS is `value`.  The other
workloads are timed the same way and reported under "workloads".  Prints one
JSON line.

Only one GPU is used: --gpus above 1 exits with an error message.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X datasheet dense peaks (TFLOP/s or TOP/s) and HBM bandwidth (GB/s).
# The 2:4 kinds are priced against twice the dense peak of their type (the
# effective rate of a 2:4 product counts the dropped half of A's products).
PEAK = {"bf16": 2516.6, "f16": 2516.6, "fp8": 5033.2, "s8": 5033.2, "sparse_f16": 5033.2,
        "sparse_bf16": 5033.2, "sparse_fp8": 10066.4, "sparse_s8": 10066.4,
        "mxfp8": 5033.2, "mxfp6": 10066.4, "mxfp4": 10066.4, "w4a16_bf16": 2516.6}
HBM_GBS = 8000.0

HEADLINE = "bf16_8192"


def _workloads():
    from sparse_tiled_gemm_amd import inputs
    return {
        "f16_128": (lambda: inputs.dense_f16(128, 128, 128), "f16"),
        "bf16_8192": (lambda: inputs.dense_bf16(8192, 8192, 8192), "bf16"),
        "bf16_skinny_16x8192x8192": (lambda: inputs.dense_bf16(16, 8192, 8192), "bf16"),
        "bf16_8192_acol_brow": (lambda: _mn_major(inputs.dense_bf16(8192, 8192, 8192)), "bf16"),
        "bf16_8192_c_bf16": (lambda: _c16(inputs.dense_bf16(8192, 8192, 8192), "bf16"), "bf16"),
        "fp8_8192_acol_brow": (lambda: _mn_major(inputs.dense_fp8(8192, 8192, 8192)), "fp8"),
        "s8_8192_acol_brow": (lambda: _mn_major(inputs.dense_s8(8192, 8192, 8192)), "s8"),
        "s8_8192": (lambda: inputs.dense_s8(8192, 8192, 8192), "s8"),
        "fp8_8192": (lambda: inputs.dense_fp8(8192, 8192, 8192), "fp8"),
        "sparse24_f16_8192": (lambda: inputs.sparse24_f16(8192, 8192, 8192), "sparse_f16"),
        "sparse24_bf16_8192": (lambda: inputs.sparse24_bf16(8192, 8192, 8192), "sparse_bf16"),
        "sparse24_s8_8192": (lambda: inputs.sparse24_s8(8192, 8192, 8192), "sparse_s8"),
        "sparse24_fp8_8192": (lambda: inputs.sparse24_fp8(8192, 8192, 8192), "sparse_fp8"),
        "mxfp8_8192": (lambda: inputs.mx_problem(8192, 8192, 8192, "e4m3", "e4m3", 9), "mxfp8"),
        "mxfp4_8192": (lambda: inputs.mx_problem(8192, 8192, 8192, "e2m1", "e2m1", 11), "mxfp4"),
        "mxfp6_8192": (lambda: inputs.mx_problem(8192, 8192, 8192, "e2m3", "e2m3", 10), "mxfp6"),
        "w4a16_bf16_8192": (lambda: inputs.w4a16_problem(8192, 8192, 8192, "bf16", 128, 12),
                            "w4a16_bf16"),
        "w4a16_bf16_16x8192x8192": (lambda: inputs.w4a16_problem(16, 8192, 8192, "bf16", 128, 13),
                                    "w4a16_bf16"),
    }


def _mn_major(p):
    """The same problem with A stored column-major ([K,M]) and B row-major
    ([K,N])."""
    p["A"] = np.ascontiguousarray(p["A"].T)
    p["B"] = np.ascontiguousarray(p["B"].T)
    p["a_col"], p["b_col"] = True, False
    return p


def _c16(p, c_type):
    """The same problem with C given as fp16 or bf16 (its fp32 values
    rounded to nearest even)."""
    from sparse_tiled_gemm_amd import inputs
    p["C"] = (inputs.to_bf16 if c_type == "bf16" else inputs.to_f16)(p["C"])
    p["c_type"] = c_type
    return p


def _dev(a):
    import torch
    a = np.ascontiguousarray(a)
    view = {1: np.uint8, 2: np.int16, 4: np.int32}[a.itemsize]
    return torch.from_numpy(a.view(view)).cuda()


def algorithmic_bytes(p, sparse=False):
    """Operand bytes read and written once: A (or values + metadata), B, C,
    bias, D."""
    from sparse_tiled_gemm_amd import gemm as G
    M, N, K = p["M"], p["N"], p["K"]
    eb = G.ELEM_BYTES
    if p.get("w4"):  # A, the packed codes, scales and zero points, D
        return (p["A"].nbytes + p["B"].nbytes + p["scales"].nbytes +
                (p["zeros"].nbytes if p["zeros"] is not None else 0) +
                (M * N * 4 if p["C"] is not None else 0) + M * N * eb[p["d_type"]])
    if p.get("mx"):  # packed elements and one scale byte per 32 K
        return (p["A"].nbytes + p["B"].nbytes + p["SA"].nbytes + p["SB"].nbytes +
                (M * N * 4 if p["C"] is not None else 0) + M * N * eb[p["d_type"]])
    if sparse:
        a = M * (K // 2) * eb[p["a_type"]] + M * ((K + 31) // 32) * 4
    else:
        a = M * K * eb[p["a_type"]]
    b = N * K * eb[p["b_type"]]
    c = M * N * (2 if p.get("c_type") in ("f16", "bf16") else 4) if p["C"] is not None else 0
    bias = N * 4 if p["bias"] is not None else 0
    d = M * N * eb[p["d_type"]]
    return a + b + c + bias + d


def run_workload(name, steps, warmup, rotate_b=3, per_call=0):
    """Time `steps` library calls; returns a dict of measurements.  B cycles
    through `rotate_b` copies, so the 256 MB memory-side cache cannot keep
    every operand of the 8192^3 workloads between calls.  With per_call > 0,
    that many further calls are then timed one by one (median, min, max;
    reported beside the mean of the timed region, which stays the result)."""
    import torch
    from sparse_tiled_gemm_amd import gemm as G
    make, kind = _workloads()[name]
    p = make()
    M, N, K = p["M"], p["N"], p["K"]
    sparse = p.get("A_logical") is not None
    mx, w4 = bool(p.get("mx")), bool(p.get("w4"))
    desc = G.make_desc(M, N, K, p["a_type"], p["b_type"], p["d_type"], c_type=p.get("c_type"),
                       has_c=p["C"] is not None, has_bias=p["bias"] is not None, alpha=p["alpha"],
                       act="relu" if p["relu"] else "none", sparse_a=sparse,
                       block_scale=32 if mx else (p["gs"] if w4 else 0),
                       a_layout="col" if p.get("a_col") else "row",
                       b_layout="row" if p.get("b_col") is False else "col")
    plan = G.gemm_plan(desc)
    Bs = [_dev(p["B"]) for _ in range(rotate_b)]
    tC = _dev(p["C"]) if p["C"] is not None else None
    tbias = _dev(p["bias"]) if p["bias"] is not None else None
    D = torch.empty(M * N * G.ELEM_BYTES[p["d_type"]], dtype=torch.uint8, device="cuda")
    if sparse:
        vb, mb = G.gemm_sparse24_sizes(M, K, p["a_type"])
        tAl = _dev(p["A_logical"])
        vals = torch.empty(vb, dtype=torch.uint8, device="cuda")
        meta = torch.empty(mb, dtype=torch.uint8, device="cuda")
        G.gemm_sparse24_compress(M, K, p["a_type"], tAl, vals, meta)
        del tAl

        def call(i):
            G.gemm_sparse24_run(plan, vals, meta, Bs[i % rotate_b], tC, tbias, D)
    elif w4:
        tA, tS = _dev(p["A"]), _dev(p["scales"])
        tZ = _dev(p["zeros"]) if p["zeros"] is not None else None

        def call(i):
            G.gemm_w4a16_run(plan, tA, Bs[i % rotate_b], tS, tZ, tC, tbias, D)
    elif mx:
        tA, tSA, tSB = _dev(p["A"]), _dev(p["SA"]), _dev(p["SB"])

        def call(i):
            G.gemm_mx_run(plan, tA, tSA, Bs[i % rotate_b], tSB, tC, tbias, D)
    else:
        tA = _dev(p["A"])

        def call(i):
            G.gemm_run(plan, tA, Bs[i % rotate_b], tC, tbias, D)

    stream = torch.cuda.current_stream()
    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        call(i)
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    flops = 2.0 * M * N * K
    out = {
        "workload": name, "kernel": plan.name, "M": M, "N": N, "K": K,
        "a_type": p["a_type"], "b_type": p["b_type"], "d_type": p["d_type"],
        "ms_per_call": ms, "us_per_call": ms * 1e3, "b_copies": rotate_b,
    }
    if per_call > 0:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(per_call)]
        for i, (e0, e1) in enumerate(evs):
            e0.record(stream)
            call(steps + i)
            e1.record(stream)
        torch.cuda.synchronize()
        us = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs)
        out["per_call_us"] = {"n": per_call, "median": us[per_call // 2], "min": us[0],
                              "max": us[-1]}
    byts = algorithmic_bytes(p, sparse)
    out["algorithmic_bytes"] = byts
    out["GBps"] = byts / (ms * 1e-3) / 1e9
    if sparse:
        # TOPS for s8 (the key names keep the float spelling)
        out["effective_TFLOPS"] = flops / (ms * 1e-3) / 1e12
        out["algorithmic_TFLOPS"] = flops / 2 / (ms * 1e-3) / 1e12
        out["frac_sparse_peak"] = out["effective_TFLOPS"] / PEAK[kind]
        out["frac_dense_peak_algorithmic"] = out["algorithmic_TFLOPS"] / (PEAK[kind] / 2)
    else:
        unit = "TOPS" if kind == "s8" else "TFLOPS"
        out[unit] = flops / (ms * 1e-3) / 1e12
        out["frac_peak"] = out[unit] / PEAK[kind]
    out["frac_hbm"] = out["GBps"] / HBM_GBS
    return out, p


def kernel_source_hash():
    """Hash of the sources the dense, skinny and sparse kernels are built from."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_tiled_gemm_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp", ".cpp")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    if it was taken on the kernel sources as they are now (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t["fetch_bytes_scaled"] + t["write_bytes_scaled"]


def cpu_baseline(p, rows=4096):
    """The CPU oracle on rows 0..rows-1 of the workload (bounded sample)."""
    from oracle import oracle
    M, N, K = p["M"], p["N"], p["K"]
    r = min(rows, M)
    t0 = time.perf_counter()
    oracle.gemm(p["A"][:r], p["B"], p["C"][:r] if p["C"] is not None else None, p["bias"], r,
                N, K, p["a_type"], p["b_type"], p["d_type"], alpha=p["alpha"], relu=p["relu"],
                want_y=False, want_s=False)
    dt = time.perf_counter() - t0
    return {"value": 2.0 * r * N * K / dt / 1e12, "unit": "TFLOPS", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": dt,
            "sample": "rows 0..%d of A: a %dx%dx%d slice of the %dx%dx%d workload, fp64 "
                      "accumulation, same epilogue" % (r - 1, r, N, K, M, N, K)}


def ceiling(steps, warmup):
    """The MFMA-only throughput ceiling (gemm_diag_mfma_loop): one workgroup
    of 8 waves per compute unit issuing nothing but MFMAs on random register
    operands; each launch sized to about a millisecond."""
    import torch
    from sparse_tiled_gemm_amd import gemm as G
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(cus * 512, dtype=torch.float32, device="cuda")
    res = {}
    # kind k (32x32 form) and k + 3 (16x16 form) do the same work per
    # iteration: 64 instructions of `flop` each per wave
    for kind, name, flop, peak in [(0, "bf16", 32768, PEAK["bf16"]), (1, "fp8", 131072, PEAK["fp8"]),
                                   (2, "s8", 65536, PEAK["s8"]),
                                   (3, "bf16_16x16", 32768, PEAK["bf16"]),
                                   (4, "fp8_16x16", 131072, PEAK["fp8"]),
                                   (5, "s8_16x16", 65536, PEAK["s8"])]:
        per_iter = cus * 8 * 64 * flop
        iters = max(1, int(0.6 * peak * 1e12 * 1e-3 / per_iter))
        for _ in range(warmup):
            G.gemm_diag_mfma_loop(kind, cus, iters, out)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            G.gemm_diag_mfma_loop(kind, cus, iters, out)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        rate = per_iter * iters / (ms * 1e-3) / 1e12
        res[name] = {"TOPS" if name.startswith("s8") else "TFLOPS": rate, "frac_peak": rate / peak,
                     "ms_per_launch": ms, "iters": iters, "workgroups": cus}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the first calls after the operands are allocated run 5-20 % slower
    # than the steady state (about 25 calls); the default warm-up covers them
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(_workloads().keys()))
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (x3), the reference kernel for "
                         "scaling the FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--ceiling", action="store_true",
                    help="run only the MFMA-only ceiling diagnostic (bf16, fp8, int8; 32x32 and "
                         "16x16 forms) and print "
                         "its rates as one JSON line")
    ap.add_argument("--force-kernel", default=None,
                    help="kernel family to force (tuning: sets STGEMM_FORCE_KERNEL)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the GEMM library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        import torch
        torch.cuda.set_device(0)
        a = torch.ones(1 << 28, device="cuda")  # 1 GiB of fp32
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": a.numel() * 4, "copies": 3}))
        return
    if args.ceiling:
        import torch
        torch.cuda.set_device(0)
        from sparse_tiled_gemm_amd import gemm as G
        G.load()
        print(json.dumps({"mfma_only_ceiling": ceiling(args.steps, args.warmup)}))
        return
    if args.force_kernel:
        os.environ["STGEMM_FORCE_KERNEL"] = args.force_kernel
    import torch
    torch.cuda.set_device(0)
    from sparse_tiled_gemm_amd import gemm as G
    G.load()

    head, p = run_workload(args.workload, args.steps, args.warmup, per_call=50)
    kind = _workloads()[args.workload][1]
    unit = "TOPS" if kind in ("s8", "sparse_s8") else "TFLOPS"
    sparse = kind.startswith("sparse_")
    value = head["effective_TFLOPS"] if sparse else head[unit]
    achieved = value
    roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK[kind],
                "unit": "TOP/s" if unit == "TOPS" else "TFLOP/s", "frac": achieved / PEAK[kind],
                "traffic": measured_traffic(args.workload), "kernel": head["kernel"],
                "algorithmic_flops_per_launch": 2.0 * p["M"] * p["N"] * p["K"]}
    result = {
        "metric": "TFLOPS (TOPS int8) at M=N=K=8192 per dtype; % of MFMA peak",
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_call"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "f16": "f16", "fp8": "fp8_e4m3xe5m2", "s8": "s8",
                  "sparse_f16": "f16", "sparse_bf16": "bf16", "sparse_fp8": "fp8_e4m3xe5m2",
                  "sparse_s8": "s8", "mxfp8": "mxfp8_e4m3", "mxfp6": "mxfp6_e2m3",
                  "mxfp4": "mxfp4_e2m1", "w4a16_bf16": "bf16_u4"}[kind],
        "data": "synthetic",
        "config": {"workload": args.workload, "M": p["M"], "N": p["N"], "K": p["K"],
                   "a_type": p["a_type"], "b_type": p["b_type"], "d_type": p["d_type"],
                   "parallelism": "none (one GPU)"},
        "frac_of_peak": value / PEAK[kind],
        "roofline": roofline,
        "per_call_us": head["per_call_us"],
    }
    result["config"]["b_copies"] = head["b_copies"]
    del p
    if not args.no_cpu_baseline:
        _, pc = None, _workloads()[args.workload][0]()
        result["cpu_baseline"] = cpu_baseline(pc)
        del pc
    if not args.no_extras:
        extras = {}
        for name in _workloads():
            if name == args.workload:
                continue
            rot = 4 if (name.startswith("bf16_skinny") or name.startswith("w4a16_bf16_16x")) else 3
            try:
                r, _ = run_workload(name, args.steps, args.warmup, rotate_b=rot)
            except Exception as e:  # report, keep the headline line
                r = {"error": str(e)}
            extras[name] = r
            torch.cuda.empty_cache()
        result["workloads"] = extras
    print(json.dumps(result))


if __name__ == "__main__":
    main()
