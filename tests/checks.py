"""Parity criteria between a GPU result and the oracle.

- Integer outputs: bit-exact.
- fp32 outputs: |D - Y| <= tol * |alpha| * S + ulp32(Y), where Y is the
  oracle's fp64 result before the cast and S = sum_k |a b| + |c| (with alpha
  = 1 and no bias this is the normalised bound max |D - D_ref| / S <= tol).
- fp16 / bf16 outputs: within 1 ulp of the oracle's correctly rounded value
  (distance of the ordered bit patterns), or, where fp32 accumulation error
  alone can exceed one output ulp (results near 0),
  |D - Y| <= ulp_out(Y) + tol * |alpha| * S.
tol = 1e-5 for fp16/bf16 inputs and 1e-4 for fp8 inputs (and the MX formats); 1e-6
for s8 inputs with a float output (the int32 sum is exact; only its fp32
conversion and the epilogue round).
- fp8 outputs: within 1 ulp of the format, or the bound above with an fp8 ulp;
  results beyond the largest finite value must equal the saturated value.
"""
import numpy as np

from exact import lib_decode

TOL = {"f16": 1e-5, "bf16": 1e-5, "e4m3": 1e-4, "e5m2": 1e-4, "e2m3": 1e-4, "e3m2": 1e-4,
       "e2m1": 1e-4, "s8": 1e-6}


def ordered16(bits):
    b = np.asarray(bits).astype(np.uint16).astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def ulp16(y, d_type):
    """Spacing of fp16 / bf16 values at |y|."""
    a = np.abs(np.asarray(y, dtype=np.float64))
    fbits, emin = (10, -14) if d_type == "f16" else (7, -126)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, emin)
    return np.ldexp(1.0, (e - fbits).astype(np.int64))


def ordered8(bits):
    b = np.asarray(bits).astype(np.uint8).astype(np.int64)
    return np.where(b & 0x80, -(b & 0x7F), b)


def ulp8(y, d_type):
    """Spacing of E4M3 / E5M2 values at |y|."""
    a = np.abs(np.asarray(y, dtype=np.float64))
    fbits, emin = (3, -6) if d_type == "e4m3" else (2, -14)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, emin)
    return np.ldexp(1.0, (e - fbits).astype(np.int64))


def ulp32(y):
    a = np.abs(np.asarray(y, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.ldexp(1.0, (np.maximum(e, -126) - 23).astype(np.int64))


class Result:
    def __init__(self, ok, n, max_norm_err=0.0, n_second_clause=0, n_bad=0, detail=""):
        self.ok, self.n, self.max_norm_err = ok, n, max_norm_err
        self.n_second_clause, self.n_bad, self.detail = n_second_clause, n_bad, detail

    def __repr__(self):
        return ("Result(ok=%s, n=%d, max_norm_err=%.3g, second_clause=%d, bad=%d %s)" %
                (self.ok, self.n, self.max_norm_err, self.n_second_clause, self.n_bad,
                 self.detail))


def check(D, d_type, D_ref, Y, S, in_type, alpha=1.0):
    """D, D_ref: raw output bits (same shape); Y, S: oracle fp64 arrays."""
    D = np.asarray(D)
    n = D.size
    if d_type == "s32":
        bad = np.asarray(D).view(np.int32) != np.asarray(D_ref).view(np.int32)
        nb = int(bad.sum())
        det = ""
        if nb:
            i = np.flatnonzero(bad.reshape(-1))[0]
            det = "first mismatch at flat %d: %d vs %d" % (
                i, D.reshape(-1).view(np.int32)[i], np.asarray(D_ref).reshape(-1).view(np.int32)[i])
        return Result(nb == 0, n, 0.0, 0, nb, det)
    tol = TOL[in_type]
    Y = np.asarray(Y, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    scale = abs(alpha) * S
    with np.errstate(divide="ignore", invalid="ignore"):
        if d_type == "f32":
            d = np.asarray(D, dtype=np.float32).astype(np.float64)
            err = np.abs(d - Y)
            ok = err <= tol * scale + ulp32(Y)
            norm = np.where(scale > 0, err / np.where(scale > 0, scale, 1), np.where(err > 0, np.inf, 0))
            nb = int((~ok).sum())
            det = ""
            if nb:
                i = np.flatnonzero(~ok.reshape(-1))[0]
                det = "first bad flat %d: D=%r Y=%r S=%r" % (i, d.reshape(-1)[i], Y.reshape(-1)[i],
                                                            S.reshape(-1)[i])
            return Result(nb == 0, n, float(norm.max()) if n else 0.0, 0, nb, det)
        if d_type in ("e4m3", "e5m2"):
            # FP8 outputs: 1 ulp of the format (ordered 8-bit codes), or the
            # accumulation bound; results past the largest finite value
            # must be that value exactly (saturation)
            d = lib_decode(d_type, np.asarray(D).astype(np.uint8))
            dist = np.abs(ordered8(D) - ordered8(D_ref))
            vmax = 448.0 if d_type == "e4m3" else 57344.0
            sat = np.abs(Y) >= vmax
            first = (dist <= 1) & ~sat | (sat & (np.asarray(D) == np.asarray(D_ref)))
            err = np.abs(d - Y)
            second = ~sat & (err <= ulp8(Y, d_type) + tol * scale)
        else:
            d = lib_decode(d_type, np.asarray(D).astype(np.uint16))
            dist = np.abs(ordered16(D) - ordered16(D_ref))
            first = dist <= 1
            err = np.abs(d - Y)
            second = err <= ulp16(Y, d_type) + tol * scale
        ok = first | second
        norm = np.where(scale > 0, err / np.where(scale > 0, scale, 1), 0.0)
        nb = int((~ok).sum())
        det = ""
        if nb:
            i = np.flatnonzero(~ok.reshape(-1))[0]
            det = "first bad flat %d: D=%r Dref bits=%r Y=%r S=%r" % (
                i, d.reshape(-1)[i], np.asarray(D_ref).reshape(-1)[i], Y.reshape(-1)[i],
                S.reshape(-1)[i])
        return Result(nb == 0, n, float(norm.max()) if n else 0.0, int((~first & second).sum()),
                      nb, det)


def check_rows(D, d_type, D_ref, Y, S, in_type, alpha=1.0, rows=512):
    """check() over an [M,N] output in blocks of `rows` rows (bounded
    temporaries at full size); one Result for the whole output whose detail
    names the first bad element's (row, column)."""
    D = np.asarray(D)
    M = D.shape[0]
    tot = Result(True, 0)
    for r0 in range(0, M, rows):
        r1 = min(M, r0 + rows)
        r = check(D[r0:r1], d_type, D_ref[r0:r1], None if Y is None else Y[r0:r1],
                  None if S is None else S[r0:r1], in_type, alpha)
        if r.n_bad and tot.ok:
            tot.detail = "rows %d..%d: %s" % (r0, r1 - 1, r.detail)
        tot.ok &= r.ok
        tot.n += r.n
        tot.max_norm_err = max(tot.max_norm_err, r.max_norm_err)
        tot.n_second_clause += r.n_second_clause
        tot.n_bad += r.n_bad
    return tot
