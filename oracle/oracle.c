/*
 * CPU oracle for D = A*B + C with a scale/bias/activation/cast epilogue and
 * the 2:4 structured-sparse-A variant.  TEST INFRASTRUCTURE ONLY (see
 * oracle.h): plain loops, fp64/int64 accumulation, k ascending, no blocking.
 *
 * Sources of each definition are cited at the functions.  Bit formats follow
 * IEEE 754 (binary16/binary32), bfloat16 (upper half of binary32) and the OCP
 * 8-bit floating point specification (E4M3, E5M2).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

/* ------------------------------------------------------------------ decode */

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double dec_f16(uint16_t h)
{
    double s = (h & 0x8000) ? -1.0 : 1.0;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    if (e == 0)
        return s * ldexp((double)f, -24);
    if (e == 31)
        return f ? NAN : s * INFINITY;
    return s * ldexp((double)(1024 + f), e - 25);
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits. */
static double dec_bf16(uint16_t h)
{
    double s = (h & 0x8000) ? -1.0 : 1.0;
    int e = (h >> 7) & 0xFF;
    int f = h & 0x7F;
    if (e == 0)
        return s * ldexp((double)f, -133);
    if (e == 255)
        return f ? NAN : s * INFINITY;
    return s * ldexp((double)(128 + f), e - 134);
}

/* OCP E4M3: 1 sign, 4 exponent (bias 7), 3 fraction bits; S.1111.111 is NaN,
 * there is no infinity, so exponent 15 with fraction 0..6 are normal values. */
static double dec_e4m3(uint8_t v)
{
    double s = (v & 0x80) ? -1.0 : 1.0;
    int e = (v >> 3) & 0xF;
    int f = v & 0x7;
    if (e == 15 && f == 7)
        return NAN;
    if (e == 0)
        return s * ldexp((double)f, -9);
    return s * ldexp((double)(8 + f), e - 10);
}

/* OCP E5M2: 1 sign, 5 exponent (bias 15), 2 fraction bits, IEEE specials. */
static double dec_e5m2(uint8_t v)
{
    double s = (v & 0x80) ? -1.0 : 1.0;
    int e = (v >> 2) & 0x1F;
    int f = v & 0x3;
    if (e == 0)
        return s * ldexp((double)f, -16);
    if (e == 31)
        return f ? NAN : s * INFINITY;
    return s * ldexp((double)(4 + f), e - 17);
}

/* OCP MX element formats: sign, e exponent bits, f fraction bits, bias;
 * exponent field 0 is subnormal (f/2^f_bits * 2^(1-bias)); no inf or NaN. */
static double dec_mx(uint32_t v, int ebits, int fbits, int bias)
{
    double s = (v >> (ebits + fbits)) & 1u ? -1.0 : 1.0;
    int e = (int)((v >> fbits) & ((1u << ebits) - 1u));
    int f = (int)(v & ((1u << fbits) - 1u));
    if (e == 0)
        return s * ldexp((double)f, 1 - bias - fbits);
    return s * ldexp((double)((1 << fbits) + f), e - bias - fbits);
}

/* element idx of a packed 6-bit row: bits 6 idx .. 6 idx + 5, little-endian */
static uint32_t get6(const void *base, int64_t idx)
{
    const uint8_t *p = (const uint8_t *)base;
    const int64_t bit = 6 * idx;
    uint32_t w = p[bit / 8];
    if ((bit % 8) > 2)
        w |= (uint32_t)p[bit / 8 + 1] << 8;
    return (w >> (bit % 8)) & 0x3Fu;
}

double oracle_decode(int type, const void *base, int64_t idx)
{
    switch (type) {
    case OR_E2M3: return dec_mx(get6(base, idx), 2, 3, 1);
    case OR_E3M2: return dec_mx(get6(base, idx), 3, 2, 3);
    case OR_E2M1: return dec_mx((((const uint8_t *)base)[idx / 2] >> (4 * (idx % 2))) & 0xFu, 2, 1, 1);
    case OR_E8M0: {
        uint8_t e = ((const uint8_t *)base)[idx];
        return e == 0xFF ? NAN : ldexp(1.0, (int)e - 127);
    }
    case OR_F16: return dec_f16(((const uint16_t *)base)[idx]);
    case OR_BF16: return dec_bf16(((const uint16_t *)base)[idx]);
    case OR_E4M3: return dec_e4m3(((const uint8_t *)base)[idx]);
    case OR_E5M2: return dec_e5m2(((const uint8_t *)base)[idx]);
    case OR_S8: return (double)((const int8_t *)base)[idx];
    case OR_U8: return (double)((const uint8_t *)base)[idx];
    case OR_F32: return (double)((const float *)base)[idx];
    case OR_S32: return (double)((const int32_t *)base)[idx];
    default: return NAN;
    }
}

/* ------------------------------------------------------------------ encode */

/* Round x to a binary format with p significand bits (implicit bit included),
 * minimum normal exponent emin and largest finite magnitude maxv, ties to
 * even; magnitudes past maxv after rounding become infinity (IEEE 754
 * roundTiesToEven overflow rule).  q is the spacing of representable values
 * in x's binade (subnormal spacing below emin); x/q is exact because q is a
 * power of two, and nearbyint rounds half to even in the default mode. */
static double round_binary(double x, int p, int emin, double maxv)
{
    if (isnan(x) || isinf(x) || x == 0.0)
        return x;
    int e;
    (void)frexp(x, &e);
    int lead = e - 1;
    if (lead < emin)
        lead = emin;
    double q = ldexp(1.0, lead - (p - 1));
    double r = nearbyint(x / q) * q;
    if (fabs(r) > maxv)
        r = copysign(INFINITY, x);
    return r;
}

/* Bit pattern of an exactly representable value r in a binary format with
 * `fbits` fraction bits, exponent bias `bias` and `ebits` exponent bits. */
static uint32_t pack_binary(double r, int ebits, int fbits, int bias, uint32_t qnan)
{
    uint32_t sign = signbit(r) ? (1u << (ebits + fbits)) : 0u;
    uint32_t emax_field = (1u << ebits) - 1u;
    if (isnan(r))
        return qnan;
    double a = fabs(r);
    if (isinf(a))
        return sign | (emax_field << fbits);
    if (a == 0.0)
        return sign;
    int e;
    (void)frexp(a, &e);
    int lead = e - 1;
    int emin = 1 - bias;
    if (lead < emin) /* subnormal: a = f * 2^(emin - fbits) */
        return sign | (uint32_t)(a / ldexp(1.0, emin - fbits));
    uint32_t f = (uint32_t)(a / ldexp(1.0, lead - fbits) - ldexp(1.0, fbits));
    return sign | ((uint32_t)(lead + bias) << fbits) | f;
}

int oracle_encode(int type, double x, void *base, int64_t idx)
{
    switch (type) {
    case OR_F16: {
        double r = round_binary(x, 11, -14, 65504.0);
        ((uint16_t *)base)[idx] = (uint16_t)pack_binary(r, 5, 10, 15, 0x7E00u);
        return 0;
    }
    case OR_BF16: {
        double r = round_binary(x, 8, -126, ldexp(255.0, 120)); /* (2 - 2^-7) * 2^127 */
        ((uint16_t *)base)[idx] = (uint16_t)pack_binary(r, 8, 7, 127, 0x7FC0u);
        return 0;
    }
    case OR_E4M3:
    case OR_E5M2: {
        /* round to nearest even, saturating: a result beyond the largest
         * finite value (or infinite) becomes that value with its sign; NaN
         * is 0x7F */
        const int e4 = type == OR_E4M3;
        const double maxv = e4 ? 448.0 : 57344.0;
        double r = e4 ? round_binary(x, 4, -6, maxv) : round_binary(x, 3, -14, maxv);
        if (isinf(r))
            r = copysign(maxv, r);
        uint32_t bits = isnan(r) ? 0x7Fu : (e4 ? pack_binary(r, 4, 3, 7, 0x7Fu)
                                                : pack_binary(r, 5, 2, 15, 0x7Fu));
        ((uint8_t *)base)[idx] = (uint8_t)bits;
        return 0;
    }
    case OR_F32: {
        double r = round_binary(x, 24, -126, ldexp(16777215.0, 104)); /* (2 - 2^-23) * 2^127 */
        uint32_t bits = pack_binary(r, 8, 23, 127, 0x7FC00000u);
        memcpy((uint32_t *)base + idx, &bits, 4);
        return 0;
    }
    case OR_S32: {
        /* two's complement wrap: reduce modulo 2^32 */
        int64_t v = (int64_t)x;
        ((int32_t *)base)[idx] = (int32_t)(uint32_t)(uint64_t)v;
        return 0;
    }
    default:
        return -1;
    }
}

void oracle_decode_array(int type, const void *base, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_decode(type, base, i);
}

int oracle_encode_array(int type, const double *x, int64_t n, void *base)
{
    for (int64_t i = 0; i < n; ++i)
        if (oracle_encode(type, x[i], base, i))
            return -1;
    return 0;
}

/* ------------------------------------------------------------------ GEMM */

static int is_int_in(int t) { return t == OR_S8 || t == OR_U8; }
static int is_int_type(int t) { return is_int_in(t) || t == OR_S32; }
static int is_float_in(int t) { return t == OR_F16 || t == OR_BF16 || t == OR_E4M3 || t == OR_E5M2; }

/* Input/accumulator/output pairing of "NVIDIA MMA", section "Input /
 * accumulate / output": float inputs accumulate in fp32 (here fp64, exact
 * products) and may be cast to fp32/fp16/bf16; s8 inputs accumulate in int32
 * and are written as int32 with no epilogue. */
static int is_float_out(int t)
{
    return t == OR_F32 || t == OR_F16 || t == OR_BF16 || t == OR_E4M3 || t == OR_E5M2;
}

/* C of a float output: fp32, or fp16 / bf16 (decoded exactly; the pages
 * keep the C type a separate choice, "NVIDIA MMA", section "Input /
 * accumulate / output") */
static int float_c_ok(int t) { return t == OR_F32 || t == OR_F16 || t == OR_BF16; }

static int check_desc(const oracle_gemm_t *g)
{
    if (g->M < 0 || g->N < 0 || g->K < 0)
        return -1;
    if (g->saturate && g->d_type != OR_S32) /* saturation applies to int32 outputs */
        return -1;
    if (is_int_in(g->a_type) || is_int_in(g->b_type)) {
        /* s8 and u8 pair freely (the INT8 rows of the Ampere table) */
        if (!is_int_in(g->a_type) || !is_int_in(g->b_type))
            return -1;
        if (g->d_type == OR_S32) {
            if (g->c_type != OR_S32 || g->alpha != 1.0f || g->has_bias || g->relu)
                return -1;
            return 0;
        }
        /* int8 -> float: the wrapped int32 sum, then the float epilogue */
        return (float_c_ok(g->c_type) && is_float_out(g->d_type)) ? 0 : -1;
    }
    if (!is_float_in(g->a_type) || !is_float_in(g->b_type))
        return -1;
    if (!float_c_ok(g->c_type))
        return -1;
    return is_float_out(g->d_type) ? 0 : -1;
}

static int64_t a_index(const oracle_gemm_t *g, int64_t m, int64_t k)
{
    return g->a_col_major ? k * g->lda + m : m * g->lda + k;
}

static int64_t b_index(const oracle_gemm_t *g, int64_t k, int64_t n)
{
    return g->b_col_major ? n * g->ldb + k : k * g->ldb + n;
}

/* Epilogue of one element: t = acc + C, then scale, bias, activation, cast,
 * in that order ("NVIDIA MMA", section "Input / accumulate / output").  The
 * integer path reduces the exact t modulo 2^32, or, when saturating, clamps
 * it to [-2^31, 2^31 - 1] (section "Ampere: FP16/BF16 and integer MMA
 * baseline": integer instructions wrap on overflow unless .satfinite asks
 * for saturation to the INT32 bounds). */
static void finish(const oracle_gemm_t *g, int64_t m, int64_t n, double acc, double sabs,
                   const void *C, const float *bias, void *D, int64_t d_idx, double *y_out,
                   double *s_out)
{
    double c = 0.0;
    if (g->has_c)
        c = oracle_decode(g->c_type, C, m * g->ldc + n);
    if (s_out)
        *s_out = sabs + fabs(c);
    if (is_int_type(g->d_type)) {
        int64_t t = (int64_t)acc + (int64_t)c;
        if (g->saturate)
            t = t > INT32_MAX ? INT32_MAX : (t < INT32_MIN ? INT32_MIN : t);
        int32_t w = (int32_t)(uint32_t)(uint64_t)t;
        oracle_encode(OR_S32, (double)w, D, d_idx);
        if (y_out)
            *y_out = (double)w;
        return;
    }
    if (is_int_type(g->a_type)) /* int8 -> float: the int32 accumulator's value */
        acc = (double)(int32_t)(uint32_t)(uint64_t)(int64_t)acc;
    double t = acc + c;
    double y = (double)g->alpha * t;
    if (g->has_bias)
        y += (double)bias[n];
    if (g->relu)
        y = (y > 0.0) ? y : 0.0;
    oracle_encode(g->d_type, y, D, d_idx);
    if (y_out)
        *y_out = y;
}

/* D[m,n] = sum_k A[m,k] B[k,n] + C[m,n]: "NVIDIA MMA", section "From FMA to
 * MMA to GEMM", the GEMM element equation; the same sum is written for the
 * accumulator in section "Input / accumulate / output". */
int oracle_gemm(const oracle_gemm_t *g, const void *A, const void *B, const void *C,
                const float *bias, void *D, double *Y, double *S)
{
    if (check_desc(g))
        return -1;
    const int64_t M = g->M, N = g->N, K = g->K;
    if (M == 0 || N == 0)
        return 0;
    const int integer = is_int_type(g->a_type);

    /* Decode B once as Bt[n][k] so the inner loop walks k with unit stride. */
    double *Bt = (double *)malloc(sizeof(double) * (size_t)(N * (K ? K : 1)));
    if (!Bt)
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            Bt[n * K + k] = oracle_decode(g->b_type, B, b_index(g, k, n));

    int fail = 0;
#pragma omp parallel
    {
        double *arow = (double *)malloc(sizeof(double) * (size_t)(K ? K : 1));
        if (!arow) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t m = 0; m < M; ++m) {
            if (!arow)
                continue;
            for (int64_t k = 0; k < K; ++k)
                arow[k] = oracle_decode(g->a_type, A, a_index(g, m, k));
            for (int64_t n = 0; n < N; ++n) {
                const double *bcol = Bt + n * K;
                double acc = 0.0, sabs = 0.0;
                if (integer) {
                    int64_t iacc = 0, iabs = 0;
                    for (int64_t k = 0; k < K; ++k) {
                        int64_t p = (int64_t)arow[k] * (int64_t)bcol[k];
                        iacc += p;
                        iabs += p < 0 ? -p : p;
                    }
                    acc = (double)iacc;
                    sabs = (double)iabs;
                } else {
                    for (int64_t k = 0; k < K; ++k) {
                        double p = arow[k] * bcol[k];
                        acc += p;
                        sabs += fabs(p);
                    }
                }
                int64_t o = m * N + n;
                finish(g, m, n, acc, sabs, C, bias, D, m * g->ldd + n, Y ? Y + o : NULL,
                       S ? S + o : NULL);
            }
        }
        free(arow);
    }
    free(Bt);
    return fail ? -1 : 0;
}

int oracle_gemm_entries(const oracle_gemm_t *g, const void *A, const void *B, const void *C,
                        const float *bias, int64_t n_entries, const int64_t *rows,
                        const int64_t *cols, void *D_out, double *Y, double *S)
{
    if (check_desc(g))
        return -1;
    const int integer = is_int_type(g->a_type);
    for (int64_t i = 0; i < n_entries; ++i)
        if (rows[i] < 0 || rows[i] >= g->M || cols[i] < 0 || cols[i] >= g->N)
            return -1;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < n_entries; ++i) {
        int64_t m = rows[i], n = cols[i];
        double acc = 0.0, sabs = 0.0;
        if (integer) {
            int64_t iacc = 0, iabs = 0;
            for (int64_t k = 0; k < g->K; ++k) {
                int64_t p = (int64_t)oracle_decode(g->a_type, A, a_index(g, m, k)) *
                            (int64_t)oracle_decode(g->b_type, B, b_index(g, k, n));
                iacc += p;
                iabs += p < 0 ? -p : p;
            }
            acc = (double)iacc;
            sabs = (double)iabs;
        } else {
            for (int64_t k = 0; k < g->K; ++k) {
                double p = oracle_decode(g->a_type, A, a_index(g, m, k)) *
                           oracle_decode(g->b_type, B, b_index(g, k, n));
                acc += p;
                sabs += fabs(p);
            }
        }
        finish(g, m, n, acc, sabs, C, bias, D_out, i, Y ? Y + i : NULL, S ? S + i : NULL);
    }
    return 0;
}

/* ------------------------------------------------------------------ MX */

static int is_mx_elem(int t)
{
    return t == OR_E4M3 || t == OR_E5M2 || t == OR_E2M3 || t == OR_E3M2 || t == OR_E2M1;
}

static int check_mx_desc(const oracle_gemm_t *g)
{
    if (g->M < 0 || g->N < 0 || g->K < 0 || g->K % 32)
        return -1;
    if (!is_mx_elem(g->a_type) || !is_mx_elem(g->b_type) || g->a_col_major || !g->b_col_major)
        return -1;
    if (!float_c_ok(g->c_type))
        return -1;
    return is_float_out(g->d_type) ? 0 : -1;
}

/* One output of the block-scaled sum ("NVIDIA MMA", section "Blackwell:
 * FP4/FP6 and block-scaled MMA"): for each K block g of 32, the block's sum
 * of products, times 2^(SA-127) 2^(SB-127), added to the accumulator. */
static void mx_dot(const oracle_gemm_t *g, const void *A, const uint8_t *SA, const void *B,
                   const uint8_t *SB, int64_t m, int64_t n, double *acc_out, double *sabs_out)
{
    const int64_t KB = g->K / 32;
    double acc = 0.0, sabs = 0.0;
    for (int64_t blk = 0; blk < KB; ++blk) {
        const double sa = oracle_decode(OR_E8M0, SA, m * KB + blk);
        const double sb = oracle_decode(OR_E8M0, SB, n * KB + blk);
        double part = 0.0, pabs = 0.0;
        for (int64_t k = 32 * blk; k < 32 * blk + 32; ++k) {
            const double p = oracle_decode(g->a_type, A, m * g->lda + k) *
                             oracle_decode(g->b_type, B, n * g->ldb + k);
            part += p;
            pabs += fabs(p);
        }
        acc += sa * sb * part;
        sabs += sa * sb * pabs;
    }
    *acc_out = acc;
    *sabs_out = sabs;
}

int oracle_mx_gemm(const oracle_gemm_t *g, const void *A, const uint8_t *SA, const void *B,
                   const uint8_t *SB, const void *C, const float *bias, void *D, double *Y,
                   double *S)
{
    if (check_mx_desc(g))
        return -1;
    const int64_t M = g->M, N = g->N;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc, sabs;
            mx_dot(g, A, SA, B, SB, m, n, &acc, &sabs);
            const int64_t o = m * N + n;
            finish(g, m, n, acc, sabs, C, bias, D, m * g->ldd + n, Y ? Y + o : NULL,
                   S ? S + o : NULL);
        }
    return 0;
}

int oracle_mx_gemm_entries(const oracle_gemm_t *g, const void *A, const uint8_t *SA,
                           const void *B, const uint8_t *SB, const void *C, const float *bias,
                           int64_t n_entries, const int64_t *rows, const int64_t *cols,
                           void *D_out, double *Y, double *S)
{
    if (check_mx_desc(g))
        return -1;
    for (int64_t i = 0; i < n_entries; ++i)
        if (rows[i] < 0 || rows[i] >= g->M || cols[i] < 0 || cols[i] >= g->N)
            return -1;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < n_entries; ++i) {
        double acc, sabs;
        mx_dot(g, A, SA, B, SB, rows[i], cols[i], &acc, &sabs);
        finish(g, rows[i], cols[i], acc, sabs, C, bias, D_out, i, Y ? Y + i : NULL,
               S ? S + i : NULL);
    }
    return 0;
}

/* ------------------------------------------------------------------ W4A16 */

int oracle_w4a16_dequant(int w_type, int64_t N, int64_t K, int64_t gs, const uint8_t *Bq,
                         int64_t ldq, const void *scales, const uint8_t *zeros, void *W)
{
    if ((w_type != OR_F16 && w_type != OR_BF16) || N < 0 || K < 0 || gs <= 0 || K % gs ||
        ldq * 2 < K)
        return -1;
    const int64_t G = K / gs;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            const int q = (Bq[n * ldq + k / 2] >> (4 * (k % 2))) & 0xF;
            const int64_t g = k / gs;
            const int z = zeros ? zeros[n * G + g] : 8;
            const double sc = oracle_decode(w_type, scales, n * G + g);
            oracle_encode(w_type, (double)(q - z) * sc, W, n * K + k);
        }
    return 0;
}

int oracle_epilogue_f32(int64_t M, int64_t N, const float *T, float alpha, const float *bias,
                        int relu, int d_type, void *D)
{
    if (!is_float_out(d_type))
        return -1;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            float t = T[m * N + n];
            float y = bias ? fmaf(alpha, t, bias[n]) : alpha * t;
            if (relu)
                y = (y > 0.0f) ? y : 0.0f;
            oracle_encode(d_type, (double)y, D, m * N + n);
        }
    return 0;
}

/* ------------------------------------------------------------------ 2:4 */

/* Storage bytes of an element of a 2:4-compressible type, 0 for the others. */
static int sp_bytes(int type)
{
    switch (type) {
    case OR_F16:
    case OR_BF16: return 2;
    case OR_E4M3:
    case OR_E5M2:
    case OR_S8:
    case OR_U8: return 1;
    default: return 0;
    }
}

/* A zero of the format: +0 or -0 for the float formats (all bits but the
 * sign clear), 0 for s8 (whose 0x80 is -128, not a zero) and u8.  Every
 * other code, NaN and infinity included, is a non-zero. */
static int sp_is_zero(int type, uint32_t bits)
{
    switch (type) {
    case OR_F16:
    case OR_BF16: return (bits & 0x7FFFu) == 0;
    case OR_E4M3:
    case OR_E5M2: return (bits & 0x7Fu) == 0;
    default: return bits == 0;
    }
}

static uint32_t sp_get(const void *p, int eb, int64_t i)
{
    return eb == 2 ? ((const uint16_t *)p)[i] : ((const uint8_t *)p)[i];
}

static void sp_put(void *p, int eb, int64_t i, uint32_t v)
{
    if (eb == 2)
        ((uint16_t *)p)[i] = (uint16_t)v;
    else
        ((uint8_t *)p)[i] = (uint8_t)v;
}

/* "NVIDIA MMA", section "Dense and 2:4 structured sparse multiplication":
 * every 4 consecutive K positions of A keep 2 values and the positions they
 * came from (logical [a0,0,0,a3] -> values [a0,a3], positions [0,3]); the
 * "ordered metadata" form (section "Ampere: FP16/BF16 and integer MMA
 * baseline") lists the positions in ascending order.  The format does not
 * depend on the element type: only what counts as a zero does. */
int64_t oracle_sparse24_compress(int type, int64_t M, int64_t K, const void *A, void *values,
                                 uint32_t *meta)
{
    const int eb = sp_bytes(type);
    if (eb == 0 || M < 0 || K < 0 || (K % 4) != 0)
        return -1;
    const int64_t G = K / 4, W = (K + 31) / 32;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t w = 0; w < W; ++w)
            meta[m * W + w] = 0u;
        for (int64_t g = 0; g < G; ++g) {
            uint32_t grp[4];
            for (int i = 0; i < 4; ++i)
                grp[i] = sp_get(A, eb, m * K + 4 * g + i);
            int kept[4], nk = 0;
            for (int i = 0; i < 4; ++i)
                if (!sp_is_zero(type, grp[i]))
                    kept[nk++] = i;
            if (nk > 2)
                return m + 1;
            /* fill with the lowest positions not already kept */
            for (int i = 0; i < 4 && nk < 2; ++i) {
                int used = 0;
                for (int j = 0; j < nk; ++j)
                    used |= (kept[j] == i);
                if (!used)
                    kept[nk++] = i;
            }
            if (kept[0] > kept[1]) {
                int t = kept[0];
                kept[0] = kept[1];
                kept[1] = t;
            }
            sp_put(values, eb, m * (K / 2) + 2 * g, grp[kept[0]]);
            sp_put(values, eb, m * (K / 2) + 2 * g + 1, grp[kept[1]]);
            uint32_t nib = (uint32_t)kept[0] | ((uint32_t)kept[1] << 2);
            meta[m * W + g / 8] |= nib << (4 * (g % 8));
        }
    }
    return 0;
}

int oracle_sparse24_decompress(int type, int64_t M, int64_t K, const void *values,
                               const uint32_t *meta, void *A)
{
    const int eb = sp_bytes(type);
    if (eb == 0 || M < 0 || K < 0 || (K % 4) != 0)
        return -1;
    const int64_t G = K / 4, W = (K + 31) / 32;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t k = 0; k < K; ++k)
            sp_put(A, eb, m * K + k, 0u);
        for (int64_t g = 0; g < G; ++g) {
            uint32_t nib = (meta[m * W + g / 8] >> (4 * (g % 8))) & 0xFu;
            int i0 = (int)(nib & 3u), i1 = (int)(nib >> 2);
            if (i0 >= i1)
                return -1;
            sp_put(A, eb, m * K + 4 * g + i0, sp_get(values, eb, m * (K / 2) + 2 * g));
            sp_put(A, eb, m * K + 4 * g + i1, sp_get(values, eb, m * (K / 2) + 2 * g + 1));
        }
    }
    return 0;
}

int oracle_num_threads(void) { return omp_get_max_threads(); }
