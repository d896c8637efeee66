/*
 * CPU oracle for the tiled multiply-accumulate D = A*B + C and its epilogue.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls
 * this code: only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no source, header, table or helper with the HIP
 * library; the two agree only through the bytes of the seeded inputs.
 *
 * What it computes, and where that is defined:
 *   - "NVIDIA MMA" (rainlin-net), section "From FMA to MMA to GEMM": the GEMM
 *     element D[m,n] = sum_k A[m,k] B[k,n] + C[m,n].  Written out literally,
 *     k ascending, in fp64 (float inputs) or int64 (s8 inputs).  Every product
 *     of two fp16/bf16/fp8 values is exact in fp64, so the only rounding is the
 *     fp64 running sum.
 *   - same page, section "Input / accumulate / output": the accumulator is
 *     followed by an epilogue "scale, bias, activation, cast".  Here:
 *     y = alpha*(acc + C) + bias[n] in fp64, z = relu(y) when asked, then one
 *     round-to-nearest-even cast to the output type.
 *   - same page, section "Ampere: FP16/BF16 and integer MMA baseline": integer
 *     results that do not fit wrap modulo 2^32 (no saturation requested).
 *     s8 inputs may also produce a float output (the int8 -> float dequant
 *     epilogue): the wrapped int32 sum, then the float epilogue with an fp32
 *     C.  FP8 outputs (E4M3 / E5M2) round to nearest even and saturate at
 *     the largest finite value (NaN -> 0x7F).
 *   - same page, section "Dense and 2:4 structured sparse multiplication": the
 *     2:4 format keeps 2 of every 4 consecutive K positions of A, with their
 *     positions as metadata; ascending positions per the "ordered metadata"
 *     remark in the Ampere section.  Metadata bit packing is not on the pages;
 *     the packing used here is stated at oracle_sparse24_compress.  The
 *     sparse rows of the instruction tables in the sections "Ampere:
 *     FP16/BF16 and integer MMA baseline" (FP16, BF16, INT8) and "Ada:
 *     mma.sync adds FP8" (E4M3/E5M2, A and B formats may differ) give the
 *     element types the format applies to; the format itself is the same
 *     for all of them.
 *   - bit formats: IEEE binary16; bfloat16 = the upper 16 bits of binary32;
 *     OCP FP8 E4M3 (bias 7, no infinity, 0x7F/0xFF NaN, max 448) and E5M2
 *     (bias 15, IEEE-like infinities, max 57344), the bare FP8 formats named
 *     in the precision tables of "NVIDIA MMA"; for the block-scaled path the
 *     OCP MX element formats E2M3 (bias 1, max 7.5), E3M2 (bias 3, max 28)
 *     and E2M1 (bias 1, max 6), all without infinity or NaN, and the UE8M0
 *     scale (2^(e-127), 0xFF NaN) - the formats the pages name, defined by
 *     the OCP Microscaling specification.
 */
#ifndef ORACLE_H
#define ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types known to the oracle (its own numbering). */
enum {
    OR_F16 = 0,
    OR_BF16 = 1,
    OR_E4M3 = 2,
    OR_E5M2 = 3,
    OR_S8 = 4,
    OR_F32 = 5,
    OR_S32 = 6,
    /* the narrow formats of the MX block-scaled path; stored packed along a
     * row: E2M1 two to a byte (element i in bits 4(i%2) .. of byte i/2, the
     * even element in the low nibble), E2M3 / E3M2 as a little-endian bit
     * string (element i in bits 6i .. 6i+5, four elements in three bytes) */
    OR_E2M3 = 7,
    OR_E3M2 = 8,
    OR_E2M1 = 9,
    OR_E8M0 = 10, /* block scale: 2^(e - 127), 0xFF = NaN; one byte each */
    /* unsigned 8-bit integer 0..255: the INT8 rows of the instruction tables
     * ("NVIDIA MMA", section "Ampere: FP16/BF16 and integer MMA baseline")
     * let A and B each be signed or unsigned; any pairing of OR_S8 and OR_U8
     * accumulates in int32 like s8 x s8 */
    OR_U8 = 11
};

typedef struct {
    int64_t M, N, K;
    int a_type, b_type, c_type, d_type;
    int a_col_major; /* 0: A[m*lda + k]   1: A[k*lda + m] */
    int b_col_major; /* 1: B[n*ldb + k]   0: B[k*ldb + n] */
    int64_t lda, ldb, ldc, ldd; /* leading dimensions in elements; C, D row-major */
    float alpha;   /* widened to fp64 before use */
    int has_c;
    int has_bias;  /* bias is fp32, one value per output column n */
    int relu;
    int saturate;  /* int32 output: clamp acc + C to the int32 range (else wrap) */
} oracle_gemm_t;

/* Decode element idx of an array of the given type to fp64 (s8/s32 exact). */
double oracle_decode(int type, const void *base, int64_t idx);

/* Round x to the given float type with round-to-nearest-even (overflow goes
 * to +-inf, NaN stays NaN) and store its bit pattern at base[idx].  For OR_S32
 * x must be an integer and is reduced modulo 2^32. Returns 0, or -1 for an
 * unsupported type. */
int oracle_encode(int type, double x, void *base, int64_t idx);

/* Element-wise loops over oracle_decode / oracle_encode. */
void oracle_decode_array(int type, const void *base, int64_t n, double *out);
int oracle_encode_array(int type, const double *x, int64_t n, void *base);

/* Full GEMM + epilogue.  D receives the encoded result.  Optional outputs
 * (NULL to skip), each M*N fp64 values row-major:
 *   Y - the exact-as-possible fp64 result before the final cast
 *       (integers: the wrapped int32 value);
 *   S - sum_k |A[m,k] B[k,n]| + |C[m,n]|, the scale of the rounding error.
 * Returns 0, or -1 on an unsupported combination. */
int oracle_gemm(const oracle_gemm_t *g, const void *A, const void *B, const void *C,
                const float *bias, void *D, double *Y, double *S);

/* The same definition evaluated at n chosen (rows[i], cols[i]) entries only;
 * D_out receives n encoded elements, Y and S n values each (nullable). */
int oracle_gemm_entries(const oracle_gemm_t *g, const void *A, const void *B, const void *C,
                        const float *bias, int64_t n, const int64_t *rows, const int64_t *cols,
                        void *D_out, double *Y, double *S);

/* fp32 epilogue applied to a given fp32 tile T (= acc + C as a kernel holds
 * it), in fp32 arithmetic: y = has_bias ? fmaf(alpha, t, bias[n]) : alpha*t,
 * z = relu ? (y > 0 ? y : +0) : y, then an RNE cast of z to d_type.
 * Used to pin a fused epilogue bit for bit. */
int oracle_epilogue_f32(int64_t M, int64_t N, const float *T, float alpha, const float *bias,
                        int relu, int d_type, void *D);

/* 2:4 compression of a row-major [M,K] matrix of type `type` (OR_F16,
 * OR_BF16, OR_E4M3, OR_E5M2, OR_S8 or OR_U8; elements of 2 or 1 bytes),
 * K % 4 == 0.
 * Group g of row m is K positions 4g..4g+3.  Its kept positions i0 < i1 give
 *   values[m*(K/2) + 2g]   = A[m, 4g+i0]
 *   values[m*(K/2) + 2g+1] = A[m, 4g+i1]   (elements of the same type)
 *   nibble (i0 | i1 << 2) at bits 4*(g%8) .. 4*(g%8)+3 of meta[m*W + g/8],
 * with W = ceil(K/32) words per row and unused high nibbles 0.
 * The dropped positions are zeros: +0 and -0 of the float formats, 0 of s8
 * (0x80 is -128 there) and of u8.  A group with fewer than two non-zeros keeps its
 * non-zero positions and fills up with the lowest unused positions; NaN and
 * infinity count as non-zero.
 * Returns 0, -1 for a bad type or shape, or the 1-based row index of the
 * first row holding a group with more than two non-zeros (then the outputs
 * are unspecified). */
int64_t oracle_sparse24_compress(int type, int64_t M, int64_t K, const void *A, void *values,
                                 uint32_t *meta);

/* Inverse: logical [M,K] of `type` with all-zero bits at the dropped
 * positions.  Returns 0, or -1 for a bad type or shape or if some nibble is
 * not ascending (i0 >= i1). */
int oracle_sparse24_decompress(int type, int64_t M, int64_t K, const void *values,
                               const uint32_t *meta, void *A);

/* MX block-scaled GEMM ("NVIDIA MMA", section "Blackwell: FP4/FP6 and
 * block-scaled MMA": D = C + sum_g (A_g S_A,g)(B_g S_B,g), every scale applied
 * to its K block's partial sum before that sum joins the accumulation; the
 * "MXFP4 and NVFP4" table: UE8M0 scales, one per 32 K elements).  a_type and
 * b_type are any of OR_E4M3, OR_E5M2, OR_E2M3, OR_E3M2, OR_E2M1 (they may
 * differ); A row-major (element (m,k) at index m*lda + k of its packed
 * storage), B column-major (element (k,n) at n*ldb + k); K % 32 == 0.
 * SA[m*(K/32) + g] scales A's row m over K block g (K 32g .. 32g+31),
 * SB[n*(K/32) + g] B's column n.  Block sums in fp64 (exact products),
 * scaled by the exact powers of two, summed in block order; then C and the
 * epilogue as in oracle_gemm.  Y/S as there, S = sum over k of the scaled
 * |a b| plus |c|.  Returns 0, or -1 for an unsupported description. */
int oracle_mx_gemm(const oracle_gemm_t *g, const void *A, const uint8_t *SA, const void *B,
                   const uint8_t *SB, const void *C, const float *bias, void *D, double *Y,
                   double *S);

/* The same definition at chosen entries (rows[i], cols[i]) only. */
int oracle_mx_gemm_entries(const oracle_gemm_t *g, const void *A, const uint8_t *SA,
                           const void *B, const uint8_t *SB, const void *C, const float *bias,
                           int64_t n_entries, const int64_t *rows, const int64_t *cols,
                           void *D_out, double *Y, double *S);

/* W4A16 weight dequantisation ("NVIDIA MMA", section "How quantisation
 * configurations map to MMA": W4A16 INT4 weight-only runs an FP16 x FP16 or
 * BF16 x BF16 MMA on a weight tile dequantised first; section "Ampere:
 * FP16/BF16 and integer MMA baseline": a W4A16 kernel converts the weight
 * tile to FP16/BF16 before the float MMA).  Bq is the N x K weight matrix
 * (B stored column-major, one row per output column n) of unsigned 4-bit
 * codes, two per byte along K (element k of row n in bits 4(k%2) .. of byte
 * n*ldq + k/2, ldq in bytes); group g of row n is K positions gs*g ..
 * gs*g+gs-1 (K % gs == 0).  Output W (N x K, type w_type = OR_F16 or
 * OR_BF16): W[n,k] = RNE_w_type((q - z[n,g]) * s[n,g]), s = scales[n*(K/gs)
 * + g] of type w_type, z = zeros[n*(K/gs) + g] (0..15), or 8 for every group
 * when zeros is NULL.  The product is exact in fp64 (and in fp32), so the
 * one rounding is the cast.  Returns 0 or -1 for a bad argument. */
int oracle_w4a16_dequant(int w_type, int64_t N, int64_t K, int64_t gs, const uint8_t *Bq,
                         int64_t ldq, const void *scales, const uint8_t *zeros, void *W);

/* Threads the OpenMP loops use. */
int oracle_num_threads(void);

#ifdef __cplusplus
}
#endif

#endif
