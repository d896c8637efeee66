/*
 * gemm.h - C ABI of the MI355X (gfx950) tiled multiply-accumulate library
 * libstgemm.so:
 *
 *     D = cast( act( alpha * (A*B + C) + bias[n] ) )
 *
 * with low-precision A/B (fp16, bf16, fp8 E4M3/E5M2, s8), an fp32 or int32
 * accumulator along K, and a 2:4 structured-sparse-A variant.
 *
 * Definitions this interface follows (three public pages on tensor-core MMA):
 *  - "NVIDIA MMA" (rainlin-net), section "From FMA to MMA to GEMM":
 *    D[m,n] = sum_k A[m,k] B[k,n] + C[m,n] with A M x K, B K x N, C/D M x N;
 *    a GEMM is many tile MMAs plus data movement, a K loop and an epilogue.
 *  - same page, section "Input / accumulate / output": input types, the
 *    accumulator type and the output type are separate choices; the epilogue
 *    applies scale, bias, activation and cast, in that order.
 *  - same page, section "Dense and 2:4 structured sparse multiplication":
 *    only A is compressed (2 kept values of every 4 K positions plus their
 *    positions); B, C and D stay dense.
 *  - "CUDA 014 - MMA instruction usage" (blog-9y3), section "MMA instruction
 *    format": A row-major and B column-major is the natural operand pairing
 *    (both contiguous along K); the fast kernels here use that pairing.
 *
 * Conventions
 *  - Sizes and leading dimensions are in elements.  M, N and K must be below
 *    2^31 and every matrix (rows times leading dimension) at most 2^40
 *    elements (GEMM_ERR_INVALID_VALUE otherwise).  A is M x K, row-major
 *    (A[m*lda + k]) or column-major (A[k*lda + m]).  B is K x N, column-major
 *    (stored N x K, B[n*ldb + k]) or row-major (B[k*ldb + n]).  C and D are
 *    M x N row-major (C[m*ldc + n]).  A leading dimension of 0 means packed.
 *  - All data pointers are device pointers (HIP device memory).  The caller
 *    owns every buffer; the library never allocates device memory in
 *    gemm_run / gemm_sparse24_run and needs no workspace.
 *  - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *    Launches are asynchronous: a kernel fault surfaces at the caller's next
 *    synchronisation.  gemm_sparse24_compress alone synchronises its stream.
 *  - Every function returns a status; no exception or abort crosses the ABI.
 *    gemm_last_error() gives a thread-local message about the last failure.
 *  - A plan is immutable after gemm_plan returns: it may be shared by threads
 *    and used on any stream of the device it was made on.
 *  - The kernel a plan selects depends on M, N, K, the input types, layouts
 *    and leading dimensions (and, at run time, pointer alignment) - never on
 *    the epilogue or output type.  Two plans that differ only in epilogue or
 *    d_type therefore sum in the same order.
 */
#ifndef STGEMM_GEMM_H
#define STGEMM_GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GEMM_OK = 0,
    GEMM_ERR_NULL_POINTER = 1,  /* a required pointer argument is NULL */
    GEMM_ERR_INVALID_VALUE = 2, /* negative size, bad enum, ld too small, ... */
    GEMM_ERR_UNSUPPORTED = 3,   /* valid request outside the support matrix */
    GEMM_ERR_MISALIGNED = 4,    /* pointer alignment a call requires is not met */
    GEMM_ERR_NOT_SPARSE24 = 5,  /* a group of 4 holds more than 2 non-zeros */
    GEMM_ERR_DEVICE = 6,        /* current device is not gfx950 */
    GEMM_ERR_HIP = 7            /* a HIP runtime call failed */
} gemm_status_t;

typedef enum {
    GEMM_F16 = 1,     /* IEEE binary16 */
    GEMM_BF16 = 2,    /* bfloat16 */
    GEMM_F8_E4M3 = 3, /* OCP FP8 E4M3 (max 448, no infinity) */
    GEMM_F8_E5M2 = 4, /* OCP FP8 E5M2 (max 57344) */
    GEMM_S8 = 5,      /* int8, two's complement */
    GEMM_F32 = 6,     /* IEEE binary32 */
    GEMM_S32 = 7,     /* int32, two's complement */
    /* OCP MX element formats, block-scaled GEMM only (block_scale = 32),
     * stored packed along K: */
    GEMM_F6_E2M3 = 8, /* bias 1, max 7.5, no inf/NaN; 4 elements in 3 bytes */
    GEMM_F6_E3M2 = 9, /* bias 3, max 28, no inf/NaN; 4 elements in 3 bytes */
    GEMM_F4_E2M1 = 10, /* bias 1, max 6, no inf/NaN; 2 elements per byte */
    GEMM_U4 = 11,      /* W4A16 weight codes 0..15, two per byte along K (the
                          even element in the low nibble); B only */
    GEMM_U8 = 12       /* uint8 0..255: A and / or B of an integer GEMM, paired
                          with S8 or U8 */
} gemm_dtype_t;

typedef enum { GEMM_ROW_MAJOR = 0, GEMM_COL_MAJOR = 1 } gemm_layout_t;

typedef enum { GEMM_ACT_NONE = 0, GEMM_ACT_RELU = 1 } gemm_act_t;

/* Kernel family request.  GEMM_ALGO_AUTO lets the plan choose; any other
 * value forces that family and gemm_plan returns GEMM_ERR_UNSUPPORTED when it
 * cannot serve the descriptor (used by tests and tuning sweeps). */
typedef enum {
    GEMM_ALGO_AUTO = 0,
    GEMM_ALGO_TILED = 1,   /* LDS-staged, double-buffered MFMA kernel: K-contiguous
                              operands (A row-major, B column-major), or A column-major
                              and / or B row-major with M (resp. N) in whole 16-byte
                              chunks, fetched from LDS with transposing reads; any dense
                              type; K * element size a multiple of 64 and 16-byte rows
                              in every case */
    GEMM_ALGO_GENERIC = 2, /* any layout / shape / alignment, MFMA, no LDS */
    GEMM_ALGO_SKINNY = 3,  /* small M, bandwidth-oriented */
    GEMM_ALGO_TILED_128 = 4, /* GEMM_ALGO_TILED with 128 x 128 workgroup tiles */
    GEMM_ALGO_TILED_256 = 5  /* GEMM_ALGO_TILED with 256 x 256 workgroup tiles */
} gemm_algo_t;

/* Problem descriptor.
 *
 * Support matrix (everything else is GEMM_ERR_UNSUPPORTED):
 *   a, b in {F16}, {BF16}, or {F8_E4M3, F8_E5M2} (the two fp8 formats may
 *   differ): c_type F32, F16 or BF16 (a 16-bit C is widened exactly to fp32
 *   before the addition), d_type F32 / F16 / BF16 / F8_E4M3 /
 *   F8_E5M2, any epilogue.
 *   a, b in {S8, U8} (any pairing: the INT8 rows of the instruction tables
 *   on "NVIDIA MMA", section "Ampere: FP16/BF16 and integer MMA baseline",
 *   take signed or unsigned A and B): either c_type S32, d_type S32,
 *   alpha == 1, no bias, no activation; or (dequantising epilogue) c_type
 *   F32 / F16 / BF16, d_type F32 / F16 / BF16 / F8_E4M3 / F8_E5M2, any
 *   epilogue, where the int32 sum is first rounded to fp32 (to nearest
 *   even).  The int32 sum wraps modulo 2^32 in both.  With saturate = 1
 *   (int32 output only, and K small enough that the sum of products cannot
 *   leave the int32 range: K * max|a| * max|b| < 2^31, i.e. K < 131072 for
 *   s8 x s8, 65794 for u8 x s8 or s8 x u8, 33026 for u8 x u8) D = clamp(acc +
 *   C) to [-2^31, 2^31 - 1] instead (same section: integer MMA saturates with
 *   .satfinite, else wraps).  The fast kernels take U8 with A row-major and
 *   B column-major; other layouts of a U8 operand run the generic kernel.
 *   sparse_a = 1: any of the pairs above, A row-major and packed,
 *   K % 4 == 0; used with gemm_sparse24_run (A is then given in compressed
 *   form).  A U8 A of a 2:4 product runs the generic kernel.
 *   block_scale = 32 (MX): a, b any of F8_E4M3, F8_E5M2, F6_E2M3, F6_E3M2,
 *   F4_E2M1 (they may differ), A row-major, B column-major, K % 32 == 0,
 *   rows of whole bytes (lda, ldb in elements); c_type F32, any float
 *   d_type, any epilogue; used with gemm_mx_run.  The 6- and 4-bit
 *   formats exist only here.
 *   b = U4 (W4A16): a F16 or BF16, A row-major, B column-major (codes along
 *   K, ldb even), block_scale = the weight group size (a multiple of 32
 *   dividing K); c_type F32 / F16 / BF16, any float d_type, any epilogue;
 *   used with gemm_w4a16_run.
 * Epilogue, in fp32 for float outputs:  t = acc (+ C[m,n] if has_c);
 *   y = has_bias ? fmaf(alpha, t, bias[n]) : alpha * t;
 *   z = (act == RELU) ? (y > 0 ? y : +0) : y;  D = round-to-nearest-even(z).
 * FP8 outputs saturate: a finite z beyond the largest finite value (448 for
 * E4M3, 57344 for E5M2), and an infinity, become that value with z's sign;
 * a NaN becomes the canonical NaN byte 0x7F.
 * Accuracy with fp8 (and MX) inputs: gfx950's fp8 matrix instructions add
 * each group of 8 consecutive K products (K 8q .. 8q+7) with every product
 * truncated toward zero to a multiple of 2^(E - 13), E the exponent of the
 * group's largest product; group sums then accumulate in fp32.  An output
 * is therefore within sum_q 7 * 2^(E_q - 13) (plus fp32 rounding) of the
 * exact sum: at most about 8.5e-4 of sum_k |A B| when one product dominates
 * each group, well below 1e-4 of it for inputs without such dominance
 * (for example normal data scaled per tensor, or every code equally
 * likely).  16-bit and int8 inputs have no such truncation.
 * bias is fp32, N values, one per output column. */
typedef struct {
    int64_t M, N, K;
    int32_t a_type, b_type, c_type, d_type; /* gemm_dtype_t */
    int32_t a_layout, b_layout;             /* gemm_layout_t */
    int64_t lda, ldb, ldc, ldd;             /* 0 = packed */
    float alpha;                            /* 1.0f = no scaling */
    int32_t has_c;                          /* read C (else t = acc) */
    int32_t has_bias;
    int32_t act;                            /* gemm_act_t */
    int32_t sparse_a;                       /* 1: 2:4-compressed A */
    int32_t algo;                           /* gemm_algo_t, normally AUTO */
    int32_t block_scale;                    /* 0; 32: MX block-scaled (gemm_mx_run);
                                               W4A16: the weight group size */
    int32_t saturate;                       /* int32 output: 1 clamps acc + C to the
                                               int32 range, 0 wraps modulo 2^32 */
} gemm_desc_t;

typedef struct gemm_plan gemm_plan_t;
typedef void *gemm_stream_t; /* hipStream_t */

/* Validate a descriptor without touching any device (pure host function).
 * Returns GEMM_OK, GEMM_ERR_NULL_POINTER, GEMM_ERR_INVALID_VALUE or
 * GEMM_ERR_UNSUPPORTED. */
gemm_status_t gemm_validate_desc(const gemm_desc_t *desc);

/* Validate, check that the current HIP device is gfx950, select the kernel
 * and return a new plan in *out (host memory, owned by the caller, released
 * with gemm_plan_destroy).  On failure *out is set to NULL.  With GEMM_LOG=1
 * in the environment each successful call prints its kernel choice to
 * stderr. */
gemm_status_t gemm_plan(const gemm_desc_t *desc, gemm_plan_t **out);

/* Release a plan (NULL is accepted). */
gemm_status_t gemm_plan_destroy(gemm_plan_t *plan);

/* Write the selected kernel's name (NUL-terminated, truncated to len) into
 * buf.  For logs and tests. */
gemm_status_t gemm_plan_describe(const gemm_plan_t *plan, char *buf, size_t len);

/* Enqueue D = epilogue(A*B + C) on `stream` (dense A).  C may be NULL only
 * when the plan has has_c == 0; bias may be NULL only when has_bias == 0.
 * Returns after the launch is enqueued.  Pointers need only element
 * alignment: the fast kernels need 16-byte aligned A and B and fall back to
 * the generic kernel otherwise.  D must not share bytes with A, B, C or
 * bias, with one exception: D == C (in-place accumulate) when C and D have
 * the same element size and ldc == ldd.  Any other overlap is rejected with
 * GEMM_ERR_UNSUPPORTED before anything is launched (the same rule holds for
 * every run function below, with its own operands). */
gemm_status_t gemm_run(const gemm_plan_t *plan, const void *A, const void *B, const void *C,
                       const void *bias, void *D, gemm_stream_t stream);

/* Bytes of the compressed form of an M x K A of type a_type (f16, bf16,
 * fp8 E4M3/E5M2, s8 or u8; K % 4 == 0): values are M x K/2 elements of a_type;
 * metadata is M x ceil(K/32) uint32 whatever the type.  The sparse rows of
 * the instruction tables on "NVIDIA MMA" (sections "Ampere: FP16/BF16 and
 * integer MMA baseline" and "Ada: mma.sync adds FP8") give these types a
 * 2:4 form. */
gemm_status_t gemm_sparse24_sizes(int64_t M, int64_t K, int32_t a_type, size_t *values_bytes,
                                  size_t *meta_bytes);

/* Compress a dense row-major M x K A of type a_type (device) into the 2:4
 * form:
 *   group g of row m covers K positions 4g .. 4g+3; its kept positions
 *   i0 < i1 (the non-zeros, filled up with the lowest free positions when a
 *   group has fewer than two) give
 *     values[m*(K/2) + 2g] = A[m, 4g+i0],  values[m*(K/2) + 2g+1] = A[m, 4g+i1]
 *   and the nibble (i0 | i1 << 2) at bits 4(g%8)..4(g%8)+3 of
 *   meta[m*ceil(K/32) + g/8]; unused high nibbles are 0.
 * The zeros are +0 and -0 of the float types and 0 of s8 (whose 0x80 is
 * -128) and of u8; NaN and infinity count as non-zero.  Positions ascend, as the
 * ordered-metadata form on "NVIDIA MMA" (section "Ampere: FP16/BF16 and
 * integer MMA baseline") requires; the bit packing is this library's own.
 * Synchronises `stream` (a one-time weight preprocessing step) and returns
 * GEMM_ERR_NOT_SPARSE24 when some group holds more than two non-zeros
 * (values/meta are then unspecified).  A must be aligned to 4 elements,
 * values to 2 elements and meta to 4 bytes (GEMM_ERR_MISALIGNED). */
gemm_status_t gemm_sparse24_compress(int64_t M, int64_t K, int32_t a_type, const void *A,
                                     void *values, uint32_t *meta, gemm_stream_t stream);

/* gemm_sparse24_compress for callers that cannot allocate device memory
 * (code that must not call hipMalloc: tight serving loops, harnesses that
 * forbid allocation).  Same arguments, output, synchronisation and status
 * codes as gemm_sparse24_compress, and the same sizes are accepted (the
 * scratch it needs does not grow with M or K), but it allocates nothing:
 * the error flag gemm_sparse24_compress allocates per call lives instead in
 * a static device array of 64 ints (256 bytes) that each GPU the library
 * runs on holds until the process ends.  The flag is cleared by a kernel on
 * `stream` at the start of every call.  All calls on one GPU share that
 * array: calls that overlap on one GPU (from several host threads or
 * streams) race on the flag and may report each other's NOT_SPARSE24. */
gemm_status_t gemm_sparse24_compress_noalloc(int64_t M, int64_t K, int32_t a_type, const void *A,
                                             void *values, uint32_t *meta, gemm_stream_t stream);

/* Enqueue D = epilogue(A*B + C) with A given as (values, meta) from
 * gemm_sparse24_compress.  The plan must have sparse_a == 1; its A/B types,
 * accumulator and epilogue follow the dense rules (f16 x f16, bf16 x bf16,
 * any fp8 pair -> fp32 accumulation; s8 x s8 -> s32).  The SMFMAC kernels
 * need B column-major with 16-byte rows, K a multiple of 64 (16-bit types)
 * or 128 (8-bit types), and 16-byte aligned values, meta and B; otherwise
 * (also when only the alignment is missing at run time) the generic kernel
 * runs. */
gemm_status_t gemm_sparse24_run(const gemm_plan_t *plan, const void *values, const uint32_t *meta,
                                const void *B, const void *C, const void *bias, void *D,
                                gemm_stream_t stream);

/* Enqueue the MX block-scaled product ("NVIDIA MMA", section "Blackwell:
 * FP4/FP6 and block-scaled MMA"; UE8M0 scales per 32 K from the table in
 * "MXFP4 and NVFP4"):
 *     acc[m,n] = sum_g 2^(sa[m,g]-127) 2^(sb[n,g]-127) sum_{k in block g} A[m,k] B[k,n]
 * over K blocks g = k / 32, each block's partial sum scaled before it joins
 * the fp32 accumulation, then D = epilogue(acc + C) as for gemm_run.  The
 * plan must have block_scale == 32.
 *   A: row m at byte m*lda*bits/8, K elements packed from bit 0 up (8-bit:
 *      one per byte; E2M1: two per byte, the even element in the low
 *      nibble; 6-bit: element k in bits 6k .. 6k+5 of the row read as a
 *      little-endian bit string).
 *   B: stored N x K (column-major K x N), column n packed the same way.
 *   scale_a: M x K/32 E8M0 bytes (row-major), 2^(e-127); scale_b: N x K/32.
 *   A scale of 0xFF (NaN) gives an unspecified result.
 * Device pointers; the fast kernel (pairs of one width: both 8-bit or both
 * E2M1, K % 512 == 0, rows of whole 16 bytes) needs A, B and the scales
 * 16-byte aligned, else the generic kernel runs.  With a 6-bit operand
 * (partner 6- or 8-bit, K % 512 == 0, 6-bit rows of whole 4 bytes, 8-bit
 * rows of whole 16) the fast path first rewrites each 6-bit operand into a
 * temporary of M*K (A) or N*K (B) bytes, taken on `stream` from a memory
 * pool the library keeps per device (its blocks stay reserved for later
 * calls until the process ends) and released on `stream` after the
 * product; it needs 6-bit operands 4-byte aligned, 8-bit ones and the
 * scales 16-byte aligned, else the generic kernel runs.  A failure to get
 * the temporary is returned as GEMM_ERR_HIP. */
gemm_status_t gemm_mx_run(const gemm_plan_t *plan, const void *A, const uint8_t *scale_a,
                          const void *B, const uint8_t *scale_b, const void *C, const void *bias,
                          void *D, gemm_stream_t stream);

/* Enqueue the W4A16 weight-only product ("NVIDIA MMA", section "How
 * quantisation configurations map to MMA": INT4 weights, FP16 / BF16
 * activations, run as an FP16 / BF16 MMA on weight tiles dequantised in the
 * main loop).  The plan must have b_type == GEMM_U4.
 *   B: N x K codes q (column n at byte n*ldb/2, two codes per byte along K);
 *   scales: N x K/gs values of A's type (gs = the plan's block_scale);
 *   zeros: N x K/gs bytes z in 0..15, or NULL for z = 8 everywhere;
 *   w[k,n] = RNE((q - z[n,k/gs]) * scales[n,k/gs]) in A's type, then
 *   D = epilogue(A*w + C) with fp32 accumulation, as for gemm_run.
 * A and scales must be 2-byte aligned (GEMM_ERR_MISALIGNED); the fast kernel
 * (16-byte rows of A and of codes) needs A and B 16-byte aligned, else the
 * generic kernel runs. */
gemm_status_t gemm_w4a16_run(const gemm_plan_t *plan, const void *A, const void *B,
                             const void *scales, const uint8_t *zeros, const void *C,
                             const void *bias, void *D, gemm_stream_t stream);

/* Static text for a status code. */
const char *gemm_status_string(gemm_status_t status);

/* Thread-local detail about the most recent failure on this thread ("" if
 * none).  Valid until the thread's next call into the library. */
const char *gemm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif
