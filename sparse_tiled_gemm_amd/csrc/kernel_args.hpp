// Argument blocks passed by value to the GEMM kernels (host and device).
#pragma once

#include <stdint.h>

namespace stg {

enum OutKind { OUT_F32 = 0, OUT_F16 = 1, OUT_BF16 = 2, OUT_S32 = 3, OUT_E4M3 = 4, OUT_E5M2 = 5 };

// Epilogue inputs.  C == nullptr: no C term; bias == nullptr: no bias.
struct EpiArgs {
    int64_t M, N;
    const void *C;
    int64_t ldc;
    const float *bias;
    float alpha;
    int relu;
    int d_kind; // OutKind
    void *D;
    int64_t ldd;
    int vec; // 1: C, bias and D rows allow 16-byte (C, f32/s32 D) / 8-byte accesses
             //    at multiples of 4 columns
    int sat; // int32 output: acc + C saturates to the int32 range (else wraps)
    int c_kind; // float outputs: C elements are 0 fp32, 1 fp16, 2 bf16
};

// Dense operands.  Element (m,k) of A is at A[m*a_rs + k*a_cs] and element
// (k,n) of B at B[k*b_rs + n*b_cs] (strides in elements).  The K-contiguous
// kernels use only lda = a_rs and ldb = b_cs.
struct GemmArgs {
    const void *A;
    const void *B;
    int64_t K;
    int64_t a_rs, a_cs;
    int64_t b_rs, b_cs;
    EpiArgs e;
    // MX block scales (E8M0, one per 32 K): sa[m*(K/32) + g] for row m of A,
    // sb[n*(K/32) + g] for column n of B; nullptr outside the MX path
    const uint8_t *sa, *sb;
    // W4A16 weights (B holds unsigned 4-bit codes, two per byte along K,
    // b_cs in codes): group g = k / wgs of column n has scale ws[n*(K/wgs) + g]
    // (A's 16-bit type) and zero point wz[n*(K/wgs) + g] (8 when wz is null)
    const void *ws;
    const uint8_t *wz;
    int64_t wgs;
};

// 2:4-compressed A: values [M, K/2] fp16, meta [M, ceil(K/32)] u32.
struct SparseArgs {
    const void *values; // kept A values (elements of A's type)
    const uint32_t *meta;
    const void *B; // element (k,n) at B[k*b_rs + n*b_cs]
    int64_t K;
    int64_t b_rs, b_cs;
    EpiArgs e;
};

} // namespace stg
