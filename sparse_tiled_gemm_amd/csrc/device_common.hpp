// Device-side building blocks shared by the gfx950 GEMM kernels: operand
// vector types, one traits struct per MFMA form, and the fused epilogue.
//
// MFMA operand layout used throughout (32x32 forms, wave64):
//   A operand: lane l holds LANE_BYTES contiguous K bytes of row (l % 32),
//              starting at K byte (l / 32) * LANE_BYTES of the instruction's
//              K slice;  B operand: the same for column (l % 32).
//   Accumulator: lane l, register i holds row 8*(i/4) + 4*(l/32) + (i%4),
//              column l % 32.
// A and B are always loaded with the same per-lane K assignment, so any
// order in which the hardware pairs K positions inside one instruction
// leaves the dot products unchanged.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kernel_args.hpp"

namespace stg {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef float f16_t __attribute__((ext_vector_type(16)));
typedef int i4_t __attribute__((ext_vector_type(4)));
typedef int i8_t __attribute__((ext_vector_type(8)));
typedef int i16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- MFMA ops
// Each op: ELEM (bytes per element), LANE_BYTES (operand bytes per lane),
// KB (K bytes one 32x32 instruction consumes = 2 * LANE_BYTES), acc_t, and
// mma(a, b, acc) on LANE_BYTES/4 packed 32-bit words per operand.

struct OpF16 {
    static constexpr int ELEM = 2, LANE_BYTES = 16, KB = 32;
    static constexpr bool INT = false;
    typedef f16_t acc_t;
    __device__ static inline acc_t mma(const uint32_t *a, const uint32_t *b, acc_t c)
    {
        h8_t va = __builtin_bit_cast(h8_t, *(const u4_t *)a);
        h8_t vb = __builtin_bit_cast(h8_t, *(const u4_t *)b);
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(va, vb, c, 0, 0, 0);
    }
};

struct OpBF16 {
    static constexpr int ELEM = 2, LANE_BYTES = 16, KB = 32;
    static constexpr bool INT = false;
    typedef f16_t acc_t;
    __device__ static inline acc_t mma(const uint32_t *a, const uint32_t *b, acc_t c)
    {
        bf8_t va = __builtin_bit_cast(bf8_t, *(const u4_t *)a);
        bf8_t vb = __builtin_bit_cast(bf8_t, *(const u4_t *)b);
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, vb, c, 0, 0, 0);
    }
};

// fp8 through the gfx950 f8f6f4 form; the format selectors are 0 = E4M3 and
// 1 = E5M2, and both block scales are E8M0 127 (= 2^0), i.e. no scaling.
template <int AFMT, int BFMT>
struct OpF8 {
    static constexpr int ELEM = 1, LANE_BYTES = 32, KB = 64;
    static constexpr bool INT = false;
    typedef f16_t acc_t;
    __device__ static inline acc_t mma(const uint32_t *a, const uint32_t *b, acc_t c)
    {
        i8_t va = *(const i8_t *)a;
        i8_t vb = *(const i8_t *)b;
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, vb, c, AFMT, BFMT, 0, 127, 0,
                                                               127);
    }
};

struct OpS8 {
    static constexpr int ELEM = 1, LANE_BYTES = 16, KB = 32;
    static constexpr bool INT = true;
    typedef i16_t acc_t;
    __device__ static inline acc_t mma(const uint32_t *a, const uint32_t *b, acc_t c)
    {
        i4_t va = *(const i4_t *)a;
        i4_t vb = *(const i4_t *)b;
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(va, vb, c, 0, 0, 0);
    }
};

// ---------------------------------------------------------------- epilogue

__device__ inline uint16_t f32_to_f16_bits(float x)
{
    _Float16 h = (_Float16)x; // v_cvt_f16_f32: round to nearest even
    return __builtin_bit_cast(uint16_t, h);
}

__device__ inline uint16_t f32_to_bf16_bits(float x)
{
    __bf16 h = (__bf16)x; // gfx950 v_cvt_pk_bf16_f32: round to nearest even
    return __builtin_bit_cast(uint16_t, h);
}

// Epilogue of one accumulator value at (row, col), both in range, for output
// kind KIND: t = acc (+C); y = has_bias ? fmaf(alpha, t, bias[col]) : alpha*t;
// relu; round-to-nearest-even cast and store.  Integer: D = acc + C mod 2^32.
template <int KIND>
__device__ inline void epilogue_store(const EpiArgs &e, int64_t row, int64_t col, float acc)
{
    float t = acc;
    if (e.C)
        t += ((const float *)e.C)[row * e.ldc + col];
    float y = e.bias ? __builtin_fmaf(e.alpha, t, e.bias[col]) : e.alpha * t;
    if (e.relu)
        y = (y > 0.0f) ? y : 0.0f;
    const int64_t o = row * e.ldd + col;
    if constexpr (KIND == OUT_F32)
        ((float *)e.D)[o] = y;
    else if constexpr (KIND == OUT_F16)
        ((uint16_t *)e.D)[o] = f32_to_f16_bits(y);
    else
        ((uint16_t *)e.D)[o] = f32_to_bf16_bits(y);
}

template <int KIND>
__device__ inline void epilogue_store(const EpiArgs &e, int64_t row, int64_t col, int acc)
{
    uint32_t t = (uint32_t)acc;
    if (e.C)
        t += (uint32_t)((const int32_t *)e.C)[row * e.ldc + col];
    ((int32_t *)e.D)[row * e.ldd + col] = (int32_t)t;
}

// Store one 32x32 accumulator fragment whose top-left output is (m0, n0).
template <class OP, int KIND>
__device__ inline void epilogue_fragment_k(const EpiArgs &e, const typename OP::acc_t &acc,
                                           int64_t m0, int64_t n0, int lane)
{
    const int64_t col = n0 + (lane & 31);
    if (col >= e.N)
        return;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t row = m0 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        if (row < e.M)
            epilogue_store<KIND>(e, row, col, acc[i]);
    }
}

// Store an FM x FN grid of 32x32 fragments (fragment (i,j) at
// (m0 + 32 i, n0 + 32 j)); the output-type switch sits outside the loops.
template <class OP, int FM, int FN>
__device__ inline void epilogue_grid(const EpiArgs &e, typename OP::acc_t (&acc)[FM][FN],
                                     int64_t m0, int64_t n0, int lane)
{
    auto run = [&](auto kind) {
        constexpr int K = decltype(kind)::value;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                epilogue_fragment_k<OP, K>(e, acc[i][j], m0 + 32 * i, n0 + 32 * j, lane);
    };
    if constexpr (OP::INT) {
        run(std::integral_constant<int, OUT_S32>{});
    } else {
        switch (e.d_kind) {
        case OUT_F32: run(std::integral_constant<int, OUT_F32>{}); break;
        case OUT_F16: run(std::integral_constant<int, OUT_F16>{}); break;
        default: run(std::integral_constant<int, OUT_BF16>{}); break;
        }
    }
}

} // namespace stg
