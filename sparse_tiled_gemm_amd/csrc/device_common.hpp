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

// Device helpers and the lambdas in the kernels are always inlined: a call
// left in place would force everything passed or captured by reference (the
// accumulators, the kernel arguments) into scratch memory.
#define STG_AI __attribute__((always_inline))

// Compiler-only memory barrier: emits nothing, but no load or store is moved
// across it.  The kernels order the hardware with explicit s_waitcnt,
// s_barrier and wave barriers; the builtins that emit those are not memory
// operations to the compiler, which may otherwise move an LDS access across
// them when it can prove, from one lane's point of view, that two addresses
// differ (lanes exchange data through LDS exactly there).  A workgroup-scope
// fence would do the same but also wait for the direct global -> LDS copies
// that the pipelines keep in flight across barriers.
#define STG_COMPILER_FENCE() asm volatile("" ::: "memory")

namespace stg {

// A point where this wave's lanes exchange data through LDS: earlier LDS
// accesses of the wave are complete and no LDS access moves across it.
__device__ STG_AI inline void wave_lds_sync()
{
    __builtin_amdgcn_s_waitcnt(0xC07F); // lgkmcnt(0)
    STG_COMPILER_FENCE();
    __builtin_amdgcn_wave_barrier();
    STG_COMPILER_FENCE();
}

// Workgroup barrier for pipelines that manage their own waits: the caller has
// already waited for what must be complete; this adds lgkmcnt(0) (this
// wave's LDS reads and stores done) and keeps the compiler from moving LDS
// accesses across the barrier.
__device__ STG_AI inline void lds_barrier()
{
    __builtin_amdgcn_s_waitcnt(0xC07F); // lgkmcnt(0)
    STG_COMPILER_FENCE();
    __builtin_amdgcn_s_barrier();
    STG_COMPILER_FENCE();
}

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
    static constexpr int ELEM = 2, LANE_BYTES = 16, KB = 32, BITS = 16;
    static constexpr bool INT = false, MX = false, SPLIT = false, W4 = false;
    typedef f16_t acc_t;
    __device__ static inline acc_t mma(const uint32_t *a, const uint32_t *b, acc_t c)
    {
        h8_t va = __builtin_bit_cast(h8_t, *(const u4_t *)a);
        h8_t vb = __builtin_bit_cast(h8_t, *(const u4_t *)b);
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(va, vb, c, 0, 0, 0);
    }
};

struct OpBF16 {
    static constexpr int ELEM = 2, LANE_BYTES = 16, KB = 32, BITS = 16;
    static constexpr bool INT = false, MX = false, SPLIT = false, W4 = false;
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
    static constexpr int ELEM = 1, LANE_BYTES = 32, KB = 64, BITS = 8;
    static constexpr bool INT = false, MX = false, SPLIT = false, W4 = false;
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
    static constexpr int ELEM = 1, LANE_BYTES = 16, KB = 32, BITS = 8;
    static constexpr bool INT = true, MX = false, SPLIT = false, W4 = false;
    static constexpr bool AU = false, BU = false; // unsigned A / B (OpI8)
    typedef i16_t acc_t;
    __device__ static inline acc_t mma(const uint32_t *a, const uint32_t *b, acc_t c)
    {
        i4_t va = *(const i4_t *)a;
        i4_t vb = *(const i4_t *)b;
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(va, vb, c, 0, 0, 0);
    }
};

// 8-bit integer operands of either signedness (the INT8 rows of "NVIDIA
// MMA", section "Ampere: FP16/BF16 and integer MMA baseline", take signed or
// unsigned A and B).  gfx950's int8 MFMA is signed only, so an unsigned
// operand x (0..255) enters it as x - 128 (its bits XOR 0x80) and the exact
// sum is restored afterwards: with a = a' + 128 AU and b = b' + 128 BU,
//   sum_k a b = sum_k a' b' + 128 BU sum_k a'[m,k] + 128 AU sum_k b'[k,n]
//               + 16384 AU BU K,
// every term taken modulo 2^32 like the int32 accumulator itself, so the
// result is bit-exact (u8_correct).
template <bool A_U, bool B_U>
struct OpI8 : OpS8 {
    static constexpr bool AU = A_U, BU = B_U;
};
template <class OP>
constexpr bool au_v()
{
    if constexpr (requires { OP::AU; })
        return OP::AU;
    else
        return false;
}
template <class OP>
constexpr bool bu_v()
{
    if constexpr (requires { OP::BU; })
        return OP::BU;
    else
        return false;
}
// XOR mask that turns four packed u8 into the s8 values x - 128
constexpr uint32_t U8_FLIP = 0x80808080u;

// Sum of the four signed bytes of w, added to acc.
__device__ STG_AI inline int sum4_s8(uint32_t w, int acc)
{
    return __builtin_amdgcn_sdot4((int)w, 0x01010101, acc, false);
}

// The offset terms of OpI8 for a wave's FM x FN grid of 32x32 int32
// accumulators.  rs[i]: this lane's partial sum of the signed (shifted) A
// values of row lane % 32 of fragment row i over its half of K (the two
// lane halves hold the two halves); cs[j]: the same for column lane % 32 of
// B's fragment column j.  K: the number of K positions summed.
template <bool AU, bool BU, int FM, int FN>
__device__ STG_AI inline void u8_correct(i16_t (&acc)[FM][FN], const int (&rs)[FM],
                                         const int (&cs)[FN], int64_t K, int lane)
{
    if constexpr (AU || BU) {
        const uint32_t kc = AU && BU ? (uint32_t)((uint64_t)K * 16384u) : 0u;
        uint32_t cfull[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j)
            cfull[j] = AU ? (uint32_t)(cs[j] + __shfl_xor(cs[j], 32)) * 128u : 0u;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int rfull = BU ? rs[i] + __shfl_xor(rs[i], 32) : 0;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                // accumulator register r of this lane is row R of the fragment,
                // whose full sum lane R holds
                const int R = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const uint32_t rr = BU ? (uint32_t)__shfl(rfull, R) * 128u : 0u;
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j][r] = (int)((uint32_t)acc[i][j][r] + rr + cfull[j] + kc);
            }
        }
    }
}

// MX block-scaled product of OCP MX element formats (AF / BF: 0 = E4M3, 1 =
// E5M2, 2 = E2M3, 3 = E3M2, 4 = E2M1, the selectors of the gfx950
// v_mfma_scale_f32_32x32x64_f8f6f4) with one E8M0 scale per 32 K of every A
// row and B column.  The tiled kernel takes pairs of one width: both 8-bit,
// both 4-bit, or both 6-bit in the padded layout below (BITS is the stored
// width).  Lane layouts (measured with single-instruction probes):
//  - 8-bit operands: lane l (h = l / 32) gives bytes 0..15 = K 16h .. 16h+15
//    and bytes 16..31 = K 32+16h .. 32+16h+15 of row / column l % 32 (so
//    K block b of the instruction is bytes 16b .. 16b+15 of both lane
//    halves; the tiled kernel swaps chunks 1 and 2 of each 64-byte K tile
//    on its way into LDS, so a lane half reads two consecutive chunks);
//  - 6- and 4-bit operands: lane half h gives K 32h .. 32h+31, packed from
//    bit 0 up (4-bit: the even element in the low nibble);
//  - the scale VGPR of lane half b holds (in the byte the instruction's
//    op_sel picks) the scale of the lane's row / column over K block b.
// PAD6: both operands 6-bit, stored padded to the 8-bit geometry - each
// 32-K block's 24 packed bytes followed by 8 unused bytes, and the 64-byte
// K groups in the 8-bit chunk order (chunk h: bytes 0..15 of block h, chunk
// 2 + h: bytes 16..23 of block h and the padding), so that after the 8-bit
// chunk swap a lane half reads its block's 24 bytes as words 0..5 (the
// instruction reads six registers of a 6-bit operand).
template <int AF, int BF, bool PAD6 = false>
struct OpMX {
    static constexpr int FBITS = AF <= 1 ? 8 : (AF == 4 ? 4 : 6);
    static_assert((BF <= 1 ? 8 : (BF == 4 ? 4 : 6)) == FBITS, "one width for A and B");
    static_assert(!PAD6 || FBITS == 6, "padding: 6-bit formats");
    static constexpr int BITS = PAD6 ? 8 : FBITS; // storage bits per K
    static constexpr int ELEM = 1; // (unused: MX addressing is by BITS)
    static constexpr int LANE_BYTES = 32 * BITS / 8; // one 32-K block per lane
    static constexpr int KB = 2 * LANE_BYTES;        // row bytes per instruction (64 K)
    static constexpr bool INT = false, MX = true, W4 = false;
    static constexpr bool SPLIT = BITS == 8; // the 8-bit K order (chunks 1 and 2 swapped)
    typedef f16_t acc_t;
    // SEL: byte of sa / sb holding this instruction's scales
    template <int SEL>
    __device__ static STG_AI acc_t mma(const uint32_t *a, const uint32_t *b, acc_t c, uint32_t sa,
                                      uint32_t sb)
    {
        i8_t va = {}, vb = {};
#pragma unroll
        for (int i = 0; i < LANE_BYTES / 4; ++i) {
            va[i] = (int)a[i];
            vb[i] = (int)b[i];
        }
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, vb, c, AF, BF, SEL, (int)sa, SEL,
                                                               (int)sb);
    }
};

// W4A16 ("NVIDIA MMA", section "How quantisation configurations map to
// MMA": INT4 weight-only runs as an FP16 / BF16 MMA on a weight tile
// dequantised first): Base (OpF16 or OpBF16, or their 16x16 forms in the
// skinny kernel) multiplies A by B's unsigned 4-bit codes turned into
// Base's type in the main loop.
template <class Base>
struct OpW4 : Base {
    static constexpr bool W4 = true;
};

// Operands stored MN-major ("CUDA 014 - MMA 指令的用法详解", section "加载时转置":
// a load that transposes as it reads fits an operand whose memory order is
// the transpose of the MMA's register order): A column-major (M contiguous)
// and / or B row-major (N contiguous), 16- and 8-bit types, in the LDS-tiled
// kernel.  The tile keeps its memory order in LDS (K rows of MN values) and
// the fragments are fetched with the transposing LDS read.
template <class Base, bool AM, bool BM>
struct OpMN : Base {
    static constexpr bool A_MN = AM, B_MN = BM;
};
template <class OP>
constexpr bool a_mn_v()
{
    if constexpr (requires { OP::A_MN; })
        return OP::A_MN;
    else
        return false;
}
template <class OP>
constexpr bool b_mn_v()
{
    if constexpr (requires { OP::B_MN; })
        return OP::B_MN;
    else
        return false;
}

// 16x16 MFMA forms (skinny kernel).  Lane l holds row (or column) l % 16 and
// LANE_BYTES K bytes; accumulator register i of lane l is row 4 (l / 16) + i,
// column l % 16.  KB16 = K bytes one instruction consumes (4 lane groups).
struct Op16F16 {
    static constexpr int ELEM = 2, LANE_BYTES = 16;
    static constexpr bool INT = false, W4 = false;
    typedef f4_t acc_t;
    __device__ static inline acc_t mma(const uint32_t *a, const uint32_t *b, acc_t c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, *(const u4_t *)a),
                                                      __builtin_bit_cast(h8_t, *(const u4_t *)b),
                                                      c, 0, 0, 0);
    }
};
struct Op16BF16 {
    static constexpr int ELEM = 2, LANE_BYTES = 16;
    static constexpr bool INT = false, W4 = false;
    typedef f4_t acc_t;
    __device__ static inline acc_t mma(const uint32_t *a, const uint32_t *b, acc_t c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf8_t, *(const u4_t *)a), __builtin_bit_cast(bf8_t, *(const u4_t *)b),
            c, 0, 0, 0);
    }
};
template <int AFMT, int BFMT>
struct Op16F8 {
    static constexpr int ELEM = 1, LANE_BYTES = 32;
    static constexpr bool INT = false, W4 = false;
    typedef f4_t acc_t;
    __device__ static inline acc_t mma(const uint32_t *a, const uint32_t *b, acc_t c)
    {
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(*(const i8_t *)a, *(const i8_t *)b,
                                                                c, AFMT, BFMT, 0, 127, 0, 127);
    }
};
struct Op16S8 {
    static constexpr int ELEM = 1, LANE_BYTES = 16;
    static constexpr bool INT = true, W4 = false;
    typedef i4_t acc_t;
    __device__ static inline acc_t mma(const uint32_t *a, const uint32_t *b, acc_t c)
    {
        return __builtin_amdgcn_mfma_i32_16x16x64_i8(*(const i4_t *)a, *(const i4_t *)b, c, 0, 0, 0);
    }
};

// LE consecutive K elements (k0 ..) of one row or column of an operand read
// element by element (any stride), zero past K or for a row outside the
// matrix, packed into 32-bit words.
template <int ELEM, int LE>
__device__ STG_AI inline void load_frag_strided(uint32_t *out, const void *base, bool row_ok,
                                         int64_t row_off, int64_t kstride, int64_t k0, int64_t K)
{
    if constexpr (ELEM == 2) {
        const uint16_t *p = (const uint16_t *)base;
#pragma unroll
        for (int j = 0; j < LE; j += 2) {
            uint32_t lo = 0, hi = 0;
            if (row_ok && k0 + j < K)
                lo = p[row_off + (k0 + j) * kstride];
            if (row_ok && k0 + j + 1 < K)
                hi = p[row_off + (k0 + j + 1) * kstride];
            out[j / 2] = lo | (hi << 16);
        }
    } else {
        const uint8_t *p = (const uint8_t *)base;
#pragma unroll
        for (int j = 0; j < LE; j += 4) {
            uint32_t w = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (row_ok && k0 + j + q < K)
                    w |= (uint32_t)p[row_off + (k0 + j + q) * kstride] << (8 * q);
            out[j / 4] = w;
        }
    }
}

// ---------------------------------------------------------------- epilogue

__device__ STG_AI inline uint16_t f32_to_f16_bits(float x)
{
    _Float16 h = (_Float16)x; // v_cvt_f16_f32: round to nearest even
    return __builtin_bit_cast(uint16_t, h);
}

__device__ STG_AI inline uint16_t f32_to_bf16_bits(float x)
{
    __bf16 h = (__bf16)x; // gfx950 v_cvt_pk_bf16_f32: round to nearest even
    return __builtin_bit_cast(uint16_t, h);
}

// Eight codes of one 32-bit word (element j in bits 4j ..) dequantised to
// RNE((q - z) s) in the 16-bit type (BF: bfloat16, else fp16), two per
// output word, element order kept.  (q - z) s is exact in fp32 (a 5-bit
// integer times a 16-bit significand), so the cast is the only rounding.
template <bool BF>
__device__ STG_AI inline void w4_dequant8(uint32_t w, int z, float s, uint32_t *out)
{
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
        const float v0 = (float)((int)((w >> (4 * j)) & 15u) - z) * s;
        const float v1 = (float)((int)((w >> (4 * j + 4)) & 15u) - z) * s;
        out[j / 2] = BF ? f32_to_bf16_bits(v0) | ((uint32_t)f32_to_bf16_bits(v1) << 16)
                        : f32_to_f16_bits(v0) | ((uint32_t)f32_to_f16_bits(v1) << 16);
    }
}

// A 16-bit scale's bits (fp16, or bfloat16 when BF) as fp32.
template <bool BF>
__device__ STG_AI inline float w4_scale(uint32_t bits)
{
    return BF ? __builtin_bit_cast(float, bits << 16)
              : (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// fp32 -> OCP FP8 (E4M3 when E4, else E5M2): round to nearest even,
// saturating at the largest finite value (448 / 57344); NaN -> 0x7F.
template <bool E4>
__device__ STG_AI inline uint32_t f32_to_fp8_bits(float x)
{
    constexpr int MB = E4 ? 3 : 2, BIAS = E4 ? 7 : 15;
    constexpr float MAXV = E4 ? 448.0f : 57344.0f;
    const uint32_t sign = (__builtin_bit_cast(uint32_t, x) >> 24) & 0x80u;
    float a = __builtin_fabsf(x);
    if (!(a == a))
        return 0x7Fu;
    a = __builtin_fminf(a, MAXV); // every value past MAXV rounds to it
    // spacing of the format at a: 2^(e - MB), e = a's exponent (at least the
    // smallest normal exponent, below which the spacing stays fixed)
    int e = (int)((__builtin_bit_cast(uint32_t, a) >> 23) & 0xFFu) - 127;
    e = e < 1 - BIAS ? 1 - BIAS : e;
    const float q = __builtin_bit_cast(float, (uint32_t)(e - MB + 127) << 23);
    const float r = __builtin_rintf(a / q) * q; // exact quotient, RNE
    // encode r (0, subnormal, or normal - possibly one binade up)
    const int er = (int)((__builtin_bit_cast(uint32_t, r) >> 23) & 0xFFu) - 127;
    uint32_t code;
    if (r == 0.0f)
        code = 0;
    else if (er < 1 - BIAS)
        code = (uint32_t)(r / __builtin_bit_cast(float, (uint32_t)(1 - BIAS - MB + 127) << 23));
    else
        code = ((uint32_t)(er + BIAS) << MB) |
               ((__builtin_bit_cast(uint32_t, r) >> (23 - MB)) & ((1u << MB) - 1));
    return sign | code;
}

// Epilogue of one accumulator value at (row, col), both in range, for output
// C element idx of a float-output epilogue, widened exactly to fp32 (fp32,
// fp16 or bf16 storage).
__device__ STG_AI inline float load_c(const EpiArgs &e, int64_t idx)
{
    if (e.c_kind == 0)
        return ((const float *)e.C)[idx];
    const uint16_t h = ((const uint16_t *)e.C)[idx];
    if (e.c_kind == 1)
        return (float)__builtin_bit_cast(_Float16, h);
    return __builtin_bit_cast(float, (uint32_t)h << 16);
}

// kind KIND: t = acc (+C); y = has_bias ? fmaf(alpha, t, bias[col]) : alpha*t;
// relu; round-to-nearest-even cast and store.  Integer: D = acc + C mod 2^32.
template <int KIND>
__device__ STG_AI inline void epilogue_store(const EpiArgs &e, int64_t row, int64_t col, float acc)
{
    float t = acc;
    if (e.C)
        t += load_c(e, row * e.ldc + col);
    float y = e.bias ? __builtin_fmaf(e.alpha, t, e.bias[col]) : e.alpha * t;
    asm("" : "+v"(y)); // keep y an fp32 value: no fused multiply-add-convert
    if (e.relu)
        y = (y > 0.0f) ? y : 0.0f;
    const int64_t o = row * e.ldd + col;
    if constexpr (KIND == OUT_F32)
        ((float *)e.D)[o] = y;
    else if constexpr (KIND == OUT_F16)
        ((uint16_t *)e.D)[o] = f32_to_f16_bits(y);
    else if constexpr (KIND == OUT_BF16)
        ((uint16_t *)e.D)[o] = f32_to_bf16_bits(y);
    else
        ((uint8_t *)e.D)[o] = (uint8_t)f32_to_fp8_bits<KIND == OUT_E4M3>(y);
}

// Integer accumulator: D = acc + C mod 2^32 for int32 output; for a float
// output (the int8 -> float epilogue) the accumulator's value (RNE to fp32)
// goes through the float epilogue.
template <int KIND>
__device__ STG_AI inline void epilogue_store(const EpiArgs &e, int64_t row, int64_t col, int acc)
{
    if constexpr (KIND == OUT_S32) {
        int t = acc;
        if (e.C) {
            const int c = ((const int32_t *)e.C)[row * e.ldc + col];
            t = e.sat ? __builtin_elementwise_add_sat(acc, c) : (int)((uint32_t)acc + (uint32_t)c);
        }
        ((int32_t *)e.D)[row * e.ldd + col] = t;
    } else {
        epilogue_store<KIND>(e, row, col, (float)acc);
    }
}

// Calls f(std::integral_constant<int, KIND>) for the output kind d_kind
// (OUT_S32 only for integer accumulators).
template <bool INT, class F>
__device__ STG_AI inline void with_out_kind(int d_kind, F &&f)
{
    switch (d_kind) {
    case OUT_F32: f(std::integral_constant<int, OUT_F32>{}); break;
    case OUT_F16: f(std::integral_constant<int, OUT_F16>{}); break;
    case OUT_E4M3: f(std::integral_constant<int, OUT_E4M3>{}); break;
    case OUT_E5M2: f(std::integral_constant<int, OUT_E5M2>{}); break;
    case OUT_S32:
        if constexpr (INT)
            f(std::integral_constant<int, OUT_S32>{});
        break;
    default: f(std::integral_constant<int, OUT_BF16>{}); break;
    }
}

// Bytes of a D element of output kind `kind`.
__device__ STG_AI inline int out_bytes(int kind)
{
    return kind == OUT_F32 || kind == OUT_S32 ? 4 : (kind == OUT_E4M3 || kind == OUT_E5M2 ? 1 : 2);
}

// The finished float value y stored as element o of D in output kind
// `kind` (a uniform branch around the cast and store alone).
__device__ STG_AI inline void store_kind(const EpiArgs &e, int64_t o, float y)
{
    switch (e.d_kind) {
    case OUT_F32: ((float *)e.D)[o] = y; break;
    case OUT_F16: ((uint16_t *)e.D)[o] = f32_to_f16_bits(y); break;
    case OUT_E4M3: ((uint8_t *)e.D)[o] = (uint8_t)f32_to_fp8_bits<true>(y); break;
    case OUT_E5M2: ((uint8_t *)e.D)[o] = (uint8_t)f32_to_fp8_bits<false>(y); break;
    default: ((uint16_t *)e.D)[o] = f32_to_bf16_bits(y); break;
    }
}

// epilogue_store for the output kind e.d_kind, float accumulator: the
// epilogue arithmetic once, then the cast for the kind.
__device__ STG_AI inline void epilogue_store_any(const EpiArgs &e, int64_t row, int64_t col, float acc)
{
    float t = acc;
    if (e.C)
        t += load_c(e, row * e.ldc + col);
    float y = e.bias ? __builtin_fmaf(e.alpha, t, e.bias[col]) : e.alpha * t;
    asm("" : "+v"(y)); // keep y an fp32 value: no fused multiply-add-convert
    if (e.relu)
        y = (y > 0.0f) ? y : 0.0f;
    store_kind(e, row * e.ldd + col, y);
}

// Integer accumulator: int32 output (acc + C mod 2^32), or its value (RNE
// to fp32) through the float epilogue.
__device__ STG_AI inline void epilogue_store_any(const EpiArgs &e, int64_t row, int64_t col, int acc)
{
    if (e.d_kind == OUT_S32)
        epilogue_store<OUT_S32>(e, row, col, acc);
    else
        epilogue_store_any(e, row, col, (float)acc);
}

// Store one 32x32 accumulator fragment whose top-left output is (m0, n0).
template <class OP>
__device__ STG_AI inline void epilogue_fragment_k(const EpiArgs &e, const typename OP::acc_t &acc,
                                           int64_t m0, int64_t n0, int lane)
{
    const int64_t col = n0 + (lane & 31);
    if (col >= e.N)
        return;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t row = m0 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        if (row < e.M)
            epilogue_store_any(e, row, col, acc[i]);
    }
}

// Store an FM x FN grid of 32x32 fragments (fragment (i,j) at
// (m0 + 32 i, n0 + 32 j)); the output-type switch sits outside the loops.
template <class OP, int FM, int FN>
__device__ STG_AI inline void epilogue_grid(const EpiArgs &e, typename OP::acc_t (&acc)[FM][FN],
                                     int64_t m0, int64_t n0, int lane)
{
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            epilogue_fragment_k<OP>(e, acc[i][j], m0 + 32 * i, n0 + 32 * j, lane);
}

// ---------------------------------------------------------------- tile helpers

// Tile-local buffer resource: loads at byte offsets >= `bytes` return zero,
// so rows past the edge of the matrix need no clamping or masking.
__device__ STG_AI inline __amdgpu_buffer_rsrc_t tile_rsrc(const void *base, int64_t bytes)
{
    const int n = bytes > 0x7fffffff ? 0x7fffffff : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, n, 0x00020000);
}

__device__ STG_AI inline u4_t buf_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    return __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// Transposing 8-byte LDS read of 16-bit values (ds_read_b64_tr_b16), lane
// layout as measured on gfx950: inside each group of 16 lanes, lane i
// fetches the four values at its own address, and lane j receives value
// j % 4 of lane 4 e + j / 4 in result slot e (e = 0..3).  So when lane i of
// a group addresses row i / 4, columns 4 (i % 4) .. 4 (i % 4) + 3 of a 4 x 16
// block stored by rows, lane j receives column j, rows 0..3: four
// consecutive K values of one M (or N) index, the MFMA operand order.
// The 8-bit form (ds_read_b64_tr_b8), measured the same way: lane j
// receives byte j % 8 of lane 2 e + j / 8 in result byte e (e = 0..7), so
// lane i addressing row i / 2, columns 8 (i % 2) .. + 7 of an 8 x 16 block
// gives lane j column j, rows 0..7.  lds_read_tr<EB> picks the form for
// elements of EB bytes.
template <int EB>
__device__ STG_AI inline void lds_read_tr(const uint8_t *p, uint32_t *w)
{
    typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
    u2_t v;
    if constexpr (EB == 2) {
        typedef short s4_t __attribute__((ext_vector_type(4)));
        const s4_t r =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4_t *)p);
        v = __builtin_bit_cast(u2_t, r);
    } else {
        typedef int i2_t __attribute__((ext_vector_type(2)));
        const i2_t r =
            __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i2_t *)p);
        v = __builtin_bit_cast(u2_t, r);
    }
    w[0] = v.x;
    w[1] = v.y;
}

// 16-byte chunk slot inside a 64-byte LDS row: chunk c of row r sits at slot
// c ^ swz64(r).  Chosen by measurement on gfx950 (LDS bank-conflict counter
// over the fragment-read pattern of 32 consecutive rows): rotating the slot
// every 4 rows is conflict-free, while the textbook 32-bank XOR patterns
// ((r >> 1) & 3, r & 3, and mixes of them) stall 2- to 4-way.
// swz64(r + 32 i) == swz64(r).
__device__ STG_AI inline int swz64(int r) { return (r >> 2) & 3; }

// 16-byte chunk slot inside a 128-byte LDS row: chunk c of row r sits at
// slot c ^ swz128(r) (conflict-free for 16-byte fragment reads of 32
// consecutive rows, measured the same way).
__device__ STG_AI inline int swz128(int r) { return (r ^ (r >> 3)) & 7; }

// Number of the `total` memory instructions that follow MFMA slot q of
// `slots` when they are spread evenly.
constexpr int spread(int q, int total, int slots)
{
    return (q + 1) * total / slots - q * total / slots;
}

// Workgroup id -> (tile_m, tile_n): XCD-contiguous renumbering, then groups
// of GM tile rows walked column by column.
__device__ STG_AI inline void tile_coords(int id, int tiles_m, int tiles_n, int &tm, int &tn)
{
    constexpr int GM = 8;
    const int total = tiles_m * tiles_n;
    if ((total & 7) == 0)
        id = (id & 7) * (total >> 3) + (id >> 3);
    const int per_group = GM * tiles_n;
    const int group = id / per_group;
    const int first_m = group * GM;
    const int gsize = min(tiles_m - first_m, GM);
    const int in = id - group * per_group;
    tm = first_m + in % gsize;
    tn = in / gsize;
}

// s_waitcnt with only a vector-memory count (expcnt and lgkmcnt left free).
#define STG_WAIT_VMCNT(n) \
    __builtin_amdgcn_s_waitcnt((((n)&15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8)))

// 16-byte global -> LDS copy for a whole wave: lane l's 16 bytes land at
// lds_wave + 16 l (lds_wave must be wave-uniform).
__device__ STG_AI inline void dma16(__amdgpu_buffer_rsrc_t r, uint8_t *lds_wave, int voff, int soff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void *)lds_wave, 16, voff, soff, 0, 0);
}

// ---------------------------------------------------------------- LDS-staged epilogue

// A 64-bit value that is equal in all active lanes, as a scalar.
__device__ STG_AI inline int64_t wave_uniform(int64_t x)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Raw buffer resource over `bytes` bytes at `base` (clamped to 2^31 - 1);
// loads outside the range read zero and stores outside it are dropped.
__device__ STG_AI inline __amdgpu_buffer_rsrc_t epi_rsrc(const void *base, int64_t bytes)
{
    const int n = bytes <= 0 ? 0 : bytes > 0x7fffffff ? 0x7fffffff : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, n, 0x00020000);
}

// alpha * t (+ bias), then relu, for four fp32 values; the bias form is one
// fused multiply-add per element, the same operation the oracle's fp32
// epilogue performs.  Each fp32 result passes through an empty asm:
// otherwise the compiler may fuse the multiply-add with a following f16
// conversion (v_fma_mixlo_f16), which rounds once to f16 instead of to fp32
// and then to f16.
__device__ STG_AI inline f4_t epi_affine(const EpiArgs &e, f4_t t, f4_t b)
{
    f4_t y;
    if (e.bias) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            y[q] = __builtin_fmaf(e.alpha, t[q], b[q]);
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            y[q] = e.alpha * t[q];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
        asm("" : "+v"(y[q]));
    if (e.relu) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            y[q] = (y[q] > 0.0f) ? y[q] : 0.0f;
    }
    return y;
}

// Cache policy of the epilogue's C loads and D stores: non-temporal (each
// byte is touched once; keeping these streams out of the caches leaves them
// to the operand tiles; measured 2-4 % faster on MI355X with a C operand).
constexpr int EPI_CPOL = 2; // the NT bit of the buffer instructions' cache-policy operand

// Store four finished values at byte offset voff + soff of the D resource.
template <int KIND>
__device__ STG_AI inline void epi_store4(__amdgpu_buffer_rsrc_t rd, int voff, int soff, f4_t y)
{
    if constexpr (KIND == OUT_F32) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4_t, y), rd, voff, soff, EPI_CPOL);
    } else if constexpr (KIND == OUT_E4M3 || KIND == OUT_E5M2) {
        constexpr bool E4 = KIND == OUT_E4M3;
        const uint32_t w = f32_to_fp8_bits<E4>(y[0]) | (f32_to_fp8_bits<E4>(y[1]) << 8) |
                           (f32_to_fp8_bits<E4>(y[2]) << 16) | (f32_to_fp8_bits<E4>(y[3]) << 24);
        __builtin_amdgcn_raw_buffer_store_b32(w, rd, voff, soff, EPI_CPOL);
    } else {
        typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
        u2_t w;
        if constexpr (KIND == OUT_F16) {
            w[0] = f32_to_f16_bits(y[0]) | ((uint32_t)f32_to_f16_bits(y[1]) << 16);
            w[1] = f32_to_f16_bits(y[2]) | ((uint32_t)f32_to_f16_bits(y[3]) << 16);
        } else {
            w[0] = f32_to_bf16_bits(y[0]) | ((uint32_t)f32_to_bf16_bits(y[1]) << 16);
            w[1] = f32_to_bf16_bits(y[2]) | ((uint32_t)f32_to_bf16_bits(y[3]) << 16);
        }
        __builtin_amdgcn_raw_buffer_store_b64(w, rd, voff, soff, EPI_CPOL);
    }
}

// acc + C, four elements: fp32 addition, or int32 addition modulo 2^32
// (saturating to the int32 range when `sat`)
__device__ STG_AI inline f4_t add_c(f4_t v, f4_t c) { return v + c; }
// Four C values as fp32: c_kind 0 = fp32 in all four words; 1 = fp16 and
// 2 = bf16, packed two per word in words 0 and 1 (element q in the low half
// of word q / 2 for even q); both widen exactly.
__device__ STG_AI inline f4_t widen_c(u4_t c, int c_kind)
{
    if (c_kind == 0)
        return __builtin_bit_cast(f4_t, c);
    f4_t r;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t h = (c[q >> 1] >> (16 * (q & 1))) & 0xFFFFu;
        r[q] = c_kind == 1 ? (float)__builtin_bit_cast(_Float16, (uint16_t)h)
                           : __builtin_bit_cast(float, h << 16);
    }
    return r;
}
__device__ STG_AI inline i4_t add_c(i4_t v, i4_t c, int sat)
{
    if (sat)
        return __builtin_elementwise_add_sat(v, c);
#pragma unroll
    for (int q = 0; q < 4; ++q)
        v[q] = (int)((uint32_t)v[q] + (uint32_t)c[q]);
    return v;
}

// Epilogue of a wave's (FB FM) x (FB FN) accumulator block at (m0, n0)
// (the same in every lane; FB = 32 for the 32x32 MFMA forms, 16 for the
// 16x16 forms, whose accumulators hold 4 values per lane),
// staged through `lds_wave` (32 * (32 FN + 4) words of LDS owned by this
// wave): for each 32-row slab, the fragments are written to LDS in row-major
// order, then read back four consecutive columns per lane, so C and bias are
// read and D is written with 16- or 8-byte accesses along the rows.
//
// When every column of the block is inside the matrix and the host marked
// the operands as vector-aligned (e.vec), C and D are addressed through
// buffer resources that start at the block's first row and end at row M:
// rows past M read as zero and their stores are dropped, so no lane
// branches, the row step between passes is a scalar offset, and all C loads
// of a slab are issued before the slab is staged (their latency is paid
// once per slab).  Other blocks take an element-by-element path.
// KIND: the output kind (OUT_S32: int32 output of an integer accumulator;
// a float kind takes integer accumulators' values, RNE to fp32, first).
template <class OP, int FM, int FN, int KIND>
__device__ STG_AI inline void epilogue_slabs(const EpiArgs &e, typename OP::acc_t (&acc)[FM][FN],
                                      int64_t m0, int64_t n0, int lane, uint32_t *lds_wave)
{
    constexpr bool M16 = sizeof(typename OP::acc_t) == 16; // 16x16 fragments
    constexpr int FB = M16 ? 16 : 32;                      // fragment rows / columns
    constexpr int NSLAB = FM * FB / 32;                    // 32-row slabs
    constexpr int COLS = FB * FN, PITCH = COLS + 4, LPR = COLS / 4; // lanes per row
    constexpr int RPP = 64 / LPR;                                    // rows per pass
    constexpr int NP = 32 / RPP;                                     // passes per slab
    constexpr bool IOUT = KIND == OUT_S32;
    constexpr int DB = IOUT || KIND == OUT_F32 ? 4 : (KIND == OUT_E4M3 || KIND == OUT_E5M2 ? 1 : 2);
    // what the LDS slab holds: int32 sums for an int32 output, else fp32
    // values (integer accumulators converted, RNE, as they are staged)
    typedef std::conditional_t<IOUT, i4_t, f4_t> v4_t;
    // m0 and n0 are the same in every lane; saying so keeps the buffer
    // resources built from them in scalar registers
    m0 = wave_uniform(m0);
    n0 = wave_uniform(n0);
    const int c4 = (lane % LPR) * 4;
    const int rl = lane / LPR;          // row of this lane within a pass
    const int64_t col = n0 + c4;
    const bool has_c = e.C != nullptr;
    const bool fast = e.vec && n0 + COLS <= e.N; // uniform across the wave

    // the host enables e.vec only when 257 rows of C and of D span less
    // than 2^31 bytes, so every offset below fits in 32 bits (the resources
    // are empty when unused)
    // C elements: 4 bytes (fp32, int32) or 2 (fp16, bf16: a float output
    // only), read 4 per lane as one 16- or 8-byte load and widened exactly
    const int CB = e.c_kind == 0 ? 4 : 2;
    const int ldd_b = (int)(e.ldd * DB);
    const int ldc_b = has_c ? (int)(e.ldc * CB) : 0;
    const __amdgpu_buffer_rsrc_t rd =
        epi_rsrc((uint8_t *)e.D + m0 * e.ldd * DB, fast ? (e.M - m0) * e.ldd * DB : 0);
    const __amdgpu_buffer_rsrc_t rc =
        epi_rsrc(has_c ? (const uint8_t *)e.C + m0 * e.ldc * CB : (const uint8_t *)e.D,
                 fast && has_c ? (e.M - m0) * e.ldc * CB : 0);
    const int vd = rl * ldd_b + (int)(col * DB);
    const int vc = rl * ldc_b + (int)(col * CB);
    f4_t bv{};
    if constexpr (!IOUT) {
        if (fast && e.bias)
            bv = *(const f4_t *)(e.bias + col);
    }

    // one slab per 32 rows (slab i), expanded at compile time so that the
    // accumulator indices are constants however large the body
    auto slab = [&](auto ic) STG_AI {
        constexpr int i = decltype(ic)::value;
        // keep each slab's C loads from being hoisted above earlier slabs
        // (that would need C registers for the whole block at once)
        __builtin_amdgcn_sched_barrier(0);
        u4_t cv[NP];
        if (fast && has_c) {
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                if (IOUT || e.c_kind == 0) {
                    cv[p] = __builtin_bit_cast(
                        u4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                  rc, vc, (32 * i + p * RPP) * ldc_b, EPI_CPOL));
                } else {
                    typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
                    const u2_t h = __builtin_bit_cast(
                        u2_t, __builtin_amdgcn_raw_buffer_load_b64(
                                  rc, vc, (32 * i + p * RPP) * ldc_b, EPI_CPOL));
                    cv[p] = u4_t{h.x, h.y, 0u, 0u};
                }
            }
        }
        // (32x32: register r of lane l is row 8 (r / 4) + 4 (l / 32) + r % 4,
        // column l % 32; 16x16: row 4 (l / 16) + r, column l % 16, and a slab
        // holds fragment rows 2 i and 2 i + 1)
        auto put = [&](int row, int col, auto x) STG_AI {
            if constexpr (IOUT || !OP::INT)
                lds_wave[row * PITCH + col] = __builtin_bit_cast(uint32_t, x);
            else
                lds_wave[row * PITCH + col] = __builtin_bit_cast(uint32_t, (float)x);
        };
        if constexpr (M16) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const auto x = acc[2 * i + h][j][r];
                        put(16 * h + 4 * (lane >> 4) + r, j * 16 + (lane & 15), x);
                    }
        } else {
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    // copy the element out first: a bit_cast applied to a
                    // vector-element expression would read element 0
                    const auto x = acc[i][j][r];
                    put(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3), j * 32 + (lane & 31), x);
                }
        }
        wave_lds_sync(); // the slab is in LDS
        if (fast) {
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const int rr = p * RPP + rl;
                const v4_t v = __builtin_bit_cast(v4_t, *(const u4_t *)(lds_wave + rr * PITCH + c4));
                const int soff = (32 * i + p * RPP) * ldd_b;
                if constexpr (IOUT) {
                    const v4_t w = has_c ? add_c(v, __builtin_bit_cast(v4_t, cv[p]), e.sat) : v;
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4_t, w), rd, vd, soff,
                                                           EPI_CPOL);
                } else {
                    const f4_t f = has_c ? add_c(v, widen_c(cv[p], e.c_kind)) : v;
                    epi_store4<KIND>(rd, vd, soff, epi_affine(e, f, bv));
                }
            }
        } else {
            for (int p = 0; p < NP; ++p) {
                const int rr = p * RPP + rl;
                const int64_t row = m0 + 32 * i + rr;
                const v4_t v = __builtin_bit_cast(v4_t, *(const u4_t *)(lds_wave + rr * PITCH + c4));
                if (row < e.M) {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (col + q < e.N) {
                            epilogue_store<KIND>(e, row, col + q, v[q]);
                        }
                }
            }
        }
        wave_lds_sync(); // reads done before the next slab overwrites
    };
    [&]<int... I>(std::integer_sequence<int, I...>) STG_AI {
        (slab(std::integral_constant<int, I>{}), ...);
    }(std::make_integer_sequence<int, NSLAB>{});
}


template <class OP, int FM, int FN>
__device__ STG_AI inline void epilogue_grid_lds(const EpiArgs &e, typename OP::acc_t (&acc)[FM][FN],
                                         int64_t m0, int64_t n0, int lane, uint32_t *lds_wave)
{
    with_out_kind<OP::INT>(e.d_kind, [&](auto kind) STG_AI {
        epilogue_slabs<OP, FM, FN, decltype(kind)::value>(e, acc, m0, n0, lane, lds_wave);
    });
}

} // namespace stg
