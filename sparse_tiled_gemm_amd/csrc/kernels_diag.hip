// Diagnostic kernel: the MFMA-only throughput ceiling of gfx950 on random
// operands (no memory traffic, no LDS), the rate a GEMM main loop could at
// best sustain on this chip once its clock settles under MFMA load.  Each
// wave keeps the 128 accumulator registers of the 16-bit 8-wave GEMM kernel
// (a 4 x 2 grid of 32x32 tiles, or an 8 x 4 grid of 16x16 tiles for the
// 16x16 forms) and feeds it from a pool of 8 operand fragments of random
// finite values that rotate every K step, so each instruction sees new
// operand bits (the switching activity of a GEMM, which sets the power
// draw).  Launched as 8 waves (2 per SIMD) per workgroup, one workgroup per
// compute unit.  The two forms of a type do the same multiply-adds per
// iteration: 8 steps of 8 32x32 instructions, or 4 steps of 32 16x16 ones.
#include "device_common.hpp"
#include "internal.hpp"

namespace stg {

namespace {

// A 32-bit word of random operand bits for word w of lane l, fragment f:
// finite values of the operand type (16-bit floats with exponents near 1,
// E4M3 codes other than NaN, any int8).
template <class OP>
__device__ STG_AI uint32_t operand_word(uint32_t l, uint32_t f, uint32_t w)
{
    uint32_t h = (l + 1) * 0x9E3779B1u ^ (f + 1) * 0x85EBCA77u ^ (w + 1) * 0xC2B2AE3Du;
    h ^= h >> 15;
    h *= 0x2C1B3C6Du;
    h ^= h >> 12;
    if constexpr (OP::ELEM == 2) {
        // sign, exponent 125..128 (values in [0.25, 4)), 7 random fraction bits
        auto half = [](uint32_t x) { return (x & 0x807Fu) | ((0x3E80u + ((x >> 8) & 3u) * 0x80u)); };
        return half(h) | (half(h >> 16) << 16);
    } else if constexpr (OP::INT) {
        return h;
    } else {
        // E4M3 codes 0x00..0x7E and 0x80..0xFE (0x7F / 0xFF are NaN)
        uint32_t r = 0;
        for (int b = 0; b < 4; ++b) {
            uint32_t c = (h >> (8 * b)) & 0xFFu;
            c = (c & 0x7Fu) == 0x7Fu ? c ^ 1u : c;
            r |= c << (8 * b);
        }
        return r;
    }
}

template <class OP, int NA, int NB, int NS>
__global__ __launch_bounds__(512, 1) void k_mfma_loop(int64_t iters, float *out)
{
    constexpr int NP = 8, FW = OP::LANE_BYTES / 4;
    const uint32_t gid = blockIdx.x * 512 + threadIdx.x;
    uint32_t pool[NP][FW];
#pragma unroll
    for (int f = 0; f < NP; ++f)
#pragma unroll
        for (int w = 0; w < FW; ++w)
            pool[f][w] = operand_word<OP>(gid, f, w);
    typename OP::acc_t acc[NA][NB];
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
            acc[i][j] = typename OP::acc_t{};
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int i = 0; i < NA; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    acc[i][j] = OP::mma(pool[(s + i) % NP], pool[(s + NP / 2 + j) % NP], acc[i][j]);
    }
    constexpr int R = sizeof(typename OP::acc_t) / 4; // accumulator registers per tile
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < R; ++r)
                sum += (float)acc[i][j][r];
    out[gid] = sum; // keeps the loop's results live
}

template <class OP, int NA, int NB, int NS>
hipError_t launch_loop(int blocks, int64_t iters, float *out, hipStream_t s)
{
    hipLaunchKernelGGL((k_mfma_loop<OP, NA, NB, NS>), dim3((unsigned)blocks), dim3(512), 0, s,
                       iters, out);
    return hipGetLastError();
}

} // namespace

// kind: 0 bf16 (32x32x16), 1 fp8 E4M3 x E4M3 (32x32x64 f8f6f4, unit
// scales), 2 int8 (32x32x32); 3, 4, 5: the same types' 16x16 forms
// (16x16x32, 16x16x128, 16x16x64).  `out` holds blocks * 512 floats.
hipError_t launch_mfma_loop(int kind, int blocks, int64_t iters, float *out, hipStream_t s)
{
    switch (kind) {
    case 0: return launch_loop<OpBF16, 4, 2, 8>(blocks, iters, out, s);
    case 1: return launch_loop<OpF8<0, 0>, 4, 2, 8>(blocks, iters, out, s);
    case 2: return launch_loop<OpS8, 4, 2, 8>(blocks, iters, out, s);
    case 3: return launch_loop<Op16BF16, 8, 4, 4>(blocks, iters, out, s);
    case 4: return launch_loop<Op16F8<0, 0>, 8, 4, 4>(blocks, iters, out, s);
    case 5: return launch_loop<Op16S8, 8, 4, 4>(blocks, iters, out, s);
    default: return hipErrorInvalidValue;
    }
}

} // namespace stg
