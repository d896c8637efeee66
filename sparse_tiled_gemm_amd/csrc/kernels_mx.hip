// MX block-scaled GEMM ("NVIDIA MMA" (rainlin-net), section "Blackwell:
// FP4/FP6 and block-scaled MMA": D = C + sum_g (A_g S_A,g)(B_g S_B,g) over K
// blocks g of 32, UE8M0 scales per the "MXFP4 and NVFP4" table) on the gfx950
// scaled MFMA v_mfma_scale_f32_32x32x64_f8f6f4, which applies one E8M0 scale
// per 32 K of each A row and B column inside the instruction.
//
// k_mx_generic: one wave per 32x32 output tile, operands gathered byte by
//   byte from global memory into the instruction's lane layout (OpMX in
//   device_common.hpp), any pair of the five element formats, any M, N and
//   K % 32 == 0.  The fast path for pairs of one width (both 8-bit or both
//   4-bit) is k_tiled<OpMX<...>> in kernels_dense.hip.
#include "device_common.hpp"
#include "internal.hpp"

namespace stg {

template <int F>
struct MxBits {
    static constexpr int value = F <= 1 ? 8 : (F == 4 ? 4 : 6);
};

// This lane's operand words for the instruction covering K k0 .. k0+63 of the
// packed row `row` (zero when !ok or past K; K % 32 == 0, so a 32-K block is
// entirely inside or outside).
template <int F>
__device__ STG_AI void mx_operand(uint32_t (&w)[8], const uint8_t *row, bool ok, int64_t k0,
                                  int64_t K, int half)
{
    constexpr int BITS = MxBits<F>::value;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        w[i] = 0;
    if (!ok)
        return;
    if constexpr (BITS == 8) {
        // bytes 0..15: K k0+16h .. ; bytes 16..31: K k0+32+16h ..
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int64_t kb = k0 + 32 * p + 16 * half;
            if (kb < K)
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    w[4 * p + j / 4] |= (uint32_t)row[kb + j] << (8 * (j % 4));
        }
    } else {
        // K k0+32h .. k0+32h+31, packed: 16 (4-bit) or 24 (6-bit) bytes
        const int64_t kb = k0 + 32 * half;
        if (kb < K) {
            const uint8_t *p = row + kb * BITS / 8;
#pragma unroll
            for (int j = 0; j < 4 * BITS; ++j)
                w[j / 4] |= (uint32_t)p[j] << (8 * (j % 4));
        }
    }
}

template <int AF, int BF>
__global__ __launch_bounds__(256) void k_mx_generic(GemmArgs g)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t m0 = (int64_t)blockIdx.y * 64 + (wave >> 1) * 32;
    const int64_t n0 = (int64_t)blockIdx.x * 64 + (wave & 1) * 32;
    if (m0 >= g.e.M || n0 >= g.e.N)
        return;
    const int64_t am = m0 + (lane & 31), bn = n0 + (lane & 31);
    const bool a_ok = am < g.e.M, b_ok = bn < g.e.N;
    const int half = lane >> 5;
    const int64_t K = g.K, kblk = K / 32;
    const uint8_t *arow =
        (const uint8_t *)g.A + (a_ok ? am : 0) * (g.a_rs * MxBits<AF>::value / 8);
    const uint8_t *brow =
        (const uint8_t *)g.B + (b_ok ? bn : 0) * (g.b_cs * MxBits<BF>::value / 8);
    f16_t acc = {};
    for (int64_t k0 = 0; k0 < K; k0 += 64) {
        uint32_t wa[8], wb[8];
        mx_operand<AF>(wa, arow, a_ok, k0, K, half);
        mx_operand<BF>(wb, brow, b_ok, k0, K, half);
        // lane half h carries the scale of K block k0/32 + h (data past K
        // is zero, so its scale is irrelevant)
        const int64_t blk = k0 / 32 + half;
        const uint32_t sa = (a_ok && blk < kblk) ? g.sa[am * kblk + blk] : 127u;
        const uint32_t sb = (b_ok && blk < kblk) ? g.sb[bn * kblk + blk] : 127u;
        i8_t va, vb;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            va[i] = (int)wa[i];
            vb[i] = (int)wb[i];
        }
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, vb, acc, AF, BF, 0, (int)sa, 0,
                                                              (int)sb);
    }
    f16_t grid[1][1] = {{acc}};
    epilogue_grid<OpF8<0, 0>, 1, 1>(g.e, grid, m0, n0, lane);
}

template <int AF, int BF>
static hipError_t launch_mx_generic_t(const GemmArgs &g, hipStream_t s)
{
    dim3 grid((unsigned)((g.e.N + 63) / 64), (unsigned)((g.e.M + 63) / 64));
    hipLaunchKernelGGL((k_mx_generic<AF, BF>), grid, dim3(256), 0, s, g);
    return hipGetLastError();
}

template <int AF>
static hipError_t launch_mx_generic_a(int bfmt, const GemmArgs &g, hipStream_t s)
{
    switch (bfmt) {
    case 0: return launch_mx_generic_t<AF, 0>(g, s);
    case 1: return launch_mx_generic_t<AF, 1>(g, s);
    case 2: return launch_mx_generic_t<AF, 2>(g, s);
    case 3: return launch_mx_generic_t<AF, 3>(g, s);
    case 4: return launch_mx_generic_t<AF, 4>(g, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_mx(int family, int afmt, int bfmt, const GemmArgs &g, hipStream_t s)
{
    if (family == KF_MX_TILED)
        return launch_mx_tiled(afmt, bfmt, g, s);
    if (family != KF_MX_GENERIC)
        return hipErrorInvalidValue;
    switch (afmt) {
    case 0: return launch_mx_generic_a<0>(bfmt, g, s);
    case 1: return launch_mx_generic_a<1>(bfmt, g, s);
    case 2: return launch_mx_generic_a<2>(bfmt, g, s);
    case 3: return launch_mx_generic_a<3>(bfmt, g, s);
    case 4: return launch_mx_generic_a<4>(bfmt, g, s);
    default: return hipErrorInvalidValue;
    }
}

} // namespace stg
