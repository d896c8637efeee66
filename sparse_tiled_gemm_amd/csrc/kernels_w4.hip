// W4A16 weight-only GEMM ("NVIDIA MMA" (rainlin-net), section "How
// quantisation configurations map to MMA": INT4 weights, FP16 / BF16
// activations, run as an FP16 x FP16 or BF16 x BF16 MMA on a weight tile
// dequantised first; the section "Ampere: FP16/BF16 and integer MMA
// baseline" notes that INT4 MMA needs both operands in INT4, so a W4A16
// kernel converts the weight tile instead).
//
// k_w4_generic: one wave per 32x32 output tile; each lane reads its 8 K of
//   A and dequantises its 8 K of B (codes, group scale, zero point) straight
//   from global memory into the dense 32x32x16 MFMA's fragment.  Any M, N,
//   K % 32 == 0, any row pitch and alignment.  The fast path is
//   k_tiled<OpW4<...>> in kernels_dense.hip (dequantisation between the
//   global load and the LDS store of each B tile).
#include "device_common.hpp"
#include "internal.hpp"

namespace stg {

template <class BASE>
__global__ __launch_bounds__(256) void k_w4_generic(GemmArgs g)
{
    constexpr bool BF = std::is_same<BASE, OpBF16>::value;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t m0 = (int64_t)blockIdx.y * 64 + (wave >> 1) * 32;
    const int64_t n0 = (int64_t)blockIdx.x * 64 + (wave & 1) * 32;
    if (m0 >= g.e.M || n0 >= g.e.N)
        return;
    const int64_t am = m0 + (lane & 31), bn = n0 + (lane & 31);
    const bool a_ok = am < g.e.M, b_ok = bn < g.e.N;
    const int64_t K = g.K, gpr = K / g.wgs;
    const uint8_t *codes = (const uint8_t *)g.B + (b_ok ? bn : 0) * (g.b_cs / 2);
    const uint16_t *scales = (const uint16_t *)g.ws + (b_ok ? bn : 0) * gpr;
    const uint8_t *zeros = g.wz ? g.wz + (b_ok ? bn : 0) * gpr : nullptr;
    f16_t acc = {};
    for (int64_t k0 = 0; k0 < K; k0 += 16) {
        const int64_t kb = k0 + (lane >> 5) * 8; // this lane's 8 K (inside one group)
        uint32_t a[4], b[4] = {0, 0, 0, 0};
        load_frag_strided<2, 8>(a, g.A, a_ok, am * g.a_rs, g.a_cs, kb, K);
        if (b_ok) {
            const int64_t grp = kb / g.wgs;
            const float sc = w4_scale<BF>(scales[grp]);
            const int z = zeros ? (int)zeros[grp] : 8;
            // 8 codes = 4 bytes at byte kb / 2 (kb is even)
            const uint32_t w = (uint32_t)codes[kb / 2] | ((uint32_t)codes[kb / 2 + 1] << 8) |
                               ((uint32_t)codes[kb / 2 + 2] << 16) |
                               ((uint32_t)codes[kb / 2 + 3] << 24);
            w4_dequant8<BF>(w, z, sc, b);
        }
        acc = BASE::mma(a, b, acc);
    }
    f16_t grid[1][1] = {{acc}};
    epilogue_grid<BASE, 1, 1>(g.e, grid, m0, n0, lane);
}

hipError_t launch_w4(int family, int op, const GemmArgs &g, hipStream_t s)
{
    if (family == KF_W4_TILED)
        return launch_w4_tiled(op, g, s);
    if (family == KF_W4_TILED16)
        return launch_w4_tiled16(op, g, s);
    if (family == KF_W4_SKINNY)
        return launch_w4_skinny(op, g, s);
    if (family != KF_W4_GENERIC)
        return hipErrorInvalidValue;
    dim3 grid((unsigned)((g.e.N + 63) / 64), (unsigned)((g.e.M + 63) / 64));
    if (op == OPK_F16)
        hipLaunchKernelGGL(k_w4_generic<OpF16>, grid, dim3(256), 0, s, g);
    else if (op == OPK_BF16)
        hipLaunchKernelGGL(k_w4_generic<OpBF16>, grid, dim3(256), 0, s, g);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

} // namespace stg
