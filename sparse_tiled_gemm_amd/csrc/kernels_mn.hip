// MN-major operands on the LDS-tiled kernel (k_tiled, tiled_kernel.hpp): A
// column-major and / or B row-major, read from LDS with the transposing
// loads ("CUDA 014 - MMA 指令的用法详解", section "加载时转置").  One
// translation unit of its own so that it compiles beside kernels_dense.hip.
// Each input type gets the 256 x 256 wave arrangement its K-contiguous form
// uses (16-bit 2 x 4 waves, fp8 2 x 2, int8 4 x 2) and the 128 x 128 tile.
#include "tiled_kernel.hpp"

namespace stg {

typedef hipError_t (*mn_launch_fn)(const GemmArgs &, hipStream_t);

template <class OP, int BM, int BN, int GM, int GN>
static mn_launch_fn mn_pick(int layout)
{
    switch (layout) {
    case 1: return launch_tiled_t<OpMN<OP, true, false>, BM, BN, GM, GN>;
    case 2: return launch_tiled_t<OpMN<OP, false, true>, BM, BN, GM, GN>;
    case 3: return launch_tiled_t<OpMN<OP, true, true>, BM, BN, GM, GN>;
    default: return nullptr;
    }
}

template <int BM, int BN>
static mn_launch_fn mn_table(int op, int layout)
{
    constexpr bool BIG = BM == 256;
    switch (op) {
    case OPK_F16: return mn_pick<OpF16, BM, BN, 2, BIG ? 4 : 2>(layout);
    case OPK_BF16: return mn_pick<OpBF16, BM, BN, 2, BIG ? 4 : 2>(layout);
    case OPK_F8_E4E4: return mn_pick<OpF8<0, 0>, BM, BN, 2, 2>(layout);
    case OPK_F8_E4E5: return mn_pick<OpF8<0, 1>, BM, BN, 2, 2>(layout);
    case OPK_F8_E5E4: return mn_pick<OpF8<1, 0>, BM, BN, 2, 2>(layout);
    case OPK_F8_E5E5: return mn_pick<OpF8<1, 1>, BM, BN, 2, 2>(layout);
    case OPK_S8: return mn_pick<OpS8, BM, BN, BIG ? 4 : 2, 2>(layout);
    default: return nullptr;
    }
}

hipError_t launch_dense_mn(int family, int op, int layout, const GemmArgs &g, hipStream_t s)
{
    const bool is16 = op == OPK_F16 || op == OPK_BF16, is_s8 = op == OPK_S8;
    mn_launch_fn fn = nullptr;
    if (family == KF_TILED_128)
        fn = mn_table<128, 128>(op, layout);
    else if ((family == KF_TILED_256W8 && is16) || (family == KF_TILED_256W8T && is_s8) ||
             (family == KF_TILED_256 && !is16 && !is_s8))
        fn = mn_table<256, 256>(op, layout);
    if (!fn)
        return hipErrorInvalidValue;
    return fn(g, s);
}

} // namespace stg
