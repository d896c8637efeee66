// Dense GEMM kernels for gfx950 (MI355X): D = epilogue(A*B + C).
//
// k_generic: one wave per 32x32 output tile, operands read element by element
//   straight from global memory (any layout, stride, alignment or shape), one
//   32x32 MFMA per K slice.  This is the tile-per-wave structure of the naive
//   one-warp MMA GEMM on "Tensor Core three calling levels" (chenxutan),
//   section 3, with the MFMA form of each input type.
//
// k_tiled: the block-tiled GEMM of "CUDA 014 - MMA instruction usage"
//   (blog-9y3), section "Implementing general matrix multiply-add with MMA":
//   the output is cut into BM x BN workgroup tiles that walk K in steps, and
//   the waves of a workgroup split the tile.  gfx950 specifics:
//   - both operands are K-contiguous (A row-major, B stored N x K), so a K
//     tile of 64 bytes per row is copied global -> LDS with 16-byte buffer
//     loads, 4 consecutive threads per row; the buffer resource is based at
//     the tile's first row and bounded by the matrix, so rows past M or N
//     read as zero;
//   - software pipeline with three LDS stages: while tile t is multiplied,
//     tile t+2 (loaded into registers during tile t-1) is written to LDS and
//     tile t+3 is fetched into the other register set; MFMA fragments are
//     double-buffered in registers, so the next K step's (or next tile's
//     first) fragments are read from LDS during the current step's MFMAs;
//     one barrier per K tile;
//   - 16-byte chunks are XOR-swizzled within a row (chunk c of row r sits at
//     slot c ^ ((r >> 2) & 3)) so the 32 rows that one fragment read touches
//     spread over all banks - the bank-conflict remedy of the same page's
//     section "Avoiding bank conflicts" (its swizzle figure did not survive;
//     this function is this library's own);
//   - each wave owns a (BM/2) x (BN/2) sub-tile of 32x32 MFMA fragments; per
//     K slice it reads its A and B fragments once with ds_read_b128 and
//     reuses them across the fragment grid;
//   - workgroups are renumbered so consecutive tiles land on the same XCD
//     (workgroups are dealt round-robin to the 8 XCDs, each with its own L2),
//     then ordered in groups of 8 tile rows for L2 reuse.
#include "device_common.hpp"
#include "internal.hpp"
#include "tiled_kernel.hpp"

namespace stg {

// ---------------------------------------------------------------- generic

template <class OP>
__global__ __launch_bounds__(256) void k_generic(GemmArgs g)
{
    constexpr int LE = OP::LANE_BYTES / OP::ELEM; // elements per lane per slice
    constexpr int KI = OP::KB / OP::ELEM;         // elements per instruction
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t m0 = (int64_t)blockIdx.y * 64 + (wave >> 1) * 32;
    const int64_t n0 = (int64_t)blockIdx.x * 64 + (wave & 1) * 32;
    if (m0 >= g.e.M || n0 >= g.e.N)
        return; // whole wave idle
    const int64_t am = m0 + (lane & 31), bn = n0 + (lane & 31);
    const bool a_ok = am < g.e.M, b_ok = bn < g.e.N;
    constexpr bool AU = au_v<OP>(), BU = bu_v<OP>();
    int rs[1] = {0}, cs[1] = {0}; // unsigned operands: sums of the shifted values
    typename OP::acc_t acc = {};
    for (int64_t k0 = 0; k0 < g.K; k0 += KI) {
        uint32_t a[OP::LANE_BYTES / 4], b[OP::LANE_BYTES / 4];
        const int64_t kb = k0 + (lane >> 5) * LE;
        load_frag_strided<OP::ELEM, LE>(a, g.A, a_ok, am * g.a_rs, g.a_cs, kb, g.K);
        load_frag_strided<OP::ELEM, LE>(b, g.B, b_ok, bn * g.b_cs, g.b_rs, kb, g.K);
        if constexpr (AU || BU) {
            // an unsigned value x enters the MFMA as x - 128; bytes past K
            // stay 0 (they must add nothing), the rows past the edge are
            // never stored
#pragma unroll
            for (int w = 0; w < OP::LANE_BYTES / 4; ++w) {
                uint32_t m = 0;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    m |= (kb + 4 * w + q < g.K ? 0x80u : 0u) << (8 * q);
                if constexpr (AU)
                    a[w] ^= m;
                if constexpr (BU)
                    b[w] ^= m;
                if constexpr (BU)
                    rs[0] = sum4_s8(a[w], rs[0]);
                if constexpr (AU)
                    cs[0] = sum4_s8(b[w], cs[0]);
            }
        }
        acc = OP::mma(a, b, acc);
    }
    typename OP::acc_t grid[1][1] = {{acc}};
    if constexpr (AU || BU)
        u8_correct<AU, BU>(grid, rs, cs, g.K, lane);
    epilogue_grid<OP, 1, 1>(g.e, grid, m0, n0, lane);
}

// ---------------------------------------------------------------- skinny

// Small-M GEMM (M <= 16), bound by streaming B once from HBM.  One workgroup
// owns 32 output columns (two 16x16 MFMA fragments); its 8 waves split K
// (chunk c of 256 K bytes goes to wave c % 8; 8 waves keep twice the bytes in
// flight of 4 and measured 3-22 % faster), feed 16x16 MFMAs directly from
// global memory and reduce their partial sums through LDS before the
// epilogue.  Within a chunk, lane l (group g = l / 16) loads 64 contiguous
// bytes of its row at byte 64 g, and MFMA step j uses bytes 16 j.. of every
// lane's 64 (32 j.. for fp8): A and B use the same lane <-> K assignment, so
// each product pairs equal K.  Each row's 256 bytes are fetched by 4 lanes as
// whole cache lines; two chunks are kept in flight per wave.  B (the stream
// from HBM) is loaded 1 KB per instruction instead -- rows 4k .. 4k+3 of
// the chunk, 16 lanes per row -- into the wave's own LDS buffer (16-byte
// chunk q of row r at slot q ^ (r & 15), so the 16 rows a fragment read
// touches fall on 16 different slots of a 256-byte bank window) and read
// back in the layout above: a load-only probe of this kernel's B stream
// moved 4.6 TB/s with such loads against 3.6 TB/s with fragment-shaped
// ones.  (A, 16 rows read by every workgroup, comes from L2; W4A16 keeps
// its register path.)
template <class OP>
__global__ __launch_bounds__(512, 1) void k_skinny(GemmArgs g)
{
    constexpr int WAVES = 8;
    constexpr int CB = 256;                      // K bytes per chunk
    constexpr int LB = 64;                       // bytes per lane per chunk
    constexpr int NLD = LB / 16;                 // 16-byte loads per row-fragment per chunk
    constexpr int STEPS = LB / OP::LANE_BYTES;   // MFMAs per fragment per chunk
    constexpr int FW = OP::LANE_BYTES / 4;
    __shared__ __attribute__((aligned(16))) uint32_t red[WAVES][2][64][4];
    // per wave: 32 B rows x 256 bytes (one buffer: a wave's LDS accesses are
    // ordered, so a chunk's stores cannot overtake the previous chunk's reads)
    __shared__ __attribute__((aligned(16))) uint8_t bst[OP::W4 ? 16 : WAVES * 32 * 256];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t n_blk = (int64_t)blockIdx.x * 32;
    // W4A16: B holds 4-bit codes, a lane's 64 bytes of a chunk arrive as 16
    // code bytes (32 K) and are dequantised in registers before the MFMAs
    constexpr bool W4 = OP::W4;
    constexpr bool BF = std::is_base_of<Op16BF16, OP>::value;
    const int64_t lda_b = g.a_rs * OP::ELEM;
    const int64_t ldb_b = W4 ? g.b_cs / 2 : g.b_cs * OP::ELEM;
    const int64_t kbytes = g.K * OP::ELEM, kbytes_b = W4 ? g.K / 2 : kbytes;
    const int NC = (int)(kbytes / CB);
    const __amdgpu_buffer_rsrc_t ra = tile_rsrc(g.A, (g.e.M - 1) * lda_b + kbytes);
    const __amdgpu_buffer_rsrc_t rb =
        tile_rsrc((const uint8_t *)g.B + n_blk * ldb_b, (g.e.N - n_blk - 1) * ldb_b + kbytes_b);
    const int row = lane & 15, grp = lane >> 4;
    const int va = row * (int)lda_b + grp * LB;
    const int vb0 = row * (int)ldb_b + grp * (W4 ? LB / 4 : LB), vb1 = vb0 + 16 * (int)ldb_b;
    // W4A16 group scales / zero points of the block's 32 columns
    const int64_t wgr = W4 ? g.K / g.wgs : 0;
    const __amdgpu_buffer_rsrc_t rws =
        tile_rsrc((const uint8_t *)g.ws + n_blk * wgr * 2, W4 ? (g.e.N - n_blk) * wgr * 2 : 0);
    const __amdgpu_buffer_rsrc_t rwz = tile_rsrc(g.wz ? g.wz + n_blk * wgr : (const uint8_t *)g.B,
                                                 W4 && g.wz ? (g.e.N - n_blk) * wgr : 0);
    const bool has_wz = g.wz != nullptr;

    u4_t pa[2][NLD], pb[2][2][W4 ? 1 : NLD];
    // B chunk loaded 1 KB per instruction: load k, lane l holds row 4 k + l / 16,
    // bytes 16 (l % 16) of the chunk
    u4_t pc[2][W4 ? 1 : 8];
    const int vc0 = (lane >> 4) * (int)ldb_b + 16 * (lane & 15);
    uint8_t *bwave = bst + (W4 ? 0 : wave * 32 * 256);
    auto bslot = [](int r, int q) STG_AI { return r * 256 + ((q ^ (r & 15)) << 4); };
    uint32_t wsb[2][2], wzb[2][2];
    auto load = [&](auto set, int c) STG_AI {
        constexpr int S = decltype(set)::value;
        const int soff = c * CB;
#pragma unroll
        for (int j = 0; j < NLD; ++j)
            pa[S][j] = buf_load16(ra, va + 16 * j, soff);
        if constexpr (W4) {
            // K chunk c covers K (CB/2) c ..; this lane's 32 K sit in one group
            const int kg = (int)(((int64_t)c * (CB / 2) + 32 * grp) / g.wgs);
            pb[S][0][0] = buf_load16(rb, vb0, c * (CB / 4));
            pb[S][1][0] = buf_load16(rb, vb1, c * (CB / 4));
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                const int o = (16 * f + row) * (int)wgr + kg;
                wsb[S][f] = __builtin_amdgcn_raw_buffer_load_b16(rws, 2 * o, 0, 0);
                wzb[S][f] = __builtin_amdgcn_raw_buffer_load_b8(rwz, o, 0, 0);
            }
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k)
                pc[S][k] = buf_load16(rb, vc0 + 4 * k * (int)ldb_b, soff);
        }
    };
    typename OP::acc_t acc[2] = {typename OP::acc_t{}, typename OP::acc_t{}};
    auto compute = [&](auto set) STG_AI {
        constexpr int S = decltype(set)::value;
        const uint32_t *a = (const uint32_t *)pa[S];
        if constexpr (W4) {
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                // 32 codes -> the 64 bytes the 16-bit path would have loaded
                u4_t bq[NLD];
                const float sc = w4_scale<BF>(wsb[S][f]);
                const int z = has_wz ? (int)wzb[S][f] : 8;
#pragma unroll
                for (int j = 0; j < NLD; ++j)
                    w4_dequant8<BF>(pb[S][f][0][j], z, sc, (uint32_t *)&bq[j]);
#pragma unroll
                for (int st = 0; st < STEPS; ++st)
                    acc[f] = OP::mma(a + st * FW, (const uint32_t *)bq + st * FW, acc[f]);
            }
        } else {
            // the chunk through this wave's LDS buffer into the fragment layout
            uint8_t *buf = bwave;
#pragma unroll
            for (int k = 0; k < 8; ++k)
                *(u4_t *)(buf + bslot(4 * k + (lane >> 4), lane & 15)) = pc[S][k];
            wave_lds_sync();
#pragma unroll
            for (int f = 0; f < 2; ++f)
#pragma unroll
                for (int j = 0; j < NLD; ++j)
                    pb[S][f][j] = *(const u4_t *)(buf + bslot(16 * f + row, 4 * grp + j));
#pragma unroll
            for (int st = 0; st < STEPS; ++st)
#pragma unroll
                for (int f = 0; f < 2; ++f)
                    acc[f] = OP::mma(a + st * FW, (const uint32_t *)pb[S][f] + st * FW, acc[f]);
        }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    int c = wave;
    if (c < NC)
        load(I0{}, c);
    for (; c < NC; c += 2 * WAVES) {
        if (c + WAVES < NC)
            load(I1{}, c + WAVES);
        compute(I0{});
        if (c + WAVES >= NC)
            break;
        if (c + 2 * WAVES < NC)
            load(I0{}, c + 2 * WAVES);
        compute(I1{});
    }

    // reduce the waves' partial sums, then one wave stores 16 x 32
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const auto x = acc[f][i];
            red[wave][f][lane][i] = __builtin_bit_cast(uint32_t, x);
        }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            typename OP::acc_t t = acc[f];
#pragma unroll
            for (int w = 1; w < WAVES; ++w)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t u = red[w][f][lane][i];
                    if constexpr (OP::INT)
                        t[i] = (int)((uint32_t)t[i] + u);
                    else
                        t[i] += __builtin_bit_cast(float, u);
                }
            const int64_t col = n_blk + 16 * f + (lane & 15);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t r = 4 * (lane >> 4) + i;
                if (r < g.e.M && col < g.e.N)
                    epilogue_store_any(g.e, r, col, t[i]);
            }
        }
    }
}

// ---------------------------------------------------------------- launch

template <class OP>
static hipError_t launch_generic_t(const GemmArgs &g, hipStream_t s)
{
    dim3 grid((unsigned)((g.e.N + 63) / 64), (unsigned)((g.e.M + 63) / 64));
    hipLaunchKernelGGL(k_generic<OP>, grid, dim3(256), 0, s, g);
    return hipGetLastError();
}

typedef hipError_t (*dense_launch_fn)(const GemmArgs &, hipStream_t);

static dense_launch_fn generic_table(int op)
{
    switch (op) {
    case OPK_F16: return launch_generic_t<OpF16>;
    case OPK_BF16: return launch_generic_t<OpBF16>;
    case OPK_F8_E4E4: return launch_generic_t<OpF8<0, 0>>;
    case OPK_F8_E4E5: return launch_generic_t<OpF8<0, 1>>;
    case OPK_F8_E5E4: return launch_generic_t<OpF8<1, 0>>;
    case OPK_F8_E5E5: return launch_generic_t<OpF8<1, 1>>;
    case OPK_S8: return launch_generic_t<OpS8>;
    case OPK_U8S8: return launch_generic_t<OpI8<true, false>>;
    case OPK_S8U8: return launch_generic_t<OpI8<false, true>>;
    case OPK_U8U8: return launch_generic_t<OpI8<true, true>>;
    default: return nullptr;
    }
}

template <int BM, int BN, int GM = 2, int GN = 2, int WPC = 1>
static dense_launch_fn tiled_table_t(int op)
{
    switch (op) {
    case OPK_F16: return launch_tiled_t<OpF16, BM, BN, GM, GN, WPC>;
    case OPK_BF16: return launch_tiled_t<OpBF16, BM, BN, GM, GN, WPC>;
    case OPK_F8_E4E4: return launch_tiled_t<OpF8<0, 0>, BM, BN, GM, GN, WPC>;
    case OPK_F8_E4E5: return launch_tiled_t<OpF8<0, 1>, BM, BN, GM, GN, WPC>;
    case OPK_F8_E5E4: return launch_tiled_t<OpF8<1, 0>, BM, BN, GM, GN, WPC>;
    case OPK_F8_E5E5: return launch_tiled_t<OpF8<1, 1>, BM, BN, GM, GN, WPC>;
    case OPK_S8: return launch_tiled_t<OpS8, BM, BN, GM, GN, WPC>;
    default: break;
    }
    // unsigned 8-bit operands: on the tiles the plan uses for int8 (the
    // 128 x 128 tile and the 8-wave 64 x 128-per-wave 256 x 256 one)
    if constexpr (BM == 128 || GM == 4) {
        switch (op) {
        case OPK_U8S8: return launch_tiled_t<OpI8<true, false>, BM, BN, GM, GN, WPC>;
        case OPK_S8U8: return launch_tiled_t<OpI8<false, true>, BM, BN, GM, GN, WPC>;
        case OPK_U8U8: return launch_tiled_t<OpI8<true, true>, BM, BN, GM, GN, WPC>;
        default: break;
        }
    }
    return nullptr;
}

template <class OP>
static hipError_t launch_skinny_t(const GemmArgs &g, hipStream_t s)
{
    const unsigned blocks = (unsigned)((g.e.N + 31) / 32);
    hipLaunchKernelGGL(k_skinny<OP>, dim3(blocks), dim3(512), 0, s, g);
    return hipGetLastError();
}

static dense_launch_fn skinny_table(int op)
{
    switch (op) {
    case OPK_F16: return launch_skinny_t<Op16F16>;
    case OPK_BF16: return launch_skinny_t<Op16BF16>;
    case OPK_F8_E4E4: return launch_skinny_t<Op16F8<0, 0>>;
    case OPK_F8_E4E5: return launch_skinny_t<Op16F8<0, 1>>;
    case OPK_F8_E5E4: return launch_skinny_t<Op16F8<1, 0>>;
    case OPK_F8_E5E5: return launch_skinny_t<Op16F8<1, 1>>;
    case OPK_S8: return launch_skinny_t<Op16S8>;
    default: return nullptr;
    }
}

// MX block-scaled pairs of one width on the 4-wave 256x256 tile (the fp8
// choice); afmt / bfmt are the OpMX selectors.
template <class OP>
static hipError_t launch_mx_tiled_t(const GemmArgs &g, hipStream_t s)
{
    const int tiles_m = (int)((g.e.M + 255) / 256), tiles_n = (int)((g.e.N + 255) / 256);
    hipLaunchKernelGGL((k_tiled<OP, 256, 256>), dim3((unsigned)(tiles_m * tiles_n)), dim3(256), 0,
                       s, g, tiles_m, tiles_n);
    return hipGetLastError();
}

// W4A16 with M <= 16 on the skinny kernel.
hipError_t launch_w4_skinny(int op, const GemmArgs &g, hipStream_t s)
{
    const unsigned blocks = (unsigned)((g.e.N + 31) / 32);
    if (op == OPK_F16)
        hipLaunchKernelGGL(k_skinny<OpW4<Op16F16>>, dim3(blocks), dim3(512), 0, s, g);
    else if (op == OPK_BF16)
        hipLaunchKernelGGL(k_skinny<OpW4<Op16BF16>>, dim3(blocks), dim3(512), 0, s, g);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

// W4A16 on the 4-wave 256x256 tile (one B column per thread).
hipError_t launch_w4_tiled(int op, const GemmArgs &g, hipStream_t s)
{
    const int tiles_m = (int)((g.e.M + 255) / 256), tiles_n = (int)((g.e.N + 255) / 256);
    if (op == OPK_F16)
        hipLaunchKernelGGL((k_tiled<OpW4<OpF16>, 256, 256>), dim3((unsigned)(tiles_m * tiles_n)),
                           dim3(256), 0, s, g, tiles_m, tiles_n);
    else if (op == OPK_BF16)
        hipLaunchKernelGGL((k_tiled<OpW4<OpBF16>, 256, 256>), dim3((unsigned)(tiles_m * tiles_n)),
                           dim3(256), 0, s, g, tiles_m, tiles_n);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_mx_tiled(int afmt, int bfmt, const GemmArgs &g, hipStream_t s)
{
    switch (afmt * 8 + bfmt) {
    case 0 * 8 + 0: return launch_mx_tiled_t<OpMX<0, 0>>(g, s);
    case 0 * 8 + 1: return launch_mx_tiled_t<OpMX<0, 1>>(g, s);
    case 1 * 8 + 0: return launch_mx_tiled_t<OpMX<1, 0>>(g, s);
    case 1 * 8 + 1: return launch_mx_tiled_t<OpMX<1, 1>>(g, s);
    case 4 * 8 + 4: return launch_mx_tiled_t<OpMX<4, 4>>(g, s);
    default: return hipErrorInvalidValue;
    }
}

// Both operands 6-bit (E2M3 / E3M2), stored in OpMX's padded layout.
hipError_t launch_mx_tiled_pad6(int afmt, int bfmt, const GemmArgs &g, hipStream_t s)
{
    switch (afmt * 8 + bfmt) {
    case 2 * 8 + 2: return launch_mx_tiled_t<OpMX<2, 2, true>>(g, s);
    case 2 * 8 + 3: return launch_mx_tiled_t<OpMX<2, 3, true>>(g, s);
    case 3 * 8 + 2: return launch_mx_tiled_t<OpMX<3, 2, true>>(g, s);
    case 3 * 8 + 3: return launch_mx_tiled_t<OpMX<3, 3, true>>(g, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_dense(int family, int op, int layout, const GemmArgs &g, hipStream_t s)
{
    dense_launch_fn fn = nullptr;
    if (layout != 0 && family != KF_GENERIC)
        return launch_dense_mn(family, op, layout, g, s);
    switch (family) {
    case KF_GENERIC: fn = generic_table(op); break;
    case KF_TILED_256: fn = tiled_table_t<256, 256>(op); break;
    case KF_TILED_128: fn = tiled_table_t<128, 128>(op); break;
    case KF_SKINNY: fn = skinny_table(op); break;
    case KF_TILED_256W8: fn = tiled_table_t<256, 256, 2, 4>(op); break;
    case KF_TILED_256W8K16: return launch_tiled16(op, g, s);
    case KF_TILED_256W8TK16: return launch_tiled16t(op, g, s);
    case KF_TILED_256W8T: fn = tiled_table_t<256, 256, 4, 2>(op); break;
    default: break;
    }
    if (!fn)
        return hipErrorInvalidValue;
    return fn(g, s);
}

} // namespace stg
