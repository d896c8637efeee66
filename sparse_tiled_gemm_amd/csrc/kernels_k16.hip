// The 256 x 256 LDS-tiled GEMM for 16-bit and int8 inputs on the 16x16 MFMA
// forms (16x16x32 f16 / bf16, 16x16x64 i8)
// ("Tensor Core 三种调用层次…", section 3: a workgroup tile staged through
// shared memory, each warp's sub-tile accumulated from fragments; here eight
// 64-lane waves, 128 x 64 each).
//
// The 16x16 forms do the work of the 32x32 ones in the same number of MFMA
// passes but, under this chip's power limit, sustain a higher clock
// (MFMA-only loops: 2015 vs 1771 TFLOP/s for bf16, 4118 vs 3488 TOP/s for
// int8).  Their fragments cover twice the K per instruction, so
// double-buffering every fragment as the 32x32 kernel does would need 96
// registers beside the 128 accumulators; instead each K tile (64 bytes of K
// = one instruction step) runs row block by row block, and A fragment i of
// the next tile is read as soon as row block i's four MFMAs have been issued
// (one A buffer), while the four B fragments are double-buffered.
//
// Fragment layout (16 bytes per lane): lane l holds row (A) or column (B)
// l % 16; lane group l / 16 takes 16-byte chunk l / 16 of the tile's 64-byte
// row, the same K for A and B.  Accumulator register r of lane l is row
// 4 (l / 16) + r, column l % 16 of its 16 x 16 block.
//
// Global -> LDS staging, the LDS layout (64-byte rows of 16-byte chunks),
// the three-stage ring and the epilogue are those of k_tiled
// (tiled_kernel.hpp), except the chunk slot: c ^ swz16(r).
//
// W4A16 (OpW4<Op16F16 / Op16BF16>): B holds 4-bit weight codes (16 bytes per
// column per 32-K tile); threads 2c and 2c + 1 load 8 code bytes each of
// column c with the group's scale and zero point and write the 16 values,
// dequantised as in k_tiled (w4_dequant8), as chunks 2h and 2h + 1 of the
// column's row of the B tile.
#include "device_common.hpp"
#include "internal.hpp"

namespace stg {

// 16-byte chunk slot within a 64-byte LDS row for the 16x16 fragment reads
// (16 consecutive rows per lane group, the four lane groups on the four
// chunks): chunk c of row r at slot c ^ swz16(r).  Chosen by measurement on
// gfx950 (LDS bank-conflict counter on a probe replaying this read
// pattern): k_tiled's swz64, (r >> 2) & 3, is 2-way conflicted here (half
// the LDS cycles), r & 3 and several rotations too; (r >> 1) & 3 is
// conflict-free.  swz16(r + 16 i) == swz16(r).
__device__ STG_AI inline int swz16(int r) { return (r >> 1) & 3; }

// GM x GN waves (2 x 4: 128 x 64 each, A fragments roll; 4 x 2: 64 x 128
// each, B fragments roll and A is double-buffered).  OP: a 16x16 form (16
// bytes of K per lane: one 16-byte read per fragment) or the 32x32x64 fp8
// form OpF8 (32x32 blocks, 32 bytes per lane: two reads, chunks 2 h and
// 2 h + 1 of the row for lane half h -- a K order the MFMA reads as its own
// permutation of the tile's 64 K, the same for A and B, so the sum is
// unchanged -- with k_tiled's slot function swz64, conflict-free for
// 32-row reads).
template <class OP, int GM, int GN>
__global__ __launch_bounds__(512, 1) void k_tiled16(GemmArgs g, int tiles_m, int tiles_n)
{
    constexpr bool M16 = sizeof(typename OP::acc_t) == 16; // 16x16 form
    constexpr int FB = M16 ? 16 : 32;                      // rows / columns per fragment
    constexpr int NRD = OP::LANE_BYTES / 16;               // 16-byte reads per fragment
    static_assert((M16 && NRD == 1) || (!M16 && NRD == 2), "one 64-byte K tile per instruction");
    static_assert(GM * GN == 8, "eight waves");
    constexpr int NT = 512, BM = 256, BN = 256;
    constexpr int BKB = 64, CH = BKB / 16, RPP = NT / CH; // 128 rows per load pass
    constexpr int A_LD = BM / RPP, B_LD = BN / RPP;
    constexpr int WM = BM / GM, WN = BN / GN;   // 128 x 64 per wave
    constexpr int FI = WM / FB, FJ = WN / FB;   // fragments (8 x 4 for 16x16, 2 x 4 ...)
    auto swz = [](int r) STG_AI { return M16 ? swz16(r) : swz64(r); };
    constexpr int NSTAGE = 3;
    constexpr int A_TILE = BM * BKB, STAGE = (BM + BN) * BKB;
    constexpr int EPI = GM * GN * 32 * (WN + 4) * 4;
    constexpr int KLOOP = NSTAGE * STAGE;
    constexpr int LDS_BYTES = KLOOP > EPI ? KLOOP : EPI;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int64_t m_blk = (int64_t)tm * BM, n_blk = (int64_t)tn * BN;
    constexpr bool W4 = OP::W4;
    static_assert(!W4 || M16, "W4A16 on the 16x16 forms");
    constexpr bool BF = std::is_base_of<Op16BF16, OP>::value;
    const int64_t lda_b = g.a_rs * OP::ELEM, ldb_b = W4 ? g.b_cs / 2 : g.b_cs * OP::ELEM;
    const int64_t kbytes = g.K * OP::ELEM, kbytes_b = W4 ? g.K / 2 : kbytes;
    const int KT = (int)(kbytes / BKB);
    // bounded by the last byte of the last row: loads past it return zero
    const __amdgpu_buffer_rsrc_t ra =
        tile_rsrc((const uint8_t *)g.A + m_blk * lda_b, (g.e.M - m_blk - 1) * lda_b + kbytes);
    const __amdgpu_buffer_rsrc_t rb =
        tile_rsrc((const uint8_t *)g.B + n_blk * ldb_b, (g.e.N - n_blk - 1) * ldb_b + kbytes_b);
    // W4A16 group scales and zero points of the tile's columns (zero points
    // absent: a zero-length resource, whose loads return 0, and z = 8)
    const int64_t wgr = W4 ? g.K / g.wgs : 0; // groups per column
    const __amdgpu_buffer_rsrc_t rws =
        tile_rsrc((const uint8_t *)g.ws + n_blk * wgr * 2, W4 ? (g.e.N - n_blk) * wgr * 2 : 0);
    const __amdgpu_buffer_rsrc_t rwz = tile_rsrc(g.wz ? g.wz + n_blk * wgr : (const uint8_t *)g.B,
                                                 W4 && g.wz ? (g.e.N - n_blk) * wgr : 0);
    const bool has_wz = g.wz != nullptr;
    const int wcol = tid >> 1, whalf = tid & 1; // W4A16: column and half of the codes

    // global -> LDS copy: thread owns chunk `ch` of rows r0 + i RPP
    const int ch = tid % CH, r0 = tid / CH;
    const int va0 = r0 * (int)lda_b + ch * 16, vb0 = r0 * (int)ldb_b + ch * 16;
    const int va_step = RPP * (int)lda_b, vb_step = RPP * (int)ldb_b;
    const int l0 = r0 * BKB + ((ch ^ swz(r0)) << 4); // + i RPP BKB (swz is RPP-periodic)
    u4_t ga[2][A_LD], gb[2][W4 ? 1 : B_LD];
    uint32_t gw[2][2], wsb[2], wzb[2]; // W4A16: 8 code bytes, scale bits, zero point
    auto gload = [&](auto set, int kt) STG_AI {
        constexpr int S = decltype(set)::value;
        const int soff = kt * BKB;
#pragma unroll
        for (int i = 0; i < A_LD; ++i)
            ga[S][i] = buf_load16(ra, va0 + i * va_step, soff);
        if constexpr (W4) {
            typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
            const u2_t c = __builtin_bit_cast(
                u2_t, __builtin_amdgcn_raw_buffer_load_b64(rb, wcol * (int)ldb_b + 8 * whalf,
                                                           kt * (BKB / 4), 0));
            gw[S][0] = c.x;
            gw[S][1] = c.y;
            const int grp = (int)((int64_t)kt * (BKB / 2) / g.wgs);
            wsb[S] = __builtin_amdgcn_raw_buffer_load_b16(rws, (wcol * (int)wgr + grp) * 2, 0, 0);
            wzb[S] = __builtin_amdgcn_raw_buffer_load_b8(rwz, wcol * (int)wgr + grp, 0, 0);
        } else {
#pragma unroll
            for (int i = 0; i < B_LD; ++i)
                gb[S][i] = buf_load16(rb, vb0 + i * vb_step, soff);
        }
    };
    auto lstore = [&](auto set, uint8_t *__restrict__ stage_base) STG_AI {
        constexpr int S = decltype(set)::value;
#pragma unroll
        for (int i = 0; i < A_LD; ++i)
            *(u4_t *)(stage_base + l0 + i * RPP * BKB) = ga[S][i];
        if constexpr (W4) {
            const float sc = w4_scale<BF>(wsb[S]);
            const int z = has_wz ? (int)wzb[S] : 8;
            uint8_t *brow = stage_base + A_TILE + wcol * BKB;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                u4_t v;
                w4_dequant8<BF>(gw[S][q], z, sc, (uint32_t *)&v);
                *(u4_t *)(brow + (((2 * whalf + q) ^ swz16(wcol)) << 4)) = v;
            }
        } else {
#pragma unroll
            for (int i = 0; i < B_LD; ++i)
                *(u4_t *)(stage_base + A_TILE + l0 + i * RPP * BKB) = gb[S][i];
        }
    };

    // fragments: A block i is rows wm WM + FB i + l % FB, B block j rows
    // wn WN + FB j + l % FB of the B tile; chunks l / 16 (16x16) or
    // 2 (l / 32) + q, q < 2 (32x32)
    const int wm = wave / GN, wn = wave % GN;
    const int arow = wm * WM + (lane & (FB - 1)), brow = wn * WN + (lane & (FB - 1));
    const int grp = M16 ? lane >> 4 : 2 * (lane >> 5);
    int a_off[NRD], b_off[NRD];
#pragma unroll
    for (int q = 0; q < NRD; ++q) {
        a_off[q] = arow * BKB + (((grp + q) ^ swz(arow)) << 4);
        b_off[q] = A_TILE + brow * BKB + (((grp + q) ^ swz(brow)) << 4);
    }
    // the operand with more fragments rolls (one buffer), the other is
    // double-buffered; FR / FD fragments, R = rolling, D = double
    constexpr bool ROLLB = FJ > FI;
    constexpr int FR = ROLLB ? FJ : FI, FD = ROLLB ? FI : FJ;
    u4_t fr[FR][NRD], fd[2][FD][NRD];
    auto read_r = [&](const uint8_t *stage_base, int i) STG_AI {
#pragma unroll
        for (int q = 0; q < NRD; ++q)
            fr[i][q] = *(const u4_t *)(stage_base + (ROLLB ? b_off[q] : a_off[q]) + i * FB * BKB);
    };
    auto read_d = [&](auto set, const uint8_t *stage_base, int j) STG_AI {
        constexpr int S = decltype(set)::value;
#pragma unroll
        for (int q = 0; q < NRD; ++q)
            fd[S][j][q] = *(const u4_t *)(stage_base + (ROLLB ? a_off[q] : b_off[q]) + j * FB * BKB);
    };

    typename OP::acc_t acc[FI][FJ];
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j)
            acc[i][j] = typename OP::acc_t{};

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;

    // prologue: tiles 0 and 1 in stages 0 and 1, tile 2 in register set 0,
    // tile 0's fragments in registers (the last A fragment is read at the
    // start of each tile)
    gload(I0{}, 0);
    gload(I1{}, 1);
    lstore(I0{}, lds);
    lstore(I1{}, lds + STAGE);
    gload(I0{}, 2);
    __syncthreads();
#pragma unroll
    for (int i = 0; i + 1 < FR; ++i)
        read_r(lds, i);
#pragma unroll
    for (int j = 0; j < FD; ++j)
        read_d(I0{}, lds, j);

    // One K tile t (parity P): tile t+3 into register set P^1; rolling
    // fragment FR-1 of tile t; block i of the rolling operand times the FD
    // double-buffered fragments, then rolling fragment i of tile t+1 (i <
    // FR-1; the double-buffered fragments of tile t+1 with the first FD
    // blocks); register set P (tile t+2) into its stage.  The last rolling
    // fragment of a tile is read at the tile's start rather than after the
    // previous tile's last MFMAs, so no fragment read is still in flight at
    // the barrier.  Instruction order (MFMA q of the tile's FR x FD, block
    // q / FD): the current tile's last rolling fragment after MFMA 0, the
    // next tile's rolling fragment b after block b's last MFMA (b < FR-1, so
    // the last one still has a block of MFMAs to complete under), its
    // double-buffered fragments after MFMAs 1, 5, 9, 13; global loads at
    // MFMAs 0, 8, 16, 24 and LDS stores at 4, 12, 20, 28.
    constexpr int NM = FI * FJ, NL = A_LD + (W4 ? 3 : B_LD), NW = A_LD + B_LD;
    auto nread = [](int q) constexpr {
        return (q == 0 ? 1 : 0) + (q % FD == FD - 1 && q / FD < FR - 1 ? 1 : 0) +
               (q % FD == 1 && q / FD < FD ? 1 : 0);
    };
    static_assert(
        [&]() constexpr {
            int n = 0;
            for (int q = 0; q < NM; ++q)
                n += nread(q);
            return n;
        }() == FR + FD,
        "every fragment read has a slot");
    auto schedule = [&]() STG_AI {
        [&]<int... Q>(std::integer_sequence<int, Q...>) STG_AI {
            (
                [&]() STG_AI {
                    constexpr int nr = nread(Q) * NRD;
                    constexpr int nl = spread((Q + NM / NL - 1) % NM, NL, NM);
                    constexpr int nw = spread(((Q + NM / NW - 5) % NM + NM) % NM, NW, NM);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); // MFMA
                    if constexpr (nr > 0)
                        __builtin_amdgcn_sched_group_barrier(0x100, nr, 0); // DS read
                    if constexpr (nl > 0)
                        __builtin_amdgcn_sched_group_barrier(0x020, nl, 0); // VMEM read
                    if constexpr (nw > 0)
                        __builtin_amdgcn_sched_group_barrier(0x200, nw, 0); // DS write
                }(),
                ...);
        }(std::make_integer_sequence<int, NM>{});
    };

    int st = 0; // LDS stage of tile t
    auto iter = [&](auto par, int t) STG_AI {
        constexpr int P = decltype(par)::value;
        const int st1 = st == NSTAGE - 1 ? 0 : st + 1;
        const int st2 = st1 == NSTAGE - 1 ? 0 : st1 + 1;
        auto body = [&](const uint8_t *__restrict__ cur, const uint8_t *__restrict__ nxt,
                        uint8_t *__restrict__ wr) STG_AI {
            gload(std::integral_constant<int, P ^ 1>{}, t + 3);
            read_r(cur, FR - 1);
#pragma unroll
            for (int i = 0; i < FR; ++i) {
#pragma unroll
                for (int j = 0; j < FD; ++j) {
                    if constexpr (ROLLB)
                        acc[j][i] = OP::mma((const uint32_t *)&fd[P][j], (const uint32_t *)&fr[i],
                                            acc[j][i]);
                    else
                        acc[i][j] = OP::mma((const uint32_t *)&fr[i], (const uint32_t *)&fd[P][j],
                                            acc[i][j]);
                }
                if (i + 1 < FR)
                    read_r(nxt, i);
                if (i < FD)
                    read_d(std::integral_constant<int, P ^ 1>{}, nxt, i);
            }
            lstore(std::integral_constant<int, P>{}, wr);
            schedule();
        };
        body(lds + st * STAGE, lds + st1 * STAGE, lds + st2 * STAGE);
        __syncthreads();
        st = st1;
    };

    int t = 0;
    for (; t + 1 < KT; t += 2) {
        iter(I0{}, t);
        iter(I1{}, t + 1);
    }
    if (t < KT)
        iter(I0{}, t);

    __syncthreads(); // every wave is done with the LDS stages
    epilogue_grid_lds<OP, FI, FJ>(g.e, acc, m_blk + wm * WM, n_blk + wn * WN, lane,
                                  (uint32_t *)lds + wave * 32 * (WN + 4));
}

template <int GM, int GN>
static hipError_t launch_t16(int op, const GemmArgs &g, hipStream_t s)
{
    const int tiles_m = (int)((g.e.M + 255) / 256), tiles_n = (int)((g.e.N + 255) / 256);
    const dim3 grid((unsigned)(tiles_m * tiles_n));
    if (op == OPK_F16)
        hipLaunchKernelGGL((k_tiled16<Op16F16, GM, GN>), grid, dim3(512), 0, s, g, tiles_m, tiles_n);
    else if (op == OPK_BF16)
        hipLaunchKernelGGL((k_tiled16<Op16BF16, GM, GN>), grid, dim3(512), 0, s, g, tiles_m,
                           tiles_n);
    else if (op == OPK_S8)
        hipLaunchKernelGGL((k_tiled16<Op16S8, GM, GN>), grid, dim3(512), 0, s, g, tiles_m, tiles_n);
    else if (op == OPK_F8_E4E4)
        hipLaunchKernelGGL((k_tiled16<OpF8<0, 0>, GM, GN>), grid, dim3(512), 0, s, g, tiles_m, tiles_n);
    else if (op == OPK_F8_E4E5)
        hipLaunchKernelGGL((k_tiled16<OpF8<0, 1>, GM, GN>), grid, dim3(512), 0, s, g, tiles_m, tiles_n);
    else if (op == OPK_F8_E5E4)
        hipLaunchKernelGGL((k_tiled16<OpF8<1, 0>, GM, GN>), grid, dim3(512), 0, s, g, tiles_m, tiles_n);
    else if (op == OPK_F8_E5E5)
        hipLaunchKernelGGL((k_tiled16<OpF8<1, 1>, GM, GN>), grid, dim3(512), 0, s, g, tiles_m, tiles_n);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_tiled16(int op, const GemmArgs &g, hipStream_t s)
{
    return launch_t16<2, 4>(op, g, s);
}
hipError_t launch_tiled16t(int op, const GemmArgs &g, hipStream_t s)
{
    return launch_t16<4, 2>(op, g, s);
}

// W4A16 on the 2 x 4 arrangement (op: the activations' type)
hipError_t launch_w4_tiled16(int op, const GemmArgs &g, hipStream_t s)
{
    const int tiles_m = (int)((g.e.M + 255) / 256), tiles_n = (int)((g.e.N + 255) / 256);
    const dim3 grid((unsigned)(tiles_m * tiles_n));
    if (op == OPK_F16)
        hipLaunchKernelGGL((k_tiled16<OpW4<Op16F16>, 2, 4>), grid, dim3(512), 0, s, g, tiles_m,
                           tiles_n);
    else if (op == OPK_BF16)
        hipLaunchKernelGGL((k_tiled16<OpW4<Op16BF16>, 2, 4>), grid, dim3(512), 0, s, g, tiles_m,
                           tiles_n);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

} // namespace stg
