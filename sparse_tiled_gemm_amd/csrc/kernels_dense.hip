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
    typename OP::acc_t acc = {};
    for (int64_t k0 = 0; k0 < g.K; k0 += KI) {
        uint32_t a[OP::LANE_BYTES / 4], b[OP::LANE_BYTES / 4];
        const int64_t kb = k0 + (lane >> 5) * LE;
        load_frag_strided<OP::ELEM, LE>(a, g.A, a_ok, am * g.a_rs, g.a_cs, kb, g.K);
        load_frag_strided<OP::ELEM, LE>(b, g.B, b_ok, bn * g.b_cs, g.b_rs, kb, g.K);
        acc = OP::mma(a, b, acc);
    }
    typename OP::acc_t grid[1][1] = {{acc}};
    epilogue_grid<OP, 1, 1>(g.e, grid, m0, n0, lane);
}

// ---------------------------------------------------------------- tiled, LDS DMA

// Same tile structure as k_tiled, but global -> LDS copies are direct
// (buffer_load ... lds): no staging registers and no LDS store instructions,
// so NSTAGE LDS stages can be in flight.  Tile t+NSTAGE-1 is requested while
// tile t is multiplied; before the barrier that ends tile t the wave waits for
// its copies of tile t+2 (vmcnt counts the newer requests still in flight),
// so the MFMA fragments of tile t+1 can be read during tile t's last K step.
// Each wave instruction fills 1 KB of LDS = 16 rows of 64 bytes; lane l
// writes slot l % 4 of row l / 4 and therefore fetches the chunk that the
// swizzle maps to that slot.
template <class OP, int BM, int BN, int NSTAGE>
__global__ __launch_bounds__(256, 1) void k_tiled_dma(GemmArgs g, int tiles_m, int tiles_n)
{
    constexpr int BKB = 64, CH = 4;
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int FM = WM / 32, FN = WN / 32;
    constexpr int STAGE = (BM + BN) * BKB;
    constexpr int NV = OP::LANE_BYTES / 16;
    constexpr int FW = OP::LANE_BYTES / 4;
    constexpr int KS = BKB / OP::KB;
    constexpr int ROWS_PER_INST = 1024 / BKB;          // 16
    constexpr int A_INST = BM / ROWS_PER_INST / 4;     // per wave
    constexpr int B_INST = BN / ROWS_PER_INST / 4;
    constexpr int NI = A_INST + B_INST;                // DMA instructions per wave per tile
    static_assert(NSTAGE >= 4, "the fragment prefetch needs tile t+1 two tiles early");
    static_assert(4 * 32 * (WN + 4) * 4 <= NSTAGE * STAGE, "epilogue staging fits in LDS");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[NSTAGE * STAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int64_t m_blk = (int64_t)tm * BM, n_blk = (int64_t)tn * BN;
    const int64_t lda_b = g.a_rs * OP::ELEM, ldb_b = g.b_cs * OP::ELEM;
    const int64_t kbytes = g.K * OP::ELEM;
    const int KT = (int)(kbytes / BKB);
    const __amdgpu_buffer_rsrc_t ra = tile_rsrc((const uint8_t *)g.A + m_blk * lda_b,
                                                (g.e.M - m_blk - 1) * lda_b + kbytes);
    const __amdgpu_buffer_rsrc_t rb = tile_rsrc((const uint8_t *)g.B + n_blk * ldb_b,
                                                (g.e.N - n_blk - 1) * ldb_b + kbytes);

    // this lane's source offsets for each of the wave's DMA instructions
    int voff[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const bool is_a = i < A_INST;
        const int blk = is_a ? wave * A_INST + i : wave * B_INST + (i - A_INST);
        const int row = blk * ROWS_PER_INST + (lane >> 2);
        const int c = (lane & 3) ^ swz64(row);
        voff[i] = row * (int)(is_a ? lda_b : ldb_b) + c * 16;
    }
    auto dma_tile = [&](int stage, int kt) STG_AI {
        uint8_t *base = lds + stage * STAGE;
        const int soff = kt * BKB;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const bool is_a = i < A_INST;
            const int blk = is_a ? wave * A_INST + i : BM / ROWS_PER_INST + wave * B_INST + (i - A_INST);
            dma16(is_a ? ra : rb, base + blk * 1024, voff[i], soff);
        }
    };

    const int wm = wave >> 1, wn = wave & 1;
    const int arow = wm * WM + (lane & 31), brow = wn * WN + (lane & 31);
    const int half = lane >> 5;
    const int sa = swz64(arow), sb = swz64(brow);
    const int a_off = arow * BKB, b_off = BM * BKB + brow * BKB;

    uint32_t fa[2][FM][FW], fb[2][FN][FW];
    auto lread = [&](auto set, int stage, int s) STG_AI {
        constexpr int S = decltype(set)::value;
        const uint8_t *lsa = lds + stage * STAGE + a_off;
        const uint8_t *lsb = lds + stage * STAGE + b_off;
        const int c0 = (s * OP::KB + half * OP::LANE_BYTES) >> 4;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int oa = ((c0 + v) ^ sa) << 4, ob = ((c0 + v) ^ sb) << 4;
#pragma unroll
            for (int i = 0; i < FM; ++i)
                *(u4_t *)&fa[S][i][4 * v] = *(const u4_t *)(lsa + i * 32 * BKB + oa);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                *(u4_t *)&fb[S][j][4 * v] = *(const u4_t *)(lsb + j * 32 * BKB + ob);
        }
    };

    typename OP::acc_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = typename OP::acc_t{};
    auto mma = [&](auto set) STG_AI {
        constexpr int S = decltype(set)::value;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = OP::mma(fa[S][i], fb[S][j], acc[i][j]);
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;

    // prologue: request tiles 0 .. NSTAGE-2; tiles 0 and 1 complete
#pragma unroll
    for (int p = 0; p < NSTAGE - 1; ++p)
        dma_tile(p, p);
    STG_WAIT_VMCNT((NSTAGE - 3) * NI);
    lds_barrier();
    lread(I0{}, 0, 0);

    // fragment reads spread over each step's MFMAs, DMA requests spread over
    // the whole tile (see k_tiled)
    constexpr int NM = FM * FN, NR = (FM + FN) * NV;
    constexpr int NMT = KS * NM;
    auto schedule = [&]() STG_AI {
        [&]<int... Q>(std::integer_sequence<int, Q...>) STG_AI {
            (
                [&]() STG_AI {
                    constexpr int m = Q % NM;
                    constexpr int nr = spread(m, NR, NM), nl = spread(Q, NI, NMT);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); // MFMA
                    if constexpr (nr > 0)
                        __builtin_amdgcn_sched_group_barrier(0x100, nr, 0); // DS read
                    if constexpr (nl > 0)
                        __builtin_amdgcn_sched_group_barrier(0x020, nl, 0); // VMEM read
                }(),
                ...);
        }(std::make_integer_sequence<int, NMT>{});
    };

    int st = 0; // LDS stage of tile t
    auto iter = [&](auto par, int t) STG_AI {
        constexpr int P = decltype(par)::value;
        const int st1 = st == NSTAGE - 1 ? 0 : st + 1;
        const int stn = st == 0 ? NSTAGE - 1 : st - 1; // stage of tile t + NSTAGE - 1
        dma_tile(stn, t + NSTAGE - 1);
        [&]<int... S>(std::integer_sequence<int, S...>) STG_AI {
            (
                [&]() STG_AI {
                    constexpr int F = (P * KS + S) & 1;
                    if constexpr (S + 1 < KS)
                        lread(std::integral_constant<int, F ^ 1>{}, st, S + 1);
                    else
                        lread(std::integral_constant<int, F ^ 1>{}, st1, 0);
                    mma(std::integral_constant<int, F>{});
                }(),
                ...);
        }(std::make_integer_sequence<int, KS>{});
        schedule();
        __builtin_amdgcn_sched_barrier(0);
        // tile t+2 complete (tiles t+3 .. t+NSTAGE-1 may still be in flight)
        STG_WAIT_VMCNT((NSTAGE - 3) * NI);
        lds_barrier();
        st = st1;
    };

    int t = 0;
    for (; t + 1 < KT; t += 2) {
        iter(I0{}, t);
        iter(I1{}, t + 1);
    }
    if (t < KT)
        iter(I0{}, t);
    STG_WAIT_VMCNT(0); // drain the requests past the last tile before exit
    __syncthreads();   // every wave is done with the LDS stages

    epilogue_grid_lds<OP, FM, FN, false>(g.e, acc, m_blk + wm * WM, n_blk + wn * WN, lane,
                                  (uint32_t *)lds + wave * 32 * (WN + 4));
}

// ---------------------------------------------------------------- 128-byte K tiles

// 256 x 256 tile, 8 waves (two per SIMD) as 2 x 4, each a 128 x 64 block of
// 32x32 fragments, with K tiles of 128 bytes per row: every row of a tile is
// one whole 128-byte line.  With 64-byte K tiles each line is requested twice,
// half at a time, one K tile apart; measured on MI355X with the operand
// pattern of an 8192^3 GEMM, L2 delivers 21.5 TB/s to the CUs for whole-line
// rows against 13.2 TB/s for half lines (a tile-packed copy of the operands
// would give 23.2).  A stage is then 64 KB, so there are two, filled by
// direct global -> LDS copies: tile t+1 is requested at the start of tile t
// into the stage tile t-1 used, and waited for at the end of tile t.
// Fragments are double-buffered within a tile; the first step's fragment
// reads of each tile are covered by the other wave on the SIMD.
template <class OP>
__global__ __launch_bounds__(512, 1) void k_tiled_w8l(GemmArgs g, int tiles_m, int tiles_n)
{
    constexpr int BM = 256, BN = 256, BKB = 128, NSTAGE = 2;
    constexpr int WM = 128, WN = 64, FM = WM / 32, FN = WN / 32, GN = BN / WN;
    constexpr int STAGE = (BM + BN) * BKB;
    constexpr int NV = OP::LANE_BYTES / 16; // 16-byte LDS reads per operand fragment
    constexpr int FW = OP::LANE_BYTES / 4;  // 32-bit words per operand fragment
    constexpr int KS = BKB / OP::KB;        // MFMA K steps per tile
    constexpr int ROWS_PER_INST = 1024 / BKB;            // 8
    constexpr int A_I = BM / ROWS_PER_INST / 8;          // copies per wave per tile (4)
    constexpr int B_I = BN / ROWS_PER_INST / 8;
    constexpr int NI = A_I + B_I;
    constexpr int EPI = 8 * 32 * (WN + 4) * 4;
    constexpr int LDS_BYTES = NSTAGE * STAGE > EPI ? NSTAGE * STAGE : EPI;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int64_t m_blk = (int64_t)tm * BM, n_blk = (int64_t)tn * BN;
    const int64_t lda_b = g.a_rs * OP::ELEM, ldb_b = g.b_cs * OP::ELEM;
    const int64_t kbytes = g.K * OP::ELEM;
    const int KT = (int)(kbytes / BKB);
    const __amdgpu_buffer_rsrc_t ra = tile_rsrc((const uint8_t *)g.A + m_blk * lda_b,
                                                (g.e.M - m_blk - 1) * lda_b + kbytes);
    const __amdgpu_buffer_rsrc_t rb = tile_rsrc((const uint8_t *)g.B + n_blk * ldb_b,
                                                (g.e.N - n_blk - 1) * ldb_b + kbytes);

    // a copy instruction fills 1 KB of LDS = 8 rows of 128 bytes; lane l
    // writes slot l % 8 of row l / 8 and fetches the chunk the swizzle maps
    // there
    int voff[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const bool is_a = i < A_I;
        const int blk = is_a ? wave * A_I + i : wave * B_I + (i - A_I);
        const int row = blk * ROWS_PER_INST + (lane >> 3);
        voff[i] = row * (int)(is_a ? lda_b : ldb_b) + (((lane & 7) ^ swz128(row)) << 4);
    }
    auto dma_tile = [&](int stage, int kt) STG_AI {
        uint8_t *base = lds + stage * STAGE;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const bool is_a = i < A_I;
            const int blk = is_a ? wave * A_I + i : BM / ROWS_PER_INST + wave * B_I + (i - A_I);
            dma16(is_a ? ra : rb, base + blk * 1024, voff[i], kt * BKB);
        }
    };

    const int wm = wave / GN, wn = wave % GN;
    const int arow = wm * WM + (lane & 31), brow = wn * WN + (lane & 31);
    const int half = lane >> 5;
    int sa[FM], sb[FN]; // swz128 is not 32-row periodic
#pragma unroll
    for (int i = 0; i < FM; ++i)
        sa[i] = swz128(arow + 32 * i);
#pragma unroll
    for (int j = 0; j < FN; ++j)
        sb[j] = swz128(brow + 32 * j);
    const int a_off = arow * BKB, b_off = BM * BKB + brow * BKB;

    uint32_t fa[2][FM][FW], fb[2][FN][FW];
    auto lread = [&](auto set, const uint8_t *stage_base, int s) STG_AI {
        constexpr int S = decltype(set)::value;
        const uint8_t *lsa = stage_base + a_off;
        const uint8_t *lsb = stage_base + b_off;
        const int c0 = (s * OP::KB + half * OP::LANE_BYTES) >> 4;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
                *(u4_t *)&fa[S][i][4 * v] =
                    *(const u4_t *)(lsa + i * 32 * BKB + (((c0 + v) ^ sa[i]) << 4));
#pragma unroll
            for (int j = 0; j < FN; ++j)
                *(u4_t *)&fb[S][j][4 * v] =
                    *(const u4_t *)(lsb + j * 32 * BKB + (((c0 + v) ^ sb[j]) << 4));
        }
    };

    typename OP::acc_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = typename OP::acc_t{};
    auto mma = [&](auto set) STG_AI {
        constexpr int S = decltype(set)::value;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = OP::mma(fa[S][i], fb[S][j], acc[i][j]);
    };

    // the first step's fragment reads, then each step's MFMAs with the next
    // step's reads spread over them, and the copies of the next tile spread
    // over the whole tile
    constexpr int NM = FM * FN, NR = (FM + FN) * NV, NMT = KS * NM;
    auto schedule = [&]() STG_AI {
        __builtin_amdgcn_sched_group_barrier(0x100, NR, 0); // step 0 DS reads
        [&]<int... Q>(std::integer_sequence<int, Q...>) STG_AI {
            (
                [&]() STG_AI {
                    constexpr int m = Q % NM;
                    constexpr int nr = Q < NMT - NM ? spread(m, NR, NM) : 0;
                    constexpr int nl = spread(Q, NI, NMT);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); // MFMA
                    if constexpr (nr > 0)
                        __builtin_amdgcn_sched_group_barrier(0x100, nr, 0); // DS read
                    if constexpr (nl > 0)
                        __builtin_amdgcn_sched_group_barrier(0x020, nl, 0); // VMEM read
                }(),
                ...);
        }(std::make_integer_sequence<int, NMT>{});
    };

    // prologue: tile 0 into stage 0
    dma_tile(0, 0);
    STG_WAIT_VMCNT(0);
    lds_barrier();

    for (int t = 0; t < KT; ++t) {
        const uint8_t *cur = lds + (t & 1) * STAGE;
        // tile t+1 into the stage of tile t-1 (the copy past the last tile
        // reads bytes that are never used, or zeros past the resource)
        dma_tile((t + 1) & 1, t + 1);
        lread(std::integral_constant<int, 0>{}, cur, 0);
        [&]<int... S>(std::integer_sequence<int, S...>) STG_AI {
            (
                [&]() STG_AI {
                    if constexpr (S + 1 < KS)
                        lread(std::integral_constant<int, (S + 1) & 1>{}, cur, S + 1);
                    mma(std::integral_constant<int, S & 1>{});
                }(),
                ...);
        }(std::make_integer_sequence<int, KS>{});
        schedule();
        __builtin_amdgcn_sched_barrier(0);
        STG_WAIT_VMCNT(0); // this wave's copies of tile t+1 complete
        lds_barrier();     // ... and every wave's; tile t's stage is free
    }

    __syncthreads(); // every wave is done with the LDS stages
    epilogue_grid_lds<OP, FM, FN, false>(g.e, acc, m_blk + wm * WM, n_blk + wn * WN, lane,
                                  (uint32_t *)lds + wave * 32 * (WN + 4));
}

// ---------------------------------------------------------------- ping-pong

// 256 x 256 tile, 8 waves in two groups of four (one wave of each group per
// SIMD): group 0 owns output columns 0..127 of the tile, group 1 columns
// 128..255, each wave a 128 x 64 block of 32x32 fragments.  The groups run
// out of phase: in phase 1 of K tile t group 0 multiplies tile t while group
// 1 reads its fragments of tile t from LDS and issues direct global -> LDS
// copies of a future tile; in phase 2 the roles swap (group 1 multiplies,
// group 0 reads tile t+1's fragments and issues copies).  One barrier ends
// each phase, so each SIMD always has one wave issuing MFMAs from registers
// while the other wave's memory work is in flight.
// Copies: tile u's A operand is requested by group 0 in phase 2 of tile
// u - NSTAGE, its B operand by group 1 in phase 1 of tile u - NSTAGE + 1;
// both are waited for (by the requesting waves) before the barrier that ends
// phase 1 of tile u - 1, the last point before tile u is first read.
template <class OP, int NSTAGE>
__global__ __launch_bounds__(512, 1) void k_pingpong(GemmArgs g, int tiles_m, int tiles_n)
{
    constexpr int BM = 256, BN = 256, BKB = 64;
    constexpr int WM = 128, WN = 64, FM = WM / 32, FN = WN / 32;
    constexpr int STAGE = (BM + BN) * BKB;
    constexpr int NV = OP::LANE_BYTES / 16;
    constexpr int FW = OP::LANE_BYTES / 4;
    constexpr int KS = BKB / OP::KB;
    constexpr int NI = (BM * BKB / 1024) / 4; // copy instructions per wave per operand half
    constexpr int EPI = 8 * 32 * (WN + 4) * 4;
    constexpr int LDS_BYTES = NSTAGE * STAGE > EPI ? NSTAGE * STAGE : EPI;
    static_assert(NSTAGE >= 3 && LDS_BYTES <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2, wq = wave & 3;
    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int64_t m_blk = (int64_t)tm * BM, n_blk = (int64_t)tn * BN;
    const int64_t lda_b = g.a_rs * OP::ELEM, ldb_b = g.b_cs * OP::ELEM;
    const int64_t kbytes = g.K * OP::ELEM;
    const int KT = (int)(kbytes / BKB);
    const __amdgpu_buffer_rsrc_t ra = tile_rsrc((const uint8_t *)g.A + m_blk * lda_b,
                                                (g.e.M - m_blk - 1) * lda_b + kbytes);
    const __amdgpu_buffer_rsrc_t rb = tile_rsrc((const uint8_t *)g.B + n_blk * ldb_b,
                                                (g.e.N - n_blk - 1) * ldb_b + kbytes);

    // copies: group 0 fills the A half of a stage, group 1 the B half; wave
    // wq of a group owns 1 KB blocks wq*NI .. wq*NI+NI-1 (16 rows each)
    const __amdgpu_buffer_rsrc_t rsrc = grp == 0 ? ra : rb;
    const int64_t ld_b = grp == 0 ? lda_b : ldb_b;
    int voff[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int row = (wq * NI + i) * 16 + (lane >> 2);
        voff[i] = row * (int)ld_b + (((lane & 3) ^ swz64(row)) << 4);
    }
    const int half_off = grp * BM * BKB;
    auto copy_tile = [&](int stage, int kt) STG_AI {
        uint8_t *base = lds + stage * STAGE + half_off + wq * NI * 1024;
#pragma unroll
        for (int i = 0; i < NI; ++i)
            dma16(rsrc, base + i * 1024, voff[i], kt * BKB);
    };

    // fragments of this wave: rows wm*128 + 32 i of A, columns grp*128 + wn*64 + 32 j of B
    const int wm = wq >> 1, wn = wq & 1;
    const int arow = wm * WM + (lane & 31), brow = grp * 128 + wn * WN + (lane & 31);
    const int half = lane >> 5;
    const int sa = swz64(arow), sb = swz64(brow);
    const int a_off = arow * BKB, b_off = BM * BKB + brow * BKB;
    uint32_t fa[KS][FM][FW], fb[KS][FN][FW];
    auto lread = [&](const uint8_t *__restrict__ stage_base) STG_AI {
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int c0 = (s * OP::KB + half * OP::LANE_BYTES) >> 4;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int oa = ((c0 + v) ^ sa) << 4, ob = ((c0 + v) ^ sb) << 4;
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    *(u4_t *)&fa[s][i][4 * v] = *(const u4_t *)(stage_base + a_off + i * 32 * BKB + oa);
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    *(u4_t *)&fb[s][j][4 * v] = *(const u4_t *)(stage_base + b_off + j * 32 * BKB + ob);
            }
        }
    };
    typename OP::acc_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = typename OP::acc_t{};
    auto compute = [&]() STG_AI {
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = OP::mma(fa[s][i], fb[s][j], acc[i][j]);
    };
    auto stage_of = [&](int kt) STG_AI { return kt % NSTAGE; };

    // prologue: tiles 0 .. NSTAGE-2 (both halves) and the A half of tile
    // NSTAGE-1, in the same per-group order the loop continues
#pragma unroll
    for (int u = 0; u < NSTAGE - 1; ++u)
        copy_tile(u, u);
    if (grp == 0)
        copy_tile(NSTAGE - 1, NSTAGE - 1);
    STG_WAIT_VMCNT(0);
    lds_barrier();
    if (grp == 0)
        lread(lds);

    for (int t = 0; t < KT; ++t) {
        // ---- phase 1: group 0 multiplies tile t; group 1 reads tile t and
        // requests the B half of tile t + NSTAGE - 1
        if (grp == 0) {
            compute();
            // this wave's requests up to tile t+1 complete (tiles t+2 ..
            // t+NSTAGE-1 may still be in flight)
            STG_WAIT_VMCNT((NSTAGE - 2) * NI);
        } else {
            lread(lds + stage_of(t) * STAGE);
            copy_tile(stage_of(t + NSTAGE - 1), t + NSTAGE - 1);
            STG_WAIT_VMCNT((NSTAGE - 2) * NI);
        }
        lds_barrier();
        // ---- phase 2: group 1 multiplies tile t; group 0 reads tile t+1 and
        // requests the A half of tile t + NSTAGE
        if (grp == 1) {
            compute();
        } else {
            lread(lds + stage_of(t + 1) * STAGE);
            copy_tile(stage_of(t + NSTAGE), t + NSTAGE);
        }
        lds_barrier();
    }
    STG_WAIT_VMCNT(0);
    __syncthreads();
    epilogue_grid_lds<OP, FM, FN, false>(g.e, acc, m_blk + wm * WM, n_blk + grp * 128 + wn * WN, lane,
                                  (uint32_t *)lds + wave * 32 * (WN + 4));
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
// whole cache lines; two chunks are kept in flight per wave.
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
            for (int j = 0; j < NLD; ++j) {
                pb[S][0][j] = buf_load16(rb, vb0 + 16 * j, soff);
                pb[S][1][j] = buf_load16(rb, vb1 + 16 * j, soff);
            }
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
    default: return nullptr;
    }
}

template <class OP>
static hipError_t launch_w8l_t(const GemmArgs &g, hipStream_t s)
{
    const int tiles_m = (int)((g.e.M + 255) / 256), tiles_n = (int)((g.e.N + 255) / 256);
    hipLaunchKernelGGL(k_tiled_w8l<OP>, dim3((unsigned)(tiles_m * tiles_n)), dim3(512), 0, s, g,
                       tiles_m, tiles_n);
    return hipGetLastError();
}

static dense_launch_fn w8l_table(int op)
{
    switch (op) {
    case OPK_F16: return launch_w8l_t<OpF16>;
    case OPK_BF16: return launch_w8l_t<OpBF16>;
    case OPK_F8_E4E4: return launch_w8l_t<OpF8<0, 0>>;
    case OPK_F8_E4E5: return launch_w8l_t<OpF8<0, 1>>;
    case OPK_F8_E5E4: return launch_w8l_t<OpF8<1, 0>>;
    case OPK_F8_E5E5: return launch_w8l_t<OpF8<1, 1>>;
    case OPK_S8: return launch_w8l_t<OpS8>;
    default: return nullptr;
    }
}

template <class OP, int NS>
static hipError_t launch_pingpong_t(const GemmArgs &g, hipStream_t s)
{
    const int tiles_m = (int)((g.e.M + 255) / 256), tiles_n = (int)((g.e.N + 255) / 256);
    hipLaunchKernelGGL((k_pingpong<OP, NS>), dim3((unsigned)(tiles_m * tiles_n)), dim3(512), 0, s,
                       g, tiles_m, tiles_n);
    return hipGetLastError();
}

template <int NS>
static dense_launch_fn pingpong_table(int op)
{
    switch (op) {
    case OPK_F16: return launch_pingpong_t<OpF16, NS>;
    case OPK_BF16: return launch_pingpong_t<OpBF16, NS>;
    case OPK_F8_E4E4: return launch_pingpong_t<OpF8<0, 0>, NS>;
    case OPK_F8_E4E5: return launch_pingpong_t<OpF8<0, 1>, NS>;
    case OPK_F8_E5E4: return launch_pingpong_t<OpF8<1, 0>, NS>;
    case OPK_F8_E5E5: return launch_pingpong_t<OpF8<1, 1>, NS>;
    case OPK_S8: return launch_pingpong_t<OpS8, NS>;
    default: return nullptr;
    }
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

template <class OP, int BM, int BN, int NS>
static hipError_t launch_dma_t(const GemmArgs &g, hipStream_t s)
{
    const int tiles_m = (int)((g.e.M + BM - 1) / BM), tiles_n = (int)((g.e.N + BN - 1) / BN);
    hipLaunchKernelGGL((k_tiled_dma<OP, BM, BN, NS>), dim3((unsigned)(tiles_m * tiles_n)),
                       dim3(256), 0, s, g, tiles_m, tiles_n);
    return hipGetLastError();
}

template <int BM, int BN, int NS>
static dense_launch_fn dma_table_t(int op)
{
    switch (op) {
    case OPK_F16: return launch_dma_t<OpF16, BM, BN, NS>;
    case OPK_BF16: return launch_dma_t<OpBF16, BM, BN, NS>;
    case OPK_F8_E4E4: return launch_dma_t<OpF8<0, 0>, BM, BN, NS>;
    case OPK_F8_E4E5: return launch_dma_t<OpF8<0, 1>, BM, BN, NS>;
    case OPK_F8_E5E4: return launch_dma_t<OpF8<1, 0>, BM, BN, NS>;
    case OPK_F8_E5E5: return launch_dma_t<OpF8<1, 1>, BM, BN, NS>;
    case OPK_S8: return launch_dma_t<OpS8, BM, BN, NS>;
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
    case KF_TILED_256W8T: fn = tiled_table_t<256, 256, 4, 2>(op); break;
    case KF_PINGPONG4: fn = pingpong_table<4>(op); break;
    case KF_PINGPONG5: fn = pingpong_table<5>(op); break;
    case KF_TILED_256W8L: fn = w8l_table(op); break;
    case KF_TILED_DMA4: fn = dma_table_t<256, 256, 4>(op); break;
    case KF_TILED_DMA5: fn = dma_table_t<256, 256, 5>(op); break;
    default: break;
    }
    if (!fn)
        return hipErrorInvalidValue;
    return fn(g, s);
}

} // namespace stg
