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

// ---------------------------------------------------------------- tiled


template <class OP, int BM, int BN, int GM = 2, int GN = 2, int WG_PER_CU = 1>
__global__ __launch_bounds__(64 * GM * GN, WG_PER_CU) void k_tiled(GemmArgs g, int tiles_m,
                                                                   int tiles_n)
{
    constexpr int NT = 64 * GM * GN;        // GM x GN waves
    constexpr int BKB = 64;                 // K bytes per tile
    constexpr int CH = BKB / 16;            // 16-byte chunks per row
    constexpr int RPP = NT / CH;            // rows covered per load pass
    constexpr int A_LD = BM / RPP, B_LD = BN / RPP;
    constexpr int WM = BM / GM, WN = BN / GN; // wave sub-tile
    constexpr int FM = WM / 32, FN = WN / 32;
    constexpr int NSTAGE = 3;
    // MN-major operands (16-bit; A column-major, B row-major): the tile stays
    // in LDS as 32 K rows of MN values, pitch MN bytes + 64, K row r stored at
    // row slot mn_slot(r) (bits 2 and 3 swapped), so that the 8 K rows one
    // transposing fragment read touches fall on 8 different 64-byte bank
    // groups and every offset inside a step is an immediate
    constexpr bool AMN = a_mn_v<OP>(), BMN = b_mn_v<OP>();
    static_assert(!(AMN || BMN) || (OP::BITS == 16 && !OP::MX && !OP::W4), "MN-major: 16-bit");
    constexpr int KR = BKB / 2; // K rows of an MN-major tile
    constexpr int APITCH = BM * 2 + 64, BPITCH = BN * 2 + 64;
    constexpr int A_TILE = AMN ? KR * APITCH : BM * BKB;
    constexpr int B_TILE = BMN ? KR * BPITCH : BN * BKB;
    constexpr int STAGE = A_TILE + B_TILE;
    constexpr int NV = OP::LANE_BYTES / 16; // 16-byte LDS reads per operand
    constexpr int FW = OP::LANE_BYTES / 4;  // 32-bit words per operand fragment
    constexpr int KS = BKB / OP::KB;        // MFMA K steps per tile
    // LDS holds the stages during the K loop and the epilogue's per-wave
    // 32-row staging slabs afterwards
    constexpr int EPI = GM * GN * 32 * (WN + 4) * 4;
    // MX: the block scales of the tile's 256 A rows and 256 B columns pass
    // through LDS in groups of QG 32-bit words per row (16 K blocks, 512 K),
    // two group slots after the stages
    constexpr int QG = 4;
    constexpr int SC_OFF = NSTAGE * STAGE;
    constexpr int SC_BYTES = OP::MX ? 2 * 2 * QG * 256 * 4 : 0;
    static_assert(!OP::MX || (BM == 256 && BN == 256 && NT == 256), "one scale row per thread");
    constexpr int KLOOP = NSTAGE * STAGE + SC_BYTES;
    constexpr int LDS_BYTES = KLOOP > EPI ? KLOOP : EPI;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int64_t m_blk = (int64_t)tm * BM, n_blk = (int64_t)tn * BN;
    // W4A16: B holds 4-bit codes (half a byte per K), dequantised into the
    // 16-bit B tile on its way into LDS
    constexpr bool W4 = OP::W4;
    static_assert(!W4 || (BN == 256 && NT == 256), "one B row per thread");
    // (row pitch in bytes: of the M or N rows, or of the K rows when MN-major)
    const int64_t lda_b = (AMN ? g.a_cs : g.a_rs) * OP::BITS / 8;
    const int64_t ldb_b = W4 ? g.b_cs / 2 : (BMN ? g.b_rs : g.b_cs) * OP::BITS / 8;
    const int64_t kbytes = g.K * OP::BITS / 8, kbytes_b = W4 ? g.K / 2 : kbytes;
    const int KT = (int)(kbytes / BKB);
    // bounded by the last byte of the last row: loads past it return zero
    // (MN-major: the tile's columns start at the base, and the whole offset
    // goes through the checked vector offset)
    const __amdgpu_buffer_rsrc_t ra =
        AMN ? tile_rsrc((const uint8_t *)g.A + m_blk * 2, ((g.K - 1) * g.a_cs + g.e.M - m_blk) * 2)
            : tile_rsrc((const uint8_t *)g.A + m_blk * lda_b, (g.e.M - m_blk - 1) * lda_b + kbytes);
    const __amdgpu_buffer_rsrc_t rb =
        BMN ? tile_rsrc((const uint8_t *)g.B + n_blk * 2, ((g.K - 1) * g.b_rs + g.e.N - n_blk) * 2)
            : tile_rsrc((const uint8_t *)g.B + n_blk * ldb_b,
                        (g.e.N - n_blk - 1) * ldb_b + kbytes_b);
    // W4A16 group scales and zero points of the tile's columns (zero points
    // absent: a zero-length resource, whose loads return 0, and z = 8)
    const int64_t wgr = W4 ? g.K / g.wgs : 0; // groups per column
    const __amdgpu_buffer_rsrc_t rws =
        tile_rsrc((const uint8_t *)g.ws + n_blk * wgr * 2, W4 ? (g.e.N - n_blk) * wgr * 2 : 0);
    const __amdgpu_buffer_rsrc_t rwz =
        tile_rsrc(g.wz ? g.wz + n_blk * wgr : (const uint8_t *)g.B, W4 && g.wz ? (g.e.N - n_blk) * wgr : 0);
    const bool has_wz = g.wz != nullptr;

    // global -> LDS copy: thread owns chunk `ch` of rows r0 + i*RPP
    const int ch = tid % CH, r0 = tid / CH;
    // (MN-major: chunk tid % CHX of K rows tid / CHX + i * RPX; the K offset
    // of tile kt is kt * KR rows)
    constexpr int CHA = BM * 2 / 16, CHB = BN * 2 / 16, RPA = NT / CHA, RPB = NT / CHB;
    static_assert(!AMN || KR / RPA == A_LD, "MN-major A: same load count");
    static_assert(!BMN || KR / RPB == B_LD, "MN-major B: same load count");
    auto mn_slot = [](int r) STG_AI { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); };
    const int va0 = AMN ? (tid / CHA) * (int)lda_b + (tid % CHA) * 16 : r0 * (int)lda_b + ch * 16;
    const int vb0 = BMN ? (tid / CHB) * (int)ldb_b + (tid % CHB) * 16 : r0 * (int)ldb_b + ch * 16;
    const int va_step = (AMN ? RPA : RPP) * (int)lda_b, vb_step = (BMN ? RPB : RPP) * (int)ldb_b;
    const int va_tile = AMN ? KR * (int)lda_b : 0, vb_tile = BMN ? KR * (int)ldb_b : 0;
    // 8-bit MX operands: chunks 1 and 2 of every 64-byte K tile trade places in
    // LDS, so that a lane half's two consecutive chunks hold K 16h .. and
    // 32+16h .. (the instruction's K blocks are the two 16-byte halves of
    // both lane halves' operands)
    constexpr bool perm = OP::MX && OP::SPLIT;
    const int lch = perm ? (((ch & 1) << 1) | (ch >> 1)) : ch;
    const int l0 = r0 * BKB + ((lch ^ swz64(r0)) << 4); // + i*RPP*BKB (swz64 is RPP-periodic)
    const int la0 = AMN ? mn_slot(tid / CHA) * APITCH + (tid % CHA) * 16 : l0;
    const int lb0 = A_TILE + (BMN ? mn_slot(tid / CHB) * BPITCH + (tid % CHB) * 16 : l0);
    // LDS offset of load pass i (mn_slot(r + i RPX) = mn_slot(r) + mn_slot(i RPX))
    auto a_pass = [&](int i) STG_AI { return AMN ? mn_slot(i * RPA) * APITCH : i * RPP * BKB; };
    auto b_pass = [&](int i) STG_AI { return BMN ? mn_slot(i * RPB) * BPITCH : i * RPP * BKB; };

    // register staging of global tiles, two sets (prefetch distance 2 tiles)
    u4_t ga[2][A_LD], gb[2][B_LD];
    uint32_t wsb[2], wzb[2]; // W4A16: the tile's group scale bits and zero point
    auto gload = [&](auto set, int kt) STG_AI {
        constexpr int S = decltype(set)::value;
        const int soff = kt * BKB;
#pragma unroll
        for (int i = 0; i < A_LD; ++i)
            ga[S][i] = AMN ? buf_load16(ra, va0 + i * va_step + kt * va_tile, 0)
                           : buf_load16(ra, va0 + i * va_step, soff);
        if constexpr (W4) {
            // thread t: the 16 code bytes (32 K) of column n_blk + t, and its
            // group's scale and zero point
            const int grp = (int)((int64_t)kt * (BKB / 2) / g.wgs);
            gb[S][0] = buf_load16(rb, tid * (int)ldb_b, kt * (BKB / 4));
            wsb[S] = __builtin_amdgcn_raw_buffer_load_b16(rws, (tid * (int)wgr + grp) * 2, 0, 0);
            wzb[S] = __builtin_amdgcn_raw_buffer_load_b8(rwz, tid * (int)wgr + grp, 0, 0);
        } else {
#pragma unroll
            for (int i = 0; i < B_LD; ++i)
                gb[S][i] = BMN ? buf_load16(rb, vb0 + i * vb_step + kt * vb_tile, 0)
                               : buf_load16(rb, vb0 + i * vb_step, soff);
        }
    };
    auto lstore = [&](auto set, uint8_t *__restrict__ stage_base) STG_AI {
        constexpr int S = decltype(set)::value;
#pragma unroll
        for (int i = 0; i < A_LD; ++i)
            *(u4_t *)(stage_base + la0 + a_pass(i)) = ga[S][i];
        if constexpr (W4) {
            // 32 codes -> 32 16-bit values: row t of the B tile, four chunks
            constexpr bool BF = std::is_same<OP, OpW4<OpBF16>>::value;
            const float sc = w4_scale<BF>(wsb[S]);
            const int z = has_wz ? (int)wzb[S] : 8;
            uint8_t *brow = stage_base + A_TILE + tid * BKB;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                u4_t v;
                w4_dequant8<BF>(gb[S][0][c], z, sc, (uint32_t *)&v);
                // chunk c holds codes 8c .. 8c+7 = one 16-byte chunk of 8 values
                *(u4_t *)(brow + ((c ^ swz64(tid)) << 4)) = v;
            }
        } else {
#pragma unroll
            for (int i = 0; i < B_LD; ++i)
                *(u4_t *)(stage_base + lb0 + b_pass(i)) = gb[S][i];
        }
    };

    // fragment reads: lane reads rows arow + 32 i (A) and brow + 32 j (B)
    const int wm = wave / GN, wn = wave % GN;
    const int arow = wm * WM + (lane & 31), brow = wn * WN + (lane & 31);
    const int half = lane >> 5;
    const int sa = swz64(arow), sb = swz64(brow); // same for every fragment row
    const int a_off = arow * BKB, b_off = A_TILE + brow * BKB;
    // MN-major fragments: two transposing reads per fragment and step, K
    // values 4 t .. 4 t + 3 of the lane half (t = 0, 1).  Lane 16 q + j reads
    // K row 16 s + 8 (q / 2) + 4 t + j / 4 (slot 16 s + 8 t + 4 (q / 2) + j / 4)
    // at MN columns 16 (q % 2) + 4 (j % 4) .. + 3 of fragment i (+ 32 i)
    const int tr_slot = 4 * (lane >> 5) + ((lane >> 2) & 3);
    const int tr_col = 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));
    const int a_tr = tr_slot * APITCH + 2 * wm * WM + tr_col;
    const int b_tr = A_TILE + tr_slot * BPITCH + 2 * wn * WN + tr_col;

    uint32_t fa[2][FM][FW], fb[2][FN][FW];
    auto lread = [&](auto set, const uint8_t *__restrict__ stage_base, int s) STG_AI {
        constexpr int S = decltype(set)::value;
        const uint8_t *lsa = stage_base + a_off;
        const uint8_t *lsb = stage_base + b_off;
        const int c0 = (s * OP::KB + half * OP::LANE_BYTES) >> 4;
        if constexpr (AMN) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    lds_read_tr16(stage_base + a_tr + (16 * s + 8 * t) * APITCH + 64 * i,
                                  &fa[S][i][2 * t]);
        }
        if constexpr (BMN) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    lds_read_tr16(stage_base + b_tr + (16 * s + 8 * t) * BPITCH + 64 * j,
                                  &fb[S][j][2 * t]);
        }
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int oa = ((c0 + v) ^ sa) << 4, ob = ((c0 + v) ^ sb) << 4;
            if constexpr (!AMN)
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    *(u4_t *)&fa[S][i][4 * v] = *(const u4_t *)(lsa + i * 32 * BKB + oa);
            if constexpr (!BMN)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    *(u4_t *)&fb[S][j][4 * v] = *(const u4_t *)(lsb + j * 32 * BKB + ob);
        }
    };

    // MX block scales.  Each MFMA needs, per fragment row / column, the
    // scale byte of the lane half's K block; in HBM the bytes of 32
    // consecutive rows lie K/32 bytes apart, so reading them straight from
    // memory costs a cache line per lane.  Instead, at the first tile of a
    // group of TG tiles (512 K, 16 blocks), each thread copies the next
    // group's 16 scale bytes of its own A row and B column straight into
    // LDS; the copies are waited for before the barrier two tiles before
    // that group starts, and the fragments read their bytes (ds_read_u8,
    // already in the byte the instruction takes) one tile ahead.  Slot s,
    // operand o (0 A, 1 B): 256 rows of 16 bytes at SC_OFF + (2 s + o) 4 KB.
    constexpr int KPT = BKB * 8 / OP::BITS;          // K per tile
    constexpr int TG = QG * 128 / KPT;               // tiles per scale group: 8 or 4
    constexpr int NSW = OP::MX ? (FM + FN) * KS : 0; // scale bytes per lane per tile
    static_assert(!OP::MX || TG >= 2, "a group spans at least two tiles");
    uint32_t scl[2][NSW > 0 ? NSW : 1];
    const int64_t kblk = g.K / 32; // scale bytes per row (a multiple of 16)
    // (not used outside MX, where the compiler drops them)
    const __amdgpu_buffer_rsrc_t rsa = tile_rsrc(g.sa + m_blk * kblk, (g.e.M - m_blk) * kblk);
    const __amdgpu_buffer_rsrc_t rsb = tile_rsrc(g.sb + n_blk * kblk, (g.e.N - n_blk) * kblk);
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    auto sc_at = [&](int slot, int o, int b, int r) STG_AI {
        return (uint32_t) * (const uint8_t *)(lds + SC_OFF + (2 * slot + o) * 4096 + 16 * r + b);
    };
    // group grp's words of this thread's A row and B column into slot grp & 1
    // (wave w's copy instruction covers rows 64 w .. 64 w + 63)
    auto sg_copy = [&](int grp) STG_AI {
        if constexpr (OP::MX) {
            uint8_t *base = lds + SC_OFF + 2 * (grp & 1) * 4096 + wave_u * 1024;
            dma16(rsa, base, tid * (int)kblk, 16 * grp);
            dma16(rsb, base + 4096, tid * (int)kblk, 16 * grp);
        }
    };
    // this lane's scale bytes for tile u into register set S: step st, lane
    // half h takes K block u KPT / 32 + 2 st + h
    auto sload = [&](auto set, int u) STG_AI {
        if constexpr (OP::MX) {
            constexpr int S = decltype(set)::value;
            const int slot = (u / TG) & 1;
            const int arow0 = (wave / GN) * (BM / GM) + (tid & 31);
            const int brow0 = (wave % GN) * (BN / GN) + (tid & 31);
#pragma unroll
            for (int st = 0; st < KS; ++st) {
                const int b = (u * KPT / 32 + 2 * st + ((tid >> 5) & 1)) % 16;
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    scl[S][st * (FM + FN) + i] = sc_at(slot, 0, b, arow0 + 32 * i);
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    scl[S][st * (FM + FN) + FM + j] = sc_at(slot, 1, b, brow0 + 32 * j);
            }
        }
    };

    typename OP::acc_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = typename OP::acc_t{};
    // fragment set F; for MX also the tile's parity P and step S
    auto mma = [&](auto set, auto pset, auto step) STG_AI {
        constexpr int S = decltype(set)::value;
        if constexpr (OP::MX) {
            constexpr int P = decltype(pset)::value, ST = decltype(step)::value;
            constexpr int o = ST * (FM + FN);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = OP::template mma<0>(fa[S][i], fb[S][j], acc[i][j], scl[P][o + i],
                                                    scl[P][o + FM + j]);
        } else {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = OP::mma(fa[S][i], fb[S][j], acc[i][j]);
        }
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;

    // prologue: tiles 0 and 1 in LDS stages 0 and 1, tile 2 in registers set 0
    // (MX: scale group 0 into its LDS slot; tile 0's words read after the
    // barrier)
    sg_copy(0);
    gload(I0{}, 0);
    gload(I1{}, 1);
    lstore(I0{}, lds);
    lstore(I1{}, lds + STAGE);
    gload(I0{}, 2);
    if constexpr (OP::MX)
        STG_WAIT_VMCNT(0); // the direct copies of scale group 0
    __syncthreads();
    sload(I0{}, 0);
    lread(I0{}, lds, 0);

    // one K tile: `P` is the parity of the tile index (register sets and the
    // fragment buffer of its first step are chosen at compile time).
    // Loads past the last tile read padding or zeros into a stage that is
    // never consumed, which keeps the loop body branch-free.
    // Instruction order inside one K tile: the fragment reads of each step
    // are spread evenly over that step's MFMAs, and the tile's global loads
    // and LDS stores are spread evenly over all of the tile's MFMAs (a load
    // every VM_EVERY MFMAs, a store half-way between), so neither the vector
    // memory pipe (64 B/clk per CU) nor the LDS write path (about half the
    // LDS read rate) backs up and stalls MFMA issue.
    // (W4A16: three loads and four LDS writes for B)
    constexpr int NL = A_LD + (W4 ? 3 : B_LD), NLW = A_LD + (W4 ? 4 : B_LD);
    constexpr int NM = FM * FN, NR = FM * (AMN ? 2 : NV) + FN * (BMN ? 2 : NV);
    constexpr int NMT = KS * NM;
    auto schedule = [&]() STG_AI {
        [&]<int... Q>(std::integer_sequence<int, Q...>) STG_AI {
            (
                [&]() STG_AI {
                    constexpr int m = Q % NM;
                    constexpr int nr = spread(m, NR, NM), nl = spread(Q, NL, NMT);
                    constexpr int nw = spread((Q + NMT / 2) % NMT, NLW, NMT);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); // MFMA
                    if constexpr (nr > 0)
                        __builtin_amdgcn_sched_group_barrier(0x100, nr, 0); // DS read
                    if constexpr (nl > 0)
                        __builtin_amdgcn_sched_group_barrier(0x020, nl, 0); // VMEM read
                    if constexpr (nw > 0)
                        __builtin_amdgcn_sched_group_barrier(0x200, nw, 0); // DS write
                }(),
                ...);
        }(std::make_integer_sequence<int, NMT>{});
    };

    int st = 0; // LDS stage of tile t
    auto iter = [&](auto par, int t) STG_AI {
        constexpr int P = decltype(par)::value;
        const int st1 = st == NSTAGE - 1 ? 0 : st + 1;
        const int st2 = st1 == NSTAGE - 1 ? 0 : st1 + 1;
        // the three stages are distinct: the tile is read from `cur`, the
        // next tile's first fragments from `nxt`, and tile t+2 is written to
        // `wr`; restrict lets the scheduler interleave the stores with reads
        auto body = [&](const uint8_t *__restrict__ cur, const uint8_t *__restrict__ nxt,
                        uint8_t *__restrict__ wr) STG_AI {
            // MX: the next scale group at the first tile of a group, and
            // the next tile's scale bytes
            if constexpr (OP::MX)
                if (t % TG == 0)
                    sg_copy(t / TG + 1);
            sload(std::integral_constant<int, P ^ 1>{}, t + 1);
            gload(std::integral_constant<int, P ^ 1>{}, t + 3);
            [&]<int... S>(std::integer_sequence<int, S...>) STG_AI {
                (
                    [&]() STG_AI {
                        constexpr int F = (P * KS + S) & 1;
                        if constexpr (S + 1 < KS)
                            lread(std::integral_constant<int, F ^ 1>{}, cur, S + 1);
                        else
                            lread(std::integral_constant<int, F ^ 1>{}, nxt, 0);
                        mma(std::integral_constant<int, F>{}, std::integral_constant<int, P>{},
                            std::integral_constant<int, S>{});
                    }(),
                    ...);
            }(std::make_integer_sequence<int, KS>{});
            lstore(std::integral_constant<int, P>{}, wr);
            schedule();
            // the next group's bytes (copied into the slot the previous
            // group used): complete before this tile's barrier, one tile
            // before their first read.  Loads retire in order and the
            // copies are older than this tile's A_LD + B_LD prefetch loads,
            // which may stay in flight.
            if constexpr (OP::MX)
                if (t % TG == TG - 2)
                    STG_WAIT_VMCNT(A_LD + B_LD);
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
    // (MX takes K in whole scale groups, so its tile count is even)
    if constexpr (!OP::MX)
        if (t < KT)
            iter(I0{}, t);

    __syncthreads(); // every wave is done with the LDS stages
    epilogue_grid_lds<OP, FM, FN>(g.e, acc, m_blk + wm * WM, n_blk + wn * WN, lane,
                                  (uint32_t *)lds + wave * 32 * (WN + 4));
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

template <class OP, int BM, int BN, int GM = 2, int GN = 2, int WPC = 1>
static hipError_t launch_tiled_t(const GemmArgs &g, hipStream_t s)
{
    const int tiles_m = (int)((g.e.M + BM - 1) / BM), tiles_n = (int)((g.e.N + BN - 1) / BN);
    hipLaunchKernelGGL((k_tiled<OP, BM, BN, GM, GN, WPC>), dim3((unsigned)(tiles_m * tiles_n)),
                       dim3(64 * GM * GN), 0, s, g, tiles_m, tiles_n);
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

// MN-major operands (layout bit 0: A column-major, bit 1: B row-major) on
// the LDS-tiled kernel, 16-bit types
template <class OP, int BM, int BN, int GM, int GN>
static dense_launch_fn mn_pick(int layout)
{
    switch (layout) {
    case 1: return launch_tiled_t<OpMN<OP, true, false>, BM, BN, GM, GN>;
    case 2: return launch_tiled_t<OpMN<OP, false, true>, BM, BN, GM, GN>;
    case 3: return launch_tiled_t<OpMN<OP, true, true>, BM, BN, GM, GN>;
    default: return nullptr;
    }
}

template <int BM, int BN, int GM = 2, int GN = 2>
static dense_launch_fn tiled_mn_table_t(int op, int layout)
{
    switch (op) {
    case OPK_F16: return mn_pick<OpF16, BM, BN, GM, GN>(layout);
    case OPK_BF16: return mn_pick<OpBF16, BM, BN, GM, GN>(layout);
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
    if (layout != 0) {
        switch (family) {
        case KF_GENERIC: fn = generic_table(op); break;
        case KF_TILED_256W8: fn = tiled_mn_table_t<256, 256, 2, 4>(op, layout); break;
        case KF_TILED_128: fn = tiled_mn_table_t<128, 128>(op, layout); break;
        default: break;
        }
        if (!fn)
            return hipErrorInvalidValue;
        return fn(g, s);
    }
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
