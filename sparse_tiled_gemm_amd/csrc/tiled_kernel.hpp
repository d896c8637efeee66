// The LDS-tiled GEMM kernel template k_tiled (described at the top of
// kernels_dense.hip) and its launcher, shared by the translation units that
// instantiate it: kernels_dense.hip (K-contiguous operands, MX, W4A16) and
// kernels_mn.hip (MN-major operands).
#pragma once
#include "device_common.hpp"
#include "internal.hpp"

namespace stg {

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
    // MN-major operands (A column-major, B row-major; 16- and 8-bit types):
    // the tile stays in LDS as KR K rows of MN values.  A transposing read
    // gives a lane TR consecutive K values (TR = 4 16-bit or 8 8-bit values,
    // from TR rows of a 16-lane group), NT_R such reads cover the lane half's
    // LANE_K values, and the two lane halves take K rows HS = TR * NT_R apart.
    // K row r = s 2HS + h HS + t TR + e sits at row slot s 2HS + t 2TR + h TR
    // + e (mn_slot), so the 2 TR rows one read of a wave touches are
    // consecutive slots; with a row pitch of MN bytes + PAD (64 or 32) they
    // fall on distinct bank groups, and every offset inside a step is an
    // immediate.
    constexpr bool AMN = a_mn_v<OP>(), BMN = b_mn_v<OP>();
    // unsigned 8-bit operands (OpI8): staged into LDS as x - 128, corrected
    // before the epilogue from per-lane operand sums
    constexpr bool AU = au_v<OP>(), BU = bu_v<OP>();
    static_assert(!(AU || BU) || !(AMN || BMN), "unsigned operands: K-contiguous layouts");
    static_assert(!(AMN || BMN) || ((OP::BITS == 16 || OP::BITS == 8) && !OP::MX && !OP::W4),
                  "MN-major: 16- and 8-bit types");
    constexpr int EB = AMN || BMN ? OP::BITS / 8 : 2; // bytes per element (MN-major)
    constexpr int KR = BKB / EB;                    // K rows of an MN-major tile
    constexpr int TR = 8 / EB;                      // K values per transposing read
    constexpr int NTR = OP::LANE_BYTES / EB / TR;   // reads per fragment and step
    constexpr int HS = TR * NTR;                    // K rows between the lane halves
    constexpr int LTR = TR == 4 ? 2 : 3, LNT = NTR == 2 ? 1 : (NTR == 4 ? 2 : 0);
    static_assert(!(AMN || BMN) || (1 << LNT) == NTR, "reads per fragment: 2 or 4");
    constexpr int PAD = EB == 2 ? 64 : 32;
    constexpr int APITCH = BM * EB + PAD, BPITCH = BN * EB + PAD;
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
        AMN ? tile_rsrc((const uint8_t *)g.A + m_blk * EB, ((g.K - 1) * g.a_cs + g.e.M - m_blk) * EB)
            : tile_rsrc((const uint8_t *)g.A + m_blk * lda_b, (g.e.M - m_blk - 1) * lda_b + kbytes);
    const __amdgpu_buffer_rsrc_t rb =
        BMN ? tile_rsrc((const uint8_t *)g.B + n_blk * EB, ((g.K - 1) * g.b_rs + g.e.N - n_blk) * EB)
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
    constexpr int CHA = BM * EB / 16, CHB = BN * EB / 16, RPA = NT / CHA, RPB = NT / CHB;
    static_assert(!AMN || KR / RPA == A_LD, "MN-major A: same load count");
    static_assert(!BMN || KR / RPB == B_LD, "MN-major B: same load count");
    auto mn_slot = [](int r) STG_AI {
        const int e = r & (TR - 1), t = (r >> LTR) & (NTR - 1), h = (r >> (LTR + LNT)) & 1;
        return (r & ~(2 * HS - 1)) | (t << (LTR + 1)) | (h << LTR) | e;
    };
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
            *(u4_t *)(stage_base + la0 + a_pass(i)) = AU ? ga[S][i] ^ U8_FLIP : ga[S][i];
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
                *(u4_t *)(stage_base + lb0 + b_pass(i)) = BU ? gb[S][i] ^ U8_FLIP : gb[S][i];
        }
    };

    // fragment reads: lane reads rows arow + 32 i (A) and brow + 32 j (B)
    const int wm = wave / GN, wn = wave % GN;
    const int arow = wm * WM + (lane & 31), brow = wn * WN + (lane & 31);
    const int half = lane >> 5;
    const int sa = swz64(arow), sb = swz64(brow); // same for every fragment row
    const int a_off = arow * BKB, b_off = A_TILE + brow * BKB;
    // MN-major fragments: NT_R transposing reads per fragment and step, K
    // values t TR .. t TR + TR - 1 of the lane half.  Lane 16 q + j reads K
    // row s 2HS + (q / 2) HS + t TR + j / (16 / TR), i.e. slot s 2HS + t 2TR +
    // (q / 2) TR + j / (16 / TR), at MN columns 16 (q % 2) + (j % (16 / TR)) TR
    // .. + TR - 1 of fragment i (+ 32 i)
    const int tr_slot = TR * (lane >> 5) + ((lane & 15) >> (4 - LTR));
    const int tr_col = EB * (16 * ((lane >> 4) & 1) + (lane & ((16 >> LTR) - 1)) * TR);
    const int a_tr = tr_slot * APITCH + EB * wm * WM + tr_col;
    const int b_tr = A_TILE + tr_slot * BPITCH + EB * wn * WN + tr_col;

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
                for (int t = 0; t < NTR; ++t)
                    lds_read_tr<EB>(stage_base + a_tr + (2 * HS * s + 2 * TR * t) * APITCH +
                                        32 * EB * i,
                                    &fa[S][i][2 * t]);
        }
        if constexpr (BMN) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int t = 0; t < NTR; ++t)
                    lds_read_tr<EB>(stage_base + b_tr + (2 * HS * s + 2 * TR * t) * BPITCH +
                                        32 * EB * j,
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
    int usum_a[FM] = {}, usum_b[FN] = {}; // unsigned operands: see mma
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
            // unsigned operands: this lane's sums of the other operand's
            // shifted values (rows of A when B is unsigned, columns of B when
            // A is unsigned)
            if constexpr (BU)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int w = 0; w < FW; ++w)
                        usum_a[i] = sum4_s8(fa[S][i][w], usum_a[i]);
            if constexpr (AU)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int w = 0; w < FW; ++w)
                        usum_b[j] = sum4_s8(fb[S][j][w], usum_b[j]);
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
    constexpr int NM = FM * FN, NR = FM * (AMN ? NTR : NV) + FN * (BMN ? NTR : NV);
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

    if constexpr (AU || BU)
        u8_correct<AU, BU>(acc, usum_a, usum_b, g.K, lane);
    __syncthreads(); // every wave is done with the LDS stages
    epilogue_grid_lds<OP, FM, FN>(g.e, acc, m_blk + wm * WM, n_blk + wn * WN, lane,
                                  (uint32_t *)lds + wave * 32 * (WN + 4));
}


template <class OP, int BM, int BN, int GM = 2, int GN = 2, int WPC = 1>
static hipError_t launch_tiled_t(const GemmArgs &g, hipStream_t s)
{
    const int tiles_m = (int)((g.e.M + BM - 1) / BM), tiles_n = (int)((g.e.N + BN - 1) / BN);
    hipLaunchKernelGGL((k_tiled<OP, BM, BN, GM, GN, WPC>), dim3((unsigned)(tiles_m * tiles_n)),
                       dim3(64 * GM * GN), 0, s, g, tiles_m, tiles_n);
    return hipGetLastError();
}

} // namespace stg
