// 2:4 structured-sparse A kernels for gfx950: the compressor, a generic path
// and the SMFMAC tiled path.
//
// Format ("NVIDIA MMA" (rainlin-net), section "Dense and 2:4 structured
// sparse multiplication"): every 4 consecutive K positions of a row of A keep
// 2 values and their positions; B, C and D stay dense.  Packing (this
// library's own; the pages give index values only): group g of row m is
// positions 4g..4g+3, its kept positions i0 < i1 are stored as the nibble
// i0 | i1 << 2 at bits 4(g%8).. of meta[m*ceil(K/32) + g/8], and its two
// values at values[m*(K/2) + 2g], [.. + 2g+1].
//
// k_sparse_generic: one wave per 32x32 output tile; each lane expands its
//   8-element K slice of A from (values, meta) into a dense fragment and runs
//   the dense 32x32x16 fp16 MFMA.  Any B layout / stride, any K % 4 == 0.
// k_sparse_tiled: the dense k_tiled structure (LDS double buffer, XOR
//   swizzle, 2x2 waves of 32x32 fragments) with A staged in compressed form
//   and multiplied by v_smfmac_f32_32x32x32_f16, which reads the 2-bit
//   positions from an index register and skips the dropped half of A - the
//   "twice the K per instruction" of the page's sparse MMA.
#include "device_common.hpp"
#include "internal.hpp"

namespace stg {

typedef _Float16 h16v_t __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------- compress

__device__ STG_AI inline bool f16_nonzero(uint32_t h) { return (h & 0x7FFFu) != 0; }

// One thread per (row, metadata word): groups 8w .. 8w+7 of row m.
__global__ __launch_bounds__(256) void k_sparse24_compress(int64_t M, int64_t K,
                                                           const uint16_t *__restrict__ A,
                                                           uint16_t *__restrict__ values,
                                                           uint32_t *__restrict__ meta, int *flag)
{
    const int64_t W = (K + 31) / 32, G = K / 4;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= M * W)
        return;
    const int64_t m = t / W, w = t % W;
    uint32_t word = 0;
    bool bad = false;
    for (int q = 0; q < 8; ++q) {
        const int64_t g = 8 * w + q;
        if (g >= G)
            break;
        // 8-byte load of the group (A is 8-byte aligned and K % 4 == 0)
        const uint2 v = *(const uint2 *)(A + m * K + 4 * g);
        const uint32_t e[4] = {v.x & 0xFFFFu, v.x >> 16, v.y & 0xFFFFu, v.y >> 16};
        int kept[2] = {0, 0}, nk = 0, nz = 0;
        for (int i = 0; i < 4; ++i)
            if (f16_nonzero(e[i])) {
                if (nk < 2)
                    kept[nk++] = i;
                ++nz;
            }
        bad |= nz > 2;
        // fewer than two non-zeros: add the lowest positions not yet kept
        for (int i = 0; i < 4 && nk < 2; ++i)
            if (nk == 0 || kept[0] != i)
                kept[nk++] = i;
        const int i0 = min(kept[0], kept[1]), i1 = max(kept[0], kept[1]);
        word |= (uint32_t)(i0 | (i1 << 2)) << (4 * q);
        *(uint32_t *)(values + m * (K / 2) + 2 * g) = e[i0] | (e[i1] << 16);
    }
    meta[m * W + w] = word;
    if (bad)
        atomicMax(flag, (int)(0x7fffffff - m));
}

hipError_t launch_sparse24_compress(int64_t M, int64_t K, const uint16_t *A, uint16_t *values,
                                    uint32_t *meta, int *flag, hipStream_t s)
{
    const int64_t threads = M * ((K + 31) / 32);
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_sparse24_compress, dim3((unsigned)blocks), dim3(256), 0, s, M, K, A,
                       values, meta, flag);
    return hipGetLastError();
}

// ---------------------------------------------------------------- generic

__global__ __launch_bounds__(256) void k_sparse_generic(SparseArgs a)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t m0 = (int64_t)blockIdx.y * 64 + (wave >> 1) * 32;
    const int64_t n0 = (int64_t)blockIdx.x * 64 + (wave & 1) * 32;
    if (m0 >= a.e.M || n0 >= a.e.N)
        return;
    const int64_t am = m0 + (lane & 31), bn = n0 + (lane & 31);
    const bool a_ok = am < a.e.M, b_ok = bn < a.e.N;
    const int64_t K = a.K, W = (K + 31) / 32;
    const uint16_t *B = (const uint16_t *)a.B;
    f16_t acc = {};
    for (int64_t k0 = 0; k0 < K; k0 += 16) {
        const int64_t kb = k0 + (lane >> 5) * 8; // this lane's 8 K positions = 2 groups
        uint16_t av[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        uint16_t bv[8];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int64_t g = kb / 4 + q;
            if (a_ok && 4 * g < K) {
                const uint32_t nib = (a.meta[am * W + g / 8] >> (4 * (g % 8))) & 0xFu;
                av[4 * q + (nib & 3)] = a.values[am * (K / 2) + 2 * g];
                av[4 * q + (nib >> 2)] = a.values[am * (K / 2) + 2 * g + 1];
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
            bv[j] = (b_ok && kb + j < K) ? B[(kb + j) * a.b_rs + bn * a.b_cs] : (uint16_t)0;
        uint32_t aw[4], bw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            aw[j] = av[2 * j] | ((uint32_t)av[2 * j + 1] << 16);
            bw[j] = bv[2 * j] | ((uint32_t)bv[2 * j + 1] << 16);
        }
        acc = OpF16::mma(aw, bw, acc);
    }
    f16_t grid[1][1] = {{acc}};
    epilogue_grid<OpF16, 1, 1>(a.e, grid, m0, n0, lane);
}

// ---------------------------------------------------------------- tiled

// Chunk swizzles: 128-byte rows (B tile) and 64-byte rows (compressed A).
__device__ STG_AI inline int swz128(int r) { return (r ^ (r >> 3)) & 7; }
__device__ STG_AI inline int swz64(int r) { return (r >> 2) & 3; }

__device__ STG_AI inline void tile_coords_sp(int id, int tiles_m, int tiles_n, int &tm, int &tn)
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

// v_smfmac_f32_32x32x32_f16 covers 32 logical K positions k0..k0+31.  Lane l
// (h = l / 32) supplies, for row l % 32 of A, the 8 kept values of logical K
// 16h .. 16h+15 (4 groups, in group order) and their position code in the
// low 16 bits of the index register (nibble g = group g, first position in
// the low 2 bits; abid selects the register's upper half instead); for
// column l % 32 of B it supplies K 8h .. 8h+7 in elements 0..7 and
// 16+8h .. 16+8h+7 in elements 8..15.  (Measured on gfx950 with single-
// instruction probes; it is exactly this library's nibble packing.)
__device__ STG_AI inline f16_t smfmac32(const uint32_t *a, const uint32_t *b, int idx, f16_t c)
{
    h8_t va = __builtin_bit_cast(h8_t, *(const u4_t *)a);
    h16v_t vb = __builtin_bit_cast(h16v_t, *(const i8_t *)b);
    return __builtin_amdgcn_smfmac_f32_32x32x32_f16(va, vb, c, idx, 0, 0);
}

template <int BM, int BN>
__global__ __launch_bounds__(256, 1) void k_sparse_tiled(SparseArgs a, int tiles_m, int tiles_n)
{
    constexpr int BK = 64;               // logical K per tile
    constexpr int AVB = BK;              // compressed value bytes per row (BK/2 halfs)
    constexpr int AMB = BK / 8;          // metadata bytes per row (BK/4 nibbles)
    constexpr int BB = BK * 2;           // B bytes per row
    constexpr int WM = BM / 2, WN = BN / 2, FM = WM / 32, FN = WN / 32;
    constexpr int OFF_M = BM * AVB, OFF_B = OFF_M + BM * AMB;
    constexpr int STAGE = OFF_B + BN * BB;
    constexpr int AV_LD = BM * (AVB / 16) / 256; // 16-byte chunks per thread
    constexpr int B_LD = BN * (BB / 16) / 256;
    static_assert(BM <= 256, "one metadata row per thread");
    static_assert(4 * 32 * (WN + 4) * 4 <= 2 * STAGE, "epilogue staging fits in LDS");
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int tm, tn;
    tile_coords_sp(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int64_t m_blk = (int64_t)tm * BM, n_blk = (int64_t)tn * BN;
    const int64_t K = a.K, KT = K / BK;
    const int64_t vpitch = K, mpitch = K / 8; // bytes per row of values / meta
    const int64_t bpitch = a.b_cs * 2;

    const uint8_t *gv[AV_LD];
    const uint8_t *gb[B_LD];
    int lv[AV_LD], lb[B_LD];
    {
        constexpr int CHV = AVB / 16, RPV = 256 / CHV;
        const int ch = tid % CHV, r0 = tid / CHV;
#pragma unroll
        for (int i = 0; i < AV_LD; ++i) {
            const int r = r0 + i * RPV;
            const int64_t gm = min(m_blk + r, a.e.M - 1);
            gv[i] = (const uint8_t *)a.values + gm * vpitch + ch * 16;
            lv[i] = r * AVB + ((ch ^ swz64(r)) << 4);
        }
    }
    {
        constexpr int CHB = BB / 16, RPB = 256 / CHB;
        const int ch = tid % CHB, r0 = tid / CHB;
#pragma unroll
        for (int i = 0; i < B_LD; ++i) {
            const int r = r0 + i * RPB;
            const int64_t gn = min(n_blk + r, a.e.N - 1);
            gb[i] = (const uint8_t *)a.B + gn * bpitch + ch * 16;
            lb[i] = OFF_B + r * BB + ((ch ^ swz128(r)) << 4);
        }
    }
    const bool meta_row = tid < BM;
    const uint8_t *gmeta =
        (const uint8_t *)a.meta + min(m_blk + (meta_row ? tid : 0), a.e.M - 1) * mpitch;

    u4_t pv[AV_LD], pb[B_LD];
    uint2 pm = {0, 0};
    // K-tile rotation: workgroup w starts its K loop at tile 2 (w / 8) mod KT
    // and wraps, so workgroups running side by side on an XCD read different
    // K slices (with power-of-two row pitches one K slice of all rows falls
    // into few L2 channels).  Measured faster here; the dense kernels, whose
    // workgroups share A and B slices in L2, are faster without it.  Each
    // tile's summation order stays fixed.
    const int rot = KT > 0 ? (int)(((blockIdx.x >> 3) * 2) % (unsigned)KT) : 0;
    auto gload = [&](int64_t kt0) STG_AI {
        const int64_t kt = kt0 + rot >= KT ? kt0 + rot - KT : kt0 + rot;
#pragma unroll
        for (int i = 0; i < AV_LD; ++i)
            pv[i] = *(const u4_t *)(gv[i] + kt * AVB);
#pragma unroll
        for (int i = 0; i < B_LD; ++i)
            pb[i] = *(const u4_t *)(gb[i] + kt * BB);
        if (meta_row)
            pm = *(const uint2 *)(gmeta + kt * AMB);
    };
    auto lstore = [&](int stage) STG_AI {
        uint8_t *base = lds + stage * STAGE;
#pragma unroll
        for (int i = 0; i < AV_LD; ++i)
            *(u4_t *)(base + lv[i]) = pv[i];
#pragma unroll
        for (int i = 0; i < B_LD; ++i)
            *(u4_t *)(base + lb[i]) = pb[i];
        if (meta_row)
            *(uint2 *)(base + OFF_M + tid * AMB) = pm;
    };

    const int wm = wave >> 1, wn = wave & 1;
    const int arow = wm * WM + (lane & 31), brow = wn * WN + (lane & 31);
    const int half = lane >> 5;

    f16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = f16_t{};

    gload(0);
    lstore(0);
    __syncthreads();

    for (int64_t kt = 0; kt < KT; ++kt) {
        const int cur = (int)(kt & 1);
        const bool more = kt + 1 < KT;
        if (more)
            gload(kt + 1);
        const uint8_t *st = lds + cur * STAGE;
#pragma unroll
        for (int s = 0; s < BK / 32; ++s) {
            uint32_t af[FM][4], bf[FN][8];
            int ix[FM];
            // compressed A: 16 bytes at value byte s*32 + half*16
            const int ca = (s * 32 + half * 16) >> 4;
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int r = arow + i * 32;
                *(u4_t *)af[i] = *(const u4_t *)(st + r * AVB + ((ca ^ swz64(r)) << 4));
                const uint32_t w = *(const uint32_t *)(st + OFF_M + r * AMB + s * 4);
                ix[i] = (int)((w >> (16 * half)) & 0xFFFFu);
            }
            // B: 16-byte chunks 4s + half (K 8h..8h+7 of the slice) and
            // 4s + half + 2 (K 16+8h..)
            const int cb = 4 * s + half;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int r = brow + j * 32;
                *(u4_t *)&bf[j][0] = *(const u4_t *)(st + OFF_B + r * BB + ((cb ^ swz128(r)) << 4));
                *(u4_t *)&bf[j][4] =
                    *(const u4_t *)(st + OFF_B + r * BB + (((cb + 2) ^ swz128(r)) << 4));
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = smfmac32(af[i], bf[j], ix[i], acc[i][j]);
        }
        if (more)
            lstore(cur ^ 1);
        __syncthreads();
    }

    __syncthreads(); // every wave is done with the LDS stages
    epilogue_grid_lds<OpF16, FM, FN>(a.e, acc, m_blk + wm * WM, n_blk + wn * WN, lane,
                                     (uint32_t *)lds + wave * 32 * (WN + 4));
}

hipError_t launch_sparse(int family, const SparseArgs &a, hipStream_t s)
{
    if (family == KF_SPARSE_GENERIC) {
        dim3 grid((unsigned)((a.e.N + 63) / 64), (unsigned)((a.e.M + 63) / 64));
        hipLaunchKernelGGL(k_sparse_generic, grid, dim3(256), 0, s, a);
        return hipGetLastError();
    }
    if (family == KF_SPARSE_TILED) {
        constexpr int BM = 256, BN = 256;
        const int tiles_m = (int)((a.e.M + BM - 1) / BM), tiles_n = (int)((a.e.N + BN - 1) / BN);
        hipLaunchKernelGGL((k_sparse_tiled<BM, BN>), dim3((unsigned)(tiles_m * tiles_n)),
                           dim3(256), 0, s, a, tiles_m, tiles_n);
        return hipGetLastError();
    }
    return hipErrorInvalidValue;
}

} // namespace stg
