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
//   - LDS holds two K tiles (double buffer): tile k+1 is loaded into registers
//     while tile k is multiplied, then written to the other buffer; one
//     barrier per K tile;
//   - 16-byte chunks are XOR-swizzled within a row (chunk c of row r sits at
//     slot c ^ (((r >> 1) ^ (r >> 3)) & 3)) so the 32 rows that one fragment
//     read touches spread over all banks - the bank-conflict remedy of the same page's
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

template <int ELEM, int LE>
__device__ inline void load_frag_strided(uint32_t *out, const void *base, bool row_ok,
                                         int64_t row_off, int64_t kstride, int64_t k0, int64_t K)
{
    if constexpr (ELEM == 2) {
        const uint16_t *p = (const uint16_t *)base;
#pragma unroll
        for (int j = 0; j < LE; j += 2) {
            uint32_t lo = 0, hi = 0;
            if (row_ok && k0 + j < K)
                lo = p[row_off + (k0 + j) * kstride];
            if (row_ok && k0 + j + 1 < K)
                hi = p[row_off + (k0 + j + 1) * kstride];
            out[j / 2] = lo | (hi << 16);
        }
    } else {
        const uint8_t *p = (const uint8_t *)base;
#pragma unroll
        for (int j = 0; j < LE; j += 4) {
            uint32_t w = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (row_ok && k0 + j + q < K)
                    w |= (uint32_t)p[row_off + (k0 + j + q) * kstride] << (8 * q);
            out[j / 4] = w;
        }
    }
}

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

// Tile-local buffer resource: loads at byte offsets >= `bytes` return zero,
// so rows past the edge of the matrix need no clamping or masking.
__device__ inline __amdgpu_buffer_rsrc_t tile_rsrc(const void *base, int64_t bytes)
{
    const int n = bytes > 0x7fffffff ? 0x7fffffff : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, n, 0x00020000);
}

__device__ inline u4_t buf_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    return __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// 16-byte chunk slot inside a 64-byte LDS row: chunk c of row r sits at slot
// c ^ swz64(r).  Any 8 consecutive rows (32 banks x 4 B) and any 16
// consecutive rows (64 banks x 4 B) reading the same chunk hit distinct
// bank groups.  swz64(r + 32 i) == swz64(r).
__device__ inline int swz64(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

// Workgroup id -> (tile_m, tile_n): XCD-contiguous renumbering, then groups
// of GM tile rows walked column by column.
__device__ inline void tile_coords(int id, int tiles_m, int tiles_n, int &tm, int &tn)
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

template <class OP, int BM, int BN>
__global__ __launch_bounds__(256, 1) void k_tiled(GemmArgs g, int tiles_m, int tiles_n)
{
    constexpr int BKB = 64;                 // K bytes per tile
    constexpr int CH = BKB / 16;            // 16-byte chunks per row
    constexpr int RPP = 256 / CH;           // rows covered per load pass
    constexpr int A_LD = BM / RPP, B_LD = BN / RPP;
    constexpr int WM = BM / 2, WN = BN / 2; // wave sub-tile (2 x 2 waves)
    constexpr int FM = WM / 32, FN = WN / 32;
    constexpr int STAGE = (BM + BN) * BKB;
    constexpr int NV = OP::LANE_BYTES / 16; // 16-byte LDS reads per operand
    constexpr int KSTEPS = BKB / OP::KB;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int64_t m_blk = (int64_t)tm * BM, n_blk = (int64_t)tn * BN;
    const int64_t lda_b = g.a_rs * OP::ELEM, ldb_b = g.b_cs * OP::ELEM;
    const int KT = (int)(g.K * OP::ELEM / BKB);
    const __amdgpu_buffer_rsrc_t ra =
        tile_rsrc((const uint8_t *)g.A + m_blk * lda_b, (g.e.M - m_blk) * lda_b);
    const __amdgpu_buffer_rsrc_t rb =
        tile_rsrc((const uint8_t *)g.B + n_blk * ldb_b, (g.e.N - n_blk) * ldb_b);

    // global -> LDS copy: thread owns chunk `ch` of rows r0 + i*RPP
    const int ch = tid % CH, r0 = tid / CH;
    const int va0 = r0 * (int)lda_b + ch * 16, vb0 = r0 * (int)ldb_b + ch * 16;
    const int va_step = RPP * (int)lda_b, vb_step = RPP * (int)ldb_b;
    const int l0 = r0 * BKB + ((ch ^ swz64(r0)) << 4); // + i*RPP*BKB (swz64 is RPP-periodic)

    u4_t pa[A_LD], pb[B_LD];
    auto gload = [&](int kt) {
        const int soff = kt * BKB;
#pragma unroll
        for (int i = 0; i < A_LD; ++i)
            pa[i] = buf_load16(ra, va0 + i * va_step, soff);
#pragma unroll
        for (int i = 0; i < B_LD; ++i)
            pb[i] = buf_load16(rb, vb0 + i * vb_step, soff);
    };
    auto lstore = [&](int stage) {
        uint8_t *base = lds + stage * STAGE + l0;
#pragma unroll
        for (int i = 0; i < A_LD; ++i)
            *(u4_t *)(base + i * RPP * BKB) = pa[i];
#pragma unroll
        for (int i = 0; i < B_LD; ++i)
            *(u4_t *)(base + BM * BKB + i * RPP * BKB) = pb[i];
    };

    // fragment reads: lane reads rows arow + 32 i (A) and brow + 32 j (B)
    const int wm = wave >> 1, wn = wave & 1;
    const int arow = wm * WM + (lane & 31), brow = wn * WN + (lane & 31);
    const int half = lane >> 5;
    const int sa = swz64(arow), sb = swz64(brow); // same for every fragment row

    typename OP::acc_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = typename OP::acc_t{};

    gload(0);
    lstore(0);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < KT;
        if (more)
            gload(kt + 1);
        const uint8_t *lsa = lds + cur * STAGE + arow * BKB;
        const uint8_t *lsb = lds + cur * STAGE + BM * BKB + brow * BKB;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            uint32_t af[FM][OP::LANE_BYTES / 4], bf[FN][OP::LANE_BYTES / 4];
            const int c0 = (s * OP::KB + half * OP::LANE_BYTES) >> 4;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int oa = ((c0 + v) ^ sa) << 4, ob = ((c0 + v) ^ sb) << 4;
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    *(u4_t *)&af[i][4 * v] = *(const u4_t *)(lsa + i * 32 * BKB + oa);
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    *(u4_t *)&bf[j][4 * v] = *(const u4_t *)(lsb + j * 32 * BKB + ob);
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = OP::mma(af[i], bf[j], acc[i][j]);
        }
        if (more)
            lstore(cur ^ 1);
        __syncthreads();
    }

    epilogue_grid<OP, FM, FN>(g.e, acc, m_blk + wm * WM, n_blk + wn * WN, lane);
}

// ---------------------------------------------------------------- launch

template <class OP>
static hipError_t launch_generic_t(const GemmArgs &g, hipStream_t s)
{
    dim3 grid((unsigned)((g.e.N + 63) / 64), (unsigned)((g.e.M + 63) / 64));
    hipLaunchKernelGGL(k_generic<OP>, grid, dim3(256), 0, s, g);
    return hipGetLastError();
}

template <class OP, int BM, int BN>
static hipError_t launch_tiled_t(const GemmArgs &g, hipStream_t s)
{
    const int tiles_m = (int)((g.e.M + BM - 1) / BM), tiles_n = (int)((g.e.N + BN - 1) / BN);
    hipLaunchKernelGGL((k_tiled<OP, BM, BN>), dim3((unsigned)(tiles_m * tiles_n)), dim3(256), 0,
                       s, g, tiles_m, tiles_n);
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

template <int BM, int BN>
static dense_launch_fn tiled_table_t(int op)
{
    switch (op) {
    case OPK_F16: return launch_tiled_t<OpF16, BM, BN>;
    case OPK_BF16: return launch_tiled_t<OpBF16, BM, BN>;
    case OPK_F8_E4E4: return launch_tiled_t<OpF8<0, 0>, BM, BN>;
    case OPK_F8_E4E5: return launch_tiled_t<OpF8<0, 1>, BM, BN>;
    case OPK_F8_E5E4: return launch_tiled_t<OpF8<1, 0>, BM, BN>;
    case OPK_F8_E5E5: return launch_tiled_t<OpF8<1, 1>, BM, BN>;
    case OPK_S8: return launch_tiled_t<OpS8, BM, BN>;
    default: return nullptr;
    }
}

hipError_t launch_dense(int family, int op, const GemmArgs &g, hipStream_t s)
{
    dense_launch_fn fn = nullptr;
    switch (family) {
    case KF_GENERIC: fn = generic_table(op); break;
    case KF_TILED_256: fn = tiled_table_t<256, 256>(op); break;
    case KF_TILED_128: fn = tiled_table_t<128, 128>(op); break;
    default: break;
    }
    if (!fn)
        return hipErrorInvalidValue;
    return fn(g, s);
}

} // namespace stg
