// 2:4 structured-sparse A kernels for gfx950: the compressor, a generic path
// and the SMFMAC tiled paths, for f16, bf16, s8 and fp8 (E4M3/E5M2) A.
//
// Format ("NVIDIA MMA" (rainlin-net), section "Dense and 2:4 structured
// sparse multiplication"; the sparse rows of the instruction tables in the
// sections "Ampere: FP16/BF16 and integer MMA baseline" and "Ada: mma.sync
// adds FP8" apply it to BF16, INT8 and FP8): every 4 consecutive K positions
// of a row of A keep 2 values and their positions; B, C and D stay dense.
// Packing (this library's own; the pages give index values only): group g of
// row m is positions 4g..4g+3, its kept positions i0 < i1 are stored as the
// nibble i0 | i1 << 2 at bits 4(g%8).. of meta[m*ceil(K/32) + g/8], and its
// two values (elements of A's type) at values[m*(K/2) + 2g], [.. + 2g+1].
//
// k_sparse_generic: one wave per 32x32 output tile; each lane expands its K
//   slice of A from (values, meta) into a dense fragment and runs the dense
//   MFMA of the type.  Any B layout / stride, any K % 4 == 0.
// k_sparse_tiled: the dense k_tiled structure (LDS double buffer, XOR
//   swizzle, 2x2 waves of 32x32 fragments) with A staged in compressed form
//   and multiplied by the SMFMAC of the type, which reads the 2-bit positions
//   from an index register and skips the dropped half of A - the "twice the
//   K per instruction" of the page's sparse MMA.
// k_sparse_dma8: 8 waves, direct global -> LDS copies (the fast path).
#include <mutex>

#include "device_common.hpp"
#include "internal.hpp"

namespace stg {

typedef _Float16 h16v_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16v_t __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------- operations

// The 2:4 operation of an A/B type pair: the gfx950 SMFMAC 32x32 form and the
// dense MFMA form (Dense) the generic kernel uses.  Every SMFMAC lane gives 16
// bytes of kept A values, 32 bytes of B and an index register (lane l, row or
// column l % 32, h = l / 32):
//  - 16-bit types, 32x32x32: the 8 kept values of logical K 16h .. 16h+15 (4
//    groups, group order) with their codes in the low 16 bits of the index
//    (nibble g = group g, first position in the low 2 bits; abid = 1 would
//    select the upper half instead); B elements 0..7 = K 8h .. 8h+7 and
//    8..15 = K 16+8h .. 16+8h+7;
//  - 8-bit types, 32x32x64: the 16 kept values of logical K 32h .. 32h+31 (8
//    groups) with their codes in all 32 bits of the index; B bytes 0..15 =
//    K 16h .. 16h+15 and 16..31 = K 32+16h .. 32+16h+15.
// In bytes the two are alike: A at byte 16h of the step's 32 value bytes, B
// in 16-byte chunks h and h+2 of the step's 64 bytes.  (Measured on gfx950
// with single-instruction probes.  A product fixes the A and B layouts only
// up to one common permutation of K; these are the forms this library uses.)
// The fp8 forms read OCP E4M3 ("fp8") and E5M2 ("bf8").
template <class D>
struct SpOpBase {
    typedef D Dense;
    typedef typename D::acc_t acc_t;
    static constexpr int ELEM = D::ELEM;
    static constexpr int KI = ELEM == 2 ? 32 : 64; // logical K per SMFMAC
    // index register of lane half `half` for K step s of a tile whose
    // metadata row is the words w[0 .. KI/8 - 1] (8 bytes per step of 8-bit
    // types, 4 of 16-bit types): its word and the bits it uses
    __device__ static STG_AI int word_of_step(int s, int half)
    {
        return ELEM == 2 ? s : 2 * s + half;
    }
    __device__ static STG_AI int index_of(uint32_t w, int half)
    {
        return ELEM == 2 ? (int)((w >> (16 * half)) & 0xFFFFu) : (int)w;
    }
};

struct SpF16 : SpOpBase<OpF16> {
    __device__ static STG_AI acc_t smfmac(const uint32_t *a, const uint32_t *b, int idx, acc_t c)
    {
        return __builtin_amdgcn_smfmac_f32_32x32x32_f16(__builtin_bit_cast(h8_t, *(const u4_t *)a),
                                                        __builtin_bit_cast(h16v_t, *(const i8_t *)b),
                                                        c, idx, 0, 0);
    }
};

struct SpBF16 : SpOpBase<OpBF16> {
    __device__ static STG_AI acc_t smfmac(const uint32_t *a, const uint32_t *b, int idx, acc_t c)
    {
        return __builtin_amdgcn_smfmac_f32_32x32x32_bf16(
            __builtin_bit_cast(bf8_t, *(const u4_t *)a), __builtin_bit_cast(bf16v_t, *(const i8_t *)b),
            c, idx, 0, 0);
    }
};

struct SpS8 : SpOpBase<OpS8> {
    __device__ static STG_AI acc_t smfmac(const uint32_t *a, const uint32_t *b, int idx, acc_t c)
    {
        return __builtin_amdgcn_smfmac_i32_32x32x64_i8(*(const i4_t *)a, *(const i8_t *)b, c, idx, 0,
                                                       0);
    }
};

// 8-bit integers of either signedness (OpI8): the signed SMFMAC on the
// shifted values x - 128 of an unsigned operand, corrected afterwards (the
// SMFMAC kernel takes an unsigned B only; an unsigned A runs the generic
// kernel, where the dropped positions are explicit zeros)
template <bool AU, bool BU>
struct SpI8 : SpOpBase<OpI8<AU, BU>> {
    typedef i16_t acc_t;
    __device__ static STG_AI acc_t smfmac(const uint32_t *a, const uint32_t *b, int idx, acc_t c)
    {
        return SpS8::smfmac(a, b, idx, c);
    }
};

// AFMT / BFMT: 0 = E4M3, 1 = E5M2 (the selectors of OpF8)
template <int AFMT, int BFMT>
struct SpF8 : SpOpBase<OpF8<AFMT, BFMT>> {
    typedef f16_t acc_t;
    __device__ static STG_AI acc_t smfmac(const uint32_t *a, const uint32_t *b, int idx, acc_t c)
    {
        const i4_t va = *(const i4_t *)a;
        const i8_t vb = *(const i8_t *)b;
        if constexpr (AFMT == 0 && BFMT == 0)
            return __builtin_amdgcn_smfmac_f32_32x32x64_fp8_fp8(va, vb, c, idx, 0, 0);
        else if constexpr (AFMT == 0)
            return __builtin_amdgcn_smfmac_f32_32x32x64_fp8_bf8(va, vb, c, idx, 0, 0);
        else if constexpr (BFMT == 0)
            return __builtin_amdgcn_smfmac_f32_32x32x64_bf8_fp8(va, vb, c, idx, 0, 0);
        else
            return __builtin_amdgcn_smfmac_f32_32x32x64_bf8_bf8(va, vb, c, idx, 0, 0);
    }
};

// ---------------------------------------------------------------- compress

// One thread per (row, metadata word): groups 8w .. 8w+7 of row m.  EB =
// element bytes; an element is a zero when (bits & zmask) == 0 (0x7FFF for
// f16/bf16 and 0x7F for fp8, so -0 is a zero; 0xFF for s8).
template <int EB>
__global__ __launch_bounds__(256) void k_sparse24_compress(int64_t M, int64_t K,
                                                           const uint8_t *__restrict__ A,
                                                           uint8_t *__restrict__ values,
                                                           uint32_t *__restrict__ meta,
                                                           uint32_t zmask, int *flag)
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
        // one load of the group's 4 elements (A is 4*EB-byte aligned and K % 4 == 0)
        uint32_t e[4];
        if constexpr (EB == 2) {
            const uint2 v = *(const uint2 *)(A + (m * K + 4 * g) * 2);
            e[0] = v.x & 0xFFFFu, e[1] = v.x >> 16, e[2] = v.y & 0xFFFFu, e[3] = v.y >> 16;
        } else {
            const uint32_t v = *(const uint32_t *)(A + m * K + 4 * g);
            e[0] = v & 0xFFu, e[1] = (v >> 8) & 0xFFu, e[2] = (v >> 16) & 0xFFu, e[3] = v >> 24;
        }
        int kept[2] = {0, 0}, nk = 0, nz = 0;
        for (int i = 0; i < 4; ++i)
            if ((e[i] & zmask) != 0) {
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
        if constexpr (EB == 2)
            *(uint32_t *)(values + (m * (K / 2) + 2 * g) * 2) = e[i0] | (e[i1] << 16);
        else
            *(uint16_t *)(values + m * (K / 2) + 2 * g) = (uint16_t)(e[i0] | (e[i1] << 8));
    }
    meta[m * W + w] = word;
    if (bad)
        atomicMax(flag, (int)(0x7fffffff - m));
}

// Fill n ints at p with 0 (clears the compressor's flag in device scratch
// without hipMemsetAsync).
__global__ __launch_bounds__(64) void k_zero_ints(int *p, int n)
{
    for (int i = threadIdx.x; i < n; i += 64)
        p[i] = 0;
}

hipError_t launch_sparse24_compress(int elem_bytes, uint32_t zero_mask, int64_t M, int64_t K,
                                    const void *A, void *values, uint32_t *meta, int *flag,
                                    hipStream_t s)
{
    const int64_t threads = M * ((K + 31) / 32);
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidValue;
    if (elem_bytes == 2)
        hipLaunchKernelGGL(k_sparse24_compress<2>, dim3((unsigned)blocks), dim3(256), 0, s, M, K,
                           (const uint8_t *)A, (uint8_t *)values, meta, zero_mask, flag);
    else if (elem_bytes == 1)
        hipLaunchKernelGGL(k_sparse24_compress<1>, dim3((unsigned)blocks), dim3(256), 0, s, M, K,
                           (const uint8_t *)A, (uint8_t *)values, meta, zero_mask, flag);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

} // namespace stg

// ---------------------------------------------------------------- allocation-free flag

// Device scratch of gemm_sparse24_compress_noalloc: its offending-row flag
// (element 0; the rest is headroom) lives here instead of in memory
// allocated per call.  Every GPU the library runs on holds its own copy
// until the process ends.  Host code never uses the array's name as an
// address: the device address is looked up once per device with
// hipGetSymbolAddress (below) and only that pointer reaches kernels.
static __device__ __align__(256) int scratch[stg::SPARSE24_SCRATCH_INTS];

namespace stg {

namespace {
std::mutex g_scratch_mu;
int *g_scratch_ptr[64]; // per device: the address of `scratch` on that device
} // namespace

hipError_t sparse24_scratch(int dev, int **out)
{
    if (dev < 0 || dev >= 64)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        // the caller made `dev` current
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        g_scratch_ptr[dev] = (int *)p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_zero_ints(int *p, int n, hipStream_t s)
{
    hipLaunchKernelGGL(k_zero_ints, dim3(1), dim3(64), 0, s, p, n);
    return hipGetLastError();
}

// ---------------------------------------------------------------- generic

template <class SP>
__global__ __launch_bounds__(256) void k_sparse_generic(SparseArgs a)
{
    using D = typename SP::Dense;
    constexpr int EB = D::ELEM;
    constexpr int LE = D::LANE_BYTES / EB; // K elements per lane per dense instruction
    constexpr int KI = D::KB / EB;         // K elements per dense instruction
    constexpr int NG = LE / 4;             // groups per lane
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t m0 = (int64_t)blockIdx.y * 64 + (wave >> 1) * 32;
    const int64_t n0 = (int64_t)blockIdx.x * 64 + (wave & 1) * 32;
    if (m0 >= a.e.M || n0 >= a.e.N)
        return;
    const int64_t am = m0 + (lane & 31), bn = n0 + (lane & 31);
    const bool a_ok = am < a.e.M, b_ok = bn < a.e.N;
    const int64_t K = a.K, W = (K + 31) / 32;
    const uint8_t *vals = (const uint8_t *)a.values;
    constexpr bool AU = au_v<D>(), BU = bu_v<D>();
    int rs[1] = {0}, cs[1] = {0}; // unsigned operands: sums of the shifted values
    typename D::acc_t acc = {};
    for (int64_t k0 = 0; k0 < K; k0 += KI) {
        const int64_t kb = k0 + (lane >> 5) * LE; // this lane's LE K positions = NG groups
        uint32_t aw[LE * EB / 4], bw[LE * EB / 4];
#pragma unroll
        for (int i = 0; i < LE * EB / 4; ++i)
            aw[i] = 0;
#pragma unroll
        for (int q = 0; q < NG; ++q) {
            const int64_t g = kb / 4 + q;
            if (a_ok && 4 * g < K) {
                const uint32_t nib = (a.meta[am * W + g / 8] >> (4 * (g % 8))) & 0xFu;
                const int64_t vi = am * (K / 2) + 2 * g;
                const uint32_t v0 = EB == 2 ? ((const uint16_t *)vals)[vi] : vals[vi];
                const uint32_t v1 = EB == 2 ? ((const uint16_t *)vals)[vi + 1] : vals[vi + 1];
                // element 4q + p of the lane's slice: v0 at position i0, v1 at
                // i1, zero elsewhere (compile-time p: no indexed registers)
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const uint32_t x =
                        (int)(nib & 3u) == p ? v0 : ((int)(nib >> 2) == p ? v1 : 0u);
                    const int el = 4 * q + p;
                    aw[el * EB / 4] |= x << (8 * ((el * EB) % 4));
                }
            }
        }
        load_frag_strided<EB, LE>(bw, a.B, b_ok, bn * a.b_cs, a.b_rs, kb, K);
        if constexpr (AU || BU) {
            // unsigned values x enter the MFMA as x - 128 (the dropped
            // positions of A are zeros of u8 like any other); bytes past K
            // stay 0
#pragma unroll
            for (int w = 0; w < LE * EB / 4; ++w) {
                uint32_t m = 0;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    m |= (kb + 4 * w + q < K ? 0x80u : 0u) << (8 * q);
                if constexpr (AU)
                    aw[w] ^= m;
                if constexpr (BU)
                    bw[w] ^= m;
                if constexpr (BU)
                    rs[0] = sum4_s8(aw[w], rs[0]);
                if constexpr (AU)
                    cs[0] = sum4_s8(bw[w], cs[0]);
            }
        }
        acc = D::mma(aw, bw, acc);
    }
    typename D::acc_t grid[1][1] = {{acc}};
    if constexpr (AU || BU)
        u8_correct<AU, BU>(grid, rs, cs, K, lane);
    epilogue_grid<D, 1, 1>(a.e, grid, m0, n0, lane);
}

// ---------------------------------------------------------------- tiled

// A K tile is two SMFMAC steps: 64 logical K of 16-bit types, 128 of 8-bit
// types; in bytes per row both are 64 of compressed values and 128 of B.
template <class SP, int BM, int BN>
__global__ __launch_bounds__(256, 1) void k_sparse_tiled(SparseArgs a, int tiles_m, int tiles_n)
{
    constexpr int EB = SP::ELEM;
    constexpr int BK = 2 * SP::KI;       // logical K per tile
    constexpr int AVB = BK * EB / 2;     // compressed value bytes per row (64)
    constexpr int AMB = BK / 8;          // metadata bytes per row (BK/4 nibbles)
    constexpr int BB = BK * EB;          // B bytes per row (128)
    constexpr int WM = BM / 2, WN = BN / 2, FM = WM / 32, FN = WN / 32;
    constexpr int OFF_M = BM * AVB, OFF_B = OFF_M + BM * AMB;
    constexpr int STAGE = OFF_B + BN * BB;
    constexpr int AV_LD = BM * (AVB / 16) / 256; // 16-byte chunks per thread
    constexpr int B_LD = BN * (BB / 16) / 256;
    static_assert(AVB == 64 && BB == 128, "byte geometry shared by all types");
    static_assert(BM <= 256, "one metadata row per thread");
    static_assert(4 * 32 * (WN + 4) * 4 <= 2 * STAGE, "epilogue staging fits in LDS");
    typedef typename std::conditional<AMB == 8, uint2, u4_t>::type meta_t;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int64_t m_blk = (int64_t)tm * BM, n_blk = (int64_t)tn * BN;
    const int64_t K = a.K, KT = K / BK;
    const int64_t vpitch = K * EB / 2, mpitch = K / 8; // bytes per row of values / meta
    const int64_t bpitch = a.b_cs * EB;

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
    meta_t pm = {};
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
            pm = *(const meta_t *)(gmeta + kt * AMB);
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
            *(meta_t *)(base + OFF_M + tid * AMB) = pm;
    };

    const int wm = wave >> 1, wn = wave & 1;
    const int arow = wm * WM + (lane & 31), brow = wn * WN + (lane & 31);
    const int half = lane >> 5;

    typename SP::acc_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = typename SP::acc_t{};

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
        for (int s = 0; s < 2; ++s) {
            uint32_t af[FM][4], bf[FN][8];
            int ix[FM];
            // compressed A: 16 bytes at value byte s*32 + half*16
            const int ca = (s * 32 + half * 16) >> 4;
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int r = arow + i * 32;
                *(u4_t *)af[i] = *(const u4_t *)(st + r * AVB + ((ca ^ swz64(r)) << 4));
                const uint32_t w =
                    *(const uint32_t *)(st + OFF_M + r * AMB + 4 * SP::word_of_step(s, half));
                ix[i] = SP::index_of(w, half);
            }
            // B: 16-byte chunks 4s + half and 4s + half + 2 of the row
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
                    acc[i][j] = SP::smfmac(af[i], bf[j], ix[i], acc[i][j]);
        }
        if (more)
            lstore(cur ^ 1);
        __syncthreads();
    }

    __syncthreads(); // every wave is done with the LDS stages
    epilogue_grid_lds<typename SP::Dense, FM, FN>(a.e, acc, m_blk + wm * WM, n_blk + wn * WN, lane,
                                                  (uint32_t *)lds + wave * 32 * (WN + 4));
}

// ---------------------------------------------------------------- 8 waves, LDS DMA

// 256 x 256 workgroup tile, 8 waves (two per SIMD) as 2 x 4, each a 128 x 64
// block of 32x32 fragments.  A K tile is two SMFMAC steps (64 logical K of a
// 16-bit type, 128 of an 8-bit type): compressed values (64 B per row) and B
// (128 B per row), 48 KB; three such LDS stages are filled by direct
// global -> LDS copies (tile t+2 is requested while tile t is multiplied,
// and at the barrier that ends tile t each wave has waited for its copies of
// tile t+1).  The metadata (8 or 16 B per row per tile) has a ring of its
// own: two slots of 256 logical K (32 B per row, 8 KB a slot: four tiles of
// a 16-bit type, two of an 8-bit type), the next slot requested at the
// first tile of each group.  Copying the metadata a group at a time cuts its
// L2 requests fourfold or twofold (each row's bytes are a separate request
// however few they are); 3 x 48 KB + 16 KB is the whole 160 KB of LDS.
// Within a slot, each wave's 1 KB copy holds rows 32 w .. 32 w + 31 as two
// 512-byte chunks (logical K 0-127, 128-255 of the group) of 16 bytes per
// row.
// An SMFMAC of the same cost as a dense MFMA reads twice the B bytes per
// lane; gfx950 delivers about twice the LDS read rate with two waves per
// SIMD as with one (measured), and the second wave also covers the first's
// fragment-read latency at the start of each tile.  Within a tile the
// fragments of the second K step are read while the first step's SMFMACs
// run.  Requires K % 256 == 0 (whole metadata groups, 32-byte aligned
// metadata rows).
template <class SP>
__global__ __launch_bounds__(512, 1) void k_sparse_dma8(SparseArgs a, int tiles_m, int tiles_n)
{
    constexpr int EB = SP::ELEM;
    constexpr int BM = 256, BN = 256, BK = 2 * SP::KI; // BK: logical K per tile
    // unsigned B (SpI8<false, true>): its fragments are shifted to x - 128
    // after the LDS reads and the rows' sums of A's kept values restore the
    // exact product; an unsigned A cannot be restored per row here (the
    // SMFMAC skips the dropped positions), so it never reaches this kernel
    constexpr bool BU = bu_v<typename SP::Dense>();
    static_assert(!au_v<typename SP::Dense>(), "unsigned A runs the generic 2:4 kernel");
    constexpr int NSTAGE = 3, MG = 256 / BK;         // LDS stages; tiles per metadata slot
    constexpr int AVB = BK * EB / 2, AMB = BK / 8, BB = BK * EB; // bytes per row per tile
    constexpr int WM = 128, WN = 64, FM = WM / 32, FN = WN / 32, GN = BN / WN;
    constexpr int OFF_B = BM * AVB;
    constexpr int STAGE = OFF_B + BN * BB;
    constexpr int MROW = MG * AMB;             // metadata bytes per row per slot
    constexpr int OFF_META = NSTAGE * STAGE;   // two slots of BM * MROW bytes
    constexpr int LDS_BYTES = OFF_META + 2 * BM * MROW;
    constexpr int V_I = BM * AVB / 1024 / 8;   // 16-byte copies per wave per tile: values
    constexpr int B_I = BN * BB / 1024 / 8;    // B
    constexpr int NI = V_I + B_I;
    static_assert(V_I * 8 * 1024 == BM * AVB && B_I * 8 * 1024 == BN * BB &&
                      BM * MROW == 8 * 1024,
                  "copies divide evenly over the waves; one metadata copy per wave per slot");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    static_assert(AVB == 64 && BB == 128 && MROW == 32, "byte geometry shared by all types");
    static_assert(8 * 32 * (WN + 4) * 4 <= LDS_BYTES, "epilogue staging fits in LDS");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int64_t m_blk = (int64_t)tm * BM, n_blk = (int64_t)tn * BN;
    const int64_t K = a.K;
    const int KT = (int)(K / BK);
    const int64_t vpitch = K * EB / 2, mpitch = K / 8, bpitch = a.b_cs * EB; // bytes per row
    // bounded by the last byte of the last row: copies past it read zero
    // (zero values with position code 0 contribute nothing)
    const __amdgpu_buffer_rsrc_t rv = tile_rsrc((const uint8_t *)a.values + m_blk * vpitch,
                                                (a.e.M - m_blk - 1) * vpitch + vpitch);
    const __amdgpu_buffer_rsrc_t rm =
        tile_rsrc((const uint8_t *)a.meta + m_blk * mpitch, (a.e.M - m_blk - 1) * mpitch + mpitch);
    const __amdgpu_buffer_rsrc_t rb =
        tile_rsrc((const uint8_t *)a.B + n_blk * bpitch, (a.e.N - n_blk - 1) * bpitch + EB * K);

    // this lane's source offsets: a 16-byte copy instruction fills 1 KB of
    // LDS (16 value rows, 8 B rows or 32 metadata rows), lane l writing slot
    // l of it, so the lane fetches the chunk that the row's swizzle maps to
    // that slot (metadata rows are not swizzled)
    int voff[NI];
#pragma unroll
    for (int i = 0; i < V_I; ++i) {
        const int row = (wave * V_I + i) * 16 + (lane >> 2);
        voff[i] = row * (int)vpitch + (((lane & 3) ^ swz64(row)) << 4);
    }
#pragma unroll
    for (int j = 0; j < B_I; ++j) {
        const int row = (wave * B_I + j) * 8 + (lane >> 3);
        voff[V_I + j] = row * (int)bpitch + (((lane & 7) ^ swz128(row)) << 4);
    }
    // metadata: the wave's copy covers rows 32 w .. 32 w + 31; lane l moves
    // 16-byte chunk l / 32 (128 logical K) of row 32 w + l % 32, so in LDS each
    // chunk's 32 rows sit 16 bytes apart (the fragment reads of 32
    // consecutive rows then meet each LDS bank at most twice)
    const int moff = (wave * 32 + (lane & 31)) * (int)mpitch + (lane >> 5) * 16;
    // Every workgroup walks K from the start: workgroups of one XCD that share
    // A or B rows then read the same K slices at about the same time and hit
    // in L2.  (Starting each workgroup at a different K group measured up to
    // 25 % slower here.)  Tiles requested past the end of the loop read
    // bytes that are never used (or zeros past the end of a resource).
    auto dma_tile = [&](int stage, int kt) STG_AI {
        uint8_t *base = lds + stage * STAGE;
#pragma unroll
        for (int i = 0; i < V_I; ++i)
            dma16(rv, base + (wave * V_I + i) * 1024, voff[i], kt * AVB);
#pragma unroll
        for (int j = 0; j < B_I; ++j)
            dma16(rb, base + OFF_B + (wave * B_I + j) * 1024, voff[V_I + j], kt * BB);
    };
    // metadata of tiles t .. t+MG-1 (t a multiple of MG) into ring slot (t / MG) % 2
    auto dma_meta = [&](int t) STG_AI {
        dma16(rm, lds + OFF_META + ((t / MG) & 1) * (BM * MROW) + wave * 1024, moff, t * AMB);
    };

    const int wm = wave / GN, wn = wave % GN;
    const int arow = wm * WM + (lane & 31), brow = wn * WN + (lane & 31);
    const int half = lane >> 5;
    const int sa = swz64(arow); // swz64 is 32-row periodic; swz128 is not
    int sb[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j)
        sb[j] = swz128(brow + 32 * j);

    uint32_t af[2][FM][4], bf[2][FN][8];
    uint2 mw[FM]; // this lane's metadata words of both K steps of a fragment row
    // fragment reads of K step S of tile t from stage `st`
    auto lread = [&](auto set, const uint8_t *st) STG_AI {
        constexpr int S = decltype(set)::value;
        const int ca = 2 * S + half; // value chunk: byte S*32 + half*16
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int r = arow + 32 * i;
            *(u4_t *)af[S][i] = *(const u4_t *)(st + r * AVB + ((ca ^ sa) << 4));
        }
        const int cb = 4 * S + half; // B chunks 4S + half and 4S + half + 2
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int r = brow + 32 * j;
            *(u4_t *)&bf[S][j][0] = *(const u4_t *)(st + OFF_B + r * BB + ((cb ^ sb[j]) << 4));
            *(u4_t *)&bf[S][j][4] =
                *(const u4_t *)(st + OFF_B + r * BB + (((cb + 2) ^ sb[j]) << 4));
        }
    };
    // this lane's metadata words of both K steps of tile t, read in phase B
    // of tile t - 1 (the SMFMAC's index operand must be in a register before
    // the tile's first instruction).  Group g is requested in phase B of the
    // first tile of group g - 1 and is complete and visible from the next
    // tile's barrier on; a group has at least two tiles, so its first
    // tile's metadata is read at the earliest in phase B of the second tile
    // of group g - 1.  The slot the request overwrites held group g - 2,
    // whose last read completed before the barrier of the requesting tile.
    auto mread = [&](int t, uint2 (&dst)[FM]) STG_AI {
        // row r, tile t of the group: block r / 32, chunk (t % MG) * AMB / 16,
        // row r % 32 of the chunk, byte (t % MG) * AMB % 16 of the row's 16
        const int tb = (t % MG) * AMB;
        const uint8_t *meta = lds + OFF_META + ((t / MG) & 1) * (BM * MROW) + (tb >> 4) * 512 +
                              (tb & 15);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int r = arow + 32 * i;
            // two 4-byte reads, which the compiler merges into one: with
            // an 8-byte read written as such it first waits for every
            // pending direct copy into LDS
            const int mo = (r >> 5) * 1024 + (r & 31) * 16;
            dst[i].x = *(const uint32_t *)(meta + mo + 4 * SP::word_of_step(0, half));
            dst[i].y = *(const uint32_t *)(meta + mo + 4 * SP::word_of_step(1, half));
        }
    };
    uint2 mwn[FM]; // the next tile's metadata words

    typename SP::acc_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = typename SP::acc_t{};
    int usum_a[FM] = {}, usum_b[FN] = {}; // unsigned B: row sums of A's kept values
    auto mma = [&](auto set) STG_AI {
        constexpr int S = decltype(set)::value;
        if constexpr (BU) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int w = 0; w < 8; ++w)
                    bf[S][j][w] ^= U8_FLIP;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    usum_a[i] = sum4_s8(af[S][i][w], usum_a[i]);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int idx = SP::index_of(S == 0 ? mw[i].x : mw[i].y, half);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = SP::smfmac(af[S][i], bf[S][j], idx, acc[i][j]);
        }
    };

    // Each tile runs in two phases around one barrier.  Phase A: step 0's
    // SMFMACs (their fragments were read during the previous phase B) with
    // step 1's fragment reads spread among them; then the wait for tile
    // t+1's copies and the barrier.  Phase B: tile t+1's metadata and step-0
    // fragments read, tile t's stage refilled with tile t+NSTAGE (every
    // wave's reads of it completed before the barrier), then step 1's
    // SMFMACs.  So no SMFMAC waits for an LDS read issued in its own phase,
    // and the copies of a tile have a tile and a half to land.
    constexpr int NM = FM * FN, NR = FM + 2 * FN; // SMFMACs and DS reads per step
    auto schedule_a = [&]() STG_AI {
        [&]<int... Q>(std::integer_sequence<int, Q...>) STG_AI {
            (
                [&]() STG_AI {
                    constexpr int nr = spread(Q, NR, NM);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); // MFMA
                    if constexpr (nr > 0)
                        __builtin_amdgcn_sched_group_barrier(0x100, nr, 0); // DS read
                }(),
                ...);
        }(std::make_integer_sequence<int, NM>{});
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;

    // prologue: metadata group 0 and tiles 0 .. NSTAGE-1 requested; wait for
    // group 0 and tile 0, then read tile 0's metadata and step-0 fragments
    // (the compiler fences keep the copies in program order: the waits
    // below count requests in that order)
    dma_meta(0);
    STG_COMPILER_FENCE();
#pragma unroll
    for (int p = 0; p < NSTAGE; ++p)
        dma_tile(p, p);
    STG_WAIT_VMCNT((NSTAGE - 1) * NI);
    lds_barrier();
    mread(0, mw);
    lread(I0{}, lds);

    int st = 0; // LDS stage of tile t
    for (int t = 0; t < KT; ++t) {
        const int sn = st == NSTAGE - 1 ? 0 : st + 1;
        // phase A
        lread(I1{}, lds + st * STAGE);
        mma(I0{});
        schedule_a();
        __builtin_amdgcn_sched_barrier(0);
        // tile t+1 complete: only the requests of the previous phase B (its
        // metadata request, issued first, included) are counted as in flight
        STG_WAIT_VMCNT(NI);
        lds_barrier();
        // phase B.  The reads come before the copies: an LDS read issued
        // after a direct copy into the metadata ring makes the compiler wait
        // for every copy in flight (vmcnt(0)), which would serialise the
        // copy pipeline.  Past the last tile the reads are never used.
        mread(t + 1, mwn);
        lread(I0{}, lds + sn * STAGE);
        STG_COMPILER_FENCE();
        // at the first tile of a group: the group after next's metadata,
        // into the slot whose last reads completed before this barrier
        if ((t % MG) == 0)
            dma_meta(t + MG);
        STG_COMPILER_FENCE();
        dma_tile(st, t + NSTAGE);
        mma(I1{});
        __builtin_amdgcn_sched_barrier(0);
        st = sn;
#pragma unroll
        for (int i = 0; i < FM; ++i)
            mw[i] = mwn[i];
    }
    STG_WAIT_VMCNT(0); // drain the requests past the last tile before the LDS is reused
    if constexpr (BU)
        u8_correct<false, true>(acc, usum_a, usum_b, K, lane);
    __syncthreads();

    epilogue_grid_lds<typename SP::Dense, FM, FN>(a.e, acc, m_blk + wm * WM, n_blk + wn * WN, lane,
                                                  (uint32_t *)lds + wave * 32 * (WN + 4));
}

template <class SP>
static hipError_t launch_sparse_op(int family, const SparseArgs &a, hipStream_t s)
{
    if (family == KF_SPARSE_GENERIC) {
        dim3 grid((unsigned)((a.e.N + 63) / 64), (unsigned)((a.e.M + 63) / 64));
        hipLaunchKernelGGL(k_sparse_generic<SP>, grid, dim3(256), 0, s, a);
        return hipGetLastError();
    }
    constexpr int BM = 256, BN = 256;
    const int tiles_m = (int)((a.e.M + BM - 1) / BM), tiles_n = (int)((a.e.N + BN - 1) / BN);
    constexpr bool AU = au_v<typename SP::Dense>(), BU = bu_v<typename SP::Dense>();
    if constexpr (!AU) { // unsigned A: generic only (the plan never asks otherwise)
        if (family == KF_SPARSE_DMA8) {
            hipLaunchKernelGGL(k_sparse_dma8<SP>, dim3((unsigned)(tiles_m * tiles_n)), dim3(512), 0,
                               s, a, tiles_m, tiles_n);
            return hipGetLastError();
        }
        if constexpr (!BU) {
            if (family == KF_SPARSE_TILED) {
                hipLaunchKernelGGL((k_sparse_tiled<SP, BM, BN>),
                                   dim3((unsigned)(tiles_m * tiles_n)), dim3(256), 0, s, a,
                                   tiles_m, tiles_n);
                return hipGetLastError();
            }
        }
    }
    return hipErrorInvalidValue;
}

hipError_t launch_sparse(int family, int op, const SparseArgs &a, hipStream_t s)
{
    switch (op) {
    case OPK_F16: return launch_sparse_op<SpF16>(family, a, s);
    case OPK_BF16: return launch_sparse_op<SpBF16>(family, a, s);
    case OPK_S8: return launch_sparse_op<SpS8>(family, a, s);
    case OPK_U8S8: return launch_sparse_op<SpI8<true, false>>(family, a, s);
    case OPK_S8U8: return launch_sparse_op<SpI8<false, true>>(family, a, s);
    case OPK_U8U8: return launch_sparse_op<SpI8<true, true>>(family, a, s);
    case OPK_F8_E4E4: return launch_sparse_op<SpF8<0, 0>>(family, a, s);
    case OPK_F8_E4E5: return launch_sparse_op<SpF8<0, 1>>(family, a, s);
    case OPK_F8_E5E4: return launch_sparse_op<SpF8<1, 0>>(family, a, s);
    case OPK_F8_E5E5: return launch_sparse_op<SpF8<1, 1>>(family, a, s);
    default: return hipErrorInvalidValue;
    }
}

} // namespace stg
