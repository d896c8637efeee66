// MX block-scaled GEMM ("NVIDIA MMA" (rainlin-net), section "Blackwell:
// FP4/FP6 and block-scaled MMA": D = C + sum_g (A_g S_A,g)(B_g S_B,g) over K
// blocks g of 32, UE8M0 scales per the "MXFP4 and NVFP4" table) on the gfx950
// scaled MFMA v_mfma_scale_f32_32x32x64_f8f6f4, which applies one E8M0 scale
// per 32 K of each A row and B column inside the instruction.
//
// k_mx_generic: one wave per 32x32 output tile, operands gathered byte by
//   byte from global memory into the instruction's lane layout (OpMX in
//   device_common.hpp), any pair of the five element formats, any M, N and
//   K % 32 == 0.  The fast path for pairs of one width (both 8-bit or both
//   4-bit) is k_tiled<OpMX<...>> in kernels_dense.hip.
// The fast paths for 6-bit operands (E2M3, E3M2) run the tiled kernel on a
//   copy of each 6-bit operand made once per call (an HBM-bound pass over
//   0.75 bytes in and 1 byte out per element, into stream-ordered temporary
//   buffers):
//   - both operands 6-bit (k_mx6_pad + k_tiled<OpMX<.., .., true>>): the
//     packed rows regrouped into the tiled kernel's 8-bit geometry (24 bytes
//     of each 32-K block plus 8 unused bytes), so that the MFMA still takes
//     6-bit operands, at twice the 8-bit instruction rate;
//   - a 6-bit operand with an 8-bit partner, or rows the regrouping cannot
//     read 8 bytes at a time (k_mx6_expand + the 8-bit tiled kernel): every
//     E2M3 value is exactly an E4M3 value and every E3M2 value exactly an
//     E5M2 value (the same mantissa bits in a wider exponent range), so the
//     operand becomes 8-bit codes and the pair runs as an 8-bit pair (the
//     instruction's rate for a mixed pair is the 8-bit one anyway).
//   Staging the packed rows inside the tiled kernel instead needs 96-byte K
//   tiles (three 32-byte lane blocks), which do not map onto its 256 threads
//   and 16-byte chunk swizzle.
#include <mutex>

#include "device_common.hpp"
#include "internal.hpp"

namespace stg {

template <int F>
struct MxBits {
    static constexpr int value = F <= 1 ? 8 : (F == 4 ? 4 : 6);
};

// This lane's operand words for the instruction covering K k0 .. k0+63 of the
// packed row `row` (zero when !ok or past K; K % 32 == 0, so a 32-K block is
// entirely inside or outside).
template <int F>
__device__ STG_AI void mx_operand(uint32_t (&w)[8], const uint8_t *row, bool ok, int64_t k0,
                                  int64_t K, int half)
{
    constexpr int BITS = MxBits<F>::value;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        w[i] = 0;
    if (!ok)
        return;
    if constexpr (BITS == 8) {
        // bytes 0..15: K k0+16h .. ; bytes 16..31: K k0+32+16h ..
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int64_t kb = k0 + 32 * p + 16 * half;
            if (kb < K)
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    w[4 * p + j / 4] |= (uint32_t)row[kb + j] << (8 * (j % 4));
        }
    } else {
        // K k0+32h .. k0+32h+31, packed: 16 (4-bit) or 24 (6-bit) bytes
        const int64_t kb = k0 + 32 * half;
        if (kb < K) {
            const uint8_t *p = row + kb * BITS / 8;
#pragma unroll
            for (int j = 0; j < 4 * BITS; ++j)
                w[j / 4] |= (uint32_t)p[j] << (8 * (j % 4));
        }
    }
}

template <int AF, int BF>
__global__ __launch_bounds__(256) void k_mx_generic(GemmArgs g)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t m0 = (int64_t)blockIdx.y * 64 + (wave >> 1) * 32;
    const int64_t n0 = (int64_t)blockIdx.x * 64 + (wave & 1) * 32;
    if (m0 >= g.e.M || n0 >= g.e.N)
        return;
    const int64_t am = m0 + (lane & 31), bn = n0 + (lane & 31);
    const bool a_ok = am < g.e.M, b_ok = bn < g.e.N;
    const int half = lane >> 5;
    const int64_t K = g.K, kblk = K / 32;
    const uint8_t *arow =
        (const uint8_t *)g.A + (a_ok ? am : 0) * (g.a_rs * MxBits<AF>::value / 8);
    const uint8_t *brow =
        (const uint8_t *)g.B + (b_ok ? bn : 0) * (g.b_cs * MxBits<BF>::value / 8);
    f16_t acc = {};
    for (int64_t k0 = 0; k0 < K; k0 += 64) {
        uint32_t wa[8], wb[8];
        mx_operand<AF>(wa, arow, a_ok, k0, K, half);
        mx_operand<BF>(wb, brow, b_ok, k0, K, half);
        // lane half h carries the scale of K block k0/32 + h (data past K
        // is zero, so its scale is irrelevant)
        const int64_t blk = k0 / 32 + half;
        const uint32_t sa = (a_ok && blk < kblk) ? g.sa[am * kblk + blk] : 127u;
        const uint32_t sb = (b_ok && blk < kblk) ? g.sb[bn * kblk + blk] : 127u;
        i8_t va, vb;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            va[i] = (int)wa[i];
            vb[i] = (int)wb[i];
        }
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, vb, acc, AF, BF, 0, (int)sa, 0,
                                                              (int)sb);
    }
    f16_t grid[1][1] = {{acc}};
    epilogue_grid<OpF8<0, 0>, 1, 1>(g.e, grid, m0, n0, lane);
}

template <int AF, int BF>
static hipError_t launch_mx_generic_t(const GemmArgs &g, hipStream_t s)
{
    dim3 grid((unsigned)((g.e.N + 63) / 64), (unsigned)((g.e.M + 63) / 64));
    hipLaunchKernelGGL((k_mx_generic<AF, BF>), grid, dim3(256), 0, s, g);
    return hipGetLastError();
}

template <int AF>
static hipError_t launch_mx_generic_a(int bfmt, const GemmArgs &g, hipStream_t s)
{
    switch (bfmt) {
    case 0: return launch_mx_generic_t<AF, 0>(g, s);
    case 1: return launch_mx_generic_t<AF, 1>(g, s);
    case 2: return launch_mx_generic_t<AF, 2>(g, s);
    case 3: return launch_mx_generic_t<AF, 3>(g, s);
    case 4: return launch_mx_generic_t<AF, 4>(g, s);
    default: return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------- 6 -> 8 bits

// Four packed 6-bit codes (bits 6j .. 6j+5 of a 24-bit group, the low bits
// first; bits above 23 ignored) -> four bytes.
__device__ STG_AI uint32_t unpack6x4(uint32_t g)
{
    return (g & 0x3Fu) | ((g << 2) & 0x3F00u) | ((g << 4) & 0x3F0000u) | ((g << 6) & 0x3F000000u);
}

// Four 6-bit codes, one per byte, -> the same values as 8-bit codes.
// F6 = 2: E2M3 (bias 1) -> E4M3 (bias 7); F6 = 3: E3M2 (bias 3) -> E5M2
// (bias 15).  Normal values keep their mantissa and add 6 or 12 to the
// exponent field, which in both cases adds 0x30 to the low five bits; the
// sign moves from bit 5 to bit 7.  Subnormals (exponent field 0) are m / 8
// (E2M3) or m / 16 (E3M2) for mantissa m, looked up in a byte table with
// v_perm_b32 (selector byte m picks byte m of {hi, lo}).
template <int F6>
__device__ STG_AI uint32_t widen6x4(uint32_t x)
{
    const uint32_t sign = (x & 0x20202020u) << 2;
    const uint32_t norm = (x & 0x1F1F1F1Fu) + 0x30303030u;
    uint32_t nz, sub;
    if constexpr (F6 == 2) {
        // exponent field (bits 3..4) non-zero -> bit 7 of the byte
        nz = ((x & 0x18181818u) + 0x78787878u) & 0x80808080u;
        // m / 8 for m = 0..7: 0, 2^-3, 2^-2, 1.5 2^-2, 2^-1, 1.25 2^-1, 1.5 2^-1, 1.75 2^-1
        sub = __builtin_amdgcn_perm(0x36343230u, 0x2C282000u, x & 0x07070707u);
    } else {
        // exponent field (bits 2..4) non-zero -> bit 7 of the byte
        nz = ((x & 0x1C1C1C1Cu) + 0x7C7C7C7Cu) & 0x80808080u;
        // m / 16 for m = 0..3: 0, 2^-4, 2^-3, 1.5 2^-3
        sub = __builtin_amdgcn_perm(0u, 0x32302C00u, x & 0x03030303u);
    }
    const uint32_t mask = (nz >> 7) * 0xFFu;
    return sign | (norm & mask) | (sub & ~mask);
}

// One thread per 16 elements: 12 packed bytes of row r (pitch ld_src bytes,
// 4-byte aligned) -> 16 bytes of row r of dst (pitch K bytes).  K % 16 == 0.
template <int F6>
__global__ __launch_bounds__(256) void k_mx6_expand(const uint8_t *src, int64_t ld_src,
                                                    uint8_t *dst, int64_t rows, int64_t K)
{
    const int64_t cpr = K / 16;
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= rows * cpr)
        return;
    const int64_t r = q / cpr, c = q % cpr;
    const uint32_t *w = (const uint32_t *)(src + r * ld_src + c * 12);
    const uint32_t w0 = w[0], w1 = w[1], w2 = w[2];
    u4_t o;
    o.x = widen6x4<F6>(unpack6x4(w0));
    o.y = widen6x4<F6>(unpack6x4((w0 >> 24) | (w1 << 8)));
    o.z = widen6x4<F6>(unpack6x4((w1 >> 16) | (w2 << 16)));
    o.w = widen6x4<F6>(unpack6x4(w2 >> 8));
    *(u4_t *)(dst + r * K + c * 16) = o;
}

// Packed 6-bit rows -> OpMX's padded 6-bit layout: each 64-K group's 48
// source bytes (32-K blocks 0 and 1, 24 bytes each) become 64 bytes
// [blk0 0..15][blk1 0..15][blk0 16..23, 0 x 8][blk1 16..23, 0 x 8].  One
// thread per 16-byte output chunk, so a wave's stores fill 1 KB in a row;
// source rows 8-byte aligned (pitch ld_src bytes), K % 64 == 0.
__global__ __launch_bounds__(256) void k_mx6_pad(const uint8_t *src, int64_t ld_src, uint8_t *dst,
                                                 int64_t rows, int64_t K)
{
    const int64_t gpr = K / 64;
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= rows * gpr * 4)
        return;
    const int j = (int)(q & 3);
    const int64_t grp = q >> 2, r = grp / gpr, c = grp % gpr;
    // source bytes of chunk j: [lo, lo + 8) and, for j < 2, [lo + 8, lo + 16)
    const int lo = j == 0 ? 0 : (j == 1 ? 24 : (j == 2 ? 16 : 40));
    const uint2 *p = (const uint2 *)(src + r * ld_src + c * 48 + lo);
    const uint2 a = p[0];
    uint2 b = {0u, 0u};
    if (j < 2)
        b = p[1];
    *(u4_t *)(dst + r * K + c * 64 + 16 * j) = u4_t{a.x, a.y, b.x, b.y};
}

static hipError_t launch_pad(const void *src, int64_t ld_src, uint8_t *dst, int64_t rows, int64_t K,
                             hipStream_t s)
{
    const int64_t n = rows * (K / 64) * 4;
    hipLaunchKernelGGL(k_mx6_pad, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       (const uint8_t *)src, ld_src, dst, rows, K);
    return hipGetLastError();
}

static hipError_t launch_expand(int f6, const void *src, int64_t ld_src, uint8_t *dst, int64_t rows,
                                int64_t K, hipStream_t s)
{
    const int64_t n = rows * (K / 16);
    const dim3 grid((unsigned)((n + 255) / 256));
    if (f6 == 2)
        hipLaunchKernelGGL(k_mx6_expand<2>, grid, dim3(256), 0, s, (const uint8_t *)src, ld_src,
                           dst, rows, K);
    else
        hipLaunchKernelGGL(k_mx6_expand<3>, grid, dim3(256), 0, s, (const uint8_t *)src, ld_src,
                           dst, rows, K);
    return hipGetLastError();
}

// The library's stream-ordered pool for the expanded operands, one per
// device, keeping freed blocks for the next call (release threshold: never).
static hipError_t expand_pool(int dev, hipMemPool_t *out)
{
    static std::mutex mu;
    static hipMemPool_t pools[64] = {};
    if (dev < 0 || dev >= 64)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!pools[dev]) {
        hipMemPoolProps props = {};
        props.allocType = hipMemAllocationTypePinned;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t p;
        hipError_t e = hipMemPoolCreate(&p, &props);
        if (e != hipSuccess)
            return e;
        uint64_t keep = ~0ull;
        e = hipMemPoolSetAttribute(p, hipMemPoolAttrReleaseThreshold, &keep);
        if (e != hipSuccess) {
            (void)hipMemPoolDestroy(p);
            return e;
        }
        pools[dev] = p;
    }
    *out = pools[dev];
    return hipSuccess;
}

// 6-bit operands (format selectors 2, 3): both 6-bit with 8-byte aligned
// rows -> the padded layout and the tiled kernel at the 6-bit rate;
// otherwise each 6-bit operand expanded to 8-bit codes (0, 1) and the 8-bit
// tiled kernel.  The temporaries are freed on the stream after the kernel.
static hipError_t launch_mx6(int afmt, int bfmt, const GemmArgs &g, hipStream_t s)
{
    const bool a6 = afmt == 2 || afmt == 3, b6 = bfmt == 2 || bfmt == 3;
    const int64_t M = g.e.M, N = g.e.N, K = g.K;
    const int64_t lda6 = g.a_rs * 6 / 8, ldb6 = g.b_cs * 6 / 8;
    const bool pad = a6 && b6 && lda6 % 8 == 0 && ldb6 % 8 == 0 && (uintptr_t)g.A % 8 == 0 &&
                     (uintptr_t)g.B % 8 == 0;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    hipMemPool_t pool;
    if (e == hipSuccess)
        e = expand_pool(dev, &pool);
    if (e != hipSuccess)
        return e;
    uint8_t *ea = nullptr, *eb = nullptr;
    GemmArgs h = g;
    if (a6) {
        e = hipMallocFromPoolAsync((void **)&ea, (size_t)(M * K), pool, s);
        if (e == hipSuccess)
            e = pad ? launch_pad(g.A, lda6, ea, M, K, s) : launch_expand(afmt, g.A, lda6, ea, M, K, s);
        h.A = ea;
        h.a_rs = K;
    }
    if (e == hipSuccess && b6) {
        e = hipMallocFromPoolAsync((void **)&eb, (size_t)(N * K), pool, s);
        if (e == hipSuccess)
            e = pad ? launch_pad(g.B, ldb6, eb, N, K, s) : launch_expand(bfmt, g.B, ldb6, eb, N, K, s);
        h.B = eb;
        h.b_cs = K;
    }
    if (e == hipSuccess)
        e = pad ? launch_mx_tiled_pad6(afmt, bfmt, h, s)
                : launch_mx_tiled(a6 ? afmt - 2 : afmt, b6 ? bfmt - 2 : bfmt, h, s);
    const hipError_t fa = ea ? hipFreeAsync(ea, s) : hipSuccess;
    const hipError_t fb = eb ? hipFreeAsync(eb, s) : hipSuccess;
    return e != hipSuccess ? e : (fa != hipSuccess ? fa : fb);
}

hipError_t launch_mx(int family, int afmt, int bfmt, const GemmArgs &g, hipStream_t s)
{
    if (family == KF_MX_TILED)
        return launch_mx_tiled(afmt, bfmt, g, s);
    if (family == KF_MX_TILED6)
        return launch_mx6(afmt, bfmt, g, s);
    if (family != KF_MX_GENERIC)
        return hipErrorInvalidValue;
    switch (afmt) {
    case 0: return launch_mx_generic_a<0>(bfmt, g, s);
    case 1: return launch_mx_generic_a<1>(bfmt, g, s);
    case 2: return launch_mx_generic_a<2>(bfmt, g, s);
    case 3: return launch_mx_generic_a<3>(bfmt, g, s);
    case 4: return launch_mx_generic_a<4>(bfmt, g, s);
    default: return hipErrorInvalidValue;
    }
}

} // namespace stg
