// Host-only driver of the library's C ABI layer (gemm_api.cpp) for an
// AddressSanitizer / UndefinedBehaviorSanitizer build on a machine without a
// GPU.  The HIP runtime calls that layer makes and the kernel launchers it
// calls are replaced by stubs below: a fake gfx950 device with 256 compute
// units, and launchers that check their arguments and record the call.  The
// driver then runs fixed cases and a seeded fuzz of descriptors (sizes,
// types, layouts, leading dimensions and flags from extreme sets) through
// gemm_validate_desc, gemm_plan, gemm_plan_describe, the run functions and
// the 2:4 entry points.  Exit status 0 means no sanitizer report and no
// failed expectation.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "gemm.h"
#include "gemm_diag.h"
#include "internal.hpp"

// ------------------------------------------------------------ HIP stubs
static int g_flag_store[64];
extern "C" {
hipError_t hipGetDevice(int *d)
{
    *d = 0;
    return hipSuccess;
}
hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600 *p, int)
{
    memset(p, 0, sizeof *p);
    snprintf(p->gcnArchName, sizeof p->gcnArchName, "gfx950:sramecc+:xnack-");
    p->multiProcessorCount = 256;
    return hipSuccess;
}
const char *hipGetErrorString(hipError_t) { return "stub error"; }
hipError_t hipMalloc(void **p, size_t n)
{
    if (n > sizeof g_flag_store)
        return hipErrorOutOfMemory;
    *p = g_flag_store;
    return hipSuccess;
}
hipError_t hipFree(void *) { return hipSuccess; }
hipError_t hipMemsetAsync(void *p, int v, size_t n, hipStream_t)
{
    if (p == g_flag_store && n <= sizeof g_flag_store)
        memset(p, v, n);
    return hipSuccess;
}
hipError_t hipMemcpyAsync(void *dst, const void *src, size_t n, hipMemcpyKind, hipStream_t)
{
    if (src == g_flag_store && n <= sizeof g_flag_store)
        memcpy(dst, src, n);
    return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
}

// ------------------------------------------------------------ launcher stubs
static long g_launches;
static int g_fail;
#define EXPECT(c)                                                                   \
    do {                                                                            \
        if (!(c)) {                                                                 \
            fprintf(stderr, "expectation failed at line %d: %s\n", __LINE__, #c); \
            g_fail = 1;                                                             \
        }                                                                           \
    } while (0)

static void check_epi(const stg::EpiArgs &e)
{
    EXPECT(e.M > 0 && e.N > 0 && e.D != nullptr && e.ldd >= e.N);
    EXPECT(!e.C || e.ldc >= e.N);
    EXPECT(e.d_kind >= stg::OUT_F32 && e.d_kind <= stg::OUT_E5M2);
}
namespace stg {
hipError_t launch_dense(int family, int op, int layout, const GemmArgs &g, hipStream_t)
{
    EXPECT(family >= 0 && family < KF_COUNT && op >= 0 && op < OPK_COUNT && layout >= 0 &&
           layout < 4);
    EXPECT(g.K >= 0);
    check_epi(g.e);
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_dense_mn(int, int, int, const GemmArgs &, hipStream_t) { return hipSuccess; }
hipError_t launch_mx(int family, int afmt, int bfmt, const GemmArgs &g, hipStream_t)
{
    EXPECT(family == KF_MX_GENERIC || family == KF_MX_TILED || family == KF_MX_TILED6);
    EXPECT(afmt >= 0 && afmt < 5 && bfmt >= 0 && bfmt < 5 && g.K % 32 == 0);
    check_epi(g.e);
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_mx_tiled(int, int, const GemmArgs &, hipStream_t) { return hipSuccess; }
hipError_t launch_w4(int family, int op, const GemmArgs &g, hipStream_t)
{
    EXPECT((family >= KF_W4_GENERIC && family <= KF_W4_SKINNY) || family == KF_W4_TILED16);
    EXPECT((op == OPK_F16 || op == OPK_BF16) && g.wgs >= 32 && g.K % g.wgs == 0);
    check_epi(g.e);
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_w4_tiled(int, const GemmArgs &, hipStream_t) { return hipSuccess; }
hipError_t launch_w4_skinny(int, const GemmArgs &, hipStream_t) { return hipSuccess; }
hipError_t launch_sparse(int family, int op, const SparseArgs &a, hipStream_t)
{
    EXPECT(family == KF_SPARSE_GENERIC || family == KF_SPARSE_TILED || family == KF_SPARSE_DMA8);
    EXPECT(op >= 0 && op < OPK_COUNT && a.K % 4 == 0);
    check_epi(a.e);
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_sparse24_compress(int eb, uint32_t, int64_t M, int64_t K, const void *A,
                                    void *values, uint32_t *meta, int *flag, hipStream_t)
{
    EXPECT((eb == 1 || eb == 2) && M > 0 && K > 0 && K % 4 == 0 && A && values && meta);
    EXPECT(flag != nullptr);
    ++g_launches;
    return hipSuccess;
}
hipError_t sparse24_scratch(int, int **out)
{
    *out = g_flag_store;
    return hipSuccess;
}
hipError_t launch_mfma_loop(int kind, int blocks, int64_t iters, float *out, hipStream_t)
{
    EXPECT(kind >= 0 && kind <= 5 && blocks >= 1 && iters >= 0 && out);
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_zero_ints(int *p, int n, hipStream_t)
{
    EXPECT(p == g_flag_store && n >= 1 && n <= SPARSE24_SCRATCH_INTS);
    memset(p, 0, sizeof(int) * (size_t)n);
    return hipSuccess;
}
} // namespace stg

// ------------------------------------------------------------ driver
static uint64_t g_rng = 0x9E3779B97F4A7C15ull;
static uint64_t rnd()
{
    g_rng ^= g_rng << 13;
    g_rng ^= g_rng >> 7;
    g_rng ^= g_rng << 17;
    return g_rng;
}
template <class T, size_t N> static T pick(const T (&a)[N]) { return a[rnd() % N]; }

static const int64_t SIZES[] = {-1, 0, 1, 3, 4, 16, 17, 32, 64, 100, 128, 255, 256, 512, 8192,
                                131072, (int64_t)1 << 31, (int64_t)1 << 40, INT64_MAX, INT64_MIN};
static const int64_t LDS[] = {0, 0, 0, 1, 8, 64, 130, 8192, 8200, (int64_t)1 << 33, INT64_MAX, -3};
static const int32_t TYPES[] = {0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, -1};
static const int32_t FLAGS[] = {0, 0, 1, 1, 2, -1};
static const int32_t BLOCK[] = {0, 0, 0, 32, 64, 128, 16, 33, -32};
static const float ALPHA[] = {1.0f, 1.0f, 0.5f, -2.0f};

// Fake device pointers: distinct 256-byte-aligned regions far apart, never
// dereferenced (the launcher stubs only look at them).
// (2^44 bytes apart: every matrix the descriptor checks admit, 2^40
// elements of up to 4 bytes, fits between two of them)
static void *fake(int i) { return (void *)(uintptr_t)((uint64_t)(i + 1) << 44); }

static void run_desc(const gemm_desc_t &d)
{
    const gemm_status_t v = gemm_validate_desc(&d);
    EXPECT(v == GEMM_OK || v == GEMM_ERR_INVALID_VALUE || v == GEMM_ERR_UNSUPPORTED);
    gemm_plan_t *p = nullptr;
    const gemm_status_t s = gemm_plan(&d, &p);
    // a valid descriptor may still be refused by an algorithm it forces
    EXPECT(s == v || (v == GEMM_OK && s == GEMM_ERR_UNSUPPORTED && d.algo != GEMM_ALGO_AUTO));
    EXPECT((s == GEMM_OK) == (p != nullptr));
    if (!p)
        return;
    char name[128];
    EXPECT(gemm_plan_describe(p, name, sizeof name) == GEMM_OK && name[0] != '\0');
    if (d.M <= 65536 && d.N <= 65536 && d.K <= ((int64_t)1 << 24)) {
        const void *C = d.has_c ? fake(3) : nullptr;
        const void *bias = d.has_bias ? fake(4) : nullptr;
        gemm_status_t r;
        if (d.sparse_a)
            r = gemm_sparse24_run(p, fake(1), (const uint32_t *)fake(6), fake(2), C, bias, fake(5),
                                  nullptr);
        else if (d.block_scale && d.b_type != GEMM_U4)
            r = gemm_mx_run(p, fake(1), (const uint8_t *)fake(6), fake(2),
                            (const uint8_t *)fake(7), C, bias, fake(5), nullptr);
        else if (d.b_type == GEMM_U4)
            r = gemm_w4a16_run(p, fake(1), fake(2), fake(6), (const uint8_t *)fake(7), C, bias,
                               fake(5), nullptr);
        else
            r = gemm_run(p, fake(1), fake(2), C, bias, fake(5), nullptr);
        if (r != GEMM_OK)
            fprintf(stderr, "run of %s: %s\n", name, gemm_last_error());
        EXPECT(r == GEMM_OK);
        // every run function refuses a plan of another kind
        if (!d.sparse_a)
            EXPECT(gemm_sparse24_run(p, fake(1), (const uint32_t *)fake(6), fake(2), C, bias,
                                     fake(5), nullptr) == GEMM_ERR_UNSUPPORTED);
        // D == A is refused
        if (!d.sparse_a && !d.block_scale && d.b_type != GEMM_U4 && d.M > 0 && d.N > 0 && d.K > 0)
            EXPECT(gemm_run(p, fake(1), fake(2), C, bias, fake(1), nullptr) ==
                   GEMM_ERR_UNSUPPORTED);
    }
    EXPECT(gemm_plan_destroy(p) == GEMM_OK);
}

int main(int argc, char **argv)
{
    const long iters = argc > 1 ? atol(argv[1]) : 200000;
    // fixed cases: the workloads' descriptors
    gemm_desc_t d{};
    d.M = d.N = d.K = 8192;
    d.a_type = d.b_type = GEMM_BF16;
    d.c_type = GEMM_F32;
    d.d_type = GEMM_BF16;
    d.a_layout = GEMM_ROW_MAJOR;
    d.b_layout = GEMM_COL_MAJOR;
    d.alpha = 1.0f;
    d.has_c = 1;
    run_desc(d);
    gemm_plan_t *p = nullptr;
    EXPECT(gemm_plan(&d, &p) == GEMM_OK);
    char name[64];
    gemm_plan_describe(p, name, sizeof name);
    EXPECT(strcmp(name, "tiled256w8tk16_bf16") == 0);
    gemm_plan_destroy(p);
    EXPECT(gemm_validate_desc(nullptr) == GEMM_ERR_NULL_POINTER);
    EXPECT(gemm_plan(&d, nullptr) == GEMM_ERR_NULL_POINTER);
    EXPECT(gemm_run(nullptr, fake(1), fake(2), nullptr, nullptr, fake(5), nullptr) ==
           GEMM_ERR_NULL_POINTER);
    EXPECT(gemm_last_error()[0] != '\0');
    size_t vb = 0, mb = 0;
    EXPECT(gemm_sparse24_sizes(8192, 8192, GEMM_F16, &vb, &mb) == GEMM_OK);
    EXPECT(vb == (size_t)8192 * 4096 * 2 && mb == (size_t)8192 * 256 * 4);
    EXPECT(gemm_sparse24_compress(64, 64, GEMM_F16, fake(1), fake(2), (uint32_t *)fake(3),
                                  nullptr) == GEMM_OK);
    EXPECT(gemm_sparse24_compress_noalloc(64, 64, GEMM_S8, fake(1), fake(2),
                                          (uint32_t *)fake(3), nullptr) == GEMM_OK);
    EXPECT(gemm_sparse24_compress_noalloc(64, 6, GEMM_S8, fake(1), fake(2), (uint32_t *)fake(3),
                                          nullptr) == GEMM_ERR_UNSUPPORTED);
    // the flag set by a (simulated) failing compression is reported and
    // then cleared by the next call
    g_flag_store[0] = 0x7fffffff - 5;
    EXPECT(gemm_sparse24_compress_noalloc(64, 64, GEMM_F16, fake(1), fake(2),
                                          (uint32_t *)fake(3), nullptr) == GEMM_OK);
    EXPECT(gemm_diag_mfma_loop(0, 256, 100, (float *)fake(1), nullptr) == GEMM_OK);
    EXPECT(gemm_diag_mfma_loop(5, 256, 100, (float *)fake(1), nullptr) == GEMM_OK);
    EXPECT(gemm_diag_mfma_loop(6, 256, 100, (float *)fake(1), nullptr) == GEMM_ERR_INVALID_VALUE);
    EXPECT(gemm_diag_mfma_loop(1, 0, 100, (float *)fake(1), nullptr) == GEMM_ERR_INVALID_VALUE);
    EXPECT(gemm_diag_mfma_loop(2, 8, 1, nullptr, nullptr) == GEMM_ERR_NULL_POINTER);
    for (int s = -2; s < 10; ++s)
        EXPECT(gemm_status_string((gemm_status_t)s) != nullptr);

    // fuzz: half the descriptors drawn from the extreme sets alone, half
    // from a valid (a, b, c, d) signature with extreme sizes and strides
    static const int32_t SIG[][4] = {
        {GEMM_BF16, GEMM_BF16, GEMM_F32, GEMM_BF16}, {GEMM_F16, GEMM_F16, GEMM_F32, GEMM_F32},
        {GEMM_F8_E4M3, GEMM_F8_E5M2, GEMM_F32, GEMM_F16}, {GEMM_S8, GEMM_S8, GEMM_S32, GEMM_S32},
        {GEMM_S8, GEMM_S8, GEMM_F16, GEMM_F8_E4M3}, {GEMM_BF16, GEMM_BF16, GEMM_BF16, GEMM_F32},
        {GEMM_F6_E2M3, GEMM_F4_E2M1, GEMM_F32, GEMM_BF16}, {GEMM_BF16, GEMM_U4, GEMM_F32, GEMM_BF16}};
    static const int64_t GOOD[] = {1, 16, 17, 64, 96, 256, 300, 512, 1024, 8192, 65536, 1 << 20};
    long ok = 0;
    for (long i = 0; i < iters; ++i) {
        gemm_desc_t f{};
        const bool wild = rnd() & 1;
        f.M = wild ? pick(SIZES) : pick(GOOD);
        f.N = wild ? pick(SIZES) : pick(GOOD);
        f.K = wild ? pick(SIZES) : pick(GOOD);
        if (wild) {
            f.a_type = pick(TYPES);
            f.b_type = (rnd() & 3) ? f.a_type : pick(TYPES);
            f.c_type = pick(TYPES);
            f.d_type = pick(TYPES);
        } else {
            const int32_t *g = SIG[rnd() % (sizeof SIG / sizeof SIG[0])];
            f.a_type = g[0], f.b_type = g[1], f.c_type = g[2], f.d_type = g[3];
        }
        f.a_layout = wild ? pick(FLAGS) : (int32_t)(rnd() % 4 == 0);
        f.b_layout = wild ? pick(FLAGS) : (int32_t)(rnd() % 4 != 0);
        f.lda = (wild || rnd() % 4 == 0) ? pick(LDS) : 0;
        f.ldb = (wild || rnd() % 4 == 0) ? pick(LDS) : 0;
        f.ldc = (wild || rnd() % 4 == 0) ? pick(LDS) : 0;
        f.ldd = (wild || rnd() % 4 == 0) ? pick(LDS) : 0;
        f.alpha = pick(ALPHA);
        f.has_c = wild ? pick(FLAGS) : (int32_t)(rnd() & 1);
        f.has_bias = wild ? pick(FLAGS) : (int32_t)(rnd() & 1);
        f.act = wild ? pick(FLAGS) : (int32_t)(rnd() & 1);
        f.sparse_a = (rnd() % 4 == 0) ? (wild ? pick(FLAGS) : 1) : 0;
        f.algo = (int32_t)(rnd() % 8) - 1;
        f.block_scale = wild ? pick(BLOCK) : (f.b_type == GEMM_U4 ? 128 : (f.a_type >= GEMM_F6_E2M3 ? 32 : 0));
        f.saturate = (rnd() % 4 == 0) ? (wild ? pick(FLAGS) : 1) : 0;
        if (!wild && f.d_type == GEMM_S32)
            f.alpha = 1.0f, f.has_bias = 0, f.act = 0;
        ok += gemm_validate_desc(&f) == GEMM_OK;
        run_desc(f);
    }
    printf("host driver: %ld fuzz descriptors (%ld valid), %ld launches, %s\n", iters, ok,
           g_launches, g_fail ? "FAILED" : "ok");
    return g_fail;
}
