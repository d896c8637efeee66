// C ABI of libstgemm.so: descriptor validation, plan selection and launch.
// The operation and its conventions are documented in include/gemm.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <new>

#include "gemm_diag.h"
#include "internal.hpp"

using namespace stg;

namespace {

thread_local char g_last_error[512] = "";

gemm_status_t fail(gemm_status_t st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

gemm_status_t ok()
{
    g_last_error[0] = '\0';
    return GEMM_OK;
}

gemm_status_t hip_fail(hipError_t e, const char *what)
{
    return fail(GEMM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool is_fp8(int t) { return t == GEMM_F8_E4M3 || t == GEMM_F8_E5M2; }
// MX element formats: their bits and the scaled MFMA's format selector
bool is_mx_elem(int t) { return is_fp8(t) || t == GEMM_F6_E2M3 || t == GEMM_F6_E3M2 || t == GEMM_F4_E2M1; }
int mx_bits(int t) { return is_fp8(t) ? 8 : (t == GEMM_F4_E2M1 ? 4 : 6); }
int mx_sel(int t)
{
    switch (t) {
    case GEMM_F8_E4M3: return 0;
    case GEMM_F8_E5M2: return 1;
    case GEMM_F6_E2M3: return 2;
    case GEMM_F6_E3M2: return 3;
    default: return 4;
    }
}
const char *mx_name(int sel)
{
    static const char *n[] = {"e4m3", "e5m2", "e2m3", "e3m2", "e2m1"};
    return sel >= 0 && sel < 5 ? n[sel] : "?";
}
bool is_float_in(int t) { return t == GEMM_F16 || t == GEMM_BF16 || is_fp8(t); }
bool is_float_out(int t) { return t == GEMM_F32 || t == GEMM_F16 || t == GEMM_BF16 || is_fp8(t); }
// C of a float output: fp32, or fp16 / bf16 widened exactly in the epilogue
bool float_c_ok(const gemm_desc_t &d)
{
    return d.c_type == GEMM_F32 || d.c_type == GEMM_F16 || d.c_type == GEMM_BF16 ||
           (d.c_type == 0 && !d.has_c);
}
int elem_bytes(int t)
{
    switch (t) {
    case GEMM_F16:
    case GEMM_BF16: return 2;
    case GEMM_F8_E4M3:
    case GEMM_F8_E5M2:
    case GEMM_S8:
    case GEMM_U8: return 1;
    default: return 4;
    }
}
bool is_int8(int t) { return t == GEMM_S8 || t == GEMM_U8; }
bool is_unsigned_op(int op) { return op == OPK_U8S8 || op == OPK_S8U8 || op == OPK_U8U8; }

int op_kind(int a, int b)
{
    if (a == GEMM_F16 && b == GEMM_F16)
        return OPK_F16;
    if (a == GEMM_BF16 && b == GEMM_BF16)
        return OPK_BF16;
    if (is_int8(a) && is_int8(b))
        return a == GEMM_S8 ? (b == GEMM_S8 ? OPK_S8 : OPK_S8U8)
                            : (b == GEMM_S8 ? OPK_U8S8 : OPK_U8U8);
    if (is_fp8(a) && is_fp8(b)) {
        const bool a5 = a == GEMM_F8_E5M2, b5 = b == GEMM_F8_E5M2;
        return a5 ? (b5 ? OPK_F8_E5E5 : OPK_F8_E5E4) : (b5 ? OPK_F8_E4E5 : OPK_F8_E4E4);
    }
    return -1;
}

const char *op_name(int op)
{
    static const char *names[] = {"f16",       "bf16", "e4m3xe4m3", "e4m3xe5m2", "e5m2xe4m3",
                                  "e5m2xe5m2", "s8",   "u8xs8",     "s8xu8",     "u8xu8"};
    return (op >= 0 && op < OPK_COUNT) ? names[op] : "?";
}

int out_kind(int d)
{
    switch (d) {
    case GEMM_F32: return OUT_F32;
    case GEMM_F16: return OUT_F16;
    case GEMM_BF16: return OUT_BF16;
    case GEMM_F8_E4M3: return OUT_E4M3;
    case GEMM_F8_E5M2: return OUT_E5M2;
    default: return OUT_S32;
    }
}

// a * b for a, b >= 0, saturating at INT64_MAX (size checks never overflow)
int64_t smul(int64_t a, int64_t b)
{
    return (a != 0 && b > INT64_MAX / a) ? INT64_MAX : a * b;
}

// Fill packed leading dimensions; returns false if a given one is too small.
bool normalise(gemm_desc_t &d)
{
    const int64_t a_min = d.a_layout == GEMM_ROW_MAJOR ? d.K : d.M;
    const int64_t b_min = d.b_layout == GEMM_COL_MAJOR ? d.K : d.N;
    auto fix = [](int64_t &ld, int64_t mn) {
        if (ld == 0)
            ld = mn > 0 ? mn : 1;
        return ld >= mn && ld > 0;
    };
    return fix(d.lda, a_min) & fix(d.ldb, b_min) & fix(d.ldc, d.N) & fix(d.ldd, d.N);
}

struct DeviceInfo {
    int checked = 0;
    int is_gfx950 = 0;
    int num_cu = 0;
    char arch[64] = "";
};
DeviceInfo g_dev[64];
std::mutex g_dev_mu;

gemm_status_t check_device(int *dev_out, DeviceInfo *info_out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= 64)
        return fail(GEMM_ERR_DEVICE, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lk(g_dev_mu);
    DeviceInfo &di = g_dev[dev];
    if (!di.checked) {
        hipDeviceProp_t p;
        e = hipGetDeviceProperties(&p, dev);
        if (e != hipSuccess)
            return hip_fail(e, "hipGetDeviceProperties");
        snprintf(di.arch, sizeof di.arch, "%.63s", p.gcnArchName);
        di.is_gfx950 = strncmp(p.gcnArchName, "gfx950", 6) == 0;
        di.num_cu = p.multiProcessorCount;
        di.checked = 1;
    }
    if (!di.is_gfx950)
        return fail(GEMM_ERR_DEVICE, "device %d is %s, this library is built for gfx950", dev,
                    di.arch);
    *dev_out = dev;
    if (info_out)
        *info_out = di;
    return GEMM_OK;
}

// Can the LDS-tiled kernel serve this descriptor (ignoring pointer alignment)?
bool tiled_ok(const gemm_desc_t &d)
{
    // 64-byte K tiles, 16-byte rows; 32-bit buffer offsets cover 256 rows
    // plus the K extent.  An MN-major operand (A column-major, B row-major)
    // is read in 16-byte chunks along M (N), which must not straddle the end
    // of the data (M, N in whole 16-byte chunks), and its whole offset, K
    // rows included, goes through 32 bits.
    const int eb = elem_bytes(d.a_type);
    const int64_t lim = (int64_t)1 << 30;
    const bool a_mn = d.a_layout == GEMM_COL_MAJOR, b_mn = d.b_layout == GEMM_ROW_MAJOR;
    const bool a_ok = a_mn ? (d.M * eb) % 16 == 0 && smul(smul(d.K + 256, d.lda), eb) < lim
                           : d.lda * eb * 256 < lim;
    const bool b_ok = b_mn ? (d.N * eb) % 16 == 0 && smul(smul(d.K + 256, d.ldb), eb) < lim
                           : d.ldb * eb * 256 < lim;
    return d.K > 0 && (d.K * eb) % 64 == 0 && (d.lda * eb) % 16 == 0 && (d.ldb * eb) % 16 == 0 &&
           a_ok && b_ok;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

const char *family_name(int f)
{
    switch (f) {
    case KF_GENERIC: return "generic";
    case KF_TILED_256: return "tiled256";
    case KF_TILED_128: return "tiled128";
    case KF_SKINNY: return "skinny";
    case KF_SPARSE_GENERIC: return "sparse24_generic";
    case KF_SPARSE_TILED: return "sparse24_tiled";
    case KF_SPARSE_DMA8: return "sparse24_dma8";
    case KF_TILED_256W8: return "tiled256w8";
    case KF_TILED_256W8K16: return "tiled256w8k16";
    case KF_TILED_256W8TK16: return "tiled256w8tk16";
    case KF_TILED_256W8T: return "tiled256w8t";
    case KF_MX_GENERIC: return "mx_generic";
    case KF_MX_TILED: return "mx_tiled";
    case KF_W4_GENERIC: return "w4_generic";
    case KF_W4_TILED: return "w4_tiled";
    case KF_W4_TILED16: return "w4_tiled16";
    case KF_W4_SKINNY: return "w4_skinny";
    case KF_MX_TILED6: return "mx_tiled6";
    default: return "?";
    }
}

// Skinny kernel: M <= 16, K-contiguous operands, whole 256-byte K chunks.
bool skinny_ok(const gemm_desc_t &d)
{
    const int eb = elem_bytes(d.a_type);
    const int64_t lim = (int64_t)1 << 30;
    return d.M <= 16 && d.a_layout == GEMM_ROW_MAJOR && d.b_layout == GEMM_COL_MAJOR && d.K > 0 &&
           (d.K * eb) % 256 == 0 && (d.lda * eb) % 16 == 0 && (d.ldb * eb) % 16 == 0 &&
           d.lda * eb * 16 < lim && d.ldb * eb * 32 < lim;
}

bool is_tiled(int f)
{
    return f == KF_TILED_256 || f == KF_TILED_128 || f == KF_TILED_256W8 || f == KF_TILED_256W8T ||
           f == KF_TILED_256W8K16 || f == KF_TILED_256W8TK16;
}

} // namespace

extern "C" {

const char *gemm_status_string(gemm_status_t s)
{
    switch (s) {
    case GEMM_OK: return "GEMM_OK";
    case GEMM_ERR_NULL_POINTER: return "GEMM_ERR_NULL_POINTER";
    case GEMM_ERR_INVALID_VALUE: return "GEMM_ERR_INVALID_VALUE";
    case GEMM_ERR_UNSUPPORTED: return "GEMM_ERR_UNSUPPORTED";
    case GEMM_ERR_MISALIGNED: return "GEMM_ERR_MISALIGNED";
    case GEMM_ERR_NOT_SPARSE24: return "GEMM_ERR_NOT_SPARSE24";
    case GEMM_ERR_DEVICE: return "GEMM_ERR_DEVICE";
    case GEMM_ERR_HIP: return "GEMM_ERR_HIP";
    default: return "GEMM_ERR_UNKNOWN";
    }
}

const char *gemm_last_error(void) { return g_last_error; }

gemm_status_t gemm_validate_desc(const gemm_desc_t *desc)
{
    if (!desc)
        return fail(GEMM_ERR_NULL_POINTER, "desc is NULL");
    gemm_desc_t d = *desc;
    if (d.M < 0 || d.N < 0 || d.K < 0)
        return fail(GEMM_ERR_INVALID_VALUE, "negative size M=%lld N=%lld K=%lld",
                    (long long)d.M, (long long)d.N, (long long)d.K);
    auto dtype_ok = [](int t) { return t >= GEMM_F16 && t <= GEMM_U8; };
    if (!dtype_ok(d.a_type) || !dtype_ok(d.b_type) || !dtype_ok(d.d_type) ||
        !(d.c_type == 0 || dtype_ok(d.c_type)))
        return fail(GEMM_ERR_INVALID_VALUE, "unknown dtype code");
    if ((d.a_layout != GEMM_ROW_MAJOR && d.a_layout != GEMM_COL_MAJOR) ||
        (d.b_layout != GEMM_ROW_MAJOR && d.b_layout != GEMM_COL_MAJOR))
        return fail(GEMM_ERR_INVALID_VALUE, "unknown layout code");
    if (d.act != GEMM_ACT_NONE && d.act != GEMM_ACT_RELU)
        return fail(GEMM_ERR_INVALID_VALUE, "unknown activation code");
    // saturation: int32 outputs, with K small enough that the sum of
    // products itself cannot leave the int32 range (K max|a| max|b| < 2^31),
    // so that the wrapped sum is the exact one and clamping acc + C is the
    // exact saturated result
    if (d.saturate != 0 && d.saturate != 1)
        return fail(GEMM_ERR_INVALID_VALUE, "saturate must be 0 or 1");
    if (d.saturate) {
        const int64_t ma = d.a_type == GEMM_U8 ? 255 : 128, mb = d.b_type == GEMM_U8 ? 255 : 128;
        if (d.d_type != GEMM_S32 || smul(d.K, ma * mb) >= ((int64_t)1 << 31))
            return fail(GEMM_ERR_UNSUPPORTED, "saturation applies to int32 outputs with "
                                              "K * max|a| * max|b| < 2^31");
    }
    if ((d.has_c != 0 && d.has_c != 1) || (d.has_bias != 0 && d.has_bias != 1) ||
        (d.sparse_a != 0 && d.sparse_a != 1))
        return fail(GEMM_ERR_INVALID_VALUE, "has_c / has_bias / sparse_a must be 0 or 1");
    if (d.algo < GEMM_ALGO_AUTO || d.algo > GEMM_ALGO_TILED_256)
        return fail(GEMM_ERR_INVALID_VALUE, "unknown algo code");
    if (d.lda < 0 || d.ldb < 0 || d.ldc < 0 || d.ldd < 0)
        return fail(GEMM_ERR_INVALID_VALUE, "negative leading dimension");
    // sizes the kernels' index arithmetic covers: M, N, K below 2^31, and
    // every matrix (rows x leading dimension) at most 2^40 elements
    const int64_t max_elems = (int64_t)1 << 40;
    if (d.M > INT32_MAX || d.N > INT32_MAX || d.K > INT32_MAX)
        return fail(GEMM_ERR_INVALID_VALUE, "M, N and K must be below 2^31");
    if (d.lda > max_elems || d.ldb > max_elems || d.ldc > max_elems || d.ldd > max_elems)
        return fail(GEMM_ERR_INVALID_VALUE, "leading dimension above 2^40");
    if (!normalise(d))
        return fail(GEMM_ERR_INVALID_VALUE, "leading dimension smaller than the matrix extent");
    {
        const bool ar = d.a_layout == GEMM_ROW_MAJOR, bc = d.b_layout == GEMM_COL_MAJOR;
        if (smul(ar ? d.M : d.K, d.lda) > max_elems || smul(bc ? d.N : d.K, d.ldb) > max_elems ||
            smul(d.M, d.ldc) > max_elems || smul(d.M, d.ldd) > max_elems)
            return fail(GEMM_ERR_INVALID_VALUE, "a matrix spans more than 2^40 elements");
    }
    if (d.b_type == GEMM_U4 || d.a_type == GEMM_U4) {
        // W4A16 ("NVIDIA MMA", section "How quantisation configurations map
        // to MMA"): fp16 / bf16 activations, 4-bit weight codes with a scale
        // and zero point per group of block_scale K, fp32 accumulation
        if (d.a_type != GEMM_F16 && d.a_type != GEMM_BF16)
            return fail(GEMM_ERR_UNSUPPORTED, "W4A16: A must be f16 or bf16 and B u4");
        if (d.block_scale < 32 || d.block_scale % 32 || d.K % d.block_scale)
            return fail(GEMM_ERR_UNSUPPORTED,
                        "W4A16: block_scale (the group size) must be a multiple of 32 dividing K");
        if (d.sparse_a)
            return fail(GEMM_ERR_UNSUPPORTED, "W4A16: A cannot be 2:4 sparse");
        if (d.a_layout != GEMM_ROW_MAJOR || d.b_layout != GEMM_COL_MAJOR)
            return fail(GEMM_ERR_UNSUPPORTED, "W4A16: A row-major, B column-major (codes along K)");
        if (d.ldb % 2)
            return fail(GEMM_ERR_UNSUPPORTED, "W4A16: packed weight rows must be whole bytes");
        if (!float_c_ok(d))
            return fail(GEMM_ERR_UNSUPPORTED, "float inputs take an f32, f16 or bf16 C");
        if (!is_float_out(d.d_type))
            return fail(GEMM_ERR_UNSUPPORTED, "float output must be f32, f16, bf16 or fp8");
        return ok();
    }
    if (d.block_scale != 0 && d.block_scale != 32)
        return fail(GEMM_ERR_INVALID_VALUE, "block_scale must be 0 or 32 (or a W4A16 group size)");

    if (d.block_scale == 32) {
        // MX block-scaled ("NVIDIA MMA", section "Blackwell: FP4/FP6 and
        // block-scaled MMA"): any two MX element formats, fp32 accumulation
        if (!is_mx_elem(d.a_type) || !is_mx_elem(d.b_type))
            return fail(GEMM_ERR_UNSUPPORTED,
                        "block-scaled A/B must be e4m3, e5m2, e2m3, e3m2 or e2m1");
        if (d.sparse_a)
            return fail(GEMM_ERR_UNSUPPORTED, "block-scaled A cannot be 2:4 sparse");
        if (d.a_layout != GEMM_ROW_MAJOR || d.b_layout != GEMM_COL_MAJOR)
            return fail(GEMM_ERR_UNSUPPORTED,
                        "block-scaled operands are K-contiguous: A row-major, B column-major");
        if (d.K % 32)
            return fail(GEMM_ERR_UNSUPPORTED, "block-scaled K must be a multiple of 32");
        if ((d.lda * mx_bits(d.a_type)) % 8 || (d.ldb * mx_bits(d.b_type)) % 8)
            return fail(GEMM_ERR_UNSUPPORTED, "packed rows must be whole bytes");
        if (!(d.c_type == GEMM_F32 || (d.c_type == 0 && !d.has_c)))
            return fail(GEMM_ERR_UNSUPPORTED, "block-scaled GEMM takes an f32 C");
        if (!is_float_out(d.d_type))
            return fail(GEMM_ERR_UNSUPPORTED, "float output must be f32, f16, bf16 or fp8");
        return ok();
    }
    auto narrow_mx = [](int t) { return t == GEMM_F6_E2M3 || t == GEMM_F6_E3M2 || t == GEMM_F4_E2M1; };
    if (narrow_mx(d.a_type) || narrow_mx(d.b_type))
        return fail(GEMM_ERR_UNSUPPORTED, "6- and 4-bit float formats need block_scale = 32");
    if (d.d_type > GEMM_S32 || d.c_type > GEMM_S32)
        return fail(GEMM_ERR_UNSUPPORTED, "unsupported C or D type");

    if (is_int8(d.a_type) || is_int8(d.b_type)) {
        if (!is_int8(d.a_type) || !is_int8(d.b_type))
            return fail(GEMM_ERR_UNSUPPORTED, "8-bit integers (s8, u8) pair with 8-bit integers");
        if (d.d_type == GEMM_S32) {
            if (!(d.c_type == GEMM_S32 || (d.c_type == 0 && !d.has_c)))
                return fail(GEMM_ERR_UNSUPPORTED, "s32 output takes an s32 C");
            if (d.alpha != 1.0f || d.has_bias || d.act != GEMM_ACT_NONE)
                return fail(GEMM_ERR_UNSUPPORTED, "s32 output takes no alpha, bias or activation");
        } else {
            // the int8 -> float epilogue: the int32 sum through the float epilogue
            if (!is_float_out(d.d_type))
                return fail(GEMM_ERR_UNSUPPORTED, "s8 inputs produce s32 or a float output");
            if (!float_c_ok(d))
                return fail(GEMM_ERR_UNSUPPORTED, "a float output takes an f32, f16 or bf16 C");
        }
    } else {
        if (!is_float_in(d.a_type) || !is_float_in(d.b_type))
            return fail(GEMM_ERR_UNSUPPORTED, "A/B must be f16, bf16, fp8 or s8");
        if (op_kind(d.a_type, d.b_type) < 0)
            return fail(GEMM_ERR_UNSUPPORTED, "A/B type pair not supported (f16/f16, "
                                              "bf16/bf16 or fp8/fp8)");
        if (!float_c_ok(d))
            return fail(GEMM_ERR_UNSUPPORTED, "float inputs take an f32, f16 or bf16 C");
        if (!is_float_out(d.d_type))
            return fail(GEMM_ERR_UNSUPPORTED, "float output must be f32, f16, bf16 or fp8");
    }
    if (d.sparse_a) {
        // every supported pair has a 2:4 form (the A/B pairs above)
        if (op_kind(d.a_type, d.b_type) < 0)
            return fail(GEMM_ERR_UNSUPPORTED, "2:4 sparse A: unsupported A/B type pair");
        if (d.a_layout != GEMM_ROW_MAJOR)
            return fail(GEMM_ERR_UNSUPPORTED, "2:4 sparse A must be row-major");
        if (d.K % 4 != 0)
            return fail(GEMM_ERR_UNSUPPORTED, "2:4 sparse A needs K %% 4 == 0");
        if (d.lda != d.K)
            return fail(GEMM_ERR_UNSUPPORTED, "2:4 sparse A must be packed (lda == K)");
    }
    return ok();
}

static gemm_status_t plan_impl(const gemm_desc_t *desc, gemm_plan_t **out);

// GEMM_LOG=1 in the environment: every plan prints its kernel choice (one
// line on stderr) - the shape, types, layouts and the family selected.
static void log_plan(const gemm_plan_t *p)
{
    static const int on = [] {
        const char *v = getenv("GEMM_LOG");
        return v && *v && strcmp(v, "0") != 0;
    }();
    if (!on)
        return;
    const gemm_desc_t &d = p->d;
    fprintf(stderr,
            "[stgemm] plan M=%lld N=%lld K=%lld a=%d b=%d c=%d d=%d a_layout=%s b_layout=%s "
            "sparse_a=%d block_scale=%d algo=%d -> %s (fallback on misaligned pointers: %s)\n",
            (long long)d.M, (long long)d.N, (long long)d.K, d.a_type, d.b_type, d.c_type, d.d_type,
            d.a_layout == GEMM_ROW_MAJOR ? "row" : "col", d.b_layout == GEMM_ROW_MAJOR ? "row" : "col",
            d.sparse_a, d.block_scale, d.algo, p->name, family_name(p->fallback));
}

gemm_status_t gemm_plan(const gemm_desc_t *desc, gemm_plan_t **out)
{
    const gemm_status_t st = plan_impl(desc, out);
    if (st == GEMM_OK)
        log_plan(*out);
    return st;
}

static gemm_status_t plan_impl(const gemm_desc_t *desc, gemm_plan_t **out)
{
    if (!out)
        return fail(GEMM_ERR_NULL_POINTER, "out is NULL");
    *out = nullptr;
    gemm_status_t st = gemm_validate_desc(desc);
    if (st != GEMM_OK)
        return st;
    gemm_desc_t d = *desc;
    normalise(d);
    int dev = 0;
    DeviceInfo di;
    st = check_device(&dev, &di);
    if (st != GEMM_OK)
        return st;

    gemm_plan_t *p = new (std::nothrow) gemm_plan_t();
    if (!p)
        return fail(GEMM_ERR_INVALID_VALUE, "out of host memory");
    p->d = d;
    p->device = dev;
    p->op = op_kind(d.a_type, d.b_type);
    p->fallback = KF_GENERIC;

    if (d.b_type == GEMM_U4) {
        // the 4-wave 256 x 256 kernel: 16-byte rows of A and of codes, 32-bit
        // offsets over 256 rows
        const int64_t lim = (int64_t)1 << 30, rowa = d.lda * 2, rowb = d.ldb / 2;
        const bool fast = d.K > 0 && rowa % 16 == 0 && rowb % 16 == 0 && rowa * 256 < lim &&
                          rowb * 256 < lim && (d.K / d.block_scale) * 2 * 256 < lim;
        // M <= 16: the skinny kernel (whole 128-K chunks), bound by streaming
        // the codes once
        const bool skinny = fast && d.M <= 16 && d.K % 128 == 0 && rowa * 16 < lim &&
                            rowb * 32 < lim;
        int fam = -1;
        switch (d.algo) {
        // (the 16x16-form kernel measured 1144 vs 1185 us at 8192^3, groups of 128)
        case GEMM_ALGO_AUTO: fam = skinny ? KF_W4_SKINNY : fast ? KF_W4_TILED16 : KF_W4_GENERIC; break;
        case GEMM_ALGO_SKINNY: fam = skinny ? KF_W4_SKINNY : -1; break;
        case GEMM_ALGO_TILED:
        case GEMM_ALGO_TILED_256: fam = fast ? KF_W4_TILED16 : -1; break;
        case GEMM_ALGO_GENERIC: fam = KF_W4_GENERIC; break;
        default: fam = -1;
        }
        if (fam < 0) {
            delete p;
            return fail(GEMM_ERR_UNSUPPORTED, "requested algorithm cannot serve this W4A16 problem");
        }
        if (const char *force = getenv("STGEMM_FORCE_KERNEL")) { // tuning override
            if (strcmp(force, family_name(KF_W4_GENERIC)) == 0)
                fam = KF_W4_GENERIC;
            if (strcmp(force, family_name(KF_W4_TILED)) == 0 && fast)
                fam = KF_W4_TILED;
            if (strcmp(force, family_name(KF_W4_TILED16)) == 0 && fast)
                fam = KF_W4_TILED16;
            if (strcmp(force, family_name(KF_W4_SKINNY)) == 0 && skinny)
                fam = KF_W4_SKINNY;
        }
        p->op = d.a_type == GEMM_F16 ? OPK_F16 : OPK_BF16;
        p->family = fam;
        p->fallback = KF_W4_GENERIC;
        snprintf(p->name, sizeof p->name, "%s_%s", family_name(fam), op_name(p->op));
        *out = p;
        return ok();
    }

    if (d.block_scale) {
        const int ab = mx_bits(d.a_type), bb = mx_bits(d.b_type);
        const int64_t lim = (int64_t)1 << 30, rowa = d.lda * ab / 8, rowb = d.ldb * bb / 8;
        // the 4-wave 256 x 256 kernel: one width (8 or 4 bits), K in whole
        // groups of 16 scales (K % 512: 16-byte scale copies), 16-byte rows,
        // 32-bit offsets over 256 rows
        const bool fast = ab == bb && ab != 6 && d.K % 512 == 0 && rowa % 16 == 0 &&
                          rowb % 16 == 0 && rowa * 256 < lim && rowb * 256 < lim &&
                          (d.K / 32) * 256 < lim;
        // 6-bit operands (with a 6- or 8-bit partner): expanded into K-byte
        // rows of 8-bit codes (packed 6-bit rows read 4 bytes at a time),
        // then the 8-bit kernel
        const bool fast6 = (ab == 6 || bb == 6) && ab != 4 && bb != 4 && d.K % 512 == 0 &&
                           rowa % (ab == 6 ? 4 : 16) == 0 && rowb % (bb == 6 ? 4 : 16) == 0 &&
                           d.K * 256 < lim && rowa * 256 < lim && rowb * 256 < lim &&
                           (d.K / 32) * 256 < lim;
        const int tiled_fam = fast ? KF_MX_TILED : (fast6 ? KF_MX_TILED6 : -1);
        int fam = -1;
        switch (d.algo) {
        case GEMM_ALGO_AUTO: fam = tiled_fam >= 0 ? tiled_fam : KF_MX_GENERIC; break;
        case GEMM_ALGO_TILED:
        case GEMM_ALGO_TILED_256: fam = tiled_fam; break;
        case GEMM_ALGO_GENERIC: fam = KF_MX_GENERIC; break;
        default: fam = -1;
        }
        if (fam < 0) {
            delete p;
            return fail(GEMM_ERR_UNSUPPORTED, "requested algorithm cannot serve this MX problem");
        }
        if (const char *force = getenv("STGEMM_FORCE_KERNEL")) { // tuning override
            if (strcmp(force, family_name(KF_MX_GENERIC)) == 0)
                fam = KF_MX_GENERIC;
            if (strcmp(force, family_name(KF_MX_TILED)) == 0 && fast)
                fam = KF_MX_TILED;
            if (strcmp(force, family_name(KF_MX_TILED6)) == 0 && fast6)
                fam = KF_MX_TILED6;
        }
        p->op = mx_sel(d.a_type) * 8 + mx_sel(d.b_type);
        p->family = fam;
        p->fallback = KF_MX_GENERIC;
        snprintf(p->name, sizeof p->name, "%s_%sx%s", family_name(fam), mx_name(mx_sel(d.a_type)),
                 mx_name(mx_sel(d.b_type)));
        *out = p;
        return ok();
    }

    if (d.sparse_a) {
        // K tiles of two SMFMAC steps (64 logical K of a 16-bit type, 128 of
        // an 8-bit type: 64 value bytes and 128 B bytes per row); 32-bit
        // buffer offsets cover 256 rows of values and of B; 16-byte B rows
        const int64_t eb = elem_bytes(d.a_type), lim = (int64_t)1 << 30;
        const int64_t ktile = 128 / eb;
        const bool fast = d.b_layout == GEMM_COL_MAJOR && d.K % ktile == 0 &&
                          (d.ldb * eb) % 16 == 0 && d.K * eb / 2 * 256 < lim &&
                          d.ldb * eb * 256 < lim;
        // the 8-wave kernel with direct copies measured fastest (2:4 f16,
        // 8192^3); it takes K in whole metadata groups of 256 logical K.
        // Unsigned B: that kernel only (its fragments are offset after the
        // LDS reads); unsigned A: the generic kernel (the SMFMAC skips the
        // dropped positions, so the offset correction would depend on the
        // positions of every row)
        const bool dma8 = fast && d.K % 256 == 0 && d.a_type != GEMM_U8;
        const bool fast_any = fast && (!is_unsigned_op(p->op) || dma8);
        const int tiled_fam = dma8 ? KF_SPARSE_DMA8 : KF_SPARSE_TILED;
        int fam = -1;
        switch (d.algo) {
        case GEMM_ALGO_AUTO: fam = fast_any ? tiled_fam : KF_SPARSE_GENERIC; break;
        case GEMM_ALGO_TILED:
        case GEMM_ALGO_TILED_256: fam = fast_any ? tiled_fam : -1; break;
        case GEMM_ALGO_GENERIC: fam = KF_SPARSE_GENERIC; break;
        default: fam = -1;
        }
        if (fam < 0) {
            delete p;
            return fail(GEMM_ERR_UNSUPPORTED, "requested algorithm cannot serve this sparse problem");
        }
        if (const char *force = getenv("STGEMM_FORCE_KERNEL")) { // tuning override
            for (int f : {KF_SPARSE_TILED, KF_SPARSE_DMA8, KF_SPARSE_GENERIC})
                if (strcmp(force, family_name(f)) == 0 &&
                    (f == KF_SPARSE_GENERIC ||
                     (fast_any && (f != KF_SPARSE_DMA8 || dma8) &&
                      (f != KF_SPARSE_TILED || !is_unsigned_op(p->op)))))
                    fam = f;
        }
        p->family = fam;
        p->fallback = KF_SPARSE_GENERIC;
        snprintf(p->name, sizeof p->name, "%s_%s", family_name(fam), op_name(p->op));
        *out = p;
        return ok();
    }

    const int layout = (d.a_layout == GEMM_COL_MAJOR ? 1 : 0) | (d.b_layout == GEMM_ROW_MAJOR ? 2 : 0);
    // an unsigned 8-bit operand: the K-contiguous tiled kernels and the
    // generic one (the MN-major and skinny paths take signed operands only)
    const bool uns = is_unsigned_op(p->op);
    const bool tiled = tiled_ok(d) && (!uns || layout == 0);
    const bool skinny = skinny_ok(d) && !uns;
    int fam = -1;
    const int64_t big_tiles = ceil_div(d.M, 256) * ceil_div(d.N, 256);
    // 256 x 256 tiles: the fastest variant measured per operand type on
    // MI355X at 8192^3 (K-contiguous: 16-bit and signed int8 on 8 waves of
    // 64 x 128 with the 16x16 MFMA forms, fp8 on 8 waves of 128 x 64 with
    // the 32x32x64 form, both with fragments refreshed in place; MN-major
    // 16-bit: 8 waves of 128 x 64, MN-major or unsigned int8: 8 waves of
    // 64 x 128, on the 32x32 forms; MN-major fp8: 4 waves of 128 x 128, whose
    // double-buffered 8-wave forms run short of registers)
    const int op = op_kind(d.a_type, d.b_type);
    const bool k16 = layout == 0 && !uns && (op == OPK_F16 || op == OPK_BF16 || op == OPK_S8);
    const bool f8 = op == OPK_F8_E4E4 || op == OPK_F8_E4E5 || op == OPK_F8_E5E4 || op == OPK_F8_E5E5;
    const int fam256 = k16 ? KF_TILED_256W8TK16
                       : (layout == 0 && f8) ? KF_TILED_256W8K16
                       : (op == OPK_S8 || uns) ? KF_TILED_256W8T
                       : (op == OPK_F16 || op == OPK_BF16) ? KF_TILED_256W8 : KF_TILED_256;
    const int auto_tiled = big_tiles >= di.num_cu ? fam256 : KF_TILED_128;
    switch (d.algo) {
    case GEMM_ALGO_AUTO: fam = skinny ? KF_SKINNY : tiled ? auto_tiled : KF_GENERIC; break;
    case GEMM_ALGO_SKINNY: fam = skinny ? KF_SKINNY : -1; break;
    case GEMM_ALGO_TILED: fam = tiled ? auto_tiled : -1; break;
    case GEMM_ALGO_TILED_128: fam = tiled ? KF_TILED_128 : -1; break;
    case GEMM_ALGO_TILED_256: fam = tiled ? fam256 : -1; break;
    case GEMM_ALGO_GENERIC: fam = KF_GENERIC; break;
    default: fam = -1;
    }
    if (fam < 0) {
        delete p;
        return fail(GEMM_ERR_UNSUPPORTED, "requested algorithm cannot serve this problem");
    }
    // Tuning override: STGEMM_FORCE_KERNEL=<family name> replaces the choice
    // for descriptors that family can serve (ignored otherwise).
    if (const char *force = getenv("STGEMM_FORCE_KERNEL")) {
        // MN-major operands only on the type's 256 x 256 arrangement and the
        // 128 x 128 tile
        for (int f = 0; f < KF_COUNT; ++f) {
            const bool layout_ok = layout == 0 || f == fam256 || f == KF_TILED_128;
            // unsigned 8-bit operands are built on the 128 tile and w8t only
            const bool uns_ok = !uns || f == KF_TILED_128 || f == KF_TILED_256W8T;
            // the rolling-fragment kernel: 16-bit and int8 inputs on the
            // 16x16 forms, fp8 on the 32x32 form; K-contiguous
            if ((f == KF_TILED_256W8K16 || f == KF_TILED_256W8TK16) &&
                (layout != 0 || op == OPK_U8S8 || op == OPK_S8U8 || op == OPK_U8U8))
                continue;
            if (strcmp(force, family_name(f)) == 0 &&
                (f == KF_GENERIC || (tiled && is_tiled(f) && layout_ok && uns_ok) ||
                 (skinny && f == KF_SKINNY)))
                fam = f;
        }
    }
    p->family = fam;
    p->layout = layout;
    static const char *const layout_sfx[4] = {"", "_acol", "_brow", "_acol_brow"};
    snprintf(p->name, sizeof p->name, "%s_%s%s", family_name(fam), op_name(p->op),
             layout_sfx[layout]);
    *out = p;
    return ok();
}

gemm_status_t gemm_plan_destroy(gemm_plan_t *plan)
{
    delete plan;
    return ok();
}

gemm_status_t gemm_plan_describe(const gemm_plan_t *plan, char *buf, size_t len)
{
    if (!plan || !buf)
        return fail(GEMM_ERR_NULL_POINTER, "plan or buf is NULL");
    if (len == 0)
        return fail(GEMM_ERR_INVALID_VALUE, "len is 0");
    snprintf(buf, len, "%s", plan->name);
    return ok();
}

// Byte range [lo, hi) of a matrix of `rows` rows of `cols` elements of
// `eb` bytes, `ld` elements apart.
struct Span {
    uintptr_t lo = 0, hi = 0;
};
static Span span(const void *p, int64_t rows, int64_t cols, int64_t ld, int64_t eb)
{
    Span s;
    if (!p || rows <= 0 || cols <= 0)
        return s;
    s.lo = (uintptr_t)p;
    s.hi = s.lo + (uintptr_t)(((rows - 1) * ld + cols) * eb);
    return s;
}
static bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

// D must not share bytes with any input, except that D may be C itself
// (in-place accumulate: same address, element size and leading dimension,
// so every element is read before it is written by the same thread).
// `inputs` are the operand ranges of the call.
static gemm_status_t check_d_overlap(const gemm_desc_t &d, const void *C, const void *bias,
                                     const void *D, std::initializer_list<Span> inputs)
{
    const int db = elem_bytes(d.d_type);
    const Span sd = span(D, d.M, d.N, d.ldd, db);
    if (d.has_c) {
        const int cb = (d.c_type == GEMM_F16 || d.c_type == GEMM_BF16) ? 2 : 4;
        const Span sc = span(C, d.M, d.N, d.ldc, cb);
        const bool in_place = C == D && cb == db && d.ldc == d.ldd;
        if (overlap(sc, sd) && !in_place)
            return fail(GEMM_ERR_UNSUPPORTED,
                        "D overlaps C: only D == C with the same element size and leading "
                        "dimension (in-place accumulate) is supported");
    }
    if (d.has_bias && overlap(span(bias, 1, d.N, d.N, 4), sd))
        return fail(GEMM_ERR_UNSUPPORTED, "D overlaps bias");
    for (const Span &x : inputs)
        if (overlap(x, sd))
            return fail(GEMM_ERR_UNSUPPORTED, "D overlaps an input operand");
    return GEMM_OK;
}

static gemm_status_t check_epilogue_ptrs(const gemm_desc_t &d, const void *C, const void *bias,
                                         const void *D)
{
    if (!D)
        return fail(GEMM_ERR_NULL_POINTER, "D is NULL");
    if (d.has_c && !C)
        return fail(GEMM_ERR_NULL_POINTER, "C is NULL but the plan reads C");
    if (d.has_bias && !bias)
        return fail(GEMM_ERR_NULL_POINTER, "bias is NULL but the plan adds a bias");
    const size_t c_align = (d.c_type == GEMM_F16 || d.c_type == GEMM_BF16) ? 2 : 4;
    if ((d.has_c && !aligned(C, c_align)) || (d.has_bias && !aligned(bias, 4)) ||
        !aligned(D, elem_bytes(d.d_type)))
        return fail(GEMM_ERR_MISALIGNED, "C, bias or D not aligned to its element size");
    return GEMM_OK;
}

static EpiArgs make_epi(const gemm_desc_t &d, const void *C, const void *bias, void *D)
{
    EpiArgs e;
    e.M = d.M;
    e.N = d.N;
    e.C = d.has_c ? C : nullptr;
    e.ldc = d.ldc;
    e.bias = d.has_bias ? (const float *)bias : nullptr;
    e.alpha = d.alpha;
    e.relu = d.act == GEMM_ACT_RELU;
    e.d_kind = out_kind(d.d_type);
    e.sat = d.saturate;
    e.D = D;
    e.ldd = d.ldd;
    const int db = elem_bytes(d.d_type);
    // the vector epilogue addresses a block's C and D rows with 32-bit
    // offsets: 257 rows of each must span less than 2^31 bytes
    const int64_t lim = 0x7fffffff / 257;
    // C is read 4 elements per lane: 16 bytes of fp32 / int32 or 8 of
    // fp16 / bf16 (float outputs only)
    e.c_kind = !d.has_c ? 0 : (d.c_type == GEMM_F16 ? 1 : (d.c_type == GEMM_BF16 ? 2 : 0));
    const int cb = e.c_kind == 0 ? 4 : 2;
    e.vec = (!d.has_c || (aligned(C, 4 * cb) && d.ldc % 4 == 0 && d.ldc * cb < lim)) &&
            (!d.has_bias || aligned(bias, 16)) && aligned(D, 4 * db) && d.ldd % 4 == 0 &&
            d.ldd * db < lim;
    return e;
}

gemm_status_t gemm_run(const gemm_plan_t *plan, const void *A, const void *B, const void *C,
                       const void *bias, void *D, gemm_stream_t stream)
{
    if (!plan)
        return fail(GEMM_ERR_NULL_POINTER, "plan is NULL");
    const gemm_desc_t &d = plan->d;
    if (d.sparse_a)
        return fail(GEMM_ERR_UNSUPPORTED, "plan is for 2:4 sparse A: use gemm_sparse24_run");
    if (d.b_type == GEMM_U4)
        return fail(GEMM_ERR_UNSUPPORTED, "plan is W4A16: use gemm_w4a16_run");
    if (d.block_scale)
        return fail(GEMM_ERR_UNSUPPORTED, "plan is block-scaled: use gemm_mx_run");
    if (d.M == 0 || d.N == 0)
        return ok();
    if (d.K > 0 && (!A || !B))
        return fail(GEMM_ERR_NULL_POINTER, "A or B is NULL");
    gemm_status_t st = check_epilogue_ptrs(d, C, bias, D);
    if (st != GEMM_OK)
        return st;
    const int eb = elem_bytes(d.a_type);
    if (d.K > 0 && (!aligned(A, eb) || !aligned(B, eb)))
        return fail(GEMM_ERR_MISALIGNED, "A or B not aligned to its element size");
    {
        const bool ar = d.a_layout == GEMM_ROW_MAJOR, bc = d.b_layout == GEMM_COL_MAJOR;
        st = check_d_overlap(d, C, bias, D,
                             {span(A, ar ? d.M : d.K, ar ? d.K : d.M, d.lda, eb),
                              span(B, bc ? d.N : d.K, bc ? d.K : d.N, d.ldb, eb)});
        if (st != GEMM_OK)
            return st;
    }

    GemmArgs g;
    g.A = A;
    g.B = B;
    g.K = d.K;
    if (d.a_layout == GEMM_ROW_MAJOR) {
        g.a_rs = d.lda;
        g.a_cs = 1;
    } else {
        g.a_rs = 1;
        g.a_cs = d.lda;
    }
    if (d.b_layout == GEMM_COL_MAJOR) {
        g.b_rs = 1;
        g.b_cs = d.ldb;
    } else {
        g.b_rs = d.ldb;
        g.b_cs = 1;
    }
    g.e = make_epi(d, C, bias, D);
    g.sa = g.sb = nullptr;
    g.ws = nullptr;
    g.wz = nullptr;
    g.wgs = 0;

    int fam = plan->family;
    if (fam != KF_GENERIC && (!aligned(A, 16) || !aligned(B, 16)))
        fam = plan->fallback;
    hipError_t e = launch_dense(fam, plan->op, plan->layout, g, (hipStream_t)stream);
    if (e != hipSuccess)
        return hip_fail(e, "kernel launch");
    return ok();
}

gemm_status_t gemm_sparse24_sizes(int64_t M, int64_t K, int32_t a_type, size_t *values_bytes,
                                  size_t *meta_bytes)
{
    if (!values_bytes || !meta_bytes)
        return fail(GEMM_ERR_NULL_POINTER, "output pointer is NULL");
    if (M < 0 || K < 0)
        return fail(GEMM_ERR_INVALID_VALUE, "negative size");
    if (a_type != GEMM_F16 && a_type != GEMM_BF16 && !is_int8(a_type) && !is_fp8(a_type))
        return fail(GEMM_ERR_UNSUPPORTED, "2:4 compression takes f16, bf16, fp8, s8 or u8");
    if (K % 4)
        return fail(GEMM_ERR_UNSUPPORTED, "K must be a multiple of 4");
    *values_bytes = (size_t)M * (size_t)(K / 2) * (size_t)elem_bytes(a_type);
    *meta_bytes = (size_t)M * (size_t)((K + 31) / 32) * 4;
    return ok();
}

gemm_status_t gemm_sparse24_compress(int64_t M, int64_t K, int32_t a_type, const void *A,
                                     void *values, uint32_t *meta, gemm_stream_t stream)
{
    size_t vb = 0, mb = 0;
    gemm_status_t st = gemm_sparse24_sizes(M, K, a_type, &vb, &mb);
    if (st != GEMM_OK)
        return st;
    if (M == 0 || K == 0)
        return ok();
    if (!A || !values || !meta)
        return fail(GEMM_ERR_NULL_POINTER, "A, values or meta is NULL");
    // one load per group of four elements, one store per pair of values
    const int eb = elem_bytes(a_type);
    if (!aligned(A, 4 * eb) || !aligned(values, 2 * eb) || !aligned(meta, 4))
        return fail(GEMM_ERR_MISALIGNED,
                    "A must be aligned to 4 elements, values to 2 elements, meta to 4 bytes");
    int dev = 0;
    st = check_device(&dev, nullptr);
    if (st != GEMM_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    int *flag = nullptr;
    hipError_t e = hipMalloc((void **)&flag, sizeof(int));
    if (e != hipSuccess)
        return hip_fail(e, "hipMalloc(flag)");
    int host_flag = 0;
    e = hipMemsetAsync(flag, 0, sizeof(int), s);
    if (e == hipSuccess)
        e = launch_sparse24_compress(eb, eb == 2 ? 0x7FFFu : (is_int8(a_type) ? 0xFFu : 0x7Fu),
                                     M, K, A, values, meta, flag, s);
    if (e == hipSuccess)
        e = hipMemcpyAsync(&host_flag, flag, sizeof(int), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess)
        e = hipStreamSynchronize(s);
    hipError_t ef = hipFree(flag);
    if (e != hipSuccess)
        return hip_fail(e, "sparse24 compress");
    if (ef != hipSuccess)
        return hip_fail(ef, "hipFree(flag)");
    if (host_flag)
        return fail(GEMM_ERR_NOT_SPARSE24,
                    "A has a group of 4 with more than two non-zeros (first such row: %d)",
                    0x7fffffff - host_flag);
    return ok();
}

gemm_status_t gemm_sparse24_compress_noalloc(int64_t M, int64_t K, int32_t a_type, const void *A,
                                             void *values, uint32_t *meta, gemm_stream_t stream)
{
    size_t vb = 0, mb = 0;
    gemm_status_t st = gemm_sparse24_sizes(M, K, a_type, &vb, &mb);
    if (st != GEMM_OK)
        return st;
    if (M == 0 || K == 0)
        return ok();
    if (!A || !values || !meta)
        return fail(GEMM_ERR_NULL_POINTER, "A, values or meta is NULL");
    const int eb = elem_bytes(a_type);
    if (!aligned(A, 4 * eb) || !aligned(values, 2 * eb) || !aligned(meta, 4))
        return fail(GEMM_ERR_MISALIGNED,
                    "A must be aligned to 4 elements, values to 2 elements, meta to 4 bytes");
    int dev = 0;
    st = check_device(&dev, nullptr);
    if (st != GEMM_OK)
        return st;
    // the flag is element 0 of the library's static device scratch (looked
    // up on this device's first call), cleared by a kernel on the stream
    int *flag = nullptr;
    hipError_t e = sparse24_scratch(dev, &flag);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetSymbolAddress(scratch)");
    hipStream_t s = (hipStream_t)stream;
    int host_flag = 0;
    e = launch_zero_ints(flag, 1, s);
    if (e == hipSuccess)
        e = launch_sparse24_compress(eb, eb == 2 ? 0x7FFFu : (is_int8(a_type) ? 0xFFu : 0x7Fu),
                                     M, K, A, values, meta, flag, s);
    if (e == hipSuccess)
        e = hipMemcpyAsync(&host_flag, flag, sizeof(int), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess)
        e = hipStreamSynchronize(s);
    if (e != hipSuccess)
        return hip_fail(e, "sparse24 compress (no allocation)");
    if (host_flag)
        return fail(GEMM_ERR_NOT_SPARSE24,
                    "A has a group of 4 with more than two non-zeros (first such row: %d)",
                    0x7fffffff - host_flag);
    return ok();
}

gemm_status_t gemm_sparse24_run(const gemm_plan_t *plan, const void *values, const uint32_t *meta,
                                const void *B, const void *C, const void *bias, void *D,
                                gemm_stream_t stream)
{
    if (!plan)
        return fail(GEMM_ERR_NULL_POINTER, "plan is NULL");
    const gemm_desc_t &d = plan->d;
    if (!d.sparse_a)
        return fail(GEMM_ERR_UNSUPPORTED, "plan is for dense A: use gemm_run");
    if (d.M == 0 || d.N == 0)
        return ok();
    if (d.K > 0 && (!values || !meta || !B))
        return fail(GEMM_ERR_NULL_POINTER, "values, meta or B is NULL");
    gemm_status_t st = check_epilogue_ptrs(d, C, bias, D);
    if (st != GEMM_OK)
        return st;
    const int eb = elem_bytes(d.a_type);
    if (d.K > 0 && (!aligned(values, eb) || !aligned(meta, 4) || !aligned(B, eb)))
        return fail(GEMM_ERR_MISALIGNED, "values, meta or B not aligned to its element size");
    {
        const bool bc = d.b_layout == GEMM_COL_MAJOR;
        st = check_d_overlap(d, C, bias, D,
                             {span(values, d.M, d.K / 2, d.K / 2, eb),
                              span(meta, d.M, (d.K + 31) / 32, (d.K + 31) / 32, 4),
                              span(B, bc ? d.N : d.K, bc ? d.K : d.N, d.ldb, eb)});
        if (st != GEMM_OK)
            return st;
    }
    SparseArgs a;
    a.values = values;
    a.meta = meta;
    a.B = B;
    a.K = d.K;
    if (d.b_layout == GEMM_COL_MAJOR) {
        a.b_rs = 1;
        a.b_cs = d.ldb;
    } else {
        a.b_rs = d.ldb;
        a.b_cs = 1;
    }
    a.e = make_epi(d, C, bias, D);
    int fam = plan->family;
    if (fam != KF_SPARSE_GENERIC && (!aligned(values, 16) || !aligned(B, 16) || !aligned(meta, 16)))
        fam = plan->fallback;
    hipError_t e = launch_sparse(fam, plan->op, a, (hipStream_t)stream);
    if (e != hipSuccess)
        return hip_fail(e, "kernel launch");
    return ok();
}

gemm_status_t gemm_mx_run(const gemm_plan_t *plan, const void *A, const uint8_t *scale_a,
                          const void *B, const uint8_t *scale_b, const void *C, const void *bias,
                          void *D, gemm_stream_t stream)
{
    if (!plan)
        return fail(GEMM_ERR_NULL_POINTER, "plan is NULL");
    const gemm_desc_t &d = plan->d;
    if (!d.block_scale || d.b_type == GEMM_U4)
        return fail(GEMM_ERR_UNSUPPORTED, "plan is not MX block-scaled");
    if (d.M == 0 || d.N == 0)
        return ok();
    if (d.K > 0 && (!A || !B || !scale_a || !scale_b))
        return fail(GEMM_ERR_NULL_POINTER, "A, B or a scale array is NULL");
    gemm_status_t st = check_epilogue_ptrs(d, C, bias, D);
    if (st != GEMM_OK)
        return st;
    {
        // packed rows: ld elements of mx_bits bits each
        const int64_t ra = d.lda * mx_bits(d.a_type) / 8, rb = d.ldb * mx_bits(d.b_type) / 8;
        const int64_t ka = d.K * mx_bits(d.a_type) / 8, kb = d.K * mx_bits(d.b_type) / 8;
        st = check_d_overlap(d, C, bias, D,
                             {span(A, d.M, ka, ra, 1), span(B, d.N, kb, rb, 1),
                              span(scale_a, d.M, d.K / 32, d.K / 32, 1),
                              span(scale_b, d.N, d.K / 32, d.K / 32, 1)});
        if (st != GEMM_OK)
            return st;
    }
    GemmArgs g;
    g.A = A;
    g.B = B;
    g.K = d.K;
    g.a_rs = d.lda;
    g.a_cs = 1;
    g.b_rs = 1;
    g.b_cs = d.ldb;
    g.e = make_epi(d, C, bias, D);
    g.sa = scale_a;
    g.sb = scale_b;
    g.ws = nullptr;
    g.wz = nullptr;
    g.wgs = 0;
    int fam = plan->family;
    if (fam == KF_MX_TILED &&
        (!aligned(A, 16) || !aligned(B, 16) || !aligned(scale_a, 16) || !aligned(scale_b, 16)))
        fam = plan->fallback;
    // the expansion reads a 6-bit operand 4 bytes at a time; an 8-bit one
    // goes to the tiled kernel as it is
    if (fam == KF_MX_TILED6 &&
        (!aligned(A, mx_bits(d.a_type) == 6 ? 4 : 16) ||
         !aligned(B, mx_bits(d.b_type) == 6 ? 4 : 16) || !aligned(scale_a, 16) ||
         !aligned(scale_b, 16)))
        fam = plan->fallback;
    hipError_t e = launch_mx(fam, plan->op / 8, plan->op % 8, g, (hipStream_t)stream);
    if (e != hipSuccess)
        return hip_fail(e, "kernel launch");
    return ok();
}

gemm_status_t gemm_w4a16_run(const gemm_plan_t *plan, const void *A, const void *B,
                             const void *scales, const uint8_t *zeros, const void *C,
                             const void *bias, void *D, gemm_stream_t stream)
{
    if (!plan)
        return fail(GEMM_ERR_NULL_POINTER, "plan is NULL");
    const gemm_desc_t &d = plan->d;
    if (d.b_type != GEMM_U4)
        return fail(GEMM_ERR_UNSUPPORTED, "plan is not W4A16");
    if (d.M == 0 || d.N == 0)
        return ok();
    if (d.K > 0 && (!A || !B || !scales))
        return fail(GEMM_ERR_NULL_POINTER, "A, B or scales is NULL");
    gemm_status_t st = check_epilogue_ptrs(d, C, bias, D);
    if (st != GEMM_OK)
        return st;
    if (d.K > 0 && (!aligned(A, 2) || !aligned(scales, 2)))
        return fail(GEMM_ERR_MISALIGNED, "A or scales not aligned to 2 bytes");
    {
        const int64_t groups = d.K / d.block_scale;
        st = check_d_overlap(d, C, bias, D,
                             {span(A, d.M, d.K, d.lda, 2), span(B, d.N, d.K / 2, d.ldb / 2, 1),
                              span(scales, d.N, groups, groups, 2),
                              span(zeros, d.N, groups, groups, 1)});
        if (st != GEMM_OK)
            return st;
    }
    GemmArgs g;
    g.A = A;
    g.B = B;
    g.K = d.K;
    g.a_rs = d.lda;
    g.a_cs = 1;
    g.b_rs = 1;
    g.b_cs = d.ldb;
    g.e = make_epi(d, C, bias, D);
    g.sa = g.sb = nullptr;
    g.ws = scales;
    g.wz = zeros;
    g.wgs = d.block_scale;
    int fam = plan->family;
    if ((fam == KF_W4_TILED || fam == KF_W4_TILED16 || fam == KF_W4_SKINNY) &&
        (!aligned(A, 16) || !aligned(B, 16)))
        fam = plan->fallback;
    hipError_t e = launch_w4(fam, plan->op, g, (hipStream_t)stream);
    if (e != hipSuccess)
        return hip_fail(e, "kernel launch");
    return ok();
}

gemm_status_t gemm_diag_mfma_loop(int32_t kind, int32_t blocks, int64_t iters, float *out,
                                  gemm_stream_t stream)
{
    if (!out)
        return fail(GEMM_ERR_NULL_POINTER, "out is NULL");
    if (kind < 0 || kind > 5 || blocks < 1 || blocks > (1 << 20) || iters < 0)
        return fail(GEMM_ERR_INVALID_VALUE, "kind 0..5, blocks 1..2^20, iters >= 0");
    int dev = 0;
    gemm_status_t st = check_device(&dev, nullptr);
    if (st != GEMM_OK)
        return st;
    hipError_t e = launch_mfma_loop(kind, blocks, iters, out, (hipStream_t)stream);
    if (e != hipSuccess)
        return hip_fail(e, "kernel launch");
    return ok();
}

} // extern "C"
