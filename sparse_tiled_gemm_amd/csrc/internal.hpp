// Library-internal declarations shared by the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include "gemm.h"
#include "kernel_args.hpp"

namespace stg {

// MFMA operand-pair kinds.
enum OpKind {
    OPK_F16 = 0,
    OPK_BF16,
    OPK_F8_E4E4,
    OPK_F8_E4E5,
    OPK_F8_E5E4,
    OPK_F8_E5E5,
    OPK_S8,
    OPK_U8S8, // u8 A x s8 B (int8 MFMA on A - 128, corrected in the epilogue)
    OPK_S8U8,
    OPK_U8U8,
    OPK_COUNT
};

// Kernel families a plan can select.
enum KernelFamily {
    KF_GENERIC = 0, // any layout / shape / alignment
    KF_TILED_256,   // 256 x 256 workgroup tile, LDS double buffer
    KF_TILED_128,   // 128 x 128 workgroup tile, LDS double buffer
    KF_SKINNY,      // M <= 16, bandwidth-oriented
    KF_SPARSE_GENERIC,
    KF_SPARSE_TILED,
    KF_TILED_256W8,  // 256 x 256, 8 waves (2 per SIMD) as 2 x 4, 128 x 64 per wave
    KF_TILED_256W8T, // 256 x 256, 8 waves as 4 x 2, 64 x 128 per wave
    KF_SPARSE_DMA8,  // 2:4 A, 256 x 256, 8 waves, direct global -> LDS copies, 3 stages
    KF_MX_GENERIC,   // MX block-scaled, any format pair
    KF_MX_TILED,     // MX block-scaled, 256 x 256 4-wave tile, pairs of one width (8 or 4 bits)
    KF_W4_GENERIC,   // W4A16, any shape
    KF_W4_TILED,     // W4A16, 256 x 256 4-wave tile, B dequantised into LDS
    KF_W4_SKINNY,    // W4A16, M <= 16, B streamed and dequantised in registers
    KF_MX_TILED6,    // MX with 6-bit operands: expanded to 8-bit codes, then KF_MX_TILED's kernel
    KF_TILED_256W8K16,  // k_tiled16: 256 x 256, 8 waves of 128 x 64, fragments refreshed in
                        // place (16-bit / int8 on the 16x16 forms, fp8 on 32x32x64)
    KF_TILED_256W8TK16, // the same, 8 waves of 64 x 128
    KF_W4_TILED16,      // W4A16 on the 16x16-form kernel, 8 waves of 128 x 64
    KF_COUNT
};

// layout: 0 A row-major and B column-major (K contiguous); bit 0 A
// column-major, bit 1 B row-major (generic, or see launch_dense_mn)
hipError_t launch_dense(int family, int op, int layout, const GemmArgs &g, hipStream_t s);
// KF_TILED_256W8K16 (kernels_k16.hip): op OPK_F16, OPK_BF16, OPK_S8 or an fp8
// pair, K-contiguous
hipError_t launch_tiled16(int op, const GemmArgs &g, hipStream_t s);
hipError_t launch_tiled16t(int op, const GemmArgs &g, hipStream_t s); // KF_TILED_256W8TK16
hipError_t launch_w4_tiled16(int op, const GemmArgs &g, hipStream_t s); // KF_W4_TILED16
// MN-major layouts (layout 1..3) on the tiled families that take them: the
// 128 x 128 tile, and the 256 x 256 arrangement of each input type
// (tiled256w8 16-bit, tiled256 fp8, tiled256w8t int8)
hipError_t launch_dense_mn(int family, int op, int layout, const GemmArgs &g, hipStream_t s);
// MX block-scaled: afmt / bfmt are the element-format selectors of OpMX
// (0 E4M3, 1 E5M2, 2 E2M3, 3 E3M2, 4 E2M1); g.sa / g.sb hold the scales.
hipError_t launch_mx(int family, int afmt, int bfmt, const GemmArgs &g, hipStream_t s);
hipError_t launch_mx_tiled(int afmt, int bfmt, const GemmArgs &g, hipStream_t s);
// both operands 6-bit, in the padded 8-bit geometry of OpMX<.., .., true>
hipError_t launch_mx_tiled_pad6(int afmt, int bfmt, const GemmArgs &g, hipStream_t s);
// W4A16: op is OPK_F16 or OPK_BF16 (the activations' type); g.ws / g.wz /
// g.wgs hold the weight groups' scales and zero points.
hipError_t launch_w4(int family, int op, const GemmArgs &g, hipStream_t s);
hipError_t launch_w4_tiled(int op, const GemmArgs &g, hipStream_t s);
hipError_t launch_w4_skinny(int op, const GemmArgs &g, hipStream_t s);
hipError_t launch_sparse(int family, int op, const SparseArgs &a, hipStream_t s);
// Compressor for elements of elem_bytes (2 or 1) bytes, an element being a
// zero when (bits & zero_mask) == 0: writes values/meta; *flag (device int,
// zeroed by the caller) becomes 0x7fffffff - r for the lowest row r holding a
// group with more than two non-zeros, and stays 0 otherwise.
hipError_t launch_sparse24_compress(int elem_bytes, uint32_t zero_mask, int64_t M, int64_t K,
                                    const void *A, void *values, uint32_t *meta, int *flag,
                                    hipStream_t s);
// Allocation-free compressor: the device address of this library's static
// scratch array on device `dev` (current), SPARSE24_SCRATCH_INTS ints, of
// which the flag uses element 0; and a kernel that zeroes n ints.
constexpr int SPARSE24_SCRATCH_INTS = 64;
// Diagnostic MFMA-only loop (kernels_diag.hip): kind 0 bf16, 1 fp8, 2 int8
// (32x32 forms), 3..5 the same types' 16x16 forms; `blocks` workgroups of
// 512 threads.
hipError_t launch_mfma_loop(int kind, int blocks, int64_t iters, float *out, hipStream_t s);
hipError_t sparse24_scratch(int dev, int **out);
hipError_t launch_zero_ints(int *p, int n, hipStream_t s);

} // namespace stg

struct gemm_plan {
    gemm_desc_t d;   // normalised: packed leading dimensions filled in
    int op;          // stg::OpKind
    int family;      // stg::KernelFamily
    int fallback;    // family used when run-time alignment rules out `family`
    int layout;      // dense operand layout (see launch_dense)
    int device;      // HIP device the plan was made on
    char name[96];
};
