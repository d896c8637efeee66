/*
 * gemm_diag.h - diagnostic entry point of libstgemm.so (not part of the GEMM
 * operation itself): the MFMA-only throughput ceiling of the device.
 *
 * The GEMM of "NVIDIA MMA" (section "From FMA to MMA to GEMM") is many tile
 * MMAs plus data movement; this call issues the tile MMAs alone, on random
 * register operands, so the rate it reaches bounds what any GEMM main loop
 * of the same instruction can sustain on this chip (whose clock settles
 * lower under full MFMA load than the datasheet peak assumes).
 */
#ifndef STGEMM_GEMM_DIAG_H
#define STGEMM_GEMM_DIAG_H

#include <stdint.h>

#include "gemm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Enqueue `blocks` workgroups of 8 waves (launch one per compute unit), each
 * wave running `iters` iterations of MFMAs on operands from a pool of 8
 * random fragments that rotate every K step: kinds 0..2 issue 64 32x32
 * instructions per iteration (a 4 x 2 grid of accumulators over 8 K steps)
 * of 0: v_mfma_f32_32x32x16_bf16 (32768 flop each), 1:
 * v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3 x E4M3 with unit scales (131072
 * flop), 2: v_mfma_i32_32x32x32_i8 (65536 op); kinds 3..5 issue 128 16x16
 * instructions (an 8 x 4 grid over 4 K steps) of the same types' 16x16
 * forms at half those counts (3: 16x16x32 bf16, 4: 16x16x128 f8f6f4, 5:
 * 16x16x64 i8), so kind k and k + 3 do the same work per iteration.  `out`
 * (device, owned by the caller) receives blocks * 512 floats of accumulator
 * sums, which keep the work from being optimised away.  Returns
 * GEMM_ERR_NULL_POINTER, GEMM_ERR_INVALID_VALUE (kind not 0..5, blocks not
 * 1..2^20, iters < 0), GEMM_ERR_DEVICE, GEMM_ERR_HIP or GEMM_OK;
 * asynchronous like gemm_run. */
gemm_status_t gemm_diag_mfma_loop(int32_t kind, int32_t blocks, int64_t iters, float *out,
                                  gemm_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif
