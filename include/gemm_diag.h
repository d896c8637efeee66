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
 * wave running `iters` iterations of 64 MFMAs (a 4 x 2 grid of 32x32
 * accumulators over 8 K steps; operands from a pool of 8 random fragments
 * that rotate every step) of kind 0: v_mfma_f32_32x32x16_bf16 (32768 flop
 * each), 1: v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3 x E4M3 with unit scales
 * (131072 flop), 2: v_mfma_i32_32x32x32_i8 (65536 op).  `out` (device, owned
 * by the caller) receives blocks * 512 floats of accumulator sums, which
 * keep the work from being optimised away.  Returns GEMM_ERR_NULL_POINTER,
 * GEMM_ERR_INVALID_VALUE (kind not 0..2, blocks not 1..2^20, iters < 0),
 * GEMM_ERR_DEVICE, GEMM_ERR_HIP or GEMM_OK; asynchronous like gemm_run. */
gemm_status_t gemm_diag_mfma_loop(int32_t kind, int32_t blocks, int64_t iters, float *out,
                                  gemm_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif
