/*
 * fa_bwd_calib.h -- a measurement hook of libfa_bwd.so, kept apart from the
 * method's entry points in fa_bwd.h: it computes nothing of the attention
 * backward.  It runs back-to-back bf16 MFMAs so that a benchmark can state
 * the matrix-core rate the chip sustains on given operand data (the ceiling
 * the tile kernels can approach when the clock is power-limited), next to the
 * published peak.
 */
#ifndef FA_BWD_CALIB_H
#define FA_BWD_CALIB_H

#include "fa_bwd.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Calibration kernel for the MFMA roofline (not a step of the backward): the
 * bf16 MFMA rate the chip sustains on given operand data.  `blocks` workgroups
 * of 256 threads (one wave per SIMD) each issue iters x 32 back-to-back
 * v_mfma_f32_32x32x16_bf16 per wave, four independent accumulator chains,
 * operands rotating over four register blocks, nothing else in the loop.
 *   operands: device, 16-byte aligned, 2048 x 8 bf16 (32 KiB), read only
 *             (thread t: A blocks at [t + 256 i], B blocks at [1024 + t + 256 i]).
 *   sink:     device float [blocks * 256], written (keeps the work alive).
 * Work: blocks * 4 * iters * 32 * 32768 FLOP.  Errors: FA_ERR_NULL,
 * FA_ERR_ARG (blocks or iters <= 0), FA_ERR_ALIGN (operands).
 */
fa_status fa_bwd_calib_mfma_bf16(const void* operands, float* sink, int32_t blocks, int32_t iters,
                                 fa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_BWD_CALIB_H */
