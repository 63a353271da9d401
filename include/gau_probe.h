/*
 * gau_probe.h -- measurement aid of libgau (not part of the layer).
 *
 * The layer's roofline is quoted against the MI355X's published dense bf16
 * MFMA peak (256 CUs x 4 SIMDs x 1024 FLOP/clk x 2.4 GHz = 2516.6 TFLOP/s).
 * Under a sustained matrix load the chip may run below the 2.4 GHz on which
 * that figure rests, so the benchmark also measures the rate the matrix cores
 * reach with nothing else in the way, and quotes the layer against both.
 */
#ifndef GAU_PROBE_H
#define GAU_PROBE_H

#include "gau.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Queues one launch of `blocks` workgroups of four waves; every wave issues
 * iters * 16 v_mfma_f32_32x32x16_bf16 on operands held in registers (four
 * independent accumulators, so consecutive instructions never wait on each
 * other) and reads no memory.  FLOPs per launch:
 * blocks * 4 * iters * 16 * 32768.  `out` (device, one float) is written only
 * if the accumulators sum to a sentinel they cannot reach, which keeps the
 * compiler from dropping the work; it may be any 16-byte aligned device
 * pointer.  GAU_ERR_SHAPE if blocks or iters is not in 1 .. 2^20 or
 * blocks * iters > 2^22 (a cap on one call's work: about 4.4 PFLOP, seconds
 * of the whole chip), GAU_ERR_NULL / GAU_ERR_ALIGN for `out`, GAU_ERR_HIP if
 * the launch fails.  Nothing is queued unless the status is GAU_OK.
 */
gau_status gau_probe_mfma(int blocks, int iters, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GAU_PROBE_H */
