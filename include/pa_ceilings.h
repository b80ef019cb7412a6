/*
 * Chip ceilings measured beside the published MI355X peaks (not part of the
 * attention path; bench.py --mode ceilings calls them).
 *
 * pa_ceiling_mfma: `blocks` work groups of 4 waves (one per SIMD), each wave
 *   issuing `iters` x 4 independent v_mfma_f32_32x32x16_f16 (32768 FLOP each)
 *   on operands[0..127] (16-byte fp16 fragments, device memory the caller
 *   fills); per-thread sums go to sink[blocks * 256].  clocks[2 b] and
 *   clocks[2 b + 1] receive work group b's elapsed shader-clock and 100 MHz
 *   real-time ticks.  Asynchronous on `stream` (a hipStream_t); 0 = launched, -1 = bad
 *   argument, -4 = launch error.
 * pa_ceiling_mfma_lds: the same loop, but every pair of MFMAs takes a new A
 *   fragment read from LDS (the operand traffic of attention's S^T phase):
 *   operands[0..2047] (32 KB of 16-byte fp16 fragments, copied to LDS) and
 *   operands[2048..2303] (four register fragments); per iteration 2 LDS reads
 *   and 4 MFMAs (iters is rounded down to even).  sink / clocks / return
 *   codes as pa_ceiling_mfma.
 * pa_ceiling_mfma_valu: pa_ceiling_mfma's loop with `nvalu` (0, 2, 4, 6 or
 *   8) independent vector-ALU instructions after every MFMA, v_fma_f32
 *   (kind 0) or v_exp_f32 (kind 1), on registers the MFMAs do not use; one
 *   wave per SIMD.  operands[0..127], sink, clocks and return codes as
 *   pa_ceiling_mfma (-1 also for an unsupported nvalu or kind).
 * pa_ceiling_stream_read: `blocks` x 256 threads read `bytes` (a multiple of
 *   16, 16-byte aligned) of `src` once with 16-byte non-temporal loads, each
 *   block one contiguous range; sink[blocks * 256] receives one float per
 *   thread.  Same return codes.
 */
#ifndef PA_CEILINGS_H
#define PA_CEILINGS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int pa_ceiling_mfma(const void *operands, float *sink, int32_t blocks, int32_t iters,
                    unsigned long long *clocks, void *stream);
int pa_ceiling_mfma_lds(const void *operands, float *sink, int32_t blocks, int32_t iters,
                        unsigned long long *clocks, void *stream);
int pa_ceiling_mfma_valu(const void *operands, float *sink, int32_t blocks, int32_t iters, int32_t nvalu,
                         int32_t kind, unsigned long long *clocks, void *stream);
int pa_ceiling_stream_read(const void *src, int64_t bytes, float *sink, int32_t blocks, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_CEILINGS_H */
