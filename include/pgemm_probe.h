/*
 * pgemm_probe: a measurement aid shipped beside pgemm, not part of the GEMM
 * path.  Reports how fast v_mfma_f32_16x16x32_f16 (the GEMM's instruction)
 * runs on the current HIP device with no memory traffic (1024 workgroups of
 * four waves, each wave holding the GEMM's 8 x 8 accumulator tiles and
 * alternating between two sets of operand fragments), so that a GEMM's
 * throughput can be set against the clock the chip's power limit allows as
 * well as against the nominal peak.  It is a reference point, not a bound:
 * a GEMM trades issue slots and power for data movement differently.
 */
#ifndef PGEMM_PROBE_H
#define PGEMM_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Runs the MFMA loop twice on the null stream (the second run is timed with
 * HIP events) and blocks until it ends.  zero_operands: 0 for operands
 * uniform in [-1, 1) (the bits change as in a GEMM), 1 for zero operands.
 * iters: loop trips per wave (128 MFMAs each), 1 .. 2^24; 4000 takes about
 * 5 ms.  On success writes the dense f16 TFLOP/s and the average shader
 * clock of the timed run in GHz (shader-clock counter over the 100 MHz
 * reference counter, read by one wave) and returns 0; returns 1 for bad
 * arguments, 2 if a HIP call fails.  Allocates and frees its own small
 * device buffers.
 */
int pgemm_probe_mfma(int zero_operands, int64_t iters, double *tflops, double *sclk_ghz);

#ifdef __cplusplus
}
#endif

#endif /* PGEMM_PROBE_H */
