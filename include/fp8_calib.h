/* Calibration kernels for the measurement of the FP8 path (not part of the path itself).
 *
 * libfp8calib.so, beside libscaledfp8.so.  Used by bench.py to report the GEMM's matrix-core
 * fraction against a measured ceiling as well as against the published peak.
 */
#ifndef FP8_CALIB_H
#define FP8_CALIB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Matrix-core ceiling: `blocks` workgroups of 8 waves; every wave issues `iters` x 16 scaled
 * 32x32x64 FP8 (E4M3 x E4M3) MFMAs back to back on operands read from the caller's codes.
 *   A       device FP8 codes, a_bytes >= 2048, 16-byte aligned (read in 32-byte chunks, modulo
 *           a_bytes / 32; every read stays inside the buffer)
 *   e8m0    device e8m0 scale bytes, e_bytes >= 256, 4-byte aligned (read as 4-byte words)
 *   sink    device fp32 [blocks * 512] (the accumulators' sums, so that no work is dropped)
 *   clocks  device int64 [blocks][2]: per block, core cycles and constant-rate counter ticks
 *           across wave 0's MFMA loop (clock = cycles / ticks * fp8_calib_wall_clock_khz)
 *   stream  hipStream_t as void *.
 * Returns 0, -1 (null or misaligned pointer), -2 (sizes), -5 (launch failure).  Asynchronous. */
int fp8_calib_mfma(const uint8_t *A, size_t a_bytes, const uint8_t *e8m0, size_t e_bytes, int blocks, int iters,
                   float *sink, long long *clocks, void *stream);

/* FP8 operations one fp8_calib_mfma call performs (2 per multiply-add). */
double fp8_calib_mfma_flops(int blocks, int iters);

/* The constant-rate counter's frequency in kHz, or -4 if the device query fails. */
int fp8_calib_wall_clock_khz(int device);

#ifdef __cplusplus
}
#endif

#endif
