/*
 * gdr_peaks.h -- on-device peak probes (libgdr_peaks.so), separate from the
 * computing library libgdr.so.
 *
 * The roofline of a kernel compares its achieved bytes/s and flop/s with the
 * machine's peaks.  MI355X publishes 8 TB/s of HBM3E bandwidth and 2.5
 * PFLOP/s of dense bf16 matrix math; these probes measure what one simple
 * kernel reaches on the device at hand, so a roofline fraction can be stated
 * against both the published and the measured peak.
 *
 * Both calls enqueue their kernel `reps` times on `stream` (a hipStream_t;
 * NULL = the null stream) between two HIP events, wait for the second event
 * (these calls DO synchronise, unlike libgdr) and return the mean duration of
 * one kernel in *ms_out.  Buffers are owned by the caller.  Return value: 0,
 * or -1 for invalid arguments, -4 for a HIP error.
 */
#ifndef GDR_PEAKS_H_
#define GDR_PEAKS_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Device-to-device copy of `bytes` (a multiple of 16; src and dst 16-byte
 * aligned device buffers that do not overlap): every byte is read once and
 * written once, 16 bytes per lane access.  HBM traffic per kernel = 2 bytes. */
int gdr_peak_copy(const void* src, void* dst, size_t bytes, int reps, void* stream, float* ms_out);

/* A loop of independent bf16 MFMA instructions: `workgroups` workgroups of
 * 4 waves, each wave issuing independent accumulation chains for `iters`
 * iterations: tile 16 = eight chains of V_MFMA_F32_16X16X32_BF16 per
 * iteration, tile 32 = four chains of V_MFMA_F32_32X32X16_BF16 (both 131072
 * flop per wave and iteration).  sink: device buffer of workgroups * 256
 * floats (written so the work is not optimised away).
 * Flops per kernel = workgroups * 4 * iters * 131072. */
int gdr_peak_mfma_bf16(float* sink, int tile, int iters, int workgroups, int reps, void* stream, float* ms_out);

#ifdef __cplusplus
}
#endif

#endif /* GDR_PEAKS_H_ */
