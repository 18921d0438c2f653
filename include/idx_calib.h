/*
 * idx_calib.h - measurement kernels of libidx_calib, the ceilings the indexer's
 * kernels are compared against on the device they run on (a separate library: nothing
 * in libidx calls it).
 *
 *   - idx_calib_copy / idx_calib_read: the HBM bandwidth a plain streaming kernel gets
 *     (16-byte loads, every CU busy), the practical ceiling of an HBM-bound kernel
 *     beside the published 8 TB/s;
 *   - idx_calib_mfma: the rate of the dense fp8 or fp4 16x16x128 matrix instruction
 *     the logits kernels use, from register operands, beside the published 5.0 / 10.1
 *     PFLOP/s.
 *
 * Pointers are device memory owned by the caller; each call enqueues one kernel on
 * `stream` and returns 0, or the HIP error code of a failed check or launch. The
 * caller times the launch (events on the same stream).
 */
#ifndef IDX_CALIB_H
#define IDX_CALIB_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dst[0, bytes) = src[0, bytes). bytes a multiple of 16, both 16-byte aligned. */
int32_t idx_calib_copy(const void *src, void *dst, size_t bytes, hipStream_t stream);

/* Reads src[0, bytes) and writes one 32-bit digest per workgroup to sink (at least
 * idx_calib_read_sink_words() words). bytes a multiple of 16, src 16-byte aligned. */
int32_t idx_calib_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream);
int32_t idx_calib_read_sink_words(void);

/* A grid of matrix-core loops: fmt 0 = e4m3 x e4m3, 1 = e2m1 x e2m1 (scaled form),
 * `iters` loop trips of 8 independent 16x16x128 instructions per wave, every CU
 * holding 8 waves; operands alternate between two register sets of toggling bits.
 * Writes one float per wave to sink (at least idx_calib_mfma_sink_words() floats) and
 * the launch's floating-point operation count to *flop_out (host memory). */
int32_t idx_calib_mfma(int32_t fmt, int32_t iters, float *sink, int64_t *flop_out, hipStream_t stream);
int32_t idx_calib_mfma_sink_words(void);

#ifdef __cplusplus
}
#endif

#endif /* IDX_CALIB_H */
