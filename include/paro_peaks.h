/*
 * paro_peaks.h - measurement helpers (not part of the PISA path): kernels
 * that measure the practical peaks of the GPU the path runs on, so that the
 * path's rates can be stated against measured ceilings as well as against
 * the data-sheet figures.
 *
 * Conventions as in paro.h: device pointers, `stream` a hipStream_t passed
 * as void*, work enqueued asynchronously, PARO-style return codes (0 = ok,
 * -2 = bad size, -1 = NULL pointer, -6 = HIP launch error). Nothing is
 * allocated.
 */
#ifndef PARO_PEAKS_H_
#define PARO_PEAKS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * paro_peak_mfma_bf16 - dense bf16 matrix-core throughput: `workgroups`
 * workgroups of 256 threads (4 waves); each wave runs `iters` rounds of 8
 * independent chains of v_mfma_f32_32x32x16_bf16 on register operands, then
 * folds its accumulators into sink[workgroup] (so nothing is optimised
 * away). Work = workgroups * 4 * iters * 8 * 32768 FLOP.
 * sink: at least `workgroups` floats. 1 <= workgroups <= 2^20, 1 <= iters <= 2^20.
 */
int paro_peak_mfma_bf16(int32_t workgroups, int32_t iters, float* sink, void* stream);

/*
 * paro_peak_read - HBM read throughput: sums `bytes` bytes of src (16-byte
 * loads, a grid-stride loop over `workgroups` workgroups of 256 threads)
 * into sink[workgroup]. bytes a multiple of 16 and >= 16; src 16-byte
 * aligned; sink: at least `workgroups` floats.
 */
int paro_peak_read(const void* src, size_t bytes, int32_t workgroups, float* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* PARO_PEAKS_H_ */
