/*
 * qc_bench.h -- measurement aid of the library, not part of the scan's method.
 *
 * qc_stream_copy copies nbytes from src to dst (device pointers on the current
 * HIP device, both 16-byte aligned, nbytes a multiple of 16, not
 * overlapping) with a plain streaming kernel: every byte is read once and
 * written once, 1 KiB contiguous per wave instruction, non-temporal.  Its rate
 * is the practical HBM ceiling that the scan kernels' achieved bandwidth is
 * set beside.  blocks_per_cu (1 .. 64) sets the grid: that many 256-thread
 * blocks per compute unit, each walking the buffer in 16 KiB strides.
 * Asynchronous on `stream` (a hipStream_t as void*).
 *
 * Returns 0, or the negative codes of quat_cumprod.h: QC_ERR_NULL (-1),
 * QC_ERR_ALIGN (-3), QC_ERR_ALIAS (-5), QC_ERR_HIP (-7), QC_ERR_OPTION (-8)
 * for blocks_per_cu out of range.  nbytes = 0 is a no-op.
 */
#ifndef QC_BENCH_H
#define QC_BENCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int qc_stream_copy(const void* src, void* dst, size_t nbytes, int32_t blocks_per_cu, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QC_BENCH_H */
