/*
 * gdn_measure.h -- measurement aids of libgdn.so.  Not part of the method:
 * the benchmark uses them to put the layer core's kernels next to what the
 * device can do at all.
 */
#ifndef GDN_MEASURE_H
#define GDN_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Copy `bytes` bytes from src to dst on the device with 16-byte non-temporal
 * loads and stores, one per thread: the access pattern of the decode
 * recurrence's state stream without its arithmetic, used as the achievable
 * read + write bandwidth reference.  Asynchronous on `stream`.
 *   dst, src  device pointers, 16-byte aligned, not overlapping
 *   bytes     a multiple of 16 (0: nothing is launched)
 * Returns GDN_OK, GDN_ERR_NULL, GDN_ERR_SHAPE (alignment or size),
 * GDN_ERR_ALIAS (overlap) or GDN_ERR_LAUNCH.
 */
int gdn_stream_copy(void *dst, const void *src, size_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_MEASURE_H */
