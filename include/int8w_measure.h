/*
 * int8w_measure.h -- calibration kernels exported by libint8w.so beside the
 * layer entry points of int8w.h.  They are not part of the weight path: they
 * measure what a plain stream reaches on the device, the ceiling that the
 * bandwidth-bound layer kernels (gemv, dequantize_to, quantize) are compared
 * with next to the nominal HBM peak: a read (the gemv's mix), a copy (one
 * write per byte read) and an expand (two bytes written per byte read, the
 * mix of dequantize_to).  They stream their bytes the way the layer kernels
 * stream weights: each wave a contiguous range of 1 KiB items, 16 bytes per
 * lane, non-temporal loads, two blocks of four loads in flight, 8-wave
 * workgroups (four per compute unit for the read, eight for the others).
 *
 * Conventions are those of int8w.h: DEVICE pointers, `stream` a hipStream_t
 * cast to uint64_t, validation on the host before anything is enqueued,
 * INT8W_OK or a negative INT8W_ERR_* code with int8w_last_error() set.
 */
#ifndef INT8W_MEASURE_H
#define INT8W_MEASURE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes of `src` once (a multiple of 1024, at most 2^40; src
 * 16-byte aligned).  sink is a device uint32 that the kernel writes only for
 * one improbable XOR of the data (it keeps the loads from being dead code);
 * its value means nothing.  INT8W_ERR_NULL, INT8W_ERR_SHAPE (bytes zero, not a
 * multiple of 1024, or too large), INT8W_ERR_ALIGN. */
int int8w_stream_read(const void *src, uint64_t bytes, uint32_t *sink, uint64_t stream);

/* Copy `bytes` bytes from src to dst (same rules; dst 16-byte aligned and not
 * overlapping src, else INT8W_ERR_ALIAS). */
int int8w_stream_copy(const void *src, void *dst, uint64_t bytes, uint64_t stream);

/* Widen `bytes` bytes of src to 16-bit values: ((uint16_t *)dst)[i] = src[i]
 * for i < bytes (same rules as the copy; dst holds 2 * bytes bytes, 16-byte
 * aligned and not overlapping src, else INT8W_ERR_ALIAS). */
int int8w_stream_expand(const void *src, void *dst, uint64_t bytes, uint64_t stream);

#ifdef __cplusplus
}
#endif

#endif /* INT8W_MEASURE_H */
