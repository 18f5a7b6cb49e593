/*
 * delta_measure.h -- measurement helper of the delta-rule library (not a step of the method).
 *
 * delta_measure_copy: copies `bytes` bytes from src to dst (device pointers, 16-byte aligned, bytes
 * a multiple of 16, not overlapping) with a plain streaming kernel: 256-lane workgroups, each lane
 * loading `unroll` 16-byte pieces (1, 2, 4 or 8) before storing them, `blocks` workgroups striding
 * over the buffer, non-temporal loads and stores when `nontemporal` is nonzero.  It is the
 * reference for the memory-bound kernels (the best rate it reaches is the practical ceiling of a
 * kernel that reads and writes every byte once) and a kernel of known traffic for scaling HBM
 * byte counters.  Asynchronous on `stream`.  Returns 0, or -1 (NULL pointer), -3 (unroll or blocks
 * out of range), -4 (misaligned or bytes not a multiple of 16), -6 (overlap), -7 (launch error):
 * the codes of delta.h.
 */
#ifndef DELTA_MEASURE_H
#define DELTA_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int delta_measure_copy(const void* src, void* dst, size_t bytes, int32_t unroll, int32_t blocks,
                       int32_t nontemporal, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DELTA_MEASURE_H */
