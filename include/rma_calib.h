/*
 * rma_calib.h - measurement support in librma.so: a streaming-read probe
 * that calibrates the HBM read bandwidth a plain kernel reaches on the
 * device, the yardstick next to the decode kernel's achieved bandwidth.
 * It is not part of the RMA layer step.
 */
#ifndef RMA_CALIB_H
#define RMA_CALIB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` of the DEVICE buffer `buf` (16-byte aligned, caller-owned)
 * once, with `waves` waves (a multiple of 4, one workgroup of 4 waves per
 * 4): wave w reads the w-th contiguous share with 16-byte non-temporal
 * loads, folds the words by xor and writes the result to sink[w]
 * (DEVICE memory of `waves` uint32, caller-owned).  `bytes` must be a
 * multiple of waves * 16 KiB.  Enqueued on `stream` (a hipStream_t, NULL =
 * the null stream).  Returns 0, -1 for invalid arguments (nothing
 * enqueued), or -4 if the launch failed. */
int rma_calib_stream_read(const void* buf, size_t bytes, int32_t waves, uint32_t* sink,
                          void* stream);

#ifdef __cplusplus
}
#endif
#endif /* RMA_CALIB_H */
