/*
 * w8a8_probe.h -- diagnostic entry points of the W8A8 library (not part of
 * the quantized-linear method): measured ceilings that performance reports
 * quote next to the spec peaks.  Same conventions as w8a8.h (device pointers
 * owned by the caller, 16-byte alignment, host-side checks, enqueue on
 * `stream` and return).
 */
#ifndef W8A8_PROBE_H
#define W8A8_PROBE_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "w8a8.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Number of int32 values w8a8_probe_mfma_i8 writes to `sink` on the current
 * device (256 per compute unit). */
int64_t w8a8_probe_sink_count(void);

/*
 * Sustained int8 MFMA rate on given operand bytes: one workgroup of 4 waves
 * per compute unit, each wave looping `pairs` times over 32 products
 * v_mfma_i32_32x32x32_i8 (two alternating sets of 4 x 4 fragments read once
 * from the first 64 KiB of a and of b) into 16 independent 32x32
 * accumulators.  Integer operations per call:
 *   pairs * 32 * 2 * 32 * 32 * 32 * 4 * (compute units).
 *   a, b   device bytes, at least 65536 each (e.g. activation and weight codes,
 *          so that the matrix cores see the workload's value distribution).
 *   sink   int32 [w8a8_probe_sink_count()]: an xor of each lane's results.
 * Errors: W8A8_ERR_INVALID_ARG (null pointer, pairs < 0), W8A8_ERR_ALIGN;
 * pairs == 0 is a no-op.
 */
w8a8_status w8a8_probe_mfma_i8(const void *a, const void *b, int64_t pairs, int32_t *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* W8A8_PROBE_H */
