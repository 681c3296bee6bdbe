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
 * per compute unit, each wave looping `pairs` times over 64 products
 * v_mfma_i32_16x16x64_i8 (8 x 8 fragments read once from the first 64 KiB of
 * a and of b) into 64 independent 16x16 accumulators.  Integer operations
 * per call: pairs * 64 * 2 * 16 * 16 * 64 * 4 * (compute units), which equals
 * pairs * 32 * 2 * 32 * 32 * 32 * 4 * (compute units).
 *   a, b   device bytes, at least 65536 each (e.g. activation and weight codes,
 *          so that the matrix cores see the workload's value distribution).
 *   sink   int32 [w8a8_probe_sink_count()]: an xor of each lane's results.
 * Errors: W8A8_ERR_INVALID_ARG (null pointer, pairs < 0), W8A8_ERR_ALIGN;
 * pairs == 0 is a no-op.
 */
w8a8_status w8a8_probe_mfma_i8(const void *a, const void *b, int64_t pairs, int32_t *sink, hipStream_t stream);

/*
 * The hardware e4m3 conversion the quantizers use, on consecutive f32 bit
 * patterns: codes[i] = the OCP E4M3FN code (RNE) of the f32 value whose bit
 * pattern is first_bits + i, after the quantizers' clamp to [-448, 448]
 * (v_med3_f32, then v_cvt_pk_fp8_f32).  Lets a test compare the hardware
 * encoding with a reference on every f32 of a range.
 *   codes  device bytes [n].
 * Errors: W8A8_ERR_INVALID_ARG (n < 0, null codes with n > 0, or
 * first_bits + n > 2^32), W8A8_ERR_ALIGN; n == 0 is a no-op.
 */
w8a8_status w8a8_probe_cvt_e4m3(uint32_t first_bits, int64_t n, uint8_t *codes, hipStream_t stream);

/*
 * Tile width along N (256 or 192) that w8a8_linear and
 * w8a8_linear_backward_dx choose for an M x N output on the current device
 * (every other product uses 256), so that a test can tell which kernel a
 * shape exercises.  Returns 0 for M or N below 1.  Enqueues nothing.
 */
int w8a8_probe_gemm_tile_n(int64_t M, int64_t N);

#ifdef __cplusplus
}
#endif

#endif /* W8A8_PROBE_H */
