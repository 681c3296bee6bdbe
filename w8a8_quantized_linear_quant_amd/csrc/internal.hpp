// internal.hpp -- entry points shared between the library's translation units
// (not part of the C ABI).
#pragma once

#include "common.hpp"

namespace w8a8 {

// Epilogue of the 8-bit product.
enum GemmEpilogue {
    kEpiI32 = 0,      // raw int32 accumulators
    kEpiBf16 = 1,     // bf16(acc * sx[m] * sw + bias[n])
    kEpiLowRank = 2,  // bf16(acc * sx[m] * sw + u[m,:] . l2[n,:] + bias[n])
    kEpiColScale = 3, // bf16(acc * sx[m] * sw[n] + bias[n]), one weight scale per output channel
    kEpiLowRank32 = 4, // as kEpiLowRank for r of 16 or 32, with u and l2 staged in LDS
};

struct GemmArgs {
    const uint8_t *xq;  // [M, K] codes (rows = tokens)
    const uint8_t *wq;  // [N, K] codes
    int M, N, K;
    const float *sx;       // [M]
    const float *sw;       // [1], or [N] for kEpiColScale
    const uint16_t *bias;  // [N] bf16 or null
    void *out;             // bf16 [M, N] or int32 [M, N]
    // low-rank branch: u split into bf16 hi/lo halves, [M, rp] each (zero
    // padded to rp = roundup(r, 16)); l2 bf16 [N, r].
    const uint16_t *uhi;
    const uint16_t *ulo;
    const uint16_t *l2;
    int r, rp;
};

// Compute units of the current device (queried once per device).
int device_cu_count();

w8a8_status gemm_check(const void *xq, const void *wq, int64_t M, int64_t N, int64_t K, const void *out);
w8a8_status gemm_launch(w8a8_qtype qtype, GemmEpilogue epi, const GemmArgs &a, hipStream_t stream);

w8a8_status act_quant_check(w8a8_qtype qtype, const uint16_t *x, int64_t M, int64_t K, int64_t ldx, const void *xq,
                            int64_t ldq, const float *x_scale);
w8a8_status act_quant_launch(w8a8_qtype qtype, const uint16_t *x, int64_t M, int64_t K, int64_t ldx, void *xq,
                             int64_t ldq, float *x_scale, hipStream_t stream);

}  // namespace w8a8
