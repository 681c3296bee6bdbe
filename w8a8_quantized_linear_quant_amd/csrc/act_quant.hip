// act_quant.hip -- row-wise (token-wise) absmax activation quantization.
//
// bitsandbytes #1401 "LLM.int8() Refactoring: Part 1" (Enhancements) fuses the
// row-scale calibration and the quantization into one kernel; the OneTrainer
// wiki "Quantization" (int W8A8 / float W8A8, "Technical") quantizes the
// activations token-wise.  Scale and code rules are those of entrenar's
// Q8_0::quantize (absmax / QMAX, 1e-10 floor, divide, round, clamp) with
// round-half-to-even.
//
// One wave per row, single pass: the row is loaded once into registers with
// lane-interleaved 16-byte loads (each load instruction covers 1 KB of the row
// contiguously), the absmax is taken on packed bf16 magnitude bits, reduced
// across the wave, and the codes are produced from the same registers.  Rows
// longer than the register budget take a two-pass variant (the second pass
// re-reads the row, which is then in L2).
#include "act_quant.hpp"

namespace w8a8 {
namespace {

constexpr int kRowsPerBlock = 4;  // one wave per row, 4 waves per workgroup

__device__ __forceinline__ void zero_pad(uint8_t *qrow, int K, int64_t ldq, int lane) {
    // Columns [roundup(K, 8), ldq) are zero; the chunk containing K was
    // written with zero codes for its masked tail.
    const int64_t start = ((int64_t)K + 7) / 8 * 8;
    for (int64_t c = start + (int64_t)lane * 8; c < ldq; c += 64 * 8)
        *reinterpret_cast<uint2 *>(qrow + c) = make_uint2(0u, 0u);
}

// A wave quantizes rows row0, row0 + stride, ... of X, two rows in flight:
// the loads of the next row are issued before the current row is reduced,
// quantized and stored, so reads, VALU work and writes overlap.
template <int QT, int CPL, bool FULL>
__global__ __launch_bounds__(256) void act_quant_rowwise_kernel(const uint16_t *__restrict__ x, int64_t M, int K,
                                                                int64_t ldx, uint8_t *__restrict__ xq, int64_t ldq,
                                                                float *__restrict__ scale) {
    constexpr float kQmax = QT == W8A8_INT8 ? 127.0f : 448.0f;
    const int lane = threadIdx.x & 63;
    const int64_t stride = (int64_t)gridDim.x * kRowsPerBlock;
    const int nchunks = (K + 7) >> 3;

    auto load = [&](v4u *d, int64_t row) {
        const v4u *xr = reinterpret_cast<const v4u *>(x + row * ldx);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int chunk = c * 64 + lane;
            if constexpr (FULL)  // K == 512 CPL: every lane owns CPL whole chunks
                d[c] = __builtin_nontemporal_load(xr + chunk);
            else
                d[c] = chunk < nchunks ? mask_tail(__builtin_nontemporal_load(xr + chunk), chunk * 8, K)
                                       : v4u{0u, 0u, 0u, 0u};
        }
    };
    auto process = [&](const v4u *d, int64_t row) {
        uint32_t m2 = 0;
#pragma unroll
        for (int c = 0; c < CPL; ++c) m2 = pk_max_u16(m2, chunk_absmax_bits(d[c]));
        const uint32_t mbits = wave_max_u32(max(m2 & 0xFFFFu, m2 >> 16));
        const float s = absmax_scale(bf16_bits_to_f32(mbits), kQmax);
        const float r = 1.0f / s;
        if (lane == 0) scale[row] = s;
        uint8_t *qrow = xq + row * ldq;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int chunk = c * 64 + lane;
            if (FULL || chunk < nchunks) *reinterpret_cast<uint2 *>(qrow + chunk * 8) = quantize8<QT>(d[c], s, r);
        }
        if (ldq > K) zero_pad(qrow, K, ldq, lane);
    };

    int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= M) return;
    v4u a[CPL], b[CPL];
    load(a, row);
    while (true) {
        const int64_t r1 = row + stride;
        if (r1 < M) load(b, r1);
        process(a, row);
        if (r1 >= M) break;
        const int64_t r2 = r1 + stride;
        if (r2 < M) load(a, r2);
        process(b, r1);
        if (r2 >= M) break;
        row = r2;
    }
}

// Rows too long for registers: absmax pass, then a quantize pass re-reading x.
template <int QT>
__global__ __launch_bounds__(256) void act_quant_rowwise_2pass_kernel(const uint16_t *__restrict__ x, int64_t M,
                                                                      int K, int64_t ldx, uint8_t *__restrict__ xq,
                                                                      int64_t ldq, float *__restrict__ scale) {
    constexpr float kQmax = QT == W8A8_INT8 ? 127.0f : 448.0f;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= M) return;
    const v4u *xr = reinterpret_cast<const v4u *>(x + row * ldx);
    const int nchunks = (K + 7) >> 3;
    uint32_t m2 = 0;
    for (int chunk = lane; chunk < nchunks; chunk += 64)
        m2 = pk_max_u16(m2, chunk_absmax_bits(mask_tail(xr[chunk], chunk * 8, K)));
    uint32_t mbits = (m2 & 0xFFFFu) > (m2 >> 16) ? (m2 & 0xFFFFu) : (m2 >> 16);
    mbits = wave_max_u32(mbits);
    const float s = absmax_scale(bf16_bits_to_f32(mbits), kQmax);
    const float r = 1.0f / s;
    if (lane == 0) scale[row] = s;
    uint8_t *qrow = xq + row * ldq;
    for (int chunk = lane; chunk < nchunks; chunk += 64)
        *reinterpret_cast<uint2 *>(qrow + chunk * 8) = quantize8<QT>(mask_tail(xr[chunk], chunk * 8, K), s, r);
    if (ldq > K) zero_pad(qrow, K, ldq, lane);
}

template <int QT>
void launch_act_quant(const uint16_t *x, int64_t M, int K, int64_t ldx, uint8_t *xq, int64_t ldq, float *scale,
                      hipStream_t stream) {
    // Single-pass kernel: up to four workgroups per CU, each wave walking
    // rows with a stride of the whole grid (two rows in flight per wave).
    const int64_t blocks = (M + kRowsPerBlock - 1) / kRowsPerBlock;
#ifndef W8A8_ACTQ_WG_PER_CU
#define W8A8_ACTQ_WG_PER_CU 4  // workgroups (4 rows each) per CU: one row per wave at M = 16 x CUs
#endif
    const int64_t cap = W8A8_ACTQ_WG_PER_CU * (int64_t)device_cu_count();
    const dim3 grid((unsigned)(blocks < cap ? blocks : cap)), block(64 * kRowsPerBlock);
    const dim3 grid2((unsigned)blocks);
    const int cpl = (((K + 7) / 8) + 63) / 64;  // 16-byte chunks per lane
#define W8A8_ACTQ_CASE(N)                                                                             \
    if (cpl <= N) {                                                                                   \
        if (K == 512 * N)                                                                             \
            act_quant_rowwise_kernel<QT, N, true><<<grid, block, 0, stream>>>(x, M, K, ldx, xq, ldq, scale); \
        else                                                                                          \
            act_quant_rowwise_kernel<QT, N, false><<<grid, block, 0, stream>>>(x, M, K, ldx, xq, ldq, scale); \
        return;                                                                                       \
    }
    W8A8_ACTQ_CASE(1)
    W8A8_ACTQ_CASE(2)
    W8A8_ACTQ_CASE(4)
    W8A8_ACTQ_CASE(6)
    W8A8_ACTQ_CASE(8)
    W8A8_ACTQ_CASE(12)
    W8A8_ACTQ_CASE(16)
    W8A8_ACTQ_CASE(24)
    W8A8_ACTQ_CASE(32)
#undef W8A8_ACTQ_CASE
    act_quant_rowwise_2pass_kernel<QT><<<grid2, block, 0, stream>>>(x, M, K, ldx, xq, ldq, scale);
}

}  // namespace

// Shared with the SVDQuant path (same validation, same kernels).
w8a8_status act_quant_launch(w8a8_qtype qtype, const uint16_t *x, int64_t M, int64_t K, int64_t ldx, void *xq,
                             int64_t ldq, float *x_scale, hipStream_t stream) {
    if (M == 0) return W8A8_OK;
    if (qtype == W8A8_INT8)
        launch_act_quant<W8A8_INT8>(x, M, (int)K, ldx, static_cast<uint8_t *>(xq), ldq, x_scale, stream);
    else
        launch_act_quant<W8A8_FP8_E4M3>(x, M, (int)K, ldx, static_cast<uint8_t *>(xq), ldq, x_scale, stream);
    return launch_status();
}

w8a8_status act_quant_check(w8a8_qtype qtype, const uint16_t *x, int64_t M, int64_t K, int64_t ldx, const void *xq,
                            int64_t ldq, const float *x_scale) {
    if (!valid_qtype(qtype) || M < 0 || K < 0) return W8A8_ERR_INVALID_ARG;
    if (M > 0 && (!x || !xq || !x_scale)) return W8A8_ERR_INVALID_ARG;
    if (ldx < K || ldq < K || ldx % 8 != 0 || ldq % 16 != 0 || K > (int64_t)1 << 30) return W8A8_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(xq) || !aligned16(x_scale)) return W8A8_ERR_ALIGN;
    return W8A8_OK;
}

}  // namespace w8a8

extern "C" w8a8_status w8a8_quant_act_rowwise(w8a8_qtype qtype, const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                                              void *xq, int64_t ldq, float *x_scale, hipStream_t stream) {
    w8a8_status st = w8a8::act_quant_check(qtype, x, M, K, ldx, xq, ldq, x_scale);
    if (st != W8A8_OK) return st;
    return w8a8::act_quant_launch(qtype, x, M, K, ldx, xq, ldq, x_scale, stream);
}
