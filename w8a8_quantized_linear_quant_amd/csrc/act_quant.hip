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
#include "internal.hpp"

namespace w8a8 {
namespace {

constexpr int kRowsPerBlock = 4;  // one wave per row, 4 waves per workgroup

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
    us2 x = __builtin_bit_cast(us2, a), y = __builtin_bit_cast(us2, b);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(x, y));
}

// Zero the bf16 elements of a 16-byte chunk at column index >= K.
__device__ __forceinline__ v4u mask_tail(v4u d, int first_col, int K) {
    if (first_col + 8 <= K) return d;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t keep = 0;
        if (first_col + 2 * w < K) keep |= 0x0000FFFFu;
        if (first_col + 2 * w + 1 < K) keep |= 0xFFFF0000u;
        d[w] &= keep;
    }
    return d;
}

// Eight codes (two u32 words) from eight bf16 values.
template <int QT>
__device__ __forceinline__ uint2 quantize8(v4u d, float s, float r) {
    uint32_t out[2];
    if constexpr (QT == W8A8_INT8) {
        // fl(x/s) + 1.5 * 2^23 rounds to an integer half-to-even in the add
        // (|q| <= 128 < 2^22); its two's-complement low byte is the code.
        const float magic = 12582912.0f;
        uint32_t b[8];
#pragma unroll
        // The clamp to [-128, 127] of the definition cannot bind here:
        // |x| <= absmax gives |x / s| <= 127 (1 + 2^-23), which rounds to at
        // most 127.  The sign of zero does not matter for an integer code.
        for (int w = 0; w < 4; ++w) {
            float lo = __uint_as_float(d[w] << 16), hi = __uint_as_float(d[w] & 0xFFFF0000u);
            b[2 * w] = __float_as_uint(quotient_nosign(lo, s, r) + magic);
            b[2 * w + 1] = __float_as_uint(quotient_nosign(hi, s, r) + magic);
        }
        // byte-gather: v_perm_b32 selects bytes of {src0, src1}; selector byte
        // 0..3 picks src1 bytes, 4..7 picks src0 bytes.
        uint32_t p01 = __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u);  // [b0.0, b1.0, 0, 0]
        uint32_t p23 = __builtin_amdgcn_perm(b[3], b[2], 0x04000c0cu);  // [0, 0, b2.0, b3.0]
        uint32_t p45 = __builtin_amdgcn_perm(b[5], b[4], 0x0c0c0400u);
        uint32_t p67 = __builtin_amdgcn_perm(b[7], b[6], 0x04000c0cu);
        out[0] = p01 | p23;
        out[1] = p45 | p67;
    } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            float v[4];
#pragma unroll
            for (int w = 0; w < 2; ++w) {
                uint32_t word = d[2 * h + w];
                v[2 * w] = __builtin_amdgcn_fmed3f(quotient(__uint_as_float(word << 16), s, r), -448.0f, 448.0f);
                v[2 * w + 1] =
                    __builtin_amdgcn_fmed3f(quotient(__uint_as_float(word & 0xFFFF0000u), s, r), -448.0f, 448.0f);
            }
            int pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
            pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], pk, true);
            out[h] = (uint32_t)pk;
        }
    }
    return make_uint2(out[0], out[1]);
}

__device__ __forceinline__ uint32_t chunk_absmax_bits(v4u d) {
    uint32_t m = pk_max_u16(d[0] & 0x7FFF7FFFu, d[1] & 0x7FFF7FFFu);
    m = pk_max_u16(m, pk_max_u16(d[2] & 0x7FFF7FFFu, d[3] & 0x7FFF7FFFu));
    return m;
}

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
