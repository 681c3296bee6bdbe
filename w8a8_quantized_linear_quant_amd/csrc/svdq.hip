// svdq.hip -- SVDQuant-style linear: 8-bit product of the quantized residual
// plus a bf16 low-rank branch.
//
// OneTrainer PR #1034 "SVDQuant" applies SVDQuant to every quant type; the
// wiki's SVDQuant entry keeps the low-rank factors in bfloat16 at rank 16-32.
// W ~ L2 . L1 + R: the residual R is quantized tensor-wise (as any W8A8
// weight), the factors are not quantized.  Forward:
//   y = dequant(codes(X) . codes(R)) + (X . L1^T) . L2^T + bias.
//
// Launches: (1) the row-wise act-quant kernel (X -> codes, row scales);
// (2) the down-projection u = X . L1^T on the bf16 MFMA, written to the
// workspace as two bf16 halves (u = hi + lo keeps ~16 significant bits, so
// the up-projection does not round u to 8 bits); (3) the 8-bit product whose
// epilogue adds hi . L2^T + lo . L2^T with the bf16 MFMA before the bias.
// For K <= 4096 and r <= 32, (1) and (2) are one kernel reading X once.
#include "act_quant.hpp"

namespace w8a8 {
namespace {

constexpr int kRows = 16;  // rows of X per workgroup (one 16x16x32 MFMA row block)
constexpr int kWaves = 16;  // waves splitting the K steps (4 waves: 24.7 us at X [4096, 3072]; 16: 11.9 us)
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxRp = 64;

typedef __bf16 v8bf_t __attribute__((ext_vector_type(8)));

// u[m, j] = sum_k x[m, k] l1[j, k] for 16 rows; wave w takes the 32-wide k
// steps w, w + kWaves, ...; partial sums meet in LDS.  The product is
// bound by reading X once; many waves per row block keep enough loads in
// flight to stream it (one workgroup per 16 rows).
__global__ __launch_bounds__(kThreads) void svdq_down_kernel(const uint16_t *__restrict__ x, int M, int K,
                                                             const uint16_t *__restrict__ l1, int r, int rp,
                                                             uint16_t *__restrict__ uhi, uint16_t *__restrict__ ulo) {
    __shared__ float part[kWaves][kRows][kMaxRp + 1];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m0 = blockIdx.x * kRows;
    const int row = m0 + (lane & 15);
    const int kq = (lane >> 4) * 8;  // this lane's 8 k values within a step
    const int nsteps = (K + 31) / 32;
    const int jblocks = rp / 16;

    v4f acc[kMaxRp / 16];
#pragma unroll
    for (int b = 0; b < kMaxRp / 16; ++b) acc[b] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int s = wave; s < nsteps; s += kWaves) {
        const int k = s * 32 + kq;
        v8bf_t a;
        if (row < M && k + 8 <= K) {
            a = *reinterpret_cast<const v8bf_t *>(x + (size_t)row * K + k);
        } else {
            uint16_t z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            a = __builtin_bit_cast(v8bf_t, z);
        }
#pragma unroll
        for (int b = 0; b < kMaxRp / 16; ++b) {
            if (b >= jblocks) break;
            const int j = b * 16 + (lane & 15);
            v8bf_t bv;
            if (j < r && k + 8 <= K) {
                bv = *reinterpret_cast<const v8bf_t *>(l1 + (size_t)j * K + k);
            } else {
                uint16_t z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                bv = __builtin_bit_cast(v8bf_t, z);
            }
            acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bv, acc[b], 0, 0, 0);
        }
    }
    // C layout of the 16x16 MFMA: lane l, element i -> row 4(l/16) + i, col l%16.
#pragma unroll
    for (int b = 0; b < kMaxRp / 16; ++b) {
        if (b >= jblocks) break;
#pragma unroll
        for (int i = 0; i < 4; ++i) part[wave][4 * (lane >> 4) + i][b * 16 + (lane & 15)] = acc[b][i];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < kRows * rp; idx += kThreads) {
        const int rr = idx / rp, j = idx % rp;
        const int m = m0 + rr;
        if (m >= M) continue;
        float u = part[0][rr][j];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) u += part[w][rr][j];
        const uint32_t hi = f32_to_bf16_bits(u);
        const uint32_t lo = f32_to_bf16_bits(u - bf16_bits_to_f32(hi));
        uhi[(size_t)m * rp + j] = (uint16_t)hi;
        ulo[(size_t)m * rp + j] = (uint16_t)lo;
    }
}

// Fused launches (1) + (2) for K <= kFusedMaxK: one workgroup of kWaves waves
// per 16 rows reads X once.  Each lane keeps its 16-byte chunks of the rows
// (k steps wave, wave + kWaves, ...) in registers: their absmax meets in LDS
// for the row scales, they feed the down-projection MFMAs, and they are
// quantized with the act-quant kernel's arithmetic (same codes, same scales).
constexpr int kFusedSteps = 8;  // k steps per wave held in registers
constexpr int kFusedMaxK = kWaves * kFusedSteps * 32;

template <int QT, int JB>  // JB = rp / 16 column blocks of u
__global__ __launch_bounds__(kThreads) void svdq_quant_down_kernel(const uint16_t *__restrict__ x, int M, int K,
                                                                   const uint16_t *__restrict__ l1, int r, int rp,
                                                                   uint8_t *__restrict__ xq, float *__restrict__ sx,
                                                                   uint16_t *__restrict__ uhi,
                                                                   uint16_t *__restrict__ ulo) {
    __shared__ float part[kWaves][kRows][kMaxRp + 1];
    __shared__ uint32_t rmax[kWaves][kRows];
    constexpr float kQmax = QT == W8A8_INT8 ? 127.0f : 448.0f;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m0 = blockIdx.x * kRows;
    const int row = m0 + (lane & 15);
    const int kq = (lane >> 4) * 8;  // this lane's 8 k values within a step
    const int nsteps = (K + 31) / 32;

    // K % 16 == 0: a chunk is either whole or past K
    v4u d[kFusedSteps];
#pragma unroll
    for (int i = 0; i < kFusedSteps; ++i) {
        const int k = (wave + i * kWaves) * 32 + kq;
        d[i] = (row < M && k < K) ? *reinterpret_cast<const v4u *>(x + (size_t)row * K + k) : v4u{0u, 0u, 0u, 0u};
    }
    // l1 fragments of every step, all in flight at once: rows j >= r read
    // zero (buffer range); where this lane's k is past K its x chunk is zero,
    // so whatever l1 holds there adds nothing
    const __amdgpu_buffer_rsrc_t rl1 =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(l1), (short)0, r * K * 2, kBufferRsrcWord3);
    v4u lf[kFusedSteps][JB];
#pragma unroll
    for (int i = 0; i < kFusedSteps; ++i) {
        const int s = wave + i * kWaves;
#pragma unroll
        for (int b = 0; b < JB; ++b) {
            const int j = b * 16 + (lane & 15);
            lf[i][b] = s < nsteps ? __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(
                                                                 rl1, (j * K + s * 32 + kq) * 2, 0, 0))
                                  : v4u{0u, 0u, 0u, 0u};
        }
    }
    uint32_t m2 = 0;
#pragma unroll
    for (int i = 0; i < kFusedSteps; ++i) m2 = pk_max_u16(m2, chunk_absmax_bits(d[i]));
    uint32_t mb = max(m2 & 0xFFFFu, m2 >> 16);  // bf16 magnitude bits; the 4 lanes of a row differ in bits 4, 5
    mb = max(mb, (uint32_t)__shfl_xor((int)mb, 16, 64));
    mb = max(mb, (uint32_t)__shfl_xor((int)mb, 32, 64));
    if (lane < kRows) rmax[wave][lane] = mb;

    v4f acc[JB];
#pragma unroll
    for (int b = 0; b < JB; ++b) acc[b] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kFusedSteps; ++i) {
        if (wave + i * kWaves >= nsteps) break;
        const v8bf_t a = __builtin_bit_cast(v8bf_t, d[i]);
#pragma unroll
        for (int b = 0; b < JB; ++b)
            acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(v8bf_t, lf[i][b]), acc[b], 0, 0, 0);
    }
#pragma unroll
    for (int b = 0; b < JB; ++b) {
#pragma unroll
        for (int i = 0; i < 4; ++i) part[wave][4 * (lane >> 4) + i][b * 16 + (lane & 15)] = acc[b][i];
    }
    __syncthreads();

    // row scale and codes
    uint32_t rm = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) rm = max(rm, rmax[w][lane & 15]);
    const float sc = absmax_scale(bf16_bits_to_f32(rm), kQmax);
    const float rc = 1.0f / sc;
    if (wave == 0 && lane < kRows && row < M) sx[row] = sc;
#pragma unroll
    for (int i = 0; i < kFusedSteps; ++i) {
        const int k = (wave + i * kWaves) * 32 + kq;
        if (row < M && k < K) *reinterpret_cast<uint2 *>(xq + (size_t)row * K + k) = quantize8<QT>(d[i], sc, rc);
    }

    // u = sum of the waves' partials, as hi + lo bf16 halves
    for (int idx = threadIdx.x; idx < kRows * rp; idx += kThreads) {
        const int rr = idx / rp, j = idx % rp;
        const int m = m0 + rr;
        if (m >= M) continue;
        float u = part[0][rr][j];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) u += part[w][rr][j];
        const uint32_t hi = f32_to_bf16_bits(u);
        const uint32_t lo = f32_to_bf16_bits(u - bf16_bits_to_f32(hi));
        uhi[(size_t)m * rp + j] = (uint16_t)hi;
        ulo[(size_t)m * rp + j] = (uint16_t)lo;
    }
}

inline int64_t round_up16(int64_t r) { return (r + 15) / 16 * 16; }

}  // namespace
}  // namespace w8a8

extern "C" size_t svdq_workspace_bytes(int64_t M, int64_t r) {
    if (M < 0 || r < 1 || r > w8a8::kMaxRp) return 0;
    return (size_t)(2 * M * w8a8::round_up16(r) * sizeof(uint16_t));
}

extern "C" w8a8_status svdq_linear(w8a8_qtype qtype, const uint16_t *x, int64_t M, int64_t K, const void *rq,
                                   const float *r_scale, const uint16_t *l1, const uint16_t *l2, int64_t r,
                                   const uint16_t *bias, int64_t N, uint16_t *y, void *xq_out, float *x_scale_out,
                                   void *workspace, hipStream_t stream) {
    using namespace w8a8;
    if (!valid_qtype(qtype) || r < 1 || r > kMaxRp) return W8A8_ERR_INVALID_ARG;
    w8a8_status st = gemm_check(xq_out, rq, M, N, K, y);
    if (st != W8A8_OK) return st;
    st = act_quant_check(qtype, x, M, K, K, xq_out, K, x_scale_out);
    if (st != W8A8_OK) return st;
    if (M > 0 && N > 0 && (!r_scale || !l1 || !l2 || !workspace)) return W8A8_ERR_INVALID_ARG;
    if (!aligned16(r_scale) || !aligned16(l1) || !aligned16(l2) || !aligned16(bias) || !aligned16(workspace))
        return W8A8_ERR_ALIGN;
    if (M == 0) return W8A8_OK;
    const int rp = (int)round_up16(r);
    uint16_t *uhi = static_cast<uint16_t *>(workspace);
    uint16_t *ulo = uhi + (size_t)M * rp;
    const int grid = (int)((M + kRows - 1) / kRows);
    if (N > 0 && K <= kFusedMaxK && rp <= 32) {
        uint8_t *q = static_cast<uint8_t *>(xq_out);
#define W8A8_SVDQ_FUSED(QT, JB) \
    svdq_quant_down_kernel<QT, JB><<<grid, kThreads, 0, stream>>>(x, (int)M, (int)K, l1, (int)r, rp, q, x_scale_out, uhi, ulo)
        if (qtype == W8A8_INT8) {
            if (rp == 16) W8A8_SVDQ_FUSED(W8A8_INT8, 1);
            else W8A8_SVDQ_FUSED(W8A8_INT8, 2);
        } else {
            if (rp == 16) W8A8_SVDQ_FUSED(W8A8_FP8_E4M3, 1);
            else W8A8_SVDQ_FUSED(W8A8_FP8_E4M3, 2);
        }
#undef W8A8_SVDQ_FUSED
    } else {
        st = act_quant_launch(qtype, x, M, K, K, xq_out, K, x_scale_out, stream);
        if (st != W8A8_OK || N == 0) return st;
        svdq_down_kernel<<<grid, kThreads, 0, stream>>>(x, (int)M, (int)K, l1, (int)r, rp, uhi, ulo);
    }
    st = launch_status();
    if (st != W8A8_OK) return st;
    GemmArgs a = {};
    a.xq = static_cast<const uint8_t *>(xq_out);
    a.wq = static_cast<const uint8_t *>(rq);
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.sx = x_scale_out;
    a.sw = r_scale;
    a.bias = bias;
    a.out = y;
    a.uhi = uhi;
    a.ulo = ulo;
    a.l2 = l2;
    a.r = (int)r;
    a.rp = rp;
    // r of 16 or 32: the low-rank operands are staged in LDS (r == rp keeps
    // the staged l2 rows aligned); other ranks read them from global memory
    return gemm_launch(qtype, (r == 16 || r == 32) ? kEpiLowRank32 : kEpiLowRank, a, stream);
}
