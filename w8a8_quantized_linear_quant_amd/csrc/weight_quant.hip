// weight_quant.hip -- tensor-wise absmax weight quantization.
//
// OneTrainer wiki "Quantization", int W8A8 / float W8A8 ("Technical"):
// weights are quantized tensor-wise (one scale for the whole tensor) to int8
// or float8 e4m3.  The scale and code rules are the row-wise ones of
// act_quant.hip applied to the whole tensor as one group.
//
// Done once per frozen weight, so the design favours determinism over
// latency: kernel 1 writes one partial maximum per workgroup into the
// workspace; kernel 2 lets every workgroup re-reduce those partials (a few KB
// from L2, no atomics, no clearing) and quantize its share; kernel 3, only if
// requested, writes the transposed code copy [K, N] through 64x64 LDS tiles.
#include "act_quant.hpp"

namespace w8a8 {
namespace {

constexpr int kPartials = 1024;  // workgroups of the max pass = partial count
constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t *red) {
    v = wave_max_u32(v);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    uint32_t m = red[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) m = m > red[w] ? m : red[w];
    return m;
}

// Partial maxima of |w| (as bf16 magnitude bits) over 16-byte chunks.
__global__ __launch_bounds__(kThreads) void weight_absmax_kernel(const uint16_t *__restrict__ w, int64_t nchunks,
                                                                 uint32_t *__restrict__ partial) {
    __shared__ uint32_t red[kThreads / 64];
    const v4u *p = reinterpret_cast<const v4u *>(w);
    uint32_t m2 = 0;
    for (int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x; c < nchunks; c += (int64_t)gridDim.x * kThreads) {
        v4u d = p[c];
        m2 = pk_max_u16(m2, pk_max_u16(d[0] & 0x7FFF7FFFu, d[1] & 0x7FFF7FFFu));
        m2 = pk_max_u16(m2, pk_max_u16(d[2] & 0x7FFF7FFFu, d[3] & 0x7FFF7FFFu));
    }
    uint32_t m = (m2 & 0xFFFFu) > (m2 >> 16) ? (m2 & 0xFFFFu) : (m2 >> 16);
    m = block_max_u32(m, red);
    if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

template <int QT>
__global__ __launch_bounds__(kThreads) void weight_quant_kernel(const uint16_t *__restrict__ w, int64_t nchunks,
                                                                const uint32_t *__restrict__ partial, int npartial,
                                                                uint8_t *__restrict__ wq, float *__restrict__ w_scale) {
    constexpr float kQmax = QT == W8A8_INT8 ? 127.0f : 448.0f;
    __shared__ uint32_t red[kThreads / 64];
    uint32_t m = 0;
    for (int i = threadIdx.x; i < npartial; i += kThreads) m = m > partial[i] ? m : partial[i];
    m = block_max_u32(m, red);
    const float s = absmax_scale(bf16_bits_to_f32(m), kQmax);
    if (blockIdx.x == 0 && threadIdx.x == 0) w_scale[0] = s;
    // The codes are the act-quant's (quantize8): its one-correction quotient
    // equals the IEEE quotient for every bf16 value and every scale derived
    // from a bf16 absmax, which this scale is.
    const float r = 1.0f / s;
    const v4u *p = reinterpret_cast<const v4u *>(w);
    uint2 *q = reinterpret_cast<uint2 *>(wq);
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    // four chunks per thread with their loads issued together
    for (; c + 3 * stride < nchunks; c += 4 * stride) {
        v4u d[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) d[j] = p[c + j * stride];
#pragma unroll
        for (int j = 0; j < 4; ++j) q[c + j * stride] = quantize8<QT>(d[j], s, r);
    }
    for (; c < nchunks; c += stride) q[c] = quantize8<QT>(p[c], s, r);
}

// wq [N, K] -> wq_t [K, N] bytes, 64x64 tiles through LDS.
__global__ __launch_bounds__(kThreads) void transpose_codes_kernel(const uint8_t *__restrict__ wq, int64_t N,
                                                                   int64_t K, uint8_t *__restrict__ wq_t) {
    __shared__ uint8_t tile[64][64 + 4];
    // one-dimensional grid over the 64x64 tiles, k fastest
    const int64_t kb = (K + 63) / 64;
    const int64_t n0 = ((int64_t)blockIdx.x / kb) * 64, k0 = ((int64_t)blockIdx.x % kb) * 64;
    // load: 64 rows (n) x 64 bytes (k); each thread moves 16 bytes
    {
        const int rn = threadIdx.x >> 2, ck = (threadIdx.x & 3) * 16;
        const int64_t n = n0 + rn, k = k0 + ck;
        uint8_t v[16];
        if (n < N && k + 16 <= K) {
            v4u d = *reinterpret_cast<const v4u *>(wq + n * K + k);
            __builtin_memcpy(v, &d, 16);
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] = (n < N && k + i < K) ? wq[n * K + k + i] : 0;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) tile[rn][ck + i] = v[i];
    }
    __syncthreads();
    {
        const int rk = threadIdx.x >> 2, cn = (threadIdx.x & 3) * 16;
        const int64_t k = k0 + rk, n = n0 + cn;
        uint8_t v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = tile[cn + i][rk];
        if (k < K) {
            if (n + 16 <= N) {
                v4u d;
                __builtin_memcpy(&d, v, 16);
                *reinterpret_cast<v4u *>(wq_t + k * N + n) = d;
            } else {
                for (int i = 0; i < 16 && n + i < N; ++i) wq_t[k * N + n + i] = v[i];
            }
        }
    }
}

}  // namespace
}  // namespace w8a8

extern "C" size_t w8a8_weight_workspace_bytes(int64_t N, int64_t K) {
    (void)N;
    (void)K;
    return (size_t)w8a8::kPartials * sizeof(uint32_t);
}

extern "C" w8a8_status w8a8_quant_weight_tensorwise(w8a8_qtype qtype, const uint16_t *w, int64_t N, int64_t K,
                                                    void *wq, void *wq_t, float *w_scale, void *workspace,
                                                    hipStream_t stream) {
    using namespace w8a8;
    if (!valid_qtype(qtype) || N < 0 || K < 0) return W8A8_ERR_INVALID_ARG;
    if (!w_scale || !workspace) return W8A8_ERR_INVALID_ARG;
    if (N * K > 0 && (!w || !wq)) return W8A8_ERR_INVALID_ARG;
    if (K % 8 != 0 || (wq_t && N % 16 != 0)) return W8A8_ERR_SHAPE;
    if (N > ((int64_t)1 << 31) || K > ((int64_t)1 << 31) || N * K > ((int64_t)1 << 40)) return W8A8_ERR_SHAPE;
    if (!aligned16(w) || !aligned16(wq) || !aligned16(wq_t) || !aligned16(w_scale) || !aligned16(workspace))
        return W8A8_ERR_ALIGN;
    const int64_t nchunks = N * K / 8;
    uint32_t *partial = static_cast<uint32_t *>(workspace);
    const int64_t want = (nchunks + kThreads - 1) / kThreads;
    const int grid = (int)(want < 1 ? 1 : (want < kPartials ? want : kPartials));
    weight_absmax_kernel<<<grid, kThreads, 0, stream>>>(w, nchunks, partial);
    if (qtype == W8A8_INT8)
        weight_quant_kernel<W8A8_INT8><<<grid, kThreads, 0, stream>>>(w, nchunks, partial, grid,
                                                                      static_cast<uint8_t *>(wq), w_scale);
    else
        weight_quant_kernel<W8A8_FP8_E4M3><<<grid, kThreads, 0, stream>>>(w, nchunks, partial, grid,
                                                                          static_cast<uint8_t *>(wq), w_scale);
    if (wq_t && nchunks > 0) {
        const int64_t tiles = ((K + 63) / 64) * ((N + 63) / 64);  // <= 2^28 by the limits above
        transpose_codes_kernel<<<(unsigned)tiles, kThreads, 0, stream>>>(static_cast<const uint8_t *>(wq), N, K,
                                                           static_cast<uint8_t *>(wq_t));
    }
    return launch_status();
}
