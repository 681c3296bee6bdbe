// q8_0.hip -- GGUF Q8_0 block quantize / dequantize.
//
// entrenar 0.7.8 src/quant/gguf_quant/q8_0.rs: struct Q8_0 (32 values per
// block, 34 bytes: 2-byte f16 scale + 32 int8 codes), Q8_0::quantize (block
// absmax, scale = absmax / 127 floored at 1e-10, value / scale rounded and
// clamped to [-128, 127], zero padding of the partial last block; the f32
// scale becomes f16 when the blocks are written) and Q8_0::dequantize (code * scale,
// here with the stored f16 scale).
//
// Both kernels stream: 8 lanes own one 32-value block (4 values = 16 bytes of
// f32 each), so a wave covers 8 blocks = 1 KB of f32 with one coalesced load
// and 272 bytes (= 17 x 16) of blocks.  272-byte groups stay 16-byte aligned,
// so the packed blocks go through LDS and out with aligned 16-byte stores.
#include "common.hpp"

namespace w8a8 {
namespace {

constexpr int kBlock = 32;
constexpr int kBlockBytes = 34;
constexpr int kThreads = 256;
constexpr int kBlocksPerWave = 8;
constexpr int kGroupBytes = kBlocksPerWave * kBlockBytes;  // 272
constexpr int kUnroll = 4;                                 // wave groups per iteration

template <int CTRL>
__device__ __forceinline__ float dpp_max(float v) {
    return fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false)));
}

__device__ __forceinline__ float group8_max(float v) {
    // max over the 8 lanes of one block (lanes 8b .. 8b+7), in DPP: lane ^ 1,
    // lane ^ 2 (quad permutes), then the mirror within 8 lanes, which pairs
    // every lane with one of the other quad
    v = dpp_max<0xB1>(v);   // quad_perm [1,0,3,2]
    v = dpp_max<0x4E>(v);   // quad_perm [2,3,0,1]
    return dpp_max<0x141>(v);  // row_half_mirror
}

__global__ __launch_bounds__(kThreads) void q8_0_quantize_kernel(const float *__restrict__ x, int64_t n,
                                                                 uint8_t *__restrict__ out, int64_t ngroups) {
    __shared__ __attribute__((aligned(16))) uint8_t stage[kThreads / 64][kUnroll][kGroupBytes];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t nbytes = ((n + kBlock - 1) / kBlock) * kBlockBytes;
    const int64_t waves_total = (int64_t)gridDim.x * (kThreads / 64);
    for (int64_t g0 = ((int64_t)blockIdx.x * (kThreads / 64) + wave) * kUnroll; g0 < ngroups;
         g0 += waves_total * kUnroll) {
        v4f v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t e = ((g0 + u) * kBlocksPerWave * kBlock) + (int64_t)lane * 4;  // first element
            if (e + 4 <= n) {
                v[u] = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(x + e));
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) v[u][i] = (e + i < n) ? x[e + i] : 0.0f;
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            float a = fmaxf(fmaxf(fabsf(v[u][0]), fabsf(v[u][1])), fmaxf(fabsf(v[u][2]), fabsf(v[u][3])));
            a = group8_max(a);
            const float s = absmax_scale(a, 127.0f);
            const float r = 1.0f / s;
            uint32_t word = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // value / scale (the one-correction quotient equals the IEEE
                // quotient down to 2^-20, below which both round to code 0),
                // rounded half to even by the add of 1.5 * 2^23; |q| <= 127
                // by the scale rule, so the page's clamp never acts
                word |= (__float_as_uint(quotient_nosign(v[u][i], s, r) + 12582912.0f) & 0xFFu) << (8 * i);
            }
            uint8_t *blk = &stage[wave][u][(lane >> 3) * kBlockBytes];
            const int j = lane & 7;
            // 34-byte blocks are 2-byte aligned: write halves
            *reinterpret_cast<uint16_t *>(blk + 2 + 4 * j) = (uint16_t)(word & 0xFFFFu);
            *reinterpret_cast<uint16_t *>(blk + 4 + 4 * j) = (uint16_t)(word >> 16);
            if (j == 0) {
                const _Float16 d = (_Float16)s;
                *reinterpret_cast<uint16_t *>(blk) = __builtin_bit_cast(uint16_t, d);
            }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
        __builtin_amdgcn_wave_barrier();
        // 4 groups x 272 bytes = 1088 bytes = 68 chunks of 16 bytes
        const int64_t base = g0 * kGroupBytes;
        const uint8_t *src = &stage[wave][0][0];
        for (int c = lane; c < kUnroll * kGroupBytes / 16; c += 64) {
            const int64_t off = base + (int64_t)c * 16;
            if (off + 16 <= nbytes) {
                *reinterpret_cast<v4u *>(out + off) = *reinterpret_cast<const v4u *>(src + c * 16);
            } else if (off < nbytes) {
                for (int i = 0; i < 16 && off + i < nbytes; i += 2)
                    *reinterpret_cast<uint16_t *>(out + off + i) = *reinterpret_cast<const uint16_t *>(src + c * 16 + i);
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
}

__global__ __launch_bounds__(kThreads) void q8_0_dequantize_kernel(const uint8_t *__restrict__ blocks, int64_t n,
                                                                   float *__restrict__ y) {
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;  // owns elements 4t .. 4t+3
    const int64_t e = t * 4;
    if (e >= n) return;
    const uint8_t *blk = blocks + (e / kBlock) * kBlockBytes;
    const int j = (int)((e % kBlock) / 4);
    const uint16_t dbits = *reinterpret_cast<const uint16_t *>(blk);
    const uint32_t lo = *reinterpret_cast<const uint16_t *>(blk + 2 + 4 * j);
    const uint32_t hi = *reinterpret_cast<const uint16_t *>(blk + 4 + 4 * j);
    const uint32_t word = lo | (hi << 16);
    const float d = (float)__builtin_bit_cast(_Float16, dbits);
    v4f r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (float)(int8_t)(word >> (8 * i)) * d;
    if (e + 4 <= n) {
        __builtin_nontemporal_store(r, reinterpret_cast<v4f *>(y + e));
    } else {
        for (int i = 0; i < 4 && e + i < n; ++i) y[e + i] = r[i];
    }
}

}  // namespace
}  // namespace w8a8

extern "C" size_t q8_0_nbytes(int64_t n) {
    if (n < 0) return 0;
    return (size_t)((n + w8a8::kBlock - 1) / w8a8::kBlock) * w8a8::kBlockBytes;
}

extern "C" w8a8_status q8_0_quantize(const float *x, int64_t n, void *blocks, hipStream_t stream) {
    using namespace w8a8;
    if (n < 0) return W8A8_ERR_INVALID_ARG;
    if (n == 0) return W8A8_OK;
    if (!x || !blocks) return W8A8_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(blocks)) return W8A8_ERR_ALIGN;
    const int64_t nblocks = (n + kBlock - 1) / kBlock;
    const int64_t ngroups = (nblocks + kBlocksPerWave - 1) / kBlocksPerWave;
    const int64_t waves = (ngroups + kUnroll - 1) / kUnroll;
    int64_t grid = (waves + (kThreads / 64) - 1) / (kThreads / 64);
    if (grid > 65536) grid = 65536;
    q8_0_quantize_kernel<<<(unsigned)grid, kThreads, 0, stream>>>(x, n, static_cast<uint8_t *>(blocks), ngroups);
    return launch_status();
}

extern "C" w8a8_status q8_0_dequantize(const void *blocks, int64_t n, float *y, hipStream_t stream) {
    using namespace w8a8;
    if (n < 0) return W8A8_ERR_INVALID_ARG;
    if (n == 0) return W8A8_OK;
    if (!blocks || !y) return W8A8_ERR_INVALID_ARG;
    if (!aligned16(blocks) || !aligned16(y)) return W8A8_ERR_ALIGN;
    const int64_t threads = (n + 3) / 4;
    const int64_t grid = (threads + kThreads - 1) / kThreads;
    if (grid > 0x7FFFFFFF) return W8A8_ERR_SHAPE;
    q8_0_dequantize_kernel<<<(unsigned)grid, kThreads, 0, stream>>>(static_cast<const uint8_t *>(blocks), n, y);
    return launch_status();
}
