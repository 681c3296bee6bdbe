// hadamard.hip -- Hadamard rotation before the row-wise quantization.
//
// diffusers "SDNQ" (overview) lists Hadamard rotation among the quantizer's
// options; the pages give no more.  The rotation used here is the standard
// one: the input dimension K is cut into blocks of b = min(1024, largest power
// of two dividing K) and every block is multiplied by the normalized Sylvester
// Walsh-Hadamard matrix H_b / sqrt(b), which is orthogonal and symmetric, so
// rotating the activations (every row of X) and the weight (every row of W)
// leaves X W^T unchanged while spreading outlier channels over the block.
// It is evaluated as the fast transform in f32 -- stages h = 1, 2, ..., b/2,
// each replacing (x[i], x[i + h]) (bit h of i clear) by (x[i] + x[i + h],
// x[i] - x[i + h]) -- then scaled by c = f32(1 / sqrt(b)).  Every value goes
// through the same operations in the same order whatever thread computes it,
// so the result is reproducible bit for bit.
//
// Activations: one fused kernel per row rotates and quantizes (the shared
// absmax rule on the f32 rotated values).  For b = 1024 (K % 1024 == 0) a wave
// keeps the whole row in registers: each lane loads 16 consecutive values of
// each block (stages h = 1..8 in registers), one LDS transpose regroups the
// block so that element bits 4-7 are in registers (h = 16..128) and bits 8-9
// are lane bits 4-5 (h = 256, 512: a row swap between register pairs,
// v_permlane16/32_swap, makes each of these butterflies lane-local), then the
// codes go back through LDS to leave as one 16-byte store per lane and block.
// Other block sizes use a per-wave LDS transform (two passes over the row).
// Weights: the same transform, rounded to bf16 (one-time).
#include "internal.hpp"

namespace w8a8 {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / 64;
constexpr int kMaxBlock = 1024;

inline int hadamard_block(int64_t K) {
    int b = 1;
    while (K % (2 * b) == 0 && 2 * b <= kMaxBlock) b *= 2;
    return b;
}

// Codes of 4 f32 values (one u32 word, element order) with the shared rule;
// r = f32(1 / s).  The quotient with one correction equals the IEEE quotient
// whenever its magnitude is at least 2^-20 (below that both give code 0; the
// sign of zero is restored for e4m3).
template <int QT>
__device__ __forceinline__ uint32_t codes4(const float *v, float s, float r) {
    if constexpr (QT == W8A8_INT8) {
        const float magic = 12582912.0f;  // 1.5 * 2^23: the add rounds half to even
        uint32_t b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) b[i] = __float_as_uint(quotient_nosign(v[i], s, r) + magic);
        const uint32_t lo = __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u);
        const uint32_t hi = __builtin_amdgcn_perm(b[3], b[2], 0x04000c0cu);
        return lo | hi;
    } else {
        float q[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = __builtin_amdgcn_fmed3f(quotient(v[i], s, r), -448.0f, 448.0f);
        int pk = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
        pk = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], pk, true);
        return (uint32_t)pk;
    }
}

__device__ __forceinline__ void zero_pad_row(uint8_t *qrow, int64_t K, int64_t ldq, int lane) {
    for (int64_t c = K + (int64_t)lane * 8; c < ldq; c += 64 * 8) *reinterpret_cast<uint2 *>(qrow + c) = make_uint2(0u, 0u);
}

// ---------------------------------------------------------------- b = 1024
// LDS position of element e of a block: 16 dwords of padding after every 256
// elements, so the transposed reads of the 4 element groups land in
// different banks.
__device__ __forceinline__ int pad_pos(int e) { return e + 16 * (e >> 8); }
constexpr int kPadBlockFloats = 1024 + 16 * 4;

// Butterflies of a stage whose element bit is lane bit 4 (W = 16) or 5
// (W = 32), on the register pair (x, y): v_permlane{16,32}_swap exchanges the
// W-lane rows of x that have that lane bit set with the rows of y that have it
// clear.  Afterwards every lane holds in (x, y) two values whose elements
// differ in the stage's bit alone (the one with the bit clear in x), from x's
// elements where the lane bit is clear and from y's where it is set; the
// butterfly is then the same in every lane: x <- x + y, y <- x - y.
template <int W>
__device__ __forceinline__ void swap_butterfly(float &x, float &y) {
    const auto p = W == 16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false)
                           : __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    const float a = __uint_as_float(p[0]), d = __uint_as_float(p[1]);
    x = a + d;
    y = a - d;
}

template <int QT, int NB>  // NB blocks of 1024 per row
__global__ __launch_bounds__(kThreads) void hadamard_act_quant_1024_kernel(const uint16_t *__restrict__ x, int64_t M,
                                                                           int64_t ldx, uint8_t *__restrict__ xq,
                                                                           int64_t ldq, float *__restrict__ scale) {
    __shared__ __attribute__((aligned(16))) float lds[kRowsPerBlock][kPadBlockFloats];
    constexpr float kQmax = QT == W8A8_INT8 ? 127.0f : 448.0f;
    constexpr int K = NB * 1024;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    float *sb = lds[wave];
    // layout B: lane l holds e = (l & 15) | (t << 4) | ((l >> 4) << 8), t = 0..15
    const int lo4 = lane & 15, hi2 = lane >> 4;
    // Final layout, after the swaps of stages h = 256 and 512: lane l, value i
    // is element ((l & 31) | ((i >> 2) << 5) | ((l >> 5) << 7) |
    // (((i >> 1) & 1) << 8) | ((i & 1) << 9)); byte offset of i = 0:
    const int fin = (lane & 31) | ((lane >> 5) << 7);
    const float c = 1.0f / 32.0f;  // 1 / sqrt(1024), exact
    const int64_t stride = (int64_t)gridDim.x * kRowsPerBlock;

    for (int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + wave; row < M; row += stride) {
        const uint16_t *xr = x + row * ldx;
        float vb[NB][16];  // layout B values of every block, before the scale c
        float amax = 0.0f;
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
            // layout A: lane l holds e = 16 l + t
            const v4u *src = reinterpret_cast<const v4u *>(xr + blk * 1024 + 16 * lane);
            const v4u d0 = __builtin_nontemporal_load(src), d1 = __builtin_nontemporal_load(src + 1);
            float v[16];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                v[2 * w] = __uint_as_float(d0[w] << 16);
                v[2 * w + 1] = __uint_as_float(d0[w] & 0xFFFF0000u);
                v[8 + 2 * w] = __uint_as_float(d1[w] << 16);
                v[8 + 2 * w + 1] = __uint_as_float(d1[w] & 0xFFFF0000u);
            }
            // stages h = 1, 2, 4, 8 (t bits 0..3)
#pragma unroll
            for (int h = 1; h < 16; h *= 2)
#pragma unroll
                for (int t = 0; t < 16; ++t)
                    if ((t & h) == 0) {
                        const float a = v[t], dd = v[t + h];
                        v[t] = a + dd;
                        v[t + h] = a - dd;
                    }
            // transpose through LDS: write layout A (64 contiguous bytes per lane)
            float *wp = sb + pad_pos(16 * lane);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<v4f *>(wp + 4 * q) = v4f{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
            float u[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) u[t] = sb[pad_pos(lo4 | (t << 4) | (hi2 << 8))];
            // stages h = 16, 32, 64, 128 (t' bits 0..3)
#pragma unroll
            for (int h = 1; h < 16; h *= 2)
#pragma unroll
                for (int t = 0; t < 16; ++t)
                    if ((t & h) == 0) {
                        const float a = u[t], dd = u[t + h];
                        u[t] = a + dd;
                        u[t + h] = a - dd;
                    }
            // stage h = 256 (lane bit 4) on the pairs (2j, 2j + 1): then lane
            // l, value 2j + s holds element (l & 15) | ((2j + l4) << 4) |
            // (s << 8) | (l5 << 9), with l4, l5 lane bits 4 and 5
#pragma unroll
            for (int j = 0; j < 8; ++j) swap_butterfly<16>(u[2 * j], u[2 * j + 1]);
            // stage h = 512 (lane bit 5) on the pairs (k, k + 8), into the
            // final layout: value 2k + s2 from pair k, s2 = element bit 9
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                swap_butterfly<32>(u[k], u[k + 8]);
                vb[blk][2 * k] = u[k];
                vb[blk][2 * k + 1] = u[k + 8];
            }
#pragma unroll
            for (int t = 0; t < 16; ++t) amax = fmaxf(amax, fabsf(vb[blk][t]));
        }
        // The scale c = 2^-5 is exact, so it moves from the values to the
        // divisor: scale from f32(amax c), codes from v / (32 s) with
        // reciprocal f32(1 / s) / 32 -- the same numbers as (v c) / s and its
        // one-correction quotient, scaled by a power of two.
        const float s = absmax_scale(__uint_as_float(wave_max_u32(__float_as_uint(amax))) * c, kQmax);
        const float r = 1.0f / s;
        if (lane == 0) scale[row] = s;
        const float s32 = s * 32.0f, r32 = r * c;
        uint8_t *qrow = xq + row * ldq;
        uint8_t *cb = reinterpret_cast<uint8_t *>(sb);  // 1 KB of codes per block
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
            // codes in the final layout -> bytes at their element positions
#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4) {
                if constexpr (QT == W8A8_INT8) {
                    // the code is the low byte of the magic-add result
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        cb[fin | (t4 << 5) | (((i >> 1) & 1) << 8) | ((i & 1) << 9)] =
                            (uint8_t)__float_as_uint(quotient_nosign(vb[blk][4 * t4 + i], s32, r32) + 12582912.0f);
                } else {
                    const uint32_t w = codes4<QT>(&vb[blk][4 * t4], s32, r32);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        cb[fin | (t4 << 5) | (((i >> 1) & 1) << 8) | ((i & 1) << 9)] = (uint8_t)(w >> (8 * i));
                }
            }
            // layout A out: 16 contiguous codes per lane
            const v4u out = *reinterpret_cast<const v4u *>(cb + 16 * lane);
            *reinterpret_cast<v4u *>(qrow + blk * 1024 + 16 * lane) = out;
        }
        if (ldq > K) zero_pad_row(qrow, K, ldq, lane);
    }
}

// ---------------------------------------------------------------- any b
// The wave's LDS area holds one block (b <= 1024 f32); stages run on it with
// the lanes sharing the b / 2 butterflies of a stage.  Within one wave, LDS
// operations complete in program order, so a stage reads what the previous
// one wrote.
__device__ __forceinline__ void block_fwht_lds(float *sb, int b, int lane) {
    for (int h = 1; h < b; h *= 2) {
        for (int p = lane; p < b / 2; p += 64) {
            const int i = (p / h) * 2 * h + (p % h);
            const float a = sb[i], d = sb[i + h];
            sb[i] = a + d;
            sb[i + h] = a - d;
        }
    }
}

__device__ __forceinline__ void load_block_f32(float *sb, const uint16_t *xr, int b, int lane) {
    for (int i = lane; i < b; i += 64) sb[i] = __uint_as_float((uint32_t)xr[i] << 16);
}

// MODE 0: quantize rows (pass 1: absmax of the rotated row; pass 2: rotate
// again and write codes).  MODE 1: rotated rows rounded to bf16.
template <int QT, int MODE>
__global__ __launch_bounds__(kThreads) void hadamard_rows_generic_kernel(const uint16_t *__restrict__ x, int64_t M,
                                                                         int64_t K, int64_t ldx, int b, float c,
                                                                         uint8_t *__restrict__ xq, int64_t ldq,
                                                                         float *__restrict__ scale,
                                                                         uint16_t *__restrict__ out, int64_t ldo) {
    __shared__ float lds[kRowsPerBlock][kMaxBlock];
    constexpr float kQmax = QT == W8A8_INT8 ? 127.0f : 448.0f;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    float *sb = lds[wave];
    const int64_t stride = (int64_t)gridDim.x * kRowsPerBlock;
    for (int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + wave; row < M; row += stride) {
        const uint16_t *xr = x + row * ldx;
        if constexpr (MODE == 1) {
            for (int64_t k0 = 0; k0 < K; k0 += b) {
                load_block_f32(sb, xr + k0, b, lane);
                block_fwht_lds(sb, b, lane);
                for (int i = lane; i < b; i += 64) out[row * ldo + k0 + i] = (uint16_t)f32_to_bf16_bits(sb[i] * c);
            }
        } else {
            uint32_t amax_bits = 0;
            for (int64_t k0 = 0; k0 < K; k0 += b) {
                load_block_f32(sb, xr + k0, b, lane);
                block_fwht_lds(sb, b, lane);
                for (int i = lane; i < b; i += 64) amax_bits = max(amax_bits, __float_as_uint(sb[i] * c) & 0x7FFFFFFFu);
            }
            const float s = absmax_scale(__uint_as_float(wave_max_u32(amax_bits)), kQmax);
            const float r = 1.0f / s;
            if (lane == 0) scale[row] = s;
            uint8_t *qrow = xq + row * ldq;
            for (int64_t k0 = 0; k0 < K; k0 += b) {
                load_block_f32(sb, xr + k0, b, lane);
                block_fwht_lds(sb, b, lane);
                // 4 consecutive values per lane and step (b >= 16 and K % 16 == 0)
                for (int i = 4 * lane; i < b; i += 256) {
                    const float v[4] = {sb[i] * c, sb[i + 1] * c, sb[i + 2] * c, sb[i + 3] * c};
                    *reinterpret_cast<uint32_t *>(qrow + k0 + i) = codes4<QT>(v, s, r);
                }
            }
            if (ldq > K) zero_pad_row(qrow, K, ldq, lane);
        }
    }
}

int grid_for(int64_t M) {
    const int64_t blocks = (M + kRowsPerBlock - 1) / kRowsPerBlock;
    const int64_t cap = 4 * (int64_t)device_cu_count();
    return (int)(blocks < cap ? blocks : cap);
}

}  // namespace
}  // namespace w8a8

extern "C" w8a8_status w8a8_quant_act_rowwise_hadamard(w8a8_qtype qtype, const uint16_t *x, int64_t M, int64_t K,
                                                       int64_t ldx, void *xq, int64_t ldq, float *x_scale,
                                                       hipStream_t stream) {
    using namespace w8a8;
    w8a8_status st = act_quant_check(qtype, x, M, K, ldx, xq, ldq, x_scale);
    if (st != W8A8_OK) return st;
    if (K % 16 != 0 || K == 0) return W8A8_ERR_SHAPE;
    if (M == 0) return W8A8_OK;
    const int b = hadamard_block(K);
    const int grid = grid_for(M);
    uint8_t *q = static_cast<uint8_t *>(xq);
#define W8A8_HAD_FAST(NB)                                                                                    \
    if (b == 1024 && K == NB * 1024) {                                                                       \
        if (qtype == W8A8_INT8)                                                                              \
            hadamard_act_quant_1024_kernel<W8A8_INT8, NB><<<grid, kThreads, 0, stream>>>(x, M, ldx, q, ldq, x_scale); \
        else                                                                                                 \
            hadamard_act_quant_1024_kernel<W8A8_FP8_E4M3, NB><<<grid, kThreads, 0, stream>>>(x, M, ldx, q, ldq,    \
                                                                                            x_scale);        \
        return launch_status();                                                                              \
    }
    W8A8_HAD_FAST(1)
    W8A8_HAD_FAST(2)
    W8A8_HAD_FAST(3)
    W8A8_HAD_FAST(4)
#undef W8A8_HAD_FAST
    const float c = (float)(1.0 / sqrt((double)b));
    if (qtype == W8A8_INT8)
        hadamard_rows_generic_kernel<W8A8_INT8, 0><<<grid, kThreads, 0, stream>>>(x, M, K, ldx, b, c, q, ldq, x_scale,
                                                                                  nullptr, 0);
    else
        hadamard_rows_generic_kernel<W8A8_FP8_E4M3, 0><<<grid, kThreads, 0, stream>>>(x, M, K, ldx, b, c, q, ldq,
                                                                                      x_scale, nullptr, 0);
    return launch_status();
}

extern "C" w8a8_status w8a8_hadamard_rotate(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, uint16_t *out,
                                            int64_t ldo, hipStream_t stream) {
    using namespace w8a8;
    if (M < 0 || K < 0) return W8A8_ERR_INVALID_ARG;
    if (K % 16 != 0 || ldx < K || ldo < K || K > ((int64_t)1 << 30)) return W8A8_ERR_SHAPE;
    if (M == 0 || K == 0) return W8A8_OK;
    if (!x || !out) return W8A8_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(out)) return W8A8_ERR_ALIGN;
    const int b = hadamard_block(K);
    const float c = (float)(1.0 / sqrt((double)b));
    hadamard_rows_generic_kernel<W8A8_INT8, 1><<<grid_for(M), kThreads, 0, stream>>>(x, M, K, ldx, b, c, nullptr, 0,
                                                                                     nullptr, out, ldo);
    return launch_status();
}
