// act_quant.hpp -- device helpers of the row-wise activation quantizer,
// shared by the act-quant kernel and the SVDQuant kernel that fuses the
// quantization with the low-rank down-projection.  Scale and code rules are
// those of entrenar's Q8_0::quantize (absmax / QMAX, 1e-10 floor, divide,
// round, clamp) with round-half-to-even.
#pragma once

#include "internal.hpp"

namespace w8a8 {

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

}  // namespace w8a8
