// common.hpp -- shared device helpers and host-side argument checks of the
// gfx950 W8A8 library.  Everything here is written for CDNA4 (wave64, MFMA,
// buffer loads straight into LDS); there is no other target.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/w8a8.h"

namespace w8a8 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Buffer-resource word 3 for gfx9-family targets (raw buffer, 32-bit records).
constexpr int kBufferRsrcWord3 = 0x00020000;
// A buffer offset at or beyond num_records reads as zero; this one always is.
constexpr int kOobOffset = 0x80000000;

// ---------------------------------------------------------------- host side
inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline w8a8_status launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? W8A8_OK : W8A8_ERR_HIP;
}

inline bool valid_qtype(w8a8_qtype q) { return q == W8A8_INT8 || q == W8A8_FP8_E4M3; }

// ---------------------------------------------------------------- device side
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
    return __uint_as_float(b16 << 16);
}

// f32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Two f32 -> packed bf16x2 (lo in bits 0..15), RNE; gfx950 lowers the
// conversion pair to v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    bf2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Wave-wide max of a non-negative integer (wave64): DPP row shifts reduce
// each 16-lane row into its lane 15, four lane reads combine the rows; the
// result is wave-uniform.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    // row_shr:n (dpp ctrl 0x110 + n); lanes shifted in from outside the row
    // read 0 (bound_ctrl), which is neutral for a max of non-negative values
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true));
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
    return max(max(r0, r1), max(r2, r3));
}

// Absmax scale rule of every quantizer: 1e-10 floor, else absmax / QMAX (IEEE
// f32 division, correctly rounded).
__device__ __forceinline__ float absmax_scale(float amax, float qmax) {
    return amax < 1e-10f ? 1e-10f : amax / qmax;
}

// f32(x / s) from r = f32(1 / s) with one Markstein correction:
//   q0 = x r,  e = x - q0 s (exact with an FMA),  q = q0 + e r,
// sign of zero taken from x; 3 VALU ops instead of the ~10 of a full
// division.  Wherever |x / s| >= 2^-20 it is bit-identical to the IEEE
// quotient: exhaustively for every bf16 x and every scale derived from a
// bf16 absmax (both QMAX, 2.1e9 pairs), and on 1e8 random f32 pairs
// (tests/quotient_check.c).  Below 2^-20 (x subnormal: the residual e
// underflows) its last bits may differ, but both quotients are below 2^-11
// with the sign of x, so the int8 (0) and e4m3 (+-0) codes are the same.
__device__ __forceinline__ float quotient_nosign(float x, float s, float r) {
    float q0 = x * r;
    float e = __builtin_fmaf(-q0, s, x);
    return __builtin_fmaf(e, r, q0);
}
__device__ __forceinline__ float quotient(float x, float s, float r) {
    return __builtin_copysignf(quotient_nosign(x, s, r), x);
}

}  // namespace w8a8
