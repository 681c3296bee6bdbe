// probe.hip -- measured ceiling of the int8 matrix cores, for reporting the
// GEMM's rate against what the chip sustains on the workload's data as well
// as against the spec figure (the spec assumes 2.4 GHz; under a sustained
// 8-bit MFMA load the clock settles lower, by an amount that depends on the
// operand values).
//
// One workgroup of 4 waves per CU (one wave per SIMD, as the GEMM).  Every
// wave takes 8 A and 8 B fragments of v_mfma_i32_16x16x64_i8 (the GEMM's int8
// MFMA) from the given operand bytes and loops over the 64 products of an
// 8x8 block of 16x16 accumulators -- the GEMM's k-step without its memory
// traffic.
//
// A second probe checks the hardware e4m3 conversion the quantizers use
// (clamp to +-448 with v_med3_f32, then v_cvt_pk_fp8_f32 with RNE) on every
// f32 bit pattern of a range, so that a test can compare each code with the
// oracle's encoding of the OCP E4M3FN format.
#include "../../include/w8a8_probe.h"
#include "internal.hpp"

namespace w8a8 {
namespace {

constexpr int kProbeBytes = 64 * 1024;  // operand bytes read by the probe (each of a, b)

__global__ __launch_bounds__(256) void probe_mfma_i8_kernel(const int8_t *__restrict__ a, const int8_t *__restrict__ b,
                                                            int64_t pairs, int32_t *__restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);  // global wave index
    v4i fa[8], fb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int off = ((gw * 8 + i) * 1024 + lane * 16) % kProbeBytes;
        fa[i] = *reinterpret_cast<const v4i *>(a + off);
        fb[i] = *reinterpret_cast<const v4i *>(b + off);
    }
    v4i acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = v4i{};
    for (int64_t it = 0; it < pairs; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    int32_t x = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) x ^= acc[i][j][e];
    sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = x;
}

// codes[i] = e4m3 code of the f32 whose bit pattern is first + i, by the
// quantizers' conversion sequence; 4 values per thread, grid-stride.
__global__ __launch_bounds__(256) void probe_cvt_e4m3_kernel(uint32_t first, int64_t n, uint8_t *__restrict__ codes) {
    const int64_t quads = (n + 3) / 4;
    for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < quads; q += (int64_t)gridDim.x * 256) {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v[i] = __builtin_amdgcn_fmed3f(__uint_as_float(first + (uint32_t)(4 * q + i)), -448.0f, 448.0f);
        int pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
        pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], pk, true);
        if (4 * q + 4 <= n) {
            *reinterpret_cast<uint32_t *>(codes + 4 * q) = (uint32_t)pk;
        } else {
            for (int i = 0; 4 * q + i < n; ++i) codes[4 * q + i] = (uint8_t)((uint32_t)pk >> (8 * i));
        }
    }
}

}  // namespace
}  // namespace w8a8

extern "C" w8a8_status w8a8_probe_cvt_e4m3(uint32_t first_bits, int64_t n, uint8_t *codes, hipStream_t stream) {
    using namespace w8a8;
    if (n < 0 || (n > 0 && !codes) || (uint64_t)first_bits + (uint64_t)n > (1ull << 32)) return W8A8_ERR_INVALID_ARG;
    if (!aligned16(codes)) return W8A8_ERR_ALIGN;
    if (n == 0) return W8A8_OK;
    const int64_t quads = (n + 3) / 4;
    const int64_t cap = (int64_t)device_cu_count() * 8;
    const int grid = (int)((quads + 255) / 256 < cap ? (quads + 255) / 256 : cap);
    probe_cvt_e4m3_kernel<<<grid, 256, 0, stream>>>(first_bits, n, codes);
    return launch_status();
}

extern "C" int64_t w8a8_probe_sink_count(void) { return (int64_t)w8a8::device_cu_count() * 256; }

extern "C" w8a8_status w8a8_probe_mfma_i8(const void *a, const void *b, int64_t pairs, int32_t *sink,
                                          hipStream_t stream) {
    using namespace w8a8;
    if (!a || !b || !sink || pairs < 0) return W8A8_ERR_INVALID_ARG;
    if (!aligned16(a) || !aligned16(b) || !aligned16(sink)) return W8A8_ERR_ALIGN;
    if (pairs == 0) return W8A8_OK;
    probe_mfma_i8_kernel<<<device_cu_count(), 256, 0, stream>>>(static_cast<const int8_t *>(a),
                                                               static_cast<const int8_t *>(b), pairs, sink);
    return launch_status();
}
