// probe.hip -- measured ceiling of the int8 matrix cores, for reporting the
// GEMM's rate against what the chip sustains on the workload's data as well
// as against the spec figure (the spec assumes 2.4 GHz; under a sustained
// 8-bit MFMA load the clock settles lower, by an amount that depends on the
// operand values).
//
// One workgroup of 4 waves per CU (one wave per SIMD, as the GEMM).  Every
// wave takes two sets of 4 A and 4 B fragments of v_mfma_i32_32x32x32_i8
// from the given operand bytes and loops over the 16 products of a 4x4 block
// of 32x32 accumulators, alternating the sets -- the GEMM's k-step without
// its memory traffic.
#include "../../include/w8a8_probe.h"
#include "internal.hpp"

namespace w8a8 {
namespace {

constexpr int kProbeBytes = 64 * 1024;  // operand bytes read by the probe (each of a, b)

__global__ __launch_bounds__(256) void probe_mfma_i8_kernel(const int8_t *__restrict__ a, const int8_t *__restrict__ b,
                                                            int64_t pairs, int32_t *__restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);  // global wave index
    v4i fa[2][4], fb[2][4];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int off = ((gw * 8 + s * 4 + i) * 1024 + lane * 16) % kProbeBytes;
            fa[s][i] = *reinterpret_cast<const v4i *>(a + off);
            fb[s][i] = *reinterpret_cast<const v4i *>(b + off);
        }
    v16i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v16i{};
    for (int64_t it = 0; it < pairs; ++it) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[s][i], fb[s][j], acc[i][j], 0, 0, 0);
    }
    int32_t x = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) x ^= acc[i][j][e];
    sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = x;
}

}  // namespace
}  // namespace w8a8

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
