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
#include <atomic>

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
// per 16 rows reads X once.  Wave w owns row m0 + w: it loads the row with
// lane-interleaved 16-byte loads (each instruction reads 1 KB of the row),
// takes the row absmax across the wave, writes the codes and the scale with
// the act-quant kernel's arithmetic (same codes, same scales; 8 contiguous
// code bytes per lane and chunk) and leaves the bf16 row in LDS.  The
// down-projection u = X . L1^T then reads its bf16 MFMA fragments from LDS:
// wave w takes the 32-wide k steps w, w + kWaves, ...; the l1 fragments of
// those steps are requested from global memory before the row.
constexpr int kFusedMaxK = 4096;
constexpr int kFusedCpl = kFusedMaxK / 8 / 64;          // 16-byte chunks per lane and row
constexpr int kFusedSteps = kFusedMaxK / 32 / kWaves;   // k steps per wave
constexpr int kXsChunks = kFusedMaxK / 8;               // 16-byte chunks per staged row
static_assert(kWaves == kRows, "one wave per row");
static_assert(kWaves * kRows * (kMaxRp + 1) * 4 <= kRows * kXsChunks * 16, "partials fit in the row area");

template <int QT, int JB>  // JB = rp / 16 column blocks of u
__global__ __launch_bounds__(kThreads) void svdq_quant_down_kernel(const uint16_t *__restrict__ x, int M, int K,
                                                                   const uint16_t *__restrict__ l1, int r, int rp,
                                                                   uint8_t *__restrict__ xq, float *__restrict__ sx,
                                                                   uint16_t *__restrict__ uhi,
                                                                   uint16_t *__restrict__ ulo) {
    // The block's bf16 rows: chunk c of row i in slot c ^ i, so that the
    // fragment reads of 16 rows at one chunk hit 16 distinct 16-byte bank
    // groups, while each 1 KB row write stays one permuted contiguous KB.
    // Once every wave's MFMAs are done, the same bytes hold the partial sums.
    __shared__ __attribute__((aligned(16))) v4u xs[kRows][kXsChunks];
    auto part = reinterpret_cast<float (*)[kRows][kMaxRp + 1]>(&xs[0][0]);
    constexpr float kQmax = QT == W8A8_INT8 ? 127.0f : 448.0f;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m0 = blockIdx.x * kRows;
    const int nchunks = K >> 3;  // K % 16 == 0: whole chunks
    const int nsteps = (K + 31) / 32;
    const int fi = lane & 15, fg = lane >> 4;  // fragment row and 8-value k group of this lane

    // l1 fragments of this wave's steps, all in flight at once: rows j >= r
    // read zero (buffer range); where a step's k is past K the staged row is
    // zero, so whatever l1 holds there adds nothing
    const __amdgpu_buffer_rsrc_t rl1 =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(l1), (short)0, r * K * 2, kBufferRsrcWord3);
    v4u lf[kFusedSteps][JB];
#pragma unroll
    for (int t = 0; t < kFusedSteps; ++t) {
        const int s = wave + t * kWaves;
#pragma unroll
        for (int b = 0; b < JB; ++b) {
            const int j = b * 16 + fi;
            lf[t][b] = s < nsteps ? __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(
                                                                 rl1, (j * K + s * 32 + fg * 8) * 2, 0, 0))
                                  : v4u{0u, 0u, 0u, 0u};
        }
    }

    // this wave's row: absmax, scale, codes; zeros past K and for rows past M
    const int m = m0 + wave;
    const v4u *xr = reinterpret_cast<const v4u *>(x + (size_t)(m < M ? m : 0) * K);
    v4u d[kFusedCpl];
#pragma unroll
    for (int c = 0; c < kFusedCpl; ++c) {
        const int chunk = c * 64 + lane;
        d[c] = (m < M && chunk < nchunks) ? __builtin_nontemporal_load(xr + chunk) : v4u{0u, 0u, 0u, 0u};
    }
    uint32_t m2 = 0;
#pragma unroll
    for (int c = 0; c < kFusedCpl; ++c) m2 = pk_max_u16(m2, chunk_absmax_bits(d[c]));
    const uint32_t mbits = wave_max_u32(max(m2 & 0xFFFFu, m2 >> 16));
    if (m < M) {
        const float sc = absmax_scale(bf16_bits_to_f32(mbits), kQmax);
        const float rc = 1.0f / sc;
        if (lane == 0) sx[m] = sc;
        uint8_t *qrow = xq + (size_t)m * K;
#pragma unroll
        for (int c = 0; c < kFusedCpl; ++c) {
            const int chunk = c * 64 + lane;
            if (chunk < nchunks) *reinterpret_cast<uint2 *>(qrow + chunk * 8) = quantize8<QT>(d[c], sc, rc);
        }
    }
#pragma unroll
    for (int c = 0; c < kFusedCpl; ++c) xs[wave][(c * 64 + lane) ^ wave] = d[c];
    __syncthreads();

    v4f acc[JB];
#pragma unroll
    for (int b = 0; b < JB; ++b) acc[b] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < kFusedSteps; ++t) {
        const int s = wave + t * kWaves;
        if (s >= nsteps) break;
        const v8bf_t a = __builtin_bit_cast(v8bf_t, xs[fi][(s * 4 + fg) ^ fi]);
#pragma unroll
        for (int b = 0; b < JB; ++b)
            acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(v8bf_t, lf[t][b]), acc[b], 0, 0, 0);
    }
    __syncthreads();  // every wave has read its fragments before the partials overwrite the rows
    // C layout of the 16x16 MFMA: lane l, element e -> row 4(l/16) + e, col l%16.
#pragma unroll
    for (int b = 0; b < JB; ++b) {
#pragma unroll
        for (int e = 0; e < 4; ++e) part[wave][4 * fg + e][b * 16 + fi] = acc[b][e];
    }
    __syncthreads();

    // u = sum of the waves' partials, as hi + lo bf16 halves
    for (int idx = threadIdx.x; idx < kRows * rp; idx += kThreads) {
        const int rr = idx / rp, j = idx % rp;
        const int mm = m0 + rr;
        if (mm >= M) continue;
        float u = part[0][rr][j];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) u += part[w][rr][j];
        const uint32_t hi = f32_to_bf16_bits(u);
        const uint32_t lo = f32_to_bf16_bits(u - bf16_bits_to_f32(hi));
        uhi[(size_t)mm * rp + j] = (uint16_t)hi;
        ulo[(size_t)mm * rp + j] = (uint16_t)lo;
    }
}

inline int64_t round_up16(int64_t r) { return (r + 15) / 16 * 16; }

}  // namespace
}  // namespace w8a8

extern "C" size_t svdq_workspace_bytes(int64_t M, int64_t r) {
    if (M < 0 || r < 1 || r > w8a8::kMaxRp) return 0;
    return (size_t)(2 * M * w8a8::round_up16(r) * sizeof(uint16_t));
}

namespace w8a8 {
namespace {

// Argument checks shared by svdq_linear and svdq_linear_noalloc (the
// workspace is checked by the caller).
w8a8_status svdq_check(w8a8_qtype qtype, const uint16_t *x, int64_t M, int64_t K, const void *rq,
                       const float *r_scale, const uint16_t *l1, const uint16_t *l2, int64_t r, const uint16_t *bias,
                       int64_t N, const uint16_t *y, const void *xq_out, const float *x_scale_out) {
    if (!valid_qtype(qtype) || r < 1 || r > kMaxRp) return W8A8_ERR_INVALID_ARG;
    w8a8_status st = gemm_check(xq_out, rq, M, N, K, y);
    if (st != W8A8_OK) return st;
    st = act_quant_check(qtype, x, M, K, K, xq_out, K, x_scale_out);
    if (st != W8A8_OK) return st;
    if (M > 0 && N > 0 && (!r_scale || !l1 || !l2)) return W8A8_ERR_INVALID_ARG;
    if (!aligned16(r_scale) || !aligned16(l1) || !aligned16(l2) || !aligned16(bias)) return W8A8_ERR_ALIGN;
    return W8A8_OK;
}

// The launches, on checked arguments; `workspace` holds u (hi, then lo).
w8a8_status svdq_run(w8a8_qtype qtype, const uint16_t *x, int64_t M, int64_t K, const void *rq, const float *r_scale,
                     const uint16_t *l1, const uint16_t *l2, int64_t r, const uint16_t *bias, int64_t N, uint16_t *y,
                     void *xq_out, float *x_scale_out, void *workspace, hipStream_t stream) {
    w8a8_status st = W8A8_OK;
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

}  // namespace
}  // namespace w8a8

extern "C" w8a8_status svdq_linear(w8a8_qtype qtype, const uint16_t *x, int64_t M, int64_t K, const void *rq,
                                   const float *r_scale, const uint16_t *l1, const uint16_t *l2, int64_t r,
                                   const uint16_t *bias, int64_t N, uint16_t *y, void *xq_out, float *x_scale_out,
                                   void *workspace, hipStream_t stream) {
    using namespace w8a8;
    w8a8_status st = svdq_check(qtype, x, M, K, rq, r_scale, l1, l2, r, bias, N, y, xq_out, x_scale_out);
    if (st != W8A8_OK) return st;
    if (M > 0 && N > 0 && !workspace) return W8A8_ERR_INVALID_ARG;
    if (!aligned16(workspace)) return W8A8_ERR_ALIGN;
    return svdq_run(qtype, x, M, K, rq, r_scale, l1, l2, r, bias, N, y, xq_out, x_scale_out, workspace, stream);
}

// ------------------------------------------------------------------------
// svdq_linear_noalloc: the same launches with u in a fixed device array of
// the library instead of a caller workspace, for callers that cannot
// allocate.  Each GPU holds its own copy of the array from the time the
// library's code object is loaded on it until the process ends.  u is
// written in full (every row < M, every column < rp) before it is read, so
// the contents a previous call left there never reach a result and nothing
// is cleared.  Calls that overlap on one GPU (different streams, or host
// threads) share the array and race.
static __device__ __align__(256) uint8_t scratch[W8A8_SVDQ_NOALLOC_SCRATCH_BYTES];

namespace w8a8 {
namespace {

// Device address of `scratch` on device `dev` (the current device), taken
// once per device: the name of the array in host code is a host-side
// stand-in, not a device address.  Threads racing on the first query store
// the same value.
void *scratch_address(int dev) {
    static std::atomic<void *> cached[64] = {};
    if (dev < 0 || dev >= 64) return nullptr;
    void *ptr = cached[dev].load(std::memory_order_acquire);
    if (ptr) return ptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    cached[dev].store(ptr, std::memory_order_release);
    return ptr;
}

}  // namespace
}  // namespace w8a8

extern "C" w8a8_status svdq_linear_noalloc(w8a8_qtype qtype, const uint16_t *x, int64_t M, int64_t K,
                                           const void *rq, const float *r_scale, const uint16_t *l1,
                                           const uint16_t *l2, int64_t r, const uint16_t *bias, int64_t N,
                                           uint16_t *y, void *xq_out, float *x_scale_out, hipStream_t stream) {
    using namespace w8a8;
    w8a8_status st = svdq_check(qtype, x, M, K, rq, r_scale, l1, l2, r, bias, N, y, xq_out, x_scale_out);
    if (st != W8A8_OK) return st;
    if (svdq_workspace_bytes(M, r) > (size_t)W8A8_SVDQ_NOALLOC_SCRATCH_BYTES) return W8A8_ERR_SCRATCH_LIMIT;
    if (M == 0) return W8A8_OK;
    // the scratch of the device the stream runs on, which must be current
    int dev = -1, sdev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return W8A8_ERR_HIP;
    if (stream == nullptr) sdev = dev;  // the null stream is the current device's
    else if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return W8A8_ERR_HIP;
    if (dev != sdev) return W8A8_ERR_INVALID_ARG;
    void *ws = scratch_address(dev);
    if (!ws) return W8A8_ERR_HIP;
    return svdq_run(qtype, x, M, K, rq, r_scale, l1, l2, r, bias, N, y, xq_out, x_scale_out, ws, stream);
}
