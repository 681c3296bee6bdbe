// gemm.hip -- the 8-bit product of the W8A8 linear with its fused epilogue.
//
// OneTrainer wiki "Quantization" (int W8A8 / float W8A8, "Technical"): the
// linear layer's matrix multiplication runs in int8 (int32 accumulation) or
// float8 e4m3 (f32 accumulation) on row-wise quantized activations and a
// tensor-wise quantized weight; the result is dequantized back to the train
// dtype.  The dequantization (row scale x weight scale + bias -> bf16) and
// the SVDQuant low-rank term (OneTrainer PR #1034, "SVDQuant") are fused into
// this kernel's epilogue, so the int32/f32 accumulators never leave registers.
//
// CDNA4 design:
//  * 256x256 output tile per workgroup, 4 waves in a 2x2 grid, each wave a
//    128x128 sub-tile held as 4x4 blocks of 32x32 MFMA accumulators
//    (v_mfma_i32_32x32x32_i8, or v_mfma_scale_f32_32x32x64_f8f6f4 with unit
//    scales for e4m3): 256 accumulator registers per lane.
//  * Both operands are K-contiguous ("NT"), so every lane's MFMA fragment is
//    a contiguous 16- or 32-byte run of one row.  The weight is the MFMA's A
//    operand and the activations its B operand, so each lane ends up holding
//    four consecutive output columns of one row: 8-byte bf16 stores.
//  * K is consumed in 128-byte stages.  Stages go HBM -> LDS directly with
//    buffer_load_dwordx4 ... lds (no register staging), double buffered in two
//    separate LDS arrays so the loads of stage t+1 overlap the MFMAs of stage
//    t.  Buffer loads past num_records read zero, which covers ragged M/N
//    tails and (with an out-of-range offset) the ragged K tail.
//  * Within a stage, 16-byte chunks of each 128-byte row are XOR-swizzled by
//    the row index so the fragment reads of 8 consecutive rows hit 8 distinct
//    bank groups.
//  * Tiles are numbered so that consecutive workgroups on one XCD (hardware
//    dispatches workgroup i to XCD i % 8) share operand rows in that XCD's L2.
#include <type_traits>

#include "internal.hpp"

namespace w8a8 {
namespace {

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int kThreads = 256;
constexpr int kOpBytes = 256 * BK;           // one operand tile per stage: 32 KB
constexpr int kStageBytes = 2 * kOpBytes;    // X tile then W tile
constexpr int kGroupM = 4;                   // tile-ordering group height
constexpr int kXcds = 8;

typedef __attribute__((address_space(3))) void *lds_ptr_t;

__device__ __forceinline__ int swz(int row) { return row & 7; }

struct TileCoord {
    int m0, n0;
};

__device__ __forceinline__ TileCoord tile_coord(int tiles_m, int tiles_n) {
    const int nt = tiles_m * tiles_n;
    int bid = blockIdx.x;
    // XCD-major renumbering: hardware sends workgroup b to XCD b % 8; give
    // each XCD a contiguous range of logical tiles.
    const int per = nt / kXcds;
    int t = bid < per * kXcds ? (bid % kXcds) * per + bid / kXcds : bid;
    // grouped order: kGroupM tile-rows advance together along N
    const int group = kGroupM * tiles_n;
    const int g = t / group;
    const int first_m = g * kGroupM;
    const int gm = min(tiles_m - first_m, kGroupM);
    const int in = t - g * group;
    TileCoord c;
    c.m0 = (first_m + in % gm) * BM;
    c.n0 = (in / gm) * BN;
    return c;
}

template <int QT, int EPI>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs p, int tiles_m, int tiles_n) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds0[kStageBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[kStageBytes];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const TileCoord tc = tile_coord(tiles_m, tiles_n);
    const int K = p.K;

    // Buffer descriptors starting at the tile's first row; rows past M (N)
    // fall outside num_records and read as zero.
    const int rows_x = min(p.M - tc.m0, BM), rows_w = min(p.N - tc.n0, BN);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(p.xq + (size_t)tc.m0 * K), (short)0, rows_x * K, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(p.wq + (size_t)tc.n0 * K), (short)0, rows_w * K, kBufferRsrcWord3);

    // Global -> LDS mapping: wave w fills rows [64w, 64w+64) of each operand
    // tile, 8 rows (1 KB) per instruction; lane l lands at LDS byte 16 l of
    // that KB, i.e. row 8i + l/8, physical chunk l%8 = logical chunk ^ swz.
    int goff[8], gcol[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = wave * 64 + i * 8 + (lane >> 3);
        const int c = (lane & 7) ^ swz(row);
        gcol[i] = c * 16;
        goff[i] = row * K + c * 16;
    }
    const int ktiles = (K + BK - 1) / BK;

    auto load_stage = [&](uint8_t *stage, int kt) {
        const int k0 = kt * BK;
        const bool full = k0 + BK <= K;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int o = full ? goff[i] + k0 : (k0 + gcol[i] < K ? goff[i] + k0 : kOobOffset);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr_t)(stage + (wave * 64 + i * 8) * BK), 16, o, 0, 0,
                                                     0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int o = full ? goff[i] + k0 : (k0 + gcol[i] < K ? goff[i] + k0 : kOobOffset);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_ptr_t)(stage + kOpBytes + (wave * 64 + i * 8) * BK),
                                                     16, o, 0, 0, 0);
        }
    };

    // Fragment read offsets: lane row = l & 31 within a 32-row block (so
    // swz(row) = l & 7); the k-chunk depends on the step.
    const int lrow = lane & 31, half = lane >> 5, sz = lane & 7;
    typedef typename std::conditional<QT == W8A8_INT8, v16i, v16f>::type acc_t;
    acc_t acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[a][b][e] = 0;

    auto compute_stage = [&](const uint8_t *stage) {
        const uint8_t *xs = stage + (wm * 128) * BK;            // X rows of this wave
        const uint8_t *ws = stage + kOpBytes + (wn * 128) * BK;  // W rows of this wave
        if constexpr (QT == W8A8_INT8) {
#pragma unroll
            for (int kk = 0; kk < BK / 32; ++kk) {
                const int off = lrow * BK + ((((kk * 2) + half) ^ sz) << 4);
                v4i af[4], bf[4];
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) af[nb] = *reinterpret_cast<const v4i *>(ws + nb * 32 * BK + off);
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) bf[mb] = *reinterpret_cast<const v4i *>(xs + mb * 32 * BK + off);
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                    for (int mb = 0; mb < 4; ++mb)
                        acc[nb][mb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[nb], bf[mb], acc[nb][mb], 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int kk = 0; kk < BK / 64; ++kk) {
                const int c0 = kk * 4 + half * 2;
                const int off0 = lrow * BK + ((c0 ^ sz) << 4);
                const int off1 = lrow * BK + (((c0 + 1) ^ sz) << 4);
                v8i af[4], bf[4];
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    const v4i lo = *reinterpret_cast<const v4i *>(ws + nb * 32 * BK + off0);
                    const v4i hi = *reinterpret_cast<const v4i *>(ws + nb * 32 * BK + off1);
                    af[nb] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                }
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) {
                    const v4i lo = *reinterpret_cast<const v4i *>(xs + mb * 32 * BK + off0);
                    const v4i hi = *reinterpret_cast<const v4i *>(xs + mb * 32 * BK + off1);
                    bf[mb] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                }
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                    for (int mb = 0; mb < 4; ++mb)
                        acc[nb][mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[nb], bf[mb], acc[nb][mb], 0,
                                                                                      0, 0, 127, 0, 127);
            }
        }
    };

    // Main loop: two LDS stages, loads of the next stage in flight while the
    // current one is multiplied.
    load_stage(lds0, 0);
    int kt = 0;
    for (; kt + 2 <= ktiles; kt += 2) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        load_stage(lds1, kt + 1);
        compute_stage(lds0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (kt + 2 < ktiles) load_stage(lds0, kt + 2);
        compute_stage(lds1);
    }
    if (kt < ktiles) {  // odd number of stages: the last one sits in lds0
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        compute_stage(lds0);
    }

    // ------------------------------------------------------------- epilogue
    // Block (nb, mb), register 4j+i holds output row m = mbase + (l & 31) and
    // column n = nbase + 8j + 4(l >> 5) + i.
    const int M = p.M, N = p.N;
    const int mw = tc.m0 + wm * 128, nw = tc.n0 + wn * 128;
    if constexpr (EPI == kEpiI32) {
        int32_t *out = static_cast<int32_t *>(p.out);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                const int m = mw + mb * 32 + lrow;
                if (m >= M) continue;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int n = nw + nb * 32 + 8 * j + 4 * half;
                    int32_t *dst = out + (size_t)m * N + n;
                    if ((N & 3) == 0 && n + 3 < N) {
                        v4i v = {(int)acc[nb][mb][4 * j], (int)acc[nb][mb][4 * j + 1], (int)acc[nb][mb][4 * j + 2],
                                 (int)acc[nb][mb][4 * j + 3]};
                        *reinterpret_cast<v4i *>(dst) = v;
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (n + i < N) dst[i] = (int)acc[nb][mb][4 * j + i];
                    }
                }
            }
    } else {
        uint16_t *out = static_cast<uint16_t *>(p.out);
        const float sw = p.sw[0];
        float tm[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int m = mw + mb * 32 + lrow;
            tm[mb] = m < M ? p.sx[m] * sw : 0.0f;
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            float bias[4][4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = nw + nb * 32 + 8 * j + 4 * half;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    bias[j][i] = (p.bias && n + i < N) ? bf16_bits_to_f32(p.bias[n + i]) : 0.0f;
            }
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                const int m = mw + mb * 32 + lrow;
                v16f v;
#pragma unroll
                for (int e = 0; e < 16; ++e) v[e] = (float)acc[nb][mb][e] * tm[mb];
                if constexpr (EPI == kEpiLowRank) {
                    // y += u . l2^T on the bf16 MFMA: A = l2 rows (n), B = u rows (m),
                    // u = hi + lo in bf16.
                    const int nrow = nw + nb * 32 + lrow;
                    for (int ks = 0; ks < p.rp; ks += 16) {
                        const int j0 = ks + half * 8;
                        v8bf a, bh, bl;
                        uint16_t ta[8];
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            ta[i] = (nrow < N && j0 + i < p.r) ? p.l2[(size_t)nrow * p.r + j0 + i] : (uint16_t)0;
                        a = __builtin_bit_cast(v8bf, ta);
                        if (m < M) {
                            bh = *reinterpret_cast<const v8bf *>(p.uhi + (size_t)m * p.rp + j0);
                            bl = *reinterpret_cast<const v8bf *>(p.ulo + (size_t)m * p.rp + j0);
                        } else {
                            uint16_t z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                            bh = __builtin_bit_cast(v8bf, z);
                            bl = bh;
                        }
                        v = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bh, v, 0, 0, 0);
                        v = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bl, v, 0, 0, 0);
                    }
                }
                if (m >= M) continue;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int n = nw + nb * 32 + 8 * j + 4 * half;
                    uint16_t *dst = out + (size_t)m * N + n;
                    const float y0 = v[4 * j] + bias[j][0], y1 = v[4 * j + 1] + bias[j][1];
                    const float y2 = v[4 * j + 2] + bias[j][2], y3 = v[4 * j + 3] + bias[j][3];
                    if ((N & 3) == 0 && n + 3 < N) {
                        uint2 pk = make_uint2(pack_bf16x2(y0, y1), pack_bf16x2(y2, y3));
                        *reinterpret_cast<uint2 *>(dst) = pk;
                    } else {
                        const float yy[4] = {y0, y1, y2, y3};
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (n + i < N) dst[i] = (uint16_t)f32_to_bf16_bits(yy[i]);
                    }
                }
            }
        }
    }
}

template <int QT, int EPI>
void launch(const GemmArgs &a, hipStream_t stream) {
    const int tm = (a.M + BM - 1) / BM, tn = (a.N + BN - 1) / BN;
    gemm_kernel<QT, EPI><<<tm * tn, kThreads, 0, stream>>>(a, tm, tn);
}

}  // namespace

w8a8_status gemm_check(const void *xq, const void *wq, int64_t M, int64_t N, int64_t K, const void *out) {
    if (M < 0 || N < 0 || K < 0) return W8A8_ERR_INVALID_ARG;
    if (M > 0 && N > 0 && (!xq || !wq || !out)) return W8A8_ERR_INVALID_ARG;
    if (K < 16 || K % 16 != 0 || K > (1 << 22)) return W8A8_ERR_SHAPE;
    if (M > (1 << 30) || N > (1 << 30)) return W8A8_ERR_SHAPE;
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    if (tiles > 0x7FFFFFFF) return W8A8_ERR_SHAPE;
    if (!aligned16(xq) || !aligned16(wq) || !aligned16(out)) return W8A8_ERR_ALIGN;
    return W8A8_OK;
}

w8a8_status gemm_launch(w8a8_qtype qtype, GemmEpilogue epi, const GemmArgs &a, hipStream_t stream) {
    if (a.M == 0 || a.N == 0) return W8A8_OK;
    if (qtype == W8A8_INT8) {
        if (epi == kEpiI32) launch<W8A8_INT8, kEpiI32>(a, stream);
        else if (epi == kEpiBf16) launch<W8A8_INT8, kEpiBf16>(a, stream);
        else launch<W8A8_INT8, kEpiLowRank>(a, stream);
    } else {
        if (epi == kEpiI32) return W8A8_ERR_UNSUPPORTED;
        if (epi == kEpiBf16) launch<W8A8_FP8_E4M3, kEpiBf16>(a, stream);
        else launch<W8A8_FP8_E4M3, kEpiLowRank>(a, stream);
    }
    return launch_status();
}

}  // namespace w8a8

extern "C" w8a8_status w8a8_linear(w8a8_qtype qtype, const void *xq, const float *x_scale, const void *wq,
                                   const float *w_scale, const uint16_t *bias, int64_t M, int64_t N, int64_t K,
                                   uint16_t *y, hipStream_t stream) {
    using namespace w8a8;
    if (!valid_qtype(qtype)) return W8A8_ERR_INVALID_ARG;
    w8a8_status st = gemm_check(xq, wq, M, N, K, y);
    if (st != W8A8_OK) return st;
    if (M > 0 && N > 0 && (!x_scale || !w_scale)) return W8A8_ERR_INVALID_ARG;
    if (!aligned16(x_scale) || !aligned16(w_scale) || !aligned16(bias)) return W8A8_ERR_ALIGN;
    GemmArgs a = {};
    a.xq = static_cast<const uint8_t *>(xq);
    a.wq = static_cast<const uint8_t *>(wq);
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.sx = x_scale;
    a.sw = w_scale;
    a.bias = bias;
    a.out = y;
    return gemm_launch(qtype, kEpiBf16, a, stream);
}

extern "C" w8a8_status w8a8_linear_backward_dx(w8a8_qtype qtype, const void *dyq, const float *dy_scale,
                                               const void *wq_t, const float *w_scale, int64_t M, int64_t N,
                                               int64_t K, uint16_t *dx, hipStream_t stream) {
    // dX[M, K] = dYq[M, N] . Wq[N, K] = the NT product of dYq with Wq^T [K, N]
    // over the reduction length N.
    return w8a8_linear(qtype, dyq, dy_scale, wq_t, w_scale, nullptr, M, K, N, dx, stream);
}

extern "C" w8a8_status w8a8_gemm_i32(const int8_t *xq, const int8_t *wq, int64_t M, int64_t N, int64_t K,
                                     int32_t *acc, hipStream_t stream) {
    using namespace w8a8;
    w8a8_status st = gemm_check(xq, wq, M, N, K, acc);
    if (st != W8A8_OK) return st;
    GemmArgs a = {};
    a.xq = reinterpret_cast<const uint8_t *>(xq);
    a.wq = reinterpret_cast<const uint8_t *>(wq);
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.out = acc;
    return gemm_launch(W8A8_INT8, kEpiI32, a, stream);
}
