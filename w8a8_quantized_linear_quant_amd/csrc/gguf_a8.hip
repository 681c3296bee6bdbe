// gguf_a8.hip -- weight preparation of the GGUF A8 quant types.
//
// OneTrainer wiki "Quantization", GGUF A8 int / GGUF A8 float ("Technical"):
// the weight is loaded as the GGUF file stores it and re-quantized axis-wise
// to int8 (float8 e4m3), one scale per output channel; the linear then runs
// the 8-bit product on token-wise quantized activations, with the per-channel
// weight scales applied in the product's epilogue (gguf_a8_linear, gemm.hip).
// The GGUF format here is Q8_0 (entrenar q8_0.rs, struct Q8_0: 34-byte blocks
// of an f16 scale d and 32 int8 codes); a weight row of K values is K / 32
// consecutive blocks, and its values are the exact dequantization q * d.
//
// One wave per output row.  Rows of up to kMaxRowBytes are staged whole in
// the wave's LDS area (16-byte loads from the 16-byte aligned address at or
// below the row); 8 lanes take one block (4 codes each).  Rows of K <= 4096
// are dequantized once into registers, which give both the row absmax and
// the codes; longer rows find the absmax from the staged bytes and dequantize
// again for the codes.  The codes are written in place over the blocks they
// come from (block b's 32 codes land at 32 b, at or before its source
// bytes), and the row leaves as 16-byte stores.  Rows longer than
// kMaxRowBytes are streamed through the LDS area in chunks of 64 blocks in two
// passes (absmax, then codes, the second re-staging the row from L2).
#include "internal.hpp"

namespace w8a8 {
namespace {

constexpr int kThreads = 256;            // 4 waves, one row each
constexpr int kChunkBlocks = 64;
constexpr int kStageBytes = kChunkBlocks * 34 + 32;  // chunk + alignment slack, multiple of 16
static_assert(kStageBytes % 16 == 0, "16-byte staging");
constexpr int kMaxRowBytes = 16 * 1024 - 16;  // single-pass limit: 4 waves x 16 KB of LDS

// Stage row n (row_bytes of blocks from byte s0 of the tensor) in the wave's
// LDS area st with 16-byte loads from the aligned address at or below it;
// returns the row's offset within st.  Every lane issues 4 loads before it
// writes any of them to LDS (vector indices past the row are clamped to its
// last vector: a repeated load whose data is dropped).
__device__ __forceinline__ int stage_row(__amdgpu_buffer_rsrc_t rs, uint32_t total_bytes, uint32_t s0,
                                         uint32_t row_bytes, uint8_t *st, int lane) {
    const uint32_t a0 = s0 & ~15u;
    const int off = (int)(s0 - a0);
    const int nvec = (off + (int)row_bytes + 15) / 16;
    for (int i0 = 0; i0 < nvec; i0 += 256) {
        v4u t[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int i = min(i0 + lane + 64 * j, nvec - 1);
            t[j] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rs, a0 + 16u * i, 0, 0));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int i = i0 + lane + 64 * j;
            if (i < nvec) *reinterpret_cast<v4u *>(st + 16 * i) = t[j];
        }
    }
    // The tensor's last 16 bytes may run past its end: a wide load that
    // crosses num_records reads zero as a whole, so that vector is read
    // again byte by byte (bytes past the end read zero).  Same wave, so
    // these LDS writes land after the ones above.
    const uint32_t vlast = a0 + 16u * (nvec - 1);
    if (vlast + 16u > total_bytes && lane < 16)
        st[16 * (nvec - 1) + lane] = __builtin_amdgcn_raw_buffer_load_b8(rs, vlast + lane, 0, 0);
    return off;
}

// Values q d of this lane's 4 codes (part = lane & 7) of the staged block at
// bp.  For int8 each code byte is flipped to q + 128 in [0, 255] (one XOR for
// the 4), which converts as an unsigned byte; fma(q + 128, d, -128 d) then
// gives q d exactly: both products fit in 19 bits and their difference is
// q d itself, an f32 value.  Only the sign of a zero can differ (+0 for q = 0,
// d < 0), which the int8 code ignores; e4m3 codes -0 and +0 apart, so that
// path multiplies the signed code.
template <int QT>
__device__ __forceinline__ void staged_block_vals(const uint8_t *bp, int part, float *v) {
    const uint32_t dbits = *reinterpret_cast<const uint16_t *>(bp);
    const uint32_t lo = *reinterpret_cast<const uint16_t *>(bp + 2 + 4 * part);
    const uint32_t hi = *reinterpret_cast<const uint16_t *>(bp + 4 + 4 * part);
    const float d = (float)__builtin_bit_cast(_Float16, (uint16_t)dbits);
    if constexpr (QT == W8A8_INT8) {
        const float nd = -128.0f * d;
        const uint32_t w = (lo | (hi << 16)) ^ 0x80808080u;  // q + 128 per byte
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = fmaf((float)((w >> (8 * i)) & 0xFFu), d, nd);
    } else {
        const uint32_t w = lo | (hi << 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (float)(int8_t)(w >> (8 * i)) * d;  // exact in f32
    }
}

// The code word (4 codes) of 4 values under row scale s (r = f32(1 / s)).
template <int QT>
__device__ __forceinline__ uint32_t code_word(const float *v, float s, float r) {
    if constexpr (QT == W8A8_INT8) {
        // |v / s| <= 127 by the scale rule: no clamp needed; the add of
        // 1.5 * 2^23 rounds half to even, the result's low byte is the code
        uint32_t b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) b[i] = __float_as_uint(quotient_nosign(v[i], s, r) + 12582912.0f);
        return __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u) | __builtin_amdgcn_perm(b[3], b[2], 0x04000c0cu);
    } else {
        float c[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) c[i] = __builtin_amdgcn_fmed3f(quotient(v[i], s, r), -448.0f, 448.0f);
        int pk = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
        pk = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], pk, true);
        return (uint32_t)pk;
    }
}

// Rows of at most 8 * NSTEP blocks (K <= 4096): each lane keeps the values of
// its 4 codes of NSTEP blocks in registers (block 8 q + lane / 8 of step q),
// so the row is dequantized once: its absmax and its codes come from the
// same values (the staged-row kernel below dequantizes twice).  Steps past
// the row's last block repeat that block (their writes rewrite the same
// codes).  The codes are written over the staged blocks (all reads are done
// by then) and the row leaves as 16-byte stores.  FULL: the row has exactly
// 8 * NSTEP blocks, so no step is clamped and the lane's block of step q sits
// at a fixed stride from its block of step 0: every step's LDS address is one
// per-lane base plus an immediate offset (no address arithmetic per step).
template <int QT, int NSTEP, bool FULL>
__global__ __launch_bounds__(kThreads) void gguf_a8_requant_reg_kernel(const uint8_t *__restrict__ blocks,
                                                                       uint32_t total_bytes, int N, int K,
                                                                       int row_stage, uint8_t *__restrict__ wq,
                                                                       float *__restrict__ scale) {
    extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    uint8_t *st = dyn_lds + wave * row_stage;
    const int nb = K / 32;
    const uint32_t row_bytes = (uint32_t)nb * 34u;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(blocks), (short)0, (int)total_bytes, kBufferRsrcWord3);
    const float qmax = QT == W8A8_INT8 ? 127.0f : 448.0f;
    const int blk_in_step = lane >> 3, part = lane & 7;

    for (int n = blockIdx.x * (kThreads / 64) + wave; n < N; n += gridDim.x * (kThreads / 64)) {
        const int off = stage_row(rs, total_bytes, (uint32_t)n * row_bytes, row_bytes, st, lane);
        const uint8_t *src0 = st + off + blk_in_step * 34;
        uint8_t *dst0 = st + blk_in_step * 32 + 4 * part;
        auto src = [&](int q) { return FULL ? src0 + q * (8 * 34) : st + off + min(8 * q + blk_in_step, nb - 1) * 34; };
        auto dst = [&](int q) { return FULL ? dst0 + q * (8 * 32) : st + min(8 * q + blk_in_step, nb - 1) * 32 + 4 * part; };
        float v[NSTEP][4];
        float amax = 0.0f;
#pragma unroll
        for (int q = 0; q < NSTEP; ++q) {
            staged_block_vals<QT>(src(q), part, v[q]);
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[q][0]), fabsf(v[q][1])), fmaxf(fabsf(v[q][2]), fabsf(v[q][3]))));
        }
        // non-negative floats order like their bit patterns
        const float s = absmax_scale(__uint_as_float(wave_max_u32(__float_as_uint(amax))), qmax);
        const float r = 1.0f / s;
        if (lane == 0) scale[n] = s;
#pragma unroll
        for (int q = 0; q < NSTEP; ++q) *reinterpret_cast<uint32_t *>(dst(q)) = code_word<QT>(v[q], s, r);
        // the row's codes leave as 16-byte stores, 4 LDS reads per lane at a time
        uint8_t *orow = wq + (size_t)n * K;
        const int nout = K / 16;
        for (int i0 = 0; i0 < nout; i0 += 256) {
            v4u t[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) t[j] = *reinterpret_cast<const v4u *>(st + 16 * min(i0 + lane + 64 * j, nout - 1));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = i0 + lane + 64 * j;
                if (i < nout) *reinterpret_cast<v4u *>(orow + 16 * i) = t[j];
            }
        }
    }
}

// Whole-row kernel: each wave stages one row of row_stage bytes (a multiple
// of 16, at least the row's bytes + 15) in dynamic LDS.
template <int QT>
__global__ __launch_bounds__(kThreads) void gguf_a8_requant_row_kernel(const uint8_t *__restrict__ blocks,
                                                                       uint32_t total_bytes, int N, int K,
                                                                       int row_stage, uint8_t *__restrict__ wq,
                                                                       float *__restrict__ scale) {
    extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    uint8_t *st = dyn_lds + wave * row_stage;
    const int nb = K / 32;
    const uint32_t row_bytes = (uint32_t)nb * 34u;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(blocks), (short)0, (int)total_bytes, kBufferRsrcWord3);
    const float qmax = QT == W8A8_INT8 ? 127.0f : 448.0f;
    const int blk_in_step = lane >> 3, part = lane & 7;  // 8 lanes per block, 4 codes each

    for (int n = blockIdx.x * (kThreads / 64) + wave; n < N; n += gridDim.x * (kThreads / 64)) {
        const int off = stage_row(rs, total_bytes, (uint32_t)n * row_bytes, row_bytes, st, lane);
        // |q d| of this lane's 4 codes of block b, maximized: every product is
        // exact in f32 (8-bit q, 11-bit d), so the largest is max|q| * |d|,
        // and max|q| = max(max(q + 128) - 128, 128 - min(q + 128)).
        auto block_absmax = [&](int b) {
            const uint8_t *bp = st + off + b * 34;
            const uint32_t dbits = *reinterpret_cast<const uint16_t *>(bp);
            const uint32_t lo = *reinterpret_cast<const uint16_t *>(bp + 2 + 4 * part);
            const uint32_t hi = *reinterpret_cast<const uint16_t *>(bp + 4 + 4 * part);
            const float d = (float)__builtin_bit_cast(_Float16, (uint16_t)dbits);
            const uint32_t w = (lo | (hi << 16)) ^ 0x80808080u;  // q + 128 per byte
            float u[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) u[i] = (float)((w >> (8 * i)) & 0xFFu);
            const float hi_u = fmaxf(fmaxf(u[0], u[1]), fmaxf(u[2], u[3]));
            const float lo_u = fminf(fminf(u[0], u[1]), fminf(u[2], u[3]));
            return fmaxf(hi_u - 128.0f, 128.0f - lo_u) * fabsf(d);
        };
        // Row absmax (non-negative floats order like their bit patterns), 32
        // blocks (4 steps of 8) per iteration with their LDS reads issued
        // together; block indices past the row repeat its last block.
        uint32_t amax_bits = 0;
        for (int b0 = 0; b0 < nb; b0 += 32) {
            float a[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) a[q] = block_absmax(min(b0 + 8 * q + blk_in_step, nb - 1));
#pragma unroll
            for (int q = 0; q < 4; ++q) amax_bits = max(amax_bits, __float_as_uint(a[q]));
        }
        const float s = absmax_scale(__uint_as_float(wave_max_u32(amax_bits)), qmax);
        const float r = 1.0f / s;
        if (lane == 0) scale[n] = s;
        // Codes, in place: the reads of an iteration (blocks b0..b0+31, bytes
        // from off + 34 b0 on) precede its writes (32 b0 .. 32 b0 + 1023) in
        // the wave's LDS order, and later iterations read from
        // 34 (b0 + 32) > 32 b0 + 1023 on.
        for (int b0 = 0; b0 < nb; b0 += 32) {
            float v[4][4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                staged_block_vals<QT>(st + off + min(b0 + 8 * q + blk_in_step, nb - 1) * 34, part, v[q]);
            // past the row's last block a lane rewrites that block's own word
            // with the same value (its index was clamped above)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<uint32_t *>(st + min(b0 + 8 * q + blk_in_step, nb - 1) * 32 + 4 * part) =
                    code_word<QT>(v[q], s, r);
        }
        // the row's codes leave as 16-byte stores, 4 LDS reads per lane at a time
        uint8_t *orow = wq + (size_t)n * K;
        const int nout = K / 16;
        for (int i0 = 0; i0 < nout; i0 += 256) {
            v4u t[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) t[j] = *reinterpret_cast<const v4u *>(st + 16 * min(i0 + lane + 64 * j, nout - 1));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = i0 + lane + 64 * j;
                if (i < nout) *reinterpret_cast<v4u *>(orow + 16 * i) = t[j];
            }
        }
    }
}

template <int QT>
__global__ __launch_bounds__(kThreads) void gguf_a8_requant_kernel(const uint8_t *__restrict__ blocks,
                                                                   uint32_t total_bytes, int N, int K,
                                                                   uint8_t *__restrict__ wq,
                                                                   float *__restrict__ scale) {
    __shared__ __attribute__((aligned(16))) uint8_t stage[kThreads / 64][kStageBytes];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    uint8_t *st = stage[wave];
    const int nb = K / 32;
    const uint32_t row_bytes = (uint32_t)nb * 34u;
    // Whole tensor in one descriptor (total_bytes < 2^31 is checked on the
    // host); loads past its end read zero.
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(blocks), (short)0, (int)total_bytes, kBufferRsrcWord3);
    const float qmax = QT == W8A8_INT8 ? 127.0f : 448.0f;
    const int blk_in_step = lane >> 3, part = lane & 7;  // 8 lanes per block, 4 codes each

    // Stage blocks [c0, c0 + cb) of row n; returns the byte offset of block
    // c0 within the staging area.
    auto stage_chunk = [&](int n, int c0, int cb) -> int {
        const uint32_t s0 = (uint32_t)n * row_bytes + (uint32_t)c0 * 34u;
        const uint32_t a0 = s0 & ~15u;
        const int off = (int)(s0 - a0);
        const int nvec = (off + cb * 34 + 15) / 16;
        for (int i = lane; i < nvec; i += 64) {
            const uint32_t vo = a0 + 16u * i;
            v4u v;
            if (vo + 16u <= total_bytes) {
                v = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rs, vo, 0, 0));
            } else {
                // the tensor's last 16 bytes run past its end: a wide load
                // that crosses num_records reads zero as a whole, so take the
                // remaining bytes one by one
                uint8_t t[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) t[j] = __builtin_amdgcn_raw_buffer_load_b8(rs, vo + j, 0, 0);
                v = __builtin_bit_cast(v4u, t);
            }
            *reinterpret_cast<v4u *>(st + 16 * i) = v;
        }
        return off;
    };
    // Values of this lane's 4 codes of block b of the staged chunk (0 past cb).
    auto block_vals = [&](int off, int b, int cb, float *v) {
        if (b < cb) {
            const uint8_t *bp = st + off + b * 34;
            const uint32_t dbits = *reinterpret_cast<const uint16_t *>(bp);
            const uint32_t lo = *reinterpret_cast<const uint16_t *>(bp + 2 + 4 * part);
            const uint32_t hi = *reinterpret_cast<const uint16_t *>(bp + 4 + 4 * part);
            const float d = (float)__builtin_bit_cast(_Float16, (uint16_t)dbits);
            const uint32_t w = lo | (hi << 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = (float)(int8_t)(w >> (8 * i)) * d;  // exact in f32
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = 0.0f;
        }
    };

    for (int n = blockIdx.x * (kThreads / 64) + wave; n < N; n += gridDim.x * (kThreads / 64)) {
        // pass 1: row absmax (non-negative floats order like their bit patterns)
        uint32_t amax_bits = 0;
        for (int c0 = 0; c0 < nb; c0 += kChunkBlocks) {
            const int cb = min(kChunkBlocks, nb - c0);
            const int off = stage_chunk(n, c0, cb);
            for (int b0 = 0; b0 < cb; b0 += 8) {
                float v[4];
                block_vals(off, b0 + blk_in_step, cb, v);
                const float a = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
                amax_bits = max(amax_bits, __float_as_uint(a));
            }
        }
        const float s = absmax_scale(__uint_as_float(wave_max_u32(amax_bits)), qmax);
        if (lane == 0) scale[n] = s;
        // pass 2: codes; the quotient is an IEEE division, as the oracle's
        uint8_t *orow = wq + (size_t)n * K;
        for (int c0 = 0; c0 < nb; c0 += kChunkBlocks) {
            const int cb = min(kChunkBlocks, nb - c0);
            const int off = stage_chunk(n, c0, cb);
            for (int b0 = 0; b0 < cb; b0 += 8) {
                const int b = b0 + blk_in_step;
                float v[4];
                block_vals(off, b, cb, v);
                uint32_t word = 0;
                if constexpr (QT == W8A8_INT8) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float q = __builtin_amdgcn_fmed3f(v[i] / s, -128.0f, 127.0f);
                        word |= ((uint32_t)(int)__builtin_rintf(q) & 0xFFu) << (8 * i);
                    }
                } else {
                    float q[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) q[i] = __builtin_amdgcn_fmed3f(v[i] / s, -448.0f, 448.0f);
                    int pk = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
                    pk = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], pk, true);
                    word = (uint32_t)pk;
                }
                if (b < cb) *reinterpret_cast<uint32_t *>(orow + (size_t)(c0 + b) * 32 + 4 * part) = word;
            }
        }
    }
}

}  // namespace
}  // namespace w8a8

extern "C" w8a8_status gguf_a8_requant_q8_0(w8a8_qtype qtype, const void *blocks, int64_t N, int64_t K, void *wq,
                                            float *w_scale, hipStream_t stream) {
    using namespace w8a8;
    if (!valid_qtype(qtype) || N < 0 || K < 0) return W8A8_ERR_INVALID_ARG;
    if (K % 32 != 0 || K > (1 << 24) || N > (1 << 30)) return W8A8_ERR_SHAPE;
    const int64_t total = N * (K / 32) * 34;
    if (total >= ((int64_t)1 << 31)) return W8A8_ERR_SHAPE;
    if (N == 0) return W8A8_OK;
    // K == 0: no blocks, no codes; every row is all-zero and gets the floor scale
    if (!w_scale || (K > 0 && (!blocks || !wq))) return W8A8_ERR_INVALID_ARG;
    if (!aligned16(blocks) || !aligned16(wq) || !aligned16(w_scale)) return W8A8_ERR_ALIGN;
    const int rows_per_wg = kThreads / 64;
    int64_t grid = (N + rows_per_wg - 1) / rows_per_wg;
    const int64_t cap = 8LL * device_cu_count();
    if (grid > cap) grid = cap;
    const int64_t row_bytes = (K / 32) * 34;
    if (row_bytes <= kMaxRowBytes) {
        const int row_stage = (int)((row_bytes + 15 + 15) / 16 * 16);
        const size_t lds = (size_t)row_stage * rows_per_wg;
        const int64_t steps = (K / 32 + 7) / 8;  // 8-block steps per row
        const uint8_t *b8 = static_cast<const uint8_t *>(blocks);
        uint8_t *q8 = static_cast<uint8_t *>(wq);
#define W8A8_GGUF_REG(QT, NS)                                                                                   \
    do {                                                                                                        \
        if (K / 32 == 8 * (NS))                                                                                 \
            gguf_a8_requant_reg_kernel<QT, NS, true><<<(int)grid, kThreads, lds, stream>>>(                     \
                b8, (uint32_t)total, (int)N, (int)K, row_stage, q8, w_scale);                                   \
        else                                                                                                    \
            gguf_a8_requant_reg_kernel<QT, NS, false><<<(int)grid, kThreads, lds, stream>>>(                    \
                b8, (uint32_t)total, (int)N, (int)K, row_stage, q8, w_scale);                                   \
    } while (0)
        if (steps <= 16) {  // K <= 4096: register-resident rows
            if (qtype == W8A8_INT8) {
                if (steps <= 4) W8A8_GGUF_REG(W8A8_INT8, 4);
                else if (steps <= 8) W8A8_GGUF_REG(W8A8_INT8, 8);
                else if (steps <= 12) W8A8_GGUF_REG(W8A8_INT8, 12);
                else W8A8_GGUF_REG(W8A8_INT8, 16);
            } else {
                if (steps <= 4) W8A8_GGUF_REG(W8A8_FP8_E4M3, 4);
                else if (steps <= 8) W8A8_GGUF_REG(W8A8_FP8_E4M3, 8);
                else if (steps <= 12) W8A8_GGUF_REG(W8A8_FP8_E4M3, 12);
                else W8A8_GGUF_REG(W8A8_FP8_E4M3, 16);
            }
            return launch_status();
        }
#undef W8A8_GGUF_REG
        if (qtype == W8A8_INT8)
            gguf_a8_requant_row_kernel<W8A8_INT8><<<(int)grid, kThreads, lds, stream>>>(
                static_cast<const uint8_t *>(blocks), (uint32_t)total, (int)N, (int)K, row_stage,
                static_cast<uint8_t *>(wq), w_scale);
        else
            gguf_a8_requant_row_kernel<W8A8_FP8_E4M3><<<(int)grid, kThreads, lds, stream>>>(
                static_cast<const uint8_t *>(blocks), (uint32_t)total, (int)N, (int)K, row_stage,
                static_cast<uint8_t *>(wq), w_scale);
        return launch_status();
    }
    if (qtype == W8A8_INT8)
        gguf_a8_requant_kernel<W8A8_INT8><<<(int)grid, kThreads, 0, stream>>>(
            static_cast<const uint8_t *>(blocks), (uint32_t)total, (int)N, (int)K, static_cast<uint8_t *>(wq), w_scale);
    else
        gguf_a8_requant_kernel<W8A8_FP8_E4M3><<<(int)grid, kThreads, 0, stream>>>(
            static_cast<const uint8_t *>(blocks), (uint32_t)total, (int)N, (int)K, static_cast<uint8_t *>(wq), w_scale);
    return launch_status();
}
