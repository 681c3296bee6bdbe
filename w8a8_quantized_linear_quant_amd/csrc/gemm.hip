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
//  * Persistent: one 256-thread workgroup per CU walks 256x256 output tiles
//    (or 256x192 where 256-wide tiles would leave a partial last round),
//    4 waves in a 2x2 grid, each wave a 128x128 sub-tile held as 8x8 blocks
//    of 16x16 accumulators (v_mfma_i32_16x16x64_i8) or, for e4m3, 4x4 blocks
//    of 32x32 (v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales): 256
//    accumulator registers per lane, one wave per SIMD.
//  * Both operands are K-contiguous ("NT"), so every lane's MFMA fragment is
//    a contiguous 16- or 32-byte run of one row.  The weight is the MFMA's A
//    operand and the activations its B operand, so each lane ends up holding
//    four consecutive output columns of one row.
//  * K goes HBM -> LDS in BK-byte stages through a ring of NST buffers with
//    buffer_load_dwordx4 ... lds (no register staging): int8 128-byte stages
//    in a ring of two (every load instruction reads whole 128-byte lines),
//    e4m3 64-byte stages in a ring of four.  The ring runs ahead across tile
//    boundaries.  Buffer loads past num_records
//    read zero, which covers ragged M/N tails and (with an out-of-range
//    offset) the ragged K tail.
//  * Within a stage, 16-byte chunks of each row are XOR-swizzled by the row
//    index so the fragment reads of consecutive rows hit distinct banks.
//  * Tiles are numbered so that the workgroups of one XCD (hardware sends
//    workgroup i to XCD i % 8) share operand panels in that XCD's L2.
//  * The epilogue scales, adds the bias (one FMA per value), packs to bf16
//    and stages each 32-row slice of a wave's sub-tile through LDS so that it
//    leaves as 16-byte stores covering 256-byte row segments.
#include <type_traits>
#include <utility>

#include <atomic>

#include "../../include/w8a8_probe.h"
#include "internal.hpp"

namespace w8a8 {
namespace {

constexpr int BM = 256;  // tile height along M (the tile width along N is a kernel parameter)
constexpr int kThreads = 256;
#ifndef W8A8_GEMM_GROUP_M
#define W8A8_GEMM_GROUP_M 4
#endif
constexpr int kGroupM = W8A8_GEMM_GROUP_M;  // tile-ordering group height
constexpr int kXcds = 8;

constexpr int kOutWaveBytes = 32 * 256;    // epilogue staging per wave
constexpr int kMaxRpStaged = 32;           // largest rank whose low-rank operands are staged in LDS

// Stage geometry: BK bytes of K per LDS stage, a ring of NST stage buffers.
// int8 takes 128-byte stages in a ring of two: each LDS-DMA instruction then
// reads 8 rows x one whole 128-byte line, where 64-byte stages read 16 rows x
// half a line; the vector memory path moves the same bytes ~7% faster as
// whole lines (M4096 N12288 K3072: 112.3 vs 121.2 us per launch).  e4m3
// keeps 64-byte stages in a ring of four, which measured faster for it
// (257.5 vs 263.7 us at M8192 N12288 K3072).
template <int BK_, int NST_>
struct StageGeo {
    static constexpr int BK = BK_;
    static constexpr int NST = NST_;
    static constexpr int kOpBytes = 256 * BK;          // one operand tile per stage
    static constexpr int kStageBytes = 2 * kOpBytes;   // X tile then W tile
    static constexpr int kChunks = BK / 16;            // 16-byte chunks per row
    static constexpr int kRowsPerLoad = 64 / kChunks;  // rows one wave-wide 1 KB load covers
    static constexpr int kLoadsPerOp = 64 / kRowsPerLoad;   // per wave and operand: 64 rows (of 256)
    static constexpr int kLoadsPerStage = 2 * kLoadsPerOp;  // the most a stage issues per wave
    static constexpr int kImmLoads = kLoadsPerOp < 4 ? kLoadsPerOp : 4;  // loads per M0 value (imm < 4 KB)
    static_assert(NST >= 2 && NST <= 4, "2..4 LDS stages");
    static_assert(NST * kStageBytes + 4 * kOutWaveBytes <= 160 * 1024, "LDS budget");
    static_assert((NST - 1) * kLoadsPerStage <= 63, "vmcnt range");
};
template <int QT>
using Geo = StageGeo<128, 2>;

typedef __attribute__((address_space(3))) void *lds_ptr_t;

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// in 6:4, lgkmcnt in 11:8; a field at its maximum does not wait).  Issued
// with __builtin_amdgcn_s_waitcnt, unlike inline asm, they enter the
// compiler's model of the outstanding counters, so it adds no waits of its
// own for what they already cover.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitLgkm0 = 15 | (3 << 14) | (7 << 4);

// XOR swizzle of the 16-byte chunk index by row, chosen so that the fragment
// reads of 16 consecutive rows (same logical chunk) spread over distinct bank
// groups whether the LDS serves 8 or 16 lanes of a 128-bit read per cycle.
// It depends on row % 16 only, so it is the same for every 32-row block.
template <int kChunks>
__device__ __forceinline__ int swz(int row) {
    if constexpr (kChunks == 8) return (row & 7) ^ ((row >> 3) & 1);
    else return ((row >> 1) ^ (row >> 2)) & 3;
}

// Even spread of `total` items over `groups` slots: slot g takes items
// spread_first(g) .. + spread_count(g) - 1.  The int8 stage places its next-
// stage fragment reads and its refill loads this way among its groups of 4
// MFMAs.
constexpr int spread_first(int g, int total, int groups) { return g * total / groups; }
constexpr int spread_count(int g, int total, int groups) { return (g + 1) * total / groups - g * total / groups; }

struct TileCoord {
    int m0, n0;
};

template <int BNT>
__device__ __forceinline__ TileCoord tile_coord(int tile, int tiles_m, int tiles_n) {
    const int nt = tiles_m * tiles_n;
    // XCD-major renumbering: hardware sends workgroup b to XCD b % 8, and a
    // persistent workgroup b takes tiles b, b + grid, ... (grid a multiple of
    // 8 when it is the CU count); give each XCD a contiguous range of logical
    // tiles so that the workgroups of one XCD share operand panels in its L2.
    const int per = nt / kXcds;
    const int t = tile < per * kXcds ? (tile % kXcds) * per + tile / kXcds : tile;
    // grouped order: kGroupM tile-rows advance together along N
    const int group = kGroupM * tiles_n;
    const int g = t / group;
    const int first_m = g * kGroupM;
    const int gm = min(tiles_m - first_m, kGroupM);
    const int in = t - g * group;
    TileCoord c;
    c.m0 = (first_m + in % gm) * BM;
    c.n0 = (in / gm) * BNT;
    return c;
}

// u . l2^T added to a 32x32 output block (rows n of l2, columns m of u) on
// the bf16 MFMA, u as hi + lo bf16 halves; C layout as the 8-bit product.
__device__ __forceinline__ v16f low_rank_add(const GemmArgs &p, v16f v, int nbase, int mbase, int lrow, int half) {
    const int nrow = nbase + lrow, m = mbase + lrow;
    for (int ks = 0; ks < p.rp; ks += 16) {
        const int j0 = ks + half * 8;
        uint16_t ta[8];
        if (nrow < p.N && (p.r & 7) == 0 && j0 + 8 <= p.r) {
            *reinterpret_cast<v4u *>(ta) = *reinterpret_cast<const v4u *>(p.l2 + (size_t)nrow * p.r + j0);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) ta[i] = (nrow < p.N && j0 + i < p.r) ? p.l2[(size_t)nrow * p.r + j0 + i] : 0;
        }
        const v8bf a = __builtin_bit_cast(v8bf, ta);
        v4u zh = {0u, 0u, 0u, 0u}, zl = {0u, 0u, 0u, 0u};
        if (m < p.M) {
            zh = *reinterpret_cast<const v4u *>(p.uhi + (size_t)m * p.rp + j0);
            zl = *reinterpret_cast<const v4u *>(p.ulo + (size_t)m * p.rp + j0);
        }
        v = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(v8bf, zh), v, 0, 0, 0);
        v = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(v8bf, zl), v, 0, 0, 0);
    }
    return v;
}


// The same for a 16x16 block (16x16x32 bf16 MFMA; lane l holds l2 row
// nbase + (l & 15) and u row mbase + (l & 15), rank columns 8 (l >> 4) + 0..7
// of each 32-column step; C layout as the int8 product).
__device__ __forceinline__ v4f low_rank_add16(const GemmArgs &p, v4f v, int nbase, int mbase, int brow, int lane) {
    const int nrow = nbase + brow, m = mbase + brow;
    const int jq = (lane >> 4) * 8;
    for (int ks = 0; ks < p.rp; ks += 32) {
        const int j0 = ks + jq;
        uint16_t ta[8];
        if (nrow < p.N && (p.r & 7) == 0 && j0 + 8 <= p.r) {
            *reinterpret_cast<v4u *>(ta) = *reinterpret_cast<const v4u *>(p.l2 + (size_t)nrow * p.r + j0);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) ta[i] = (nrow < p.N && j0 + i < p.r) ? p.l2[(size_t)nrow * p.r + j0 + i] : 0;
        }
        const v8bf a = __builtin_bit_cast(v8bf, ta);
        v4u zh = {0u, 0u, 0u, 0u}, zl = {0u, 0u, 0u, 0u};
        if (m < p.M && j0 < p.rp) {
            zh = *reinterpret_cast<const v4u *>(p.uhi + (size_t)m * p.rp + j0);
            zl = *reinterpret_cast<const v4u *>(p.ulo + (size_t)m * p.rp + j0);
        }
        v = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(v8bf, zh), v, 0, 0, 0);
        v = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(v8bf, zl), v, 0, 0, 0);
    }
    return v;
}

// TAIL: K is not a multiple of BK * NST, so some stages reach past K and
// need per-lane range checks; otherwise every stage is whole and the stage's
// K offset travels in the instruction's scalar offset.
// BNT: tile width along N, 256 (wave tiles 128 x 128) or 192 (128 x 96, for
// shapes whose 256-wide tiles would leave the last round of CUs half idle;
// bf16 epilogue only).
template <int QT, int EPI, bool TAIL, int BNT>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs p, int tiles_m, int tiles_n) {
    static_assert(BNT == 256 || (BNT == 192 && EPI == kEpiBf16), "192-wide tiles: bf16 epilogue only");
    using G = Geo<QT>;
    constexpr int BK = G::BK, NST = G::NST, kOpBytes = G::kOpBytes, kStageBytes = G::kStageBytes;
    constexpr int kChunks = G::kChunks, kRowsPerLoad = G::kRowsPerLoad, kLoadsPerOp = G::kLoadsPerOp;
    constexpr int kImmLoads = G::kImmLoads;
    static_assert(EPI != kEpiLowRank32 || NST != 2 || kStageBytes >= 3 * 256 * kMaxRpStaged * 2,
                  "two-stage ring: u and l2 share the last stage's buffer");
    constexpr int kWN = BNT / 2;                 // wave tile width along N
    constexpr int kRowsW = BNT / 4;              // weight rows each wave loads per stage
    constexpr int kLoadsW = kRowsW / kRowsPerLoad;
    constexpr int kLoads = kLoadsPerOp + kLoadsW;  // loads per wave and stage
    static_assert(kRowsW % kRowsPerLoad == 0, "whole weight loads per wave");
    // One distinct array per stage, so the compiler can tell the LDS-DMA writes
    // into one stage from the fragment reads of another and does not wait for
    // the former before the latter.
    __shared__ __attribute__((aligned(1024))) uint8_t lds0[kStageBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[kStageBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t lds2[NST > 2 ? kStageBytes : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t lds3[NST > 3 ? kStageBytes : 16];
    // Epilogue staging: per wave 32 rows x 128 bf16 columns (256 B rows).
    __shared__ __attribute__((aligned(1024))) uint8_t obuf[EPI == kEpiI32 ? 16 : 4 * kOutWaveBytes];
    auto buf = [&](auto s) -> uint8_t * {
        constexpr int S = decltype(s)::value;
        if constexpr (S == 0) return lds0;
        else if constexpr (S == 1) return lds1;
        else if constexpr (S == 2) return lds2;
        else return lds3;
    };

    const int lane = threadIdx.x & 63;
    // wave index as a scalar, so LDS addresses derived from it stay in SGPRs
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int K = p.K, M = p.M, N = p.N;
    const int ntiles = tiles_m * tiles_n;
    const int ktiles = (K + BK - 1) / BK;
    // Every tile runs a multiple of NST stages; stages past the end of K load
    // out-of-range offsets (zeros) and add nothing.  This keeps the loop free
    // of branches and the LDS ring aligned to the start of every tile.
    const int kt_end = (ktiles + NST - 1) / NST * NST;

    // Global -> LDS mapping: wave w fills rows [64w, 64w+64) of each operand
    // tile, kRowsPerLoad rows (1 KB) per instruction; lane l lands at LDS byte
    // 16 l of that KB: row l / kChunks, physical chunk l % kChunks, which holds
    // logical chunk (l % kChunks) ^ swz(row).
    // Loads 0 .. kLoadsPerOp - 1 of a stage fill the wave's 64 activation rows,
    // the rest its kRowsW weight rows.
    int goff[kLoads], gcol[kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
        const int i = j < kLoadsPerOp ? j : j - kLoadsPerOp;
        const int row = (j < kLoadsPerOp ? wave * 64 : wave * kRowsW) + i * kRowsPerLoad + lane / kChunks;
        const int c = (lane % kChunks) ^ swz<kChunks>(row);
        gcol[j] = c * 16;
        // the instruction's immediate offset (i KB, see load_part) is added to
        // the global address as well as to the LDS address; take it back out
        goff[j] = row * K + c * 16 - (i % kImmLoads) * 1024;
    }

    // ---- load cursor: the stage ring runs ahead across tile boundaries, so
    // the next tile's first stages are in flight during this tile's epilogue.
    int ld_tile = blockIdx.x, ld_kt = 0;
    __amdgpu_buffer_rsrc_t rx, rw;
    auto set_desc = [&]() {
        // Descriptors start at the tile's first row; rows past M (N) fall
        // outside num_records and read as zero.  Past the last tile every
        // record is out of range, so the ring keeps its constant load count.
        int rows_x = 0, rows_w = 0;
        size_t bx = 0, bw = 0;
        if (ld_tile < ntiles) {
            const TileCoord c = tile_coord<BNT>(ld_tile, tiles_m, tiles_n);
            rows_x = min(M - c.m0, BM);
            rows_w = min(N - c.n0, BNT);
            bx = (size_t)c.m0 * K;
            bw = (size_t)c.n0 * K;
        }
        rx = __builtin_amdgcn_make_buffer_rsrc((void *)(p.xq + bx), (short)0, rows_x * K, kBufferRsrcWord3);
        rw = __builtin_amdgcn_make_buffer_rsrc((void *)(p.wq + bw), (short)0, rows_w * K, kBufferRsrcWord3);
    };
    set_desc();
    // Loads of one stage, issued in NP parts (part P of NP) so that their
    // issue spreads over the k-steps of the stage being multiplied.
    // One LDS-DMA instruction writes 1 KB at M0 + immediate offset + 16 * lane.
    // Loads are grouped so that consecutive ones share M0 and differ only in
    // the immediate offset (i KB, below 4 KB): rewriting M0 between LDS-DMA
    // instructions stalls the issuing wave.
    auto load_part = [&](uint8_t *stage, auto part_c, auto np_c) {
        constexpr int P = decltype(part_c)::value, NP = decltype(np_c)::value;
        constexpr int lo = P * kLoads / NP, hi = (P + 1) * kLoads / NP;
        const int k0 = ld_kt * BK;
        const bool full = !TAIL || k0 + BK <= K;
        [&]<int... J>(std::integer_sequence<int, J...>) {
            (([&] {
                 constexpr int j = lo + J;
                 constexpr bool kX = j < kLoadsPerOp;
                 constexpr int i = kX ? j : j - kLoadsPerOp;
                 constexpr int grp = i / kImmLoads, imm = (i % kImmLoads) * 1024;
                 uint8_t *m0 = stage + (kX ? wave * 64 * BK : kOpBytes + wave * kRowsW * BK) + grp * kImmLoads * 1024;
                 if constexpr (TAIL) {
                     const int o = full ? goff[j] + k0 : (k0 + gcol[j] < K ? goff[j] + k0 : kOobOffset);
                     __builtin_amdgcn_raw_ptr_buffer_load_lds(kX ? rx : rw, (lds_ptr_t)m0, 16, o, 0, imm, 0);
                 } else {
                     // per-lane offset fixed for the whole kernel, stage offset scalar
                     // (the array element goes through a local: passed to the
                     // builtin directly, it makes the host pass drop the
                     // kernel's launch stub without a diagnostic)
                     const int o = goff[j];
                     __builtin_amdgcn_raw_ptr_buffer_load_lds(kX ? rx : rw, (lds_ptr_t)m0, 16, o, k0, imm, 0);
                 }
             }()),
             ...);
        }(std::make_integer_sequence<int, hi - lo>{});
    };
    // Move the load cursor to the next stage (outside the interleaved regions:
    // crossing into the next tile branches and recomputes the descriptors).
    auto advance_cursor = [&]() {
        if (++ld_kt == kt_end) {
            ld_kt = 0;
            ld_tile += gridDim.x;
            set_desc();
        }
    };

    // MFMA shapes.  int8: v_mfma_i32_16x16x64_i8, the wave's 128x128 as 8x8
    // blocks of 16x16 (4 accumulators per lane each).  It does the work of
    // the 32x32x32 form with half the accumulator traffic per product (4
    // accumulators read and written per 16K products instead of 16 per 32K),
    // and sustains ~22% more int8
    // operations per second than it on this chip under its power limit
    // (measured with both in a pure MFMA loop on the workload's codes).
    // e4m3: v_mfma_scale_f32_32x32x64_f8f6f4, 4x4 blocks of 32x32 (16 each).
    // Both take 64 bytes of K per lane row and instruction: one k-step per
    // 64-byte stage.
    constexpr bool kInt8 = QT == W8A8_INT8;
    constexpr int kBlk = kInt8 ? 16 : 32;  // edge of one MFMA output block
    constexpr int kNB = 128 / kBlk;        // blocks along the wave tile's 128 activation rows
    constexpr int kNBn = kWN / kBlk;       // blocks along its kWN output columns (weight rows)
    constexpr int kQuads = kBlk * kBlk / 64 / 4;  // groups of 4 consecutive columns per lane and block
    constexpr int KSTEPS = BK / 64;
    static_assert(KSTEPS >= 1, "stage too small for one MFMA k-step");
    static_assert(!kInt8 || KSTEPS == 1 || NST == 2, "int8 with several k-steps per stage: two-stage ring only");
    typedef typename std::conditional<kInt8, v4i, v8i>::type frag_t;
    typedef typename std::conditional<kInt8, v4i, v16f>::type acc_t;  // one block's accumulators
    typedef acc_t blk_t;
    const int lrow = lane & 31, half = lane >> 5;
    const int lsw = swz<kChunks>(lrow);

    acc_t acc[kNBn][kNB];  // [weight block nb][activation block mb]
    auto blk = [&](int nb, int mb) -> blk_t { return acc[nb][mb]; };
    frag_t fa[2][kNBn], fb[2][kNB];

    // int8: lane l reads row l & 15 of each 16-row block, 16-byte chunk
    // l >> 4 (the chunk XOR-swizzled by the row).  read_frags adds the lane
    // offset to the stage's base through an opaque copy, so the compiler
    // does not keep a precomputed address per stage buffer alive across the
    // loop.
    auto foff = [&](int kk) { return (lane & 15) * BK + (((kk * 4 + (lane >> 4)) ^ swz<kChunks>(lane & 15)) << 4); };
    auto read_frags = [&](const uint8_t *stage, int kk, frag_t *af, frag_t *bf) {
        const uint8_t *xs = stage + (wm * 128) * BK;            // X rows of this wave
        const uint8_t *ws = stage + kOpBytes + (wn * kWN) * BK;  // W rows of this wave
        if constexpr (kInt8) {
            int off = foff(kk);
            asm volatile("" : "+v"(off));
#pragma unroll
            for (int b = 0; b < kNBn; ++b) af[b] = *reinterpret_cast<const v4i *>(ws + b * 16 * BK + off);
#pragma unroll
            for (int b = 0; b < kNB; ++b) bf[b] = *reinterpret_cast<const v4i *>(xs + b * 16 * BK + off);
        } else {
            const int c0 = kk * 4 + half * 2;
            const int off0 = lrow * BK + ((c0 ^ lsw) << 4);
            const int off1 = lrow * BK + (((c0 + 1) ^ lsw) << 4);
#pragma unroll
            for (int b = 0; b < kNBn; ++b) {
                const v4i lo = *reinterpret_cast<const v4i *>(ws + b * 32 * BK + off0);
                const v4i hi = *reinterpret_cast<const v4i *>(ws + b * 32 * BK + off1);
                af[b] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const v4i lo = *reinterpret_cast<const v4i *>(xs + b * 32 * BK + off0);
                const v4i hi = *reinterpret_cast<const v4i *>(xs + b * 32 * BK + off1);
                bf[b] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
        }
    };

    // int8: one of the kNBn + kNB fragments of a stage (weight blocks first,
    // then activation blocks) into set af / bf; `lp` is the stage's base plus
    // this lane's offset (one address per stage, the blocks at immediate
    // offsets).
    auto read_frag_i8 = [&](const uint8_t *lp, auto idx_c, frag_t *af, frag_t *bf) {
        constexpr int I = decltype(idx_c)::value;
        if constexpr (kInt8) {
            if constexpr (I < kNBn) af[I] = *reinterpret_cast<const v4i *>(lp + kOpBytes + (wn * kWN + I * 16) * BK);
            else bf[I - kNBn] = *reinterpret_cast<const v4i *>(lp + (wm * 128 + (I - kNBn) * 16) * BK);
        }
    };

    // e4m3: half I % 2 of fragment I / 2 of a k-step (weight blocks first,
    // then activation blocks), 16 of the fragment's 32 bytes, into set af / bf.
    // lp0 / lp1: the stage's base plus this lane's offset of either half.
    auto read_half_f8 = [&](const uint8_t *lp0, const uint8_t *lp1, auto idx_c, frag_t *af, frag_t *bf) {
        constexpr int I = decltype(idx_c)::value;
        if constexpr (!kInt8) {
            constexpr int f = I / 2, h = I % 2;
            const uint8_t *lp = h ? lp1 : lp0;
            v4i v;
            if constexpr (f < kNBn) v = *reinterpret_cast<const v4i *>(lp + kOpBytes + (wn * kWN + f * 32) * BK);
            else v = *reinterpret_cast<const v4i *>(lp + (wm * 128 + (f - kNBn) * 32) * BK);
            frag_t &dst = f < kNBn ? af[f < kNBn ? f : 0] : bf[f < kNBn ? 0 : f - kNBn];
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[4 * h + e] = v[e];
        }
    };

    // FIRST: the tile's first k-step, which starts the accumulators from an
    // inline-constant zero instead of zeroing 256 registers beforehand.
    // One int8 MFMA, accumulator tied to its AGPRs.  Written as inline asm:
    // with the builtin, the register allocator kept 64 separate 4-register
    // accumulators in fixed registers only in part, and rotated the rest
    // through other AGPRs and VGPRs inside the K loop (untied MFMAs, copies
    // and s_nop waits).  The compiler does not see these as MFMAs, so the
    // K loop's consumers of their results are covered explicitly: the
    // loop's own MFMAs read an accumulator 64 MFMAs after writing it, and the
    // epilogue starts after explicit wait states.  FIRST starts from zero
    // (inline constant) instead of the accumulator.
    auto mfma_i8 = [&](v4i &c, const v4i &a, const v4i &b, auto first_c) {
        if constexpr (decltype(first_c)::value)
            asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, 0" : "=a"(c) : "v"(a), "v"(b));
        else
            asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    };
    // One e4m3 MFMA with unit block scales (E8M0 127 = 2^0), written as inline
    // asm for the same reason and tied the same way: as a builtin the
    // scheduler moved the MFMAs past the explicit order of the K loop (even
    // above the stage barrier) and issued a k-step's MFMAs back to back.
    const int scale_one = 127;
    auto mfma_f8 = [&](v16f &c, const v8i &a, const v8i &b, auto first_c) {
        if constexpr (decltype(first_c)::value)
            asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %3 op_sel_hi:[0,0,0]"
                         : "=a"(c)
                         : "v"(a), "v"(b), "v"(scale_one));
        else
            asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0]"
                         : "+a"(c)
                         : "v"(a), "v"(b), "v"(scale_one));
    };
    // MFMAs per k-step.  Each k-step's memory instructions are placed among
    // its MFMAs in an explicit program order (run_stage) so that their issue
    // (the LDS-DMA loads especially) overlaps MFMA execution instead of
    // stalling the wave in front of the matrix pipe.
    constexpr int kMfmas = kNBn * kNB;

    // Within a stage the fragments of k-step kk+1 are read while the MFMAs of
    // step kk run.  At the last step of a stage: wait until the next stage
    // has landed and every wave is done with this one (barrier), refill this
    // buffer with the stage NST ahead, read the first fragments of the next
    // stage, then issue the last MFMAs.
    // Stage kt lives in buffer kt % NST.  While stage kt is multiplied, the
    // loads of stage kt + NST - 1 go into the buffer stage kt - 1 used (free
    // since the barrier that ended stage kt - 1), one part per k-step.
    // Within a stage the fragments of k-step kk+1 are read while the MFMAs of
    // step kk run.  Before the last k-step: wait until stage kt+1 has landed
    // and every wave is done reading stage kt (barrier), then read the first
    // fragments of stage kt+1 and issue the last MFMAs of stage kt.
    // Two-stage ring (NST == 2): a stage's buffer is free only after the
    // barrier of its last k-step, so the whole refill (the stage two ahead,
    // into the buffer just freed) is issued in that k-step, and the wait at
    // the end of the next stage is for everything in flight.
    constexpr int kParts = KSTEPS;
    constexpr int kPerPart = kLoads / kParts;
    static_assert(kLoads % kParts == 0, "loads split evenly over k-steps");
    constexpr int kLoadsEarly = NST == 2 ? 0 : kPerPart;   // loads per k-step before the last
    constexpr int kLoadsLast = NST == 2 ? kLoads : kPerPart;  // loads in the last k-step
    // loads still allowed in flight when stage kt+1 must be complete: stages
    // kt+2 .. kt+NST-2 whole, and the parts of stage kt+NST-1 issued so far
    constexpr int kPending = NST == 2 ? 0 : (NST - 3) * kLoads + (kParts - 1) * kPerPart;
    constexpr int kPendingDeferred = NST == 2 ? 0 : kPending - (kParts - 1) * kPerPart;
    // e4m3 low-rank epilogue.  Buffers of the low-rank operands: u (hi, then lo) in the tile's last
    // stage's buffer, l2 in the buffer whose refill that stage defers (with
    // two stages the same 64 KB buffer, l2 after u's 32 KB).
    auto lr_ubuf = [&]() { return buf(std::integral_constant<int, NST - 1>{}); };
    auto lr_lbuf = [&]() {
        if constexpr (NST == 2) return buf(std::integral_constant<int, 1>{}) + 2 * 256 * kMaxRpStaged * 2;
        else return buf(std::integral_constant<int, NST - 2>{});
    };
    // buffer of the refill a tile's last stage defers (low-rank epilogue)
    constexpr int kDeferBuf = NST == 2 ? 1 : NST - 2;
    // e4m3 low-rank epilogue (r of 16 or 32): the tile's low-rank operands go to
    // the two ring buffers that the tile's last stage frees (its own, whose
    // fragments every wave read before the stage's barrier, and the one whose
    // refill it defers): u of the tile's 256 rows (hi, then lo, [256][rp]
    // bf16 each) and l2 of its 256 columns ([256][r], r == rp); every wave
    // fetches a quarter of each.  Issued right after that stage's barrier, so
    // the loads are in flight while its MFMAs run.  lr_mw / lr_nw: the tile's
    // wave origin, set by the tile loop.
    int lr_mw = 0, lr_nw = 0;
    auto lowrank_dma = [&]() {
        uint8_t *ub = lr_ubuf();
        uint8_t *lb = lr_lbuf();
        const int half_bytes = 256 * p.rp * 2;
        {
            const int n0 = lr_nw - wn * kWN;
            const int cols_in = min(N - n0, 256);
            const __amdgpu_buffer_rsrc_t rw2 = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(p.l2 + (size_t)n0 * p.r), (short)0, cols_in * p.r * 2, kBufferRsrcWord3);
            for (int i = 0; i < p.r / 8; ++i) {
                const int off = wave * 128 * p.r + i * 1024;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rw2, (lds_ptr_t)(lb + off), 16, off + lane * 16, 0, 0, 0);
            }
        }
        const int m0 = lr_mw - wm * 128;
        const int rows_in = min(M - m0, 256);
        const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(p.uhi + (size_t)m0 * p.rp), (short)0, rows_in * p.rp * 2, kBufferRsrcWord3);
        const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(p.ulo + (size_t)m0 * p.rp), (short)0, rows_in * p.rp * 2, kBufferRsrcWord3);
        for (int i = 0; i < p.rp / 8; ++i) {  // 128 rp bytes per wave and half, 1 KB per load
            const int off = wave * 128 * p.rp + i * 1024;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rh, (lds_ptr_t)(ub + off), 16, off + lane * 16, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (lds_ptr_t)(ub + half_bytes + off), 16, off + lane * 16, 0,
                                                     0, 0);
        }
    };
    // int8 low-rank epilogue (kLrReg): no ring buffer is held across the
    // epilogue, so every refill goes out on time.  l2 of the tile's 256
    // columns comes by LDS-DMA into the second half of the waves' staging
    // areas (wave w: tile columns 64w .. 64w + 63, [64][r] bf16) with the
    // tile's other epilogue inputs, two stages before the epilogue; u comes
    // from global memory, during the tile's last k-step, into the register
    // set that k-step would fill with the next stage's fragments: those reads
    // would be dead (the next tile re-reads its stage 0 after the epilogue).
    constexpr bool kLrReg = EPI == kEpiLowRank32 && kInt8;
    constexpr int kLrL2Off = kOutWaveBytes / 2;
    constexpr int kPLast = ((NST - 1) * KSTEPS + KSTEPS - 1) & 1;  // fragment set the tile's last k-step multiplies
    static_assert(64 * kMaxRpStaged * 2 <= kOutWaveBytes - kLrL2Off, "l2 quarter fits the staging area's second half");
    auto lowrank_l2_dma = [&](int n0) {  // n0: the tile's first column
        const int cols_in = min(N - n0, 256);
        const __amdgpu_buffer_rsrc_t rw2 = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(p.l2 + (size_t)n0 * p.r), (short)0, cols_in * p.r * 2, kBufferRsrcWord3);
        uint8_t *dst = obuf + wave * kOutWaveBytes + kLrL2Off;
        for (int i = 0; i < p.r / 8; ++i)  // 64 columns x r bf16 = 128 r bytes per wave, 1 KB per load
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw2, (lds_ptr_t)(dst + i * 1024), 16,
                                                     wave * 128 * p.r + i * 1024 + lane * 16, 0, 0, 0);
    };
    // u of the wave's 8 row blocks, hi into ah[mb] and lo into al[mb]: lane l
    // holds row 16 mb + (l & 15), rank columns 8 (l >> 4) .. + 7 (zero past
    // rp and for rows past M)
    auto lowrank_u_loads = [&](frag_t *ah, frag_t *al) {
        if constexpr (kLrReg) {
            const int m0 = lr_mw - wm * 128;
            const int rows_in = min(M - m0, 256);
            const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(p.uhi + (size_t)m0 * p.rp), (short)0, rows_in * p.rp * 2, kBufferRsrcWord3);
            const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(p.ulo + (size_t)m0 * p.rp), (short)0, rows_in * p.rp * 2, kBufferRsrcWord3);
            const int j0 = (lane >> 4) * 8;
#pragma unroll
            for (int mb = 0; mb < kNB; ++mb) {
                const int off = j0 < p.rp ? ((wm * 128 + mb * 16 + (lane & 15)) * p.rp + j0) * 2 : kOobOffset;
                ah[mb] = __builtin_bit_cast(frag_t, __builtin_amdgcn_raw_buffer_load_b128(rh, off, 0, 0));
                al[mb] = __builtin_bit_cast(frag_t, __builtin_amdgcn_raw_buffer_load_b128(rl, off, 0, 0));
            }
        }
    };
    // defer (the low-rank epilogue only, last stage of a tile): for e4m3 this
    // stage's refill -- the next tile's stage NST - 2 -- is issued after the
    // epilogue instead, so that its buffer can hold the low-rank operands
    // meanwhile; for int8 the stage's last k-step loads u into registers.
    auto run_stage = [&](auto sc, auto first_c, bool defer) {
        constexpr int S = decltype(sc)::value;
        constexpr bool FIRST = decltype(first_c)::value;
        constexpr bool kMayDefer = EPI == kEpiLowRank32 && !kInt8 && S == NST - 1;
        // int8 low-rank, the tile's last stage (`defer` then marks it)
        constexpr bool kLrRegLast = kLrReg && S == NST - 1;
        const bool issue = !kMayDefer || !defer;
        uint8_t *cur = buf(sc);
        uint8_t *nxt = buf(std::integral_constant<int, (S + 1) % NST>{});
        // NST >= 3: the buffer stage S - 1 used; two stages: this stage's own
        // (free after its last k-step's barrier)
        uint8_t *refill = buf(std::integral_constant<int, NST == 2 ? S : (S + NST - 1) % NST>{});
        [&]<int... KK>(std::integer_sequence<int, KK...>) {
            (([&] {
                 constexpr int kk = KK;
                 constexpr int P = (S * KSTEPS + kk) & 1;
                 constexpr bool kLast = kk + 1 == KSTEPS;
                 if constexpr (kLast) {
                     // without this stage's earlier parts in flight, fewer may remain
                     if (issue) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kPending));
                     else __builtin_amdgcn_s_waitcnt(waitcnt_vm(kPendingDeferred));
                     __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
                     // a bare barrier: __syncthreads() would add a release fence,
                     // i.e. a wait for every load in flight, prefetches included
                     asm volatile("s_barrier" ::: "memory");
                     __builtin_amdgcn_sched_barrier(0);
                     if constexpr (kMayDefer) {
                         if (defer) lowrank_dma();
                         __builtin_amdgcn_sched_barrier(0);
                     }
                     if constexpr (kLrRegLast) {
                         if (defer) lowrank_u_loads(fb[P ^ 1], fa[P ^ 1]);
                         __builtin_amdgcn_sched_barrier(0);
                     }
                 } else {
                     __builtin_amdgcn_sched_barrier(0);
                 }
                 if constexpr (kInt8) {
                     // kMfmas / 4 groups of 4 MFMAs (weight block nb = g / 2,
                     // activation blocks 4 (g % 2) .. + 3) in program order,
                     // each followed by its even share of the next k-step's
                     // kNBn + kNB fragment reads (into the other set; the next
                     // stage's first k-step after the barrier) and of the
                     // k-step's refill loads.  Spread over the MFMAs, the
                     // reads of the four waves leaving a barrier together do
                     // not reach the LDS at once.
                     constexpr int kGroups = kMfmas / 4, kReads = kNBn + kNB;
                     constexpr int kL = kLast ? kLoadsLast : kLoadsEarly;
                     constexpr int kPart0 = kLast ? 0 : kk;  // first load part of this k-step, in units of kL
                     int off = foff(kLast ? 0 : kk + 1);
                     asm volatile("" : "+v"(off));
                     const uint8_t *lp = (kLast ? nxt : cur) + off;
                     [&]<int... G>(std::integer_sequence<int, G...>) {
                         (([&] {
                              constexpr int g = G;
                              constexpr auto first = std::integral_constant<bool, FIRST && S == 0 && kk == 0>{};
#pragma unroll
                              for (int j = 0; j < 4; ++j)
                                  mfma_i8(acc[g / 2][(g % 2) * 4 + j], fa[P][g / 2], fb[P][(g % 2) * 4 + j], first);
                              [&]<int... R>(std::integer_sequence<int, R...>) {
                                  // (the registers hold u on the int8 low-rank tile's last k-step)
                                  if (!(kLrRegLast && kLast && defer))
                                      (read_frag_i8(lp, std::integral_constant<int, spread_first(g, kReads, kGroups) + R>{},
                                                    fa[P ^ 1], fb[P ^ 1]),
                                       ...);
                              }(std::make_integer_sequence<int, spread_count(g, kReads, kGroups)>{});
                              [&]<int... L>(std::integer_sequence<int, L...>) {
                                  if (issue)
                                      (load_part(refill,
                                                 std::integral_constant<int, kPart0 * kL + spread_first(g, kL, kGroups) + L>{},
                                                 std::integral_constant<int, kLoads>{}),
                                       ...);
                              }(std::make_integer_sequence<int, spread_count(g, kL, kGroups)>{});
                              __builtin_amdgcn_sched_barrier(0);
                          }()),
                          ...);
                     }(std::make_integer_sequence<int, kGroups>{});
                 } else {
                     // e4m3: the same explicit order with one MFMA per group
                     // (kMfmas 32x32x64 MFMAs per k-step) and the next k-step's
                     // fragments read as 16-byte halves.  Left to
                     // sched_group_barrier hints, the compiler issued a
                     // k-step's MFMAs back to back and every read and load
                     // after them, so the next k-step's first MFMA waited for
                     // the LDS.
                     constexpr int kGroups = kMfmas, kReads = 2 * (kNBn + kNB);
                     constexpr int kL = kLast ? kLoadsLast : kLoadsEarly;
                     constexpr int kPart0 = kLast ? 0 : kk;
                     constexpr int kNext = kLast ? 0 : kk + 1;
                     // the lane's offsets of the two halves, opaque to the
                     // compiler: with addresses it could trace to one stage
                     // buffer, it made some reads wait for this k-step's
                     // LDS-DMA loads into the other (vmcnt(0))
                     int off0 = lrow * BK + (((kNext * 4 + half * 2) ^ lsw) << 4);
                     int off1 = lrow * BK + (((kNext * 4 + half * 2 + 1) ^ lsw) << 4);
                     asm volatile("" : "+v"(off0), "+v"(off1));
                     const uint8_t *src = kLast ? nxt : cur;
                     const uint8_t *lp0 = src + off0, *lp1 = src + off1;
                     [&]<int... G>(std::integer_sequence<int, G...>) {
                         (([&] {
                              constexpr int g = G;
                              constexpr int nb = g / kNB, mb = g % kNB;
                              constexpr auto first = std::integral_constant<bool, FIRST && S == 0 && kk == 0>{};
                              if constexpr (!kInt8) mfma_f8(acc[nb][mb], fa[P][nb], fb[P][mb], first);
                              [&]<int... R>(std::integer_sequence<int, R...>) {
                                  (read_half_f8(lp0, lp1,
                                                std::integral_constant<int, spread_first(g, kReads, kGroups) + R>{},
                                                fa[P ^ 1], fb[P ^ 1]),
                                   ...);
                              }(std::make_integer_sequence<int, spread_count(g, kReads, kGroups)>{});
                              [&]<int... L>(std::integer_sequence<int, L...>) {
                                  if (issue)
                                      (load_part(refill,
                                                 std::integral_constant<int, kPart0 * kL + spread_first(g, kL, kGroups) + L>{},
                                                 std::integral_constant<int, kLoads>{}),
                                       ...);
                              }(std::make_integer_sequence<int, spread_count(g, kL, kGroups)>{});
                              __builtin_amdgcn_sched_barrier(0);
                          }()),
                          ...);
                     }(std::make_integer_sequence<int, kGroups>{});
                 }
             }()),
             ...);
        }(std::make_integer_sequence<int, KSTEPS>{});
        if (issue) advance_cursor();
    };
    static_assert(NST % 2 == 0 || KSTEPS % 2 == 0, "fragment parity must restart at each stage group");
    // stages FROM .. TO-1 of a group of NST
    auto run_stages = [&](auto from_c, auto to_c, auto first_c, bool defer) {
        constexpr int F = decltype(from_c)::value, T = decltype(to_c)::value;
        [&]<int... S>(std::integer_sequence<int, S...>) {
            (run_stage(std::integral_constant<int, F + S>{}, first_c, defer), ...);
        }(std::make_integer_sequence<int, T - F>{});
    };

    // Interior tiles: the row scales (128 f32) and bias (128 bf16) of this
    // wave's outputs go to the start of its staging area by LDS-DMA while the
    // tile's last stages are multiplied, so the epilogue does not open with a
    // global load queued behind the next tile's prefetches.  Lanes past the
    // 512 (256) bytes read out of range and write zeros after them.
    constexpr int kEpiSx = 0, kEpiBias = 1024;
    auto epi_dma = [&](int mw, int nw) {
        uint8_t *ob = obuf + wave * kOutWaveBytes;
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void *)(p.sx + mw), (short)0, 512, kBufferRsrcWord3);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(ob + kEpiSx), 16, lane * 16, 0, 0, 0);
        if (p.bias) {
            const __amdgpu_buffer_rsrc_t rb =
                __builtin_amdgcn_make_buffer_rsrc((void *)(p.bias + nw), (short)0, 256, kBufferRsrcWord3);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(ob + kEpiBias), 16, lane * 16, 0, 0, 0);
        }
    };

    // Prologue: stages 0 .. NST-2 in flight (0 and 1 with two stages), wait
    // for stage 0.
    constexpr int kPro = NST == 2 ? 2 : NST - 1;
    [&]<int... S>(std::integer_sequence<int, S...>) {
        ((load_part(buf(std::integral_constant<int, S>{}), std::integral_constant<int, 0>{},
                    std::integral_constant<int, 1>{}),
          advance_cursor()),
         ...);
    }(std::make_integer_sequence<int, kPro>{});
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kPro - 1) * kLoads) : "memory");
    asm volatile("s_barrier" ::: "memory");

    // bf16 epilogue of one tile: y = bf16(acc * sx[m] * sw (+ u . l2^T) + bias[n]).
    // Every lane holds, per output block, groups ("quads") of 4 consecutive
    // columns of one row:
    //   int8 (16x16 blocks): block (nb, mb), registers 0..3 -> row
    //     mb * 16 + (l & 15), columns nb * 16 + 4 (l >> 4) + 0..3;
    //   e4m3 (32x32 blocks): block (nb, mb), registers 4q..4q+3 -> row
    //     mb * 32 + (l & 31), columns nb * 32 + 8q + 4 (l >> 5) + 0..3.
    // Result rows go through this wave's LDS staging area (32 rows x 256 B,
    // 16-byte chunks XOR-swizzled by row) in four passes of 32 rows and leave
    // as 16-byte stores that cover whole 256-byte row segments.
    constexpr int kPassBlocks = 32 / kBlk;  // block rows per 32-row pass
    auto bf16_epilogue = [&](auto interior_c, int mw, int nw) {
        constexpr bool kIn = decltype(interior_c)::value;
        uint16_t *out = static_cast<uint16_t *>(p.out);
        uint8_t *ob = obuf + wave * kOutWaveBytes;
        // Re-derive the lane indices here so the staging addresses are not
        // hoisted out of the tile loop (they would stay live across the K
        // loop and spill).
        int el = lane;
        asm volatile("" : "+v"(el));
        const int brow = el & (kBlk - 1);  // the lane's row within a block
        const int cq = 4 * (el / kBlk);    // the lane's first column within a quad group
        constexpr bool kCol = EPI == kEpiColScale;
        float tm[kNB];
        uint2 bias2[kNBn][kQuads];
        v4f swc[kCol ? kNBn : 1][kCol ? kQuads : 1];  // per-channel weight scales of the lane's quads
        const float sw = kCol ? 1.0f : p.sw[0];
#pragma unroll
        for (int mb = 0; mb < kNB; ++mb) {
            const int m = mw + mb * kBlk + brow;
            if constexpr (kIn) tm[mb] = *reinterpret_cast<const float *>(ob + kEpiSx + (mb * kBlk + brow) * 4) * sw;
            else tm[mb] = m < M ? p.sx[m] * sw : 0.0f;
        }
        if constexpr (kCol) {
#pragma unroll
            for (int nb = 0; nb < kNBn; ++nb)
#pragma unroll
                for (int q = 0; q < kQuads; ++q) {
                    const int n = nw + nb * kBlk + 8 * q + cq;
                    if (kIn || ((N & 3) == 0 && n < N)) {
                        swc[nb][q] = *reinterpret_cast<const v4f *>(p.sw + n);
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i) swc[nb][q][i] = n + i < N ? p.sw[n + i] : 0.0f;
                    }
                }
        }
#pragma unroll
        for (int nb = 0; nb < kNBn; ++nb)
#pragma unroll
            for (int q = 0; q < kQuads; ++q) {
                const int n = nw + nb * kBlk + 8 * q + cq;
                uint2 b = make_uint2(0u, 0u);
                if (p.bias) {
                    if constexpr (kIn) {
                        b = *reinterpret_cast<const uint2 *>(ob + kEpiBias + (n - nw) * 2);
                    } else if ((N & 3) == 0 && n < N) {
                        b = *reinterpret_cast<const uint2 *>(p.bias + n);
                    } else {
                        uint32_t w[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) w[i] = n + i < N ? p.bias[n + i] : 0u;
                        b = make_uint2(w[0] | (w[1] << 16), w[2] | (w[3] << 16));
                    }
                }
                bias2[nb][q] = b;
            }
        // The bias as f32, one value per output column of the lane: unpacked
        // once per tile for int8 (4 columns per block), per use for e4m3 (16
        // per block, too many registers to hold).
        constexpr bool kBiasF32 = kInt8;
        float biasf[kBiasF32 ? kNBn : 1][kBiasF32 ? 4 * kQuads : 1];
        if constexpr (kBiasF32) {
#pragma unroll
            for (int nb = 0; nb < kNBn; ++nb)
#pragma unroll
                for (int q = 0; q < kQuads; ++q) {
                    biasf[nb][4 * q] = bf16_bits_to_f32(bias2[nb][q].x & 0xFFFFu);
                    biasf[nb][4 * q + 1] = bf16_bits_to_f32(bias2[nb][q].x >> 16);
                    biasf[nb][4 * q + 2] = bf16_bits_to_f32(bias2[nb][q].y & 0xFFFFu);
                    biasf[nb][4 * q + 3] = bf16_bits_to_f32(bias2[nb][q].y >> 16);
                }
        }
        auto bias_at = [&](int nb, int e) -> float {
            if constexpr (kBiasF32) return biasf[nb][e];
            const uint32_t w = (e & 2) ? bias2[nb][e / 4].y : bias2[nb][e / 4].x;
            return bf16_bits_to_f32((e & 1) ? w >> 16 : w & 0xFFFFu);
        };
        // plain epilogue: acc * (sx[m] sw) + bias[n] in one fused multiply-add
        constexpr bool kFma = EPI == kEpiBf16;
        constexpr bool kLr32 = EPI == kEpiLowRank32;
        constexpr bool kLrBatch = kLr32 && kInt8;
        uint8_t *ub = lr_ubuf();
        uint8_t *lb = lr_lbuf();
        const int half_bytes = 256 * p.rp * 2;
        if constexpr (kLr32 && !kLrBatch) {
            // e4m3: the tile's low-rank operands were issued at its last
            // stage (lowrank_dma)
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            asm volatile("s_barrier" ::: "memory");
        }
        // int8 low-rank: the l2 fragments of the wave's 8 column blocks (rows
        // n of l2, the lane's 8 of up to 32 rank columns; zero past r)
        v8bf al2[kLrBatch ? kNBn : 1];
        if constexpr (kLrBatch) {
            // from the second halves of the staging areas (lowrank_l2_dma,
            // landed and made visible by the last stages' waits and barriers);
            // every wave reads its l2 before any wave stages a pass there
            const int j0 = (el >> 4) * 8;
#pragma unroll
            for (int nb = 0; nb < kNBn; ++nb) {
                const int nl = wn * kWN + nb * 16 + brow;  // column within the tile
                al2[nb] = v8bf{};
                if (j0 < p.r)
                    al2[nb] = *reinterpret_cast<const v8bf *>(obuf + (nl >> 6) * kOutWaveBytes + kLrL2Off +
                                                             ((nl & 63) * p.r + j0) * 2);
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            asm volatile("s_barrier" ::: "memory");
        }
        // int8 low-rank: one pass's 16 blocks, dequantized with their bias
        // and then given u . l2^T
        v4f lrv[kLrBatch ? kPassBlocks : 1][kLrBatch ? kNBn : 1];
#pragma unroll
        for (int ps = 0; ps < 4; ++ps) {
            if constexpr (kLrBatch) {
                // Each block's accumulators leave the AGPRs once: converted,
                // scaled and biased in one FMA into the f32 operand C of the
                // 16x16x32 bf16 MFMA, which adds hi . l2^T and then
                // lo . l2^T (u as hi + lo).  The VALU work of one block runs
                // while the MFMAs of the block before it execute.
#pragma unroll
                for (int qb = 0; qb < kPassBlocks; ++qb) {
                    const int mb = ps * kPassBlocks + qb;
                    const v8bf uh = __builtin_bit_cast(v8bf, fb[kPLast ^ 1][mb]);
                    const v8bf ul = __builtin_bit_cast(v8bf, fa[kPLast ^ 1][mb]);
#pragma unroll
                    for (int nb = 0; nb < kNBn; ++nb) {
                        const blk_t c = blk(nb, mb);
                        v4f t;
#pragma unroll
                        for (int e = 0; e < 4; ++e) t[e] = __builtin_fmaf((float)c[e], tm[mb], bias_at(nb, e));
                        t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al2[nb], uh, t, 0, 0, 0);
                        lrv[qb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al2[nb], ul, t, 0, 0, 0);
                    }
                }
            }
#pragma unroll
            for (int qb = 0; qb < kPassBlocks; ++qb) {
                const int mb = ps * kPassBlocks + qb;
#pragma unroll
                for (int nb = 0; nb < kNBn; ++nb) {
                    typedef typename std::conditional<kInt8, v4f, v16f>::type vals_t;
                    vals_t v;
                    const blk_t c = blk(nb, mb);
                    if constexpr (kLrBatch) {
                        v = lrv[qb][nb];
                    } else {
#pragma unroll
                        for (int e = 0; e < 4 * kQuads; ++e) {
                            if constexpr (kFma) v[e] = __builtin_fmaf((float)c[e], tm[mb], bias_at(nb, e));
                            else v[e] = (float)c[e] * tm[mb];
                        }
                    }
                    if constexpr (EPI == kEpiLowRank) {
                        if constexpr (kInt8) v = low_rank_add16(p, v, nw + nb * 16, mw + mb * 16, brow, el);
                        else v = low_rank_add(p, v, nw + nb * 32, mw + mb * 32, brow, el >> 5);
                    }
                    if constexpr (kLr32 && !kLrBatch) {
                        // e4m3: u . l2^T of this block from the staged rows (the
                        // interleaved form above needs more registers than this
                        // instantiation has, and was slower)
                        const int urow = wm * 128 + mb * 32 + brow, lrow2 = wn * kWN + nb * 32 + brow;
#pragma unroll
                        for (int ks = 0; ks < 2; ++ks) {
                            if (ks * 16 >= p.rp) break;
                            const int j0 = ks * 16 + (el >> 5) * 8;
                            const v8bf a = *reinterpret_cast<const v8bf *>(lb + (lrow2 * p.r + j0) * 2);
                            const v4u uh = *reinterpret_cast<const v4u *>(ub + (urow * p.rp + j0) * 2);
                            const v4u ul = *reinterpret_cast<const v4u *>(ub + half_bytes + (urow * p.rp + j0) * 2);
                            v = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(v8bf, uh), v, 0, 0, 0);
                            v = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(v8bf, ul), v, 0, 0, 0);
                        }
                    }
                    if constexpr (kCol) {
#pragma unroll
                        for (int e = 0; e < 4 * kQuads; ++e) v[e] *= swc[nb][e / 4][e % 4];
                    }
#pragma unroll
                    for (int q = 0; q < kQuads; ++q) {
                        float y[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            y[i] = kFma || kLrBatch ? v[4 * q + i] : v[4 * q + i] + bias_at(nb, 4 * q + i);
                        const float y0 = y[0], y1 = y[1], y2 = y[2], y3 = y[3];
                        const int row = qb * kBlk + brow;           // row within the pass
                        const int col = nb * kBlk + 8 * q + cq;     // bf16 column within the wave tile
                        const int chunk = (col >> 3) ^ (row & 15);
                        *reinterpret_cast<uint2 *>(ob + row * 256 + chunk * 16 + (col & 7) * 2) =
                            make_uint2(pack_bf16x2(y0, y1), pack_bf16x2(y2, y3));
                    }
                }
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            // 32 rows x kWN / 8 chunks, read 4 rows (16 chunk slots each) per
            // wave-wide instruction.  A 128-wide wave tile leaves as whole
            // 256-byte row segments (non-temporal stores); a 96-wide one as
            // 192-byte segments, whose 128-byte lines shared with the
            // neighbouring wave's segment take cached stores so that the L2
            // merges the two halves (non-temporal partial lines would reach
            // memory as partial writes).
            constexpr int kOutChunks = kWN / 8;
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                const int r = it * 4 + (el >> 4), c = el & 15;
                if (kOutChunks < 16 && c >= kOutChunks) continue;
                const v4u d = *reinterpret_cast<const v4u *>(ob + r * 256 + ((c ^ (r & 15)) << 4));
                const int m = mw + ps * 32 + r, n = nw + c * 8;
                uint16_t *dst = out + (size_t)m * N + n;
                if constexpr (kIn && BNT != 256) {
                    const size_t seg = ((size_t)m * N + nw) * 2, at = ((size_t)m * N + n) * 2;
                    const size_t line = at & ~(size_t)127;
                    if (line >= seg && line + 128 <= seg + 2 * kWN) __builtin_nontemporal_store(d, reinterpret_cast<v4u *>(dst));
                    else *reinterpret_cast<v4u *>(dst) = d;
                } else if constexpr (kIn) {
                    __builtin_nontemporal_store(d, reinterpret_cast<v4u *>(dst));
                } else if (m < M) {
                    if ((N & 7) == 0 && n + 7 < N) {
                        __builtin_nontemporal_store(d, reinterpret_cast<v4u *>(dst));
                    } else {
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            if (n + i < N) dst[i] = (uint16_t)(d[i >> 1] >> ((i & 1) * 16));
                    }
                }
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
    };

    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const TileCoord tc = tile_coord<BNT>(tile, tiles_m, tiles_n);
        const int mw = tc.m0 + wm * 128, nw = tc.n0 + wn * kWN;
        lr_mw = mw;
        lr_nw = nw;
        // Stage 0 of this tile has landed (prologue, or the last stage of the
        // previous tile waited for it).  The copies of these fragments that
        // the previous tile's last stage read are dead across its epilogue.
        read_frags(lds0, 0, fa[0], fb[0]);

        // Interior tiles (all rows and columns in range, N % 8 == 0) take a
        // copy of the epilogue without any bounds checks.
        const bool interior = tc.m0 + BM <= M && tc.n0 + BNT <= N && (N & 7) == 0;
        constexpr bool kDma = EPI != kEpiI32;
        // The first NST stages start the accumulators (kt_end >= NST).  The
        // epilogue inputs are fetched before the second-to-last stage: the
        // waits at the ends of the last two stages cover them.
        run_stages(std::integral_constant<int, 0>{}, std::integral_constant<int, NST>{}, std::true_type{},
                   kt_end == NST);
        for (int kt0 = NST; kt0 < kt_end; kt0 += NST) {
            run_stages(std::integral_constant<int, 0>{}, std::integral_constant<int, NST - 2>{}, std::false_type{},
                       false);
            if constexpr (kDma) {
                if (interior && kt0 + NST == kt_end) epi_dma(mw, nw);
            }
            if constexpr (kLrReg) {
                if (kt0 + NST == kt_end) lowrank_l2_dma(tc.n0);
            }
            run_stages(std::integral_constant<int, NST - 2>{}, std::integral_constant<int, NST>{}, std::false_type{},
                       kt0 + NST == kt_end);
        }
        if constexpr (kDma) {
            if (interior && kt_end == NST) {
                epi_dma(mw, nw);
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
        }
        if constexpr (kLrReg) {
            // a tile of NST stages: its l2 goes out after them, and other
            // waves read it
            if (kt_end == NST) {
                lowrank_l2_dma(tc.n0);
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                asm volatile("s_barrier" ::: "memory");
            }
        }

        // --------------------------------------------------------- epilogue
        // The last MFMAs were inline asm, which the compiler's hazard tracking
        // does not see; give their results the wait states an MFMA result
        // needs before other instructions read it (24 >= the 16x16x64 int8
        // requirement, 32 >= the 16-pass 32x32x64 e4m3 one) before the
        // epilogue touches the accumulators.
        if constexpr (kInt8) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
        else asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
        // Block (nb, mb), register 4j+i holds output row m = mbase + (l & 31)
        // and column n = nbase + 8j + 4(l >> 5) + i.
        if constexpr (EPI == kEpiI32) {
            int32_t *out = static_cast<int32_t *>(p.out);
            const int brow = lane & (kBlk - 1), cq = 4 * (lane / kBlk);
#pragma unroll
            for (int nb = 0; nb < kNBn; ++nb)
#pragma unroll
                for (int mb = 0; mb < kNB; ++mb) {
                    const int m = mw + mb * kBlk + brow;
                    if (m >= M) continue;
                    const blk_t c = blk(nb, mb);
#pragma unroll
                    for (int q = 0; q < kQuads; ++q) {
                        const int n = nw + nb * kBlk + 8 * q + cq;
                        int32_t *dst = out + (size_t)m * N + n;
                        if ((N & 3) == 0 && n + 3 < N) {
                            v4i v = {(int)c[4 * q], (int)c[4 * q + 1], (int)c[4 * q + 2], (int)c[4 * q + 3]};
                            *reinterpret_cast<v4i *>(dst) = v;
                        } else {
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                if (n + i < N) dst[i] = (int)c[4 * q + i];
                        }
                    }
                }
        } else {
            if (interior) bf16_epilogue(std::true_type{}, mw, nw);
            else bf16_epilogue(std::false_type{}, mw, nw);
        }
        // e4m3: the staged u rows are read by every wave before any of them
        // starts the next tile, whose first stage refills that buffer.
        if constexpr (EPI == kEpiLowRank32 && !kInt8) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            asm volatile("s_barrier" ::: "memory");
            // the refill deferred from the tile's last stage (the next tile's
            // stage NST - 2, or stage 1 with two stages), into the buffer
            // that held l2
            load_part(buf(std::integral_constant<int, kDeferBuf>{}), std::integral_constant<int, 0>{},
                      std::integral_constant<int, 1>{});
            advance_cursor();
        }
        // The K loop counts VMEM operations in flight (vmcnt) on the premise
        // that they are all stage loads; let this tile's stores drain first.
        if constexpr (NST > 2) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    // Loads of the stages past the last tile (all out of range) may still be
    // in flight; let them land before the workgroup ends.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int QT, int EPI, int BNT>
void launch_width(const GemmArgs &a, hipStream_t stream) {
    const int tm = (a.M + BM - 1) / BM, tn = (a.N + BNT - 1) / BNT;
    const int tiles = tm * tn;
    const int grid = tiles < device_cu_count() ? tiles : device_cu_count();
    if (a.K % (Geo<QT>::BK * Geo<QT>::NST) == 0) gemm_kernel<QT, EPI, false, BNT><<<grid, kThreads, 0, stream>>>(a, tm, tn);
    else gemm_kernel<QT, EPI, true, BNT><<<grid, kThreads, 0, stream>>>(a, tm, tn);
}

// Time of `tiles` tiles on `cus` CUs, in rounds of full-chip tile time.  A
// partial last round with a fraction f of the CUs busy runs at the higher
// clock the power limit then allows and takes 0.42 + 0.58 f of a full round
// (fitted to a half round of 256 x 256 int8 tiles at K = 12288: 0.71).
double tile_rounds(int64_t tiles, int64_t cus) {
    const int64_t full = tiles / cus, rem = tiles % cus;
    return (double)full + (rem ? 0.42 + 0.58 * (double)rem / (double)cus : 0.0);
}

// Tile width for a shape (bf16 epilogue): 192-wide tiles when the product
// spans more than one round of 256-wide tiles and they finish sooner.  A
// 192-wide tile takes 0.85 of a 256-wide one's time (measured at M8192
// N3072 K12288: 0.75 of the products, but 17% more operand bytes per
// product).  E.g. M8192 N3072: 384 tiles of 256 (1.71 rounds) against 512
// of 192 (2 x 0.85 = 1.70).
bool use_192(int M, int N) {
    const int64_t cus = device_cu_count(), tm = (M + BM - 1) / BM;
    const int64_t t256 = tm * ((N + 255) / 256), t192 = tm * ((N + 191) / 192);
    if (t256 <= cus) return false;
    return 0.85 * tile_rounds(t192, cus) < tile_rounds(t256, cus);
}

template <int QT, int EPI>
void launch(const GemmArgs &a, hipStream_t stream) {
    if constexpr (EPI == kEpiBf16) {
        if (use_192(a.M, a.N)) {
            launch_width<QT, EPI, 192>(a, stream);
            return;
        }
    }
    launch_width<QT, EPI, 256>(a, stream);
}

}  // namespace

// Compute units of the current device (queried once per device; threads
// that race on the first query store the same value, atomically).
int device_cu_count() {
    static std::atomic<int> cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

w8a8_status gemm_check(const void *xq, const void *wq, int64_t M, int64_t N, int64_t K, const void *out) {
    if (M < 0 || N < 0 || K < 0) return W8A8_ERR_INVALID_ARG;
    if (M > 0 && N > 0 && (!xq || !wq || !out)) return W8A8_ERR_INVALID_ARG;
    if (K < 16 || K % 16 != 0 || K > (1 << 22)) return W8A8_ERR_SHAPE;
    if (M > (1 << 30) || N > (1 << 30)) return W8A8_ERR_SHAPE;
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + 191) / 192);  // the narrower tile's count
    if (tiles > 0x7FFFFFFF) return W8A8_ERR_SHAPE;
    if (!aligned16(xq) || !aligned16(wq) || !aligned16(out)) return W8A8_ERR_ALIGN;
    return W8A8_OK;
}

w8a8_status gemm_launch(w8a8_qtype qtype, GemmEpilogue epi, const GemmArgs &a, hipStream_t stream) {
    if (a.M == 0 || a.N == 0) return W8A8_OK;
    if (qtype == W8A8_INT8) {
        if (epi == kEpiI32) launch<W8A8_INT8, kEpiI32>(a, stream);
        else if (epi == kEpiBf16) launch<W8A8_INT8, kEpiBf16>(a, stream);
        else if (epi == kEpiLowRank) launch<W8A8_INT8, kEpiLowRank>(a, stream);
        else if (epi == kEpiLowRank32) launch<W8A8_INT8, kEpiLowRank32>(a, stream);
        else launch<W8A8_INT8, kEpiColScale>(a, stream);
    } else {
        if (epi == kEpiI32) return W8A8_ERR_UNSUPPORTED;
        if (epi == kEpiBf16) launch<W8A8_FP8_E4M3, kEpiBf16>(a, stream);
        else if (epi == kEpiLowRank) launch<W8A8_FP8_E4M3, kEpiLowRank>(a, stream);
        else if (epi == kEpiLowRank32) launch<W8A8_FP8_E4M3, kEpiLowRank32>(a, stream);
        else launch<W8A8_FP8_E4M3, kEpiColScale>(a, stream);
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

extern "C" w8a8_status gguf_a8_linear(w8a8_qtype qtype, const void *xq, const float *x_scale, const void *wq,
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
    return gemm_launch(qtype, kEpiColScale, a, stream);
}

extern "C" int w8a8_probe_gemm_tile_n(int64_t M, int64_t N) {
    using namespace w8a8;
    if (M < 1 || N < 1 || M > (1 << 30) || N > (1 << 30)) return 0;
    return use_192((int)M, (int)N) ? 192 : 256;
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
