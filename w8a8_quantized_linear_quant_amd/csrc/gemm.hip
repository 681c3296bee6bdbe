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
//  * Persistent: one 256-thread workgroup per CU walks 256x256 output tiles,
//    4 waves in a 2x2 grid, each wave a 128x128 sub-tile held as 4x4 blocks
//    of 32x32 MFMA accumulators (v_mfma_i32_32x32x32_i8, or
//    v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales for e4m3): 256
//    accumulator registers per lane, one wave per SIMD.
//  * Both operands are K-contiguous ("NT"), so every lane's MFMA fragment is
//    a contiguous 16- or 32-byte run of one row.  The weight is the MFMA's A
//    operand and the activations its B operand, so each lane ends up holding
//    four consecutive output columns of one row.
//  * K goes HBM -> LDS in BK-byte stages through a ring of NST buffers with
//    buffer_load_dwordx4 ... lds (no register staging); the ring runs NST - 1
//    stages ahead, across tile boundaries.  Buffer loads past num_records
//    read zero, which covers ragged M/N tails and (with an out-of-range
//    offset) the ragged K tail.
//  * Within a stage, 16-byte chunks of each row are XOR-swizzled by the row
//    index so the fragment reads of consecutive rows hit distinct banks.
//  * Tiles are numbered so that the workgroups of one XCD (hardware sends
//    workgroup i to XCD i % 8) share operand panels in that XCD's L2.
//  * The epilogue scales, adds the bias, packs to bf16 and stages each
//    32-row slice of a wave's sub-tile through LDS so that it leaves as
//    16-byte stores covering 256-byte row segments.
#include <type_traits>
#include <utility>

#include <atomic>

#include "internal.hpp"

namespace w8a8 {
namespace {

constexpr int BM = 256, BN = 256;
constexpr int kThreads = 256;
#ifndef W8A8_GEMM_GROUP_M
#define W8A8_GEMM_GROUP_M 4
#endif
constexpr int kGroupM = W8A8_GEMM_GROUP_M;  // tile-ordering group height
constexpr int kXcds = 8;

#ifndef W8A8_GEMM_BK
#define W8A8_GEMM_BK 64  // bytes of K per LDS stage
#endif
#ifndef W8A8_GEMM_NST
#define W8A8_GEMM_NST 4  // LDS stages (loads run NST - 1 stages ahead)
#endif
constexpr int BK = W8A8_GEMM_BK;
constexpr int NST = W8A8_GEMM_NST;
constexpr int kOpBytes = 256 * BK;         // one operand tile per stage
constexpr int kStageBytes = 2 * kOpBytes;  // X tile then W tile
constexpr int kChunks = BK / 16;           // 16-byte chunks per row
constexpr int kRowsPerLoad = 64 / kChunks; // rows one wave-wide 1 KB load covers
constexpr int kLoadsPerOp = 64 / kRowsPerLoad;  // per wave and operand: 64 rows
constexpr int kLoadsPerStage = 2 * kLoadsPerOp;
constexpr int kImmLoads = kLoadsPerOp < 4 ? kLoadsPerOp : 4;  // loads per M0 value (immediate offsets < 4 KB)
constexpr int kOutWaveBytes = 32 * 256;    // epilogue staging per wave
static_assert(NST >= 3 && NST <= 4, "3..4 LDS stages");
static_assert(NST * kStageBytes + 4 * kOutWaveBytes <= 160 * 1024, "LDS budget");
static_assert((NST - 1) * kLoadsPerStage <= 63, "vmcnt range");

typedef __attribute__((address_space(3))) void *lds_ptr_t;

// XOR swizzle of the 16-byte chunk index by row, chosen so that the fragment
// reads of 16 consecutive rows (same logical chunk) spread over distinct bank
// groups whether the LDS serves 8 or 16 lanes of a 128-bit read per cycle.
// It depends on row % 16 only, so it is the same for every 32-row block.
__device__ __forceinline__ int swz(int row) {
    if constexpr (kChunks == 8) return (row & 7) ^ ((row >> 3) & 1);
    else return ((row >> 1) ^ (row >> 2)) & 3;
}

struct TileCoord {
    int m0, n0;
};

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
    c.n0 = (in / gm) * BN;
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


// TAIL: K is not a multiple of BK * NST, so some stages reach past K and
// need per-lane range checks; otherwise every stage is whole and the stage's
// K offset travels in the instruction's scalar offset.
template <int QT, int EPI, bool TAIL>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs p, int tiles_m, int tiles_n) {
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
    int goff[kLoadsPerOp], gcol[kLoadsPerOp];
#pragma unroll
    for (int i = 0; i < kLoadsPerOp; ++i) {
        const int row = wave * 64 + i * kRowsPerLoad + lane / kChunks;
        const int c = (lane % kChunks) ^ swz(row);
        gcol[i] = c * 16;
        // the instruction's immediate offset (i KB, see load_part) is added to
        // the global address as well as to the LDS address; take it back out
        goff[i] = row * K + c * 16 - (i % kImmLoads) * 1024;
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
            const TileCoord c = tile_coord(ld_tile, tiles_m, tiles_n);
            rows_x = min(M - c.m0, BM);
            rows_w = min(N - c.n0, BN);
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
        constexpr int lo = P * kLoadsPerStage / NP, hi = (P + 1) * kLoadsPerStage / NP;
        const int k0 = ld_kt * BK;
        const bool full = !TAIL || k0 + BK <= K;
        [&]<int... J>(std::integer_sequence<int, J...>) {
            (([&] {
                 constexpr int j = lo + J;
                 constexpr int i = j % kLoadsPerOp;
                 constexpr int grp = i / kImmLoads, imm = (i % kImmLoads) * 1024;
                 uint8_t *m0 = stage + (j < kLoadsPerOp ? 0 : kOpBytes) + wave * 64 * BK + grp * kImmLoads * 1024;
                 if constexpr (TAIL) {
                     const int o = full ? goff[i] + k0 : (k0 + gcol[i] < K ? goff[i] + k0 : kOobOffset);
                     __builtin_amdgcn_raw_ptr_buffer_load_lds(j < kLoadsPerOp ? rx : rw, (lds_ptr_t)m0, 16, o, 0, imm,
                                                              0);
                 } else {
                     // per-lane offset fixed for the whole kernel, stage offset scalar
                     __builtin_amdgcn_raw_ptr_buffer_load_lds(j < kLoadsPerOp ? rx : rw, (lds_ptr_t)m0, 16, goff[i], k0,
                                                              imm, 0);
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

    // MFMA fragments: lane row = l & 31 within a 32-row block (swz(row)
    // depends on l & 15 only); int8 takes 16 bytes per lane per k-step of 32,
    // e4m3 32 bytes per k-step of 64.
    constexpr bool kInt8 = QT == W8A8_INT8;
    constexpr int KSTEPS = kInt8 ? BK / 32 : BK / 64;
    static_assert(KSTEPS >= 1, "stage too small for one MFMA k-step");
    typedef typename std::conditional<kInt8, v4i, v8i>::type frag_t;
    typedef typename std::conditional<kInt8, v16i, v16f>::type acc_t;
    const int lrow = lane & 31, half = lane >> 5;
    const int lsw = swz(lrow);

    acc_t acc[4][4];
    frag_t fa[2][4], fb[2][4];

    // int8: lane offsets of the fragment reads of k-steps 0 and 1 of a stage.
    // Each read_frags call adds one to its stage's base through an opaque
    // copy, so the compiler does not keep a precomputed address per stage
    // buffer and k-step alive across the loop (measured: ~3% faster for int8;
    // e4m3, with half as many k-steps, is faster with the addresses kept).
    int foff[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) foff[kk] = lrow * BK + (((kk * 2 + half) ^ lsw) << 4);
    auto read_frags = [&](const uint8_t *stage, int kk, frag_t *af, frag_t *bf) {
        const uint8_t *xs = stage + (wm * 128) * BK;            // X rows of this wave
        const uint8_t *ws = stage + kOpBytes + (wn * 128) * BK;  // W rows of this wave
        if constexpr (kInt8) {
            int off = foff[kk & 1];
            asm volatile("" : "+v"(off));
#pragma unroll
            for (int b = 0; b < 4; ++b) af[b] = *reinterpret_cast<const v4i *>(ws + b * 32 * BK + off);
#pragma unroll
            for (int b = 0; b < 4; ++b) bf[b] = *reinterpret_cast<const v4i *>(xs + b * 32 * BK + off);
        } else {
            const int c0 = kk * 4 + half * 2;
            const int off0 = lrow * BK + ((c0 ^ lsw) << 4);
            const int off1 = lrow * BK + (((c0 + 1) ^ lsw) << 4);
#pragma unroll
            for (int b = 0; b < 4; ++b) {
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

    // FIRST: the tile's first k-step, which starts the accumulators from an
    // inline-constant zero instead of zeroing 256 registers beforehand.
    auto mfmas = [&](const frag_t *af, const frag_t *bf, auto first_c) {
        constexpr bool FIRST = decltype(first_c)::value;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                const acc_t c = FIRST ? acc_t{} : acc[nb][mb];
                if constexpr (kInt8)
                    acc[nb][mb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[nb], bf[mb], c, 0, 0, 0);
                else
                    acc[nb][mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[nb], bf[mb], c, 0, 0, 0, 127, 0,
                                                                                  127);
            }
    };

    // Interleave the memory instructions of a k-step with its 16 MFMAs so that
    // their issue (the LDS-DMA loads especially) overlaps MFMA execution
    // instead of stalling the wave in front of the matrix pipe.
    constexpr int kDsPerStep = kInt8 ? 8 : 16;  // ds_read_b128 per fragment set
    auto interleave = [&](auto nvm_c) {
        constexpr int NVM = decltype(nvm_c)::value;
        [&]<int... I>(std::integer_sequence<int, I...>) {
            (([&] {
                 __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                 constexpr int ds = (I + 1) * kDsPerStep / 16 - I * kDsPerStep / 16;
                 if constexpr (ds > 0) __builtin_amdgcn_sched_group_barrier(0x100, ds, 0);  // DS reads
                 constexpr int vm = (I + 1) * NVM / 16 - I * NVM / 16;
                 if constexpr (vm > 0) __builtin_amdgcn_sched_group_barrier(0x020, vm, 0);  // VMEM reads
             }()),
             ...);
        }(std::make_integer_sequence<int, 16>{});
    };

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
    constexpr int kParts = KSTEPS;
    constexpr int kPerPart = kLoadsPerStage / kParts;
    static_assert(kLoadsPerStage % kParts == 0, "loads split evenly over k-steps");
    // loads still allowed in flight when stage kt+1 must be complete: stages
    // kt+2 .. kt+NST-2 whole, and the parts of stage kt+NST-1 issued so far
    constexpr int kPending = (NST - 3) * kLoadsPerStage + (kParts - 1) * kPerPart;
    // defer (the low-rank epilogue only, last stage of a tile): this stage's
    // refill -- the next tile's stage NST - 2 -- is issued after the epilogue
    // instead, so that its buffer can hold the low-rank operands meanwhile.
    auto run_stage = [&](auto sc, auto first_c, bool defer) {
        constexpr int S = decltype(sc)::value;
        constexpr bool FIRST = decltype(first_c)::value;
        constexpr bool kMayDefer = EPI == kEpiLowRank32 && S == NST - 1;
        const bool issue = !kMayDefer || !defer;
        uint8_t *cur = buf(sc);
        uint8_t *nxt = buf(std::integral_constant<int, (S + 1) % NST>{});
        uint8_t *refill = buf(std::integral_constant<int, (S + NST - 1) % NST>{});
        [&]<int... KK>(std::integer_sequence<int, KK...>) {
            (([&] {
                 constexpr int kk = KK;
                 constexpr int P = (S * KSTEPS + kk) & 1;
                 if constexpr (kk + 1 < KSTEPS) {
                     __builtin_amdgcn_sched_barrier(0);
                     read_frags(cur, kk + 1, fa[P ^ 1], fb[P ^ 1]);
                     if (issue)
                         load_part(refill, std::integral_constant<int, kk>{}, std::integral_constant<int, kParts>{});
                     mfmas(fa[P], fb[P], std::integral_constant<bool, FIRST && S == 0 && kk == 0>{});
                     interleave(std::integral_constant<int, kPerPart>{});
                     __builtin_amdgcn_sched_barrier(0);
                 } else {
                     // without this stage's earlier parts in flight, fewer may remain
                     if (issue) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kPending) : "memory");
                     else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kPending - (kParts - 1) * kPerPart) : "memory");
                     asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                     // a bare barrier: __syncthreads() would add a release fence,
                     // i.e. a wait for every load in flight, prefetches included
                     asm volatile("s_barrier" ::: "memory");
                     __builtin_amdgcn_sched_barrier(0);
                     if (issue)
                         load_part(refill, std::integral_constant<int, kk>{}, std::integral_constant<int, kParts>{});
                     read_frags(nxt, 0, fa[P ^ 1], fb[P ^ 1]);
                     mfmas(fa[P], fb[P], std::integral_constant<bool, FIRST && S == 0 && kk == 0>{});
                     interleave(std::integral_constant<int, kPerPart>{});
                     __builtin_amdgcn_sched_barrier(0);
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

    // Prologue: stages 0 .. NST-2 in flight, wait for stage 0.
    [&]<int... S>(std::integer_sequence<int, S...>) {
        ((load_part(buf(std::integral_constant<int, S>{}), std::integral_constant<int, 0>{},
                    std::integral_constant<int, 1>{}),
          advance_cursor()),
         ...);
    }(std::make_integer_sequence<int, NST - 1>{});
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NST - 2) * kLoadsPerStage) : "memory");
    asm volatile("s_barrier" ::: "memory");

    // bf16 epilogue of one tile: y = bf16(acc * sx[m] * sw (+ u . l2^T) + bias[n]).
    // Result rows go through this wave's LDS staging area (32 rows x 256 B,
    // 16-byte chunks XOR-swizzled by row) and leave as 16-byte stores that
    // cover whole 256-byte row segments.
    auto bf16_epilogue = [&](auto interior_c, int mw, int nw) {
        constexpr bool kIn = decltype(interior_c)::value;
        uint16_t *out = static_cast<uint16_t *>(p.out);
        uint8_t *ob = obuf + wave * kOutWaveBytes;
        // Re-derive the lane indices here so the staging addresses are not
        // hoisted out of the tile loop (they would stay live across the K
        // loop and spill).
        int el = lane;
        asm volatile("" : "+v"(el));
        const int erow = el & 31, ehalf = el >> 5;
        constexpr bool kCol = EPI == kEpiColScale;
        float tm[4];
        uint2 bias2[4][4];
        v4f swc[kCol ? 4 : 1][4];  // per-channel weight scales of columns nb * 32 + 8 j + 4 half + i
        const float sw = kCol ? 1.0f : p.sw[0];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int m = mw + mb * 32 + erow;
            if constexpr (kIn) tm[mb] = *reinterpret_cast<const float *>(ob + kEpiSx + (mb * 32 + erow) * 4) * sw;
            else tm[mb] = m < M ? p.sx[m] * sw : 0.0f;
        }
        if constexpr (kCol) {
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int n = nw + nb * 32 + 8 * j + 4 * ehalf;
                    if (kIn || ((N & 3) == 0 && n < N)) {
                        swc[nb][j] = *reinterpret_cast<const v4f *>(p.sw + n);
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i) swc[nb][j][i] = n + i < N ? p.sw[n + i] : 0.0f;
                    }
                }
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = nw + nb * 32 + 8 * j + 4 * ehalf;
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
                bias2[nb][j] = b;
            }
        constexpr bool kLr32 = EPI == kEpiLowRank32;
        constexpr bool kLrBatch = kLr32 && kInt8;
        uint8_t *ub = buf(std::integral_constant<int, NST - 1>{});
        uint8_t *lb = buf(std::integral_constant<int, NST - 2>{});
        const int half_bytes = 256 * p.rp * 2;
        if constexpr (kLr32) {
            // The low-rank operands of the workgroup's tile go to the two ring
            // buffers that are free during the epilogue (the last stage's, and
            // the one whose refill was deferred): u of its 256 rows (hi, then
            // lo, [256][rp] bf16 each) and l2 of its 256 columns ([256][r],
            // r == rp); every wave fetches a quarter of each.
            {
                const int n0 = nw - wn * 128;
                const int cols_in = min(N - n0, 256);
                const __amdgpu_buffer_rsrc_t rw2 = __builtin_amdgcn_make_buffer_rsrc(
                    (void *)(p.l2 + (size_t)n0 * p.r), (short)0, cols_in * p.r * 2, kBufferRsrcWord3);
                for (int i = 0; i < p.r / 8; ++i) {
                    const int off = wave * 128 * p.r + i * 1024;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rw2, (lds_ptr_t)(lb + off), 16, off + el * 16, 0, 0, 0);
                }
            }
            const int m0 = mw - wm * 128;
            const int rows_in = min(M - m0, 256);
            const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(p.uhi + (size_t)m0 * p.rp), (short)0, rows_in * p.rp * 2, kBufferRsrcWord3);
            const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(p.ulo + (size_t)m0 * p.rp), (short)0, rows_in * p.rp * 2, kBufferRsrcWord3);
            for (int i = 0; i < p.rp / 8; ++i) {  // 128 rp bytes per wave and half, 1 KB per load
                const int off = wave * 128 * p.rp + i * 1024;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rh, (lds_ptr_t)(ub + off), 16, off + el * 16, 0, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (lds_ptr_t)(ub + half_bytes + off), 16, off + el * 16, 0,
                                                         0, 0);
            }
            if constexpr (kLrBatch) {
                // int8: scale the accumulators in place while the operands land
#pragma unroll
                for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb) {
                        v16f t;
#pragma unroll
                        for (int e = 0; e < 16; ++e) t[e] = (float)acc[nb][mb][e] * tm[mb];
                        acc[nb][mb] = __builtin_bit_cast(acc_t, t);
                    }
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            asm volatile("s_barrier" ::: "memory");
        }
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            if constexpr (kLrBatch) {
                // u . l2^T of the 4 blocks of this block row from the staged
                // rows, the MFMAs interleaved over the blocks so that they
                // issue back to back rather than each waiting on the last
                const int urow = wm * 128 + mb * 32 + erow;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    if (ks * 16 >= p.rp) break;
                    const int j0 = ks * 16 + ehalf * 8;
                    v8bf a[4];
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb)
                        a[nb] = *reinterpret_cast<const v8bf *>(lb + ((wn * 128 + nb * 32 + erow) * p.r + j0) * 2);
                    const v8bf uh = *reinterpret_cast<const v8bf *>(ub + (urow * p.rp + j0) * 2);
                    const v8bf ul = *reinterpret_cast<const v8bf *>(ub + half_bytes + (urow * p.rp + j0) * 2);
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb)
                        acc[nb][mb] = __builtin_bit_cast(acc_t, __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            a[nb], uh, __builtin_bit_cast(v16f, acc[nb][mb]), 0, 0, 0));
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb)
                        acc[nb][mb] = __builtin_bit_cast(acc_t, __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            a[nb], ul, __builtin_bit_cast(v16f, acc[nb][mb]), 0, 0, 0));
                }
            }
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                v16f v;
                if constexpr (kLrBatch) {
                    v = __builtin_bit_cast(v16f, acc[nb][mb]);
                } else {
#pragma unroll
                    for (int e = 0; e < 16; ++e) v[e] = (float)acc[nb][mb][e] * tm[mb];
                }
                if constexpr (EPI == kEpiLowRank) v = low_rank_add(p, v, nw + nb * 32, mw + mb * 32, erow, ehalf);
                if constexpr (kLr32 && !kLrBatch) {
                    // e4m3: u . l2^T of this block from the staged rows (the
                    // interleaved form above needs more registers than this
                    // instantiation has, and was slower)
                    const int urow = wm * 128 + mb * 32 + erow, lrow2 = wn * 128 + nb * 32 + erow;
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        if (ks * 16 >= p.rp) break;
                        const int j0 = ks * 16 + ehalf * 8;
                        const v8bf a = *reinterpret_cast<const v8bf *>(lb + (lrow2 * p.r + j0) * 2);
                        const v4u uh = *reinterpret_cast<const v4u *>(ub + (urow * p.rp + j0) * 2);
                        const v4u ul = *reinterpret_cast<const v4u *>(ub + half_bytes + (urow * p.rp + j0) * 2);
                        v = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(v8bf, uh), v, 0, 0, 0);
                        v = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(v8bf, ul), v, 0, 0, 0);
                    }
                }
                if constexpr (kCol) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) v[e] *= swc[nb][e / 4][e % 4];
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint2 bb = bias2[nb][j];
                    const float y0 = v[4 * j] + bf16_bits_to_f32(bb.x & 0xFFFFu);
                    const float y1 = v[4 * j + 1] + bf16_bits_to_f32(bb.x >> 16);
                    const float y2 = v[4 * j + 2] + bf16_bits_to_f32(bb.y & 0xFFFFu);
                    const float y3 = v[4 * j + 3] + bf16_bits_to_f32(bb.y >> 16);
                    const int col = nb * 32 + 8 * j + 4 * ehalf;  // bf16 column within the wave tile
                    const int chunk = (col >> 3) ^ (erow & 15);
                    *reinterpret_cast<uint2 *>(ob + erow * 256 + chunk * 16 + (col & 7) * 2) =
                        make_uint2(pack_bf16x2(y0, y1), pack_bf16x2(y2, y3));
                }
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            // 32 rows x 16 chunks: 4 rows per wave-wide instruction
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                const int r = it * 4 + (el >> 4), c = el & 15;
                const v4u d = *reinterpret_cast<const v4u *>(ob + r * 256 + ((c ^ (r & 15)) << 4));
                const int m = mw + mb * 32 + r, n = nw + c * 8;
                uint16_t *dst = out + (size_t)m * N + n;
                if constexpr (kIn) {
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
        const TileCoord tc = tile_coord(tile, tiles_m, tiles_n);
        const int mw = tc.m0 + wm * 128, nw = tc.n0 + wn * 128;
        // Stage 0 of this tile has landed (prologue, or the last stage of the
        // previous tile waited for it).  The copies of these fragments that
        // the previous tile's last stage read are dead across its epilogue.
        read_frags(lds0, 0, fa[0], fb[0]);

        // Interior tiles (all rows and columns in range, N % 8 == 0) take a
        // copy of the epilogue without any bounds checks.
        const bool interior = tc.m0 + BM <= M && tc.n0 + BN <= N && (N & 7) == 0;
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
            run_stages(std::integral_constant<int, NST - 2>{}, std::integral_constant<int, NST>{}, std::false_type{},
                       kt0 + NST == kt_end);
        }
        if constexpr (kDma) {
            if (interior && kt_end == NST) {
                epi_dma(mw, nw);
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
        }

        // --------------------------------------------------------- epilogue
        // Block (nb, mb), register 4j+i holds output row m = mbase + (l & 31)
        // and column n = nbase + 8j + 4(l >> 5) + i.
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
                            v4i v = {(int)acc[nb][mb][4 * j], (int)acc[nb][mb][4 * j + 1],
                                     (int)acc[nb][mb][4 * j + 2], (int)acc[nb][mb][4 * j + 3]};
                            *reinterpret_cast<v4i *>(dst) = v;
                        } else {
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                if (n + i < N) dst[i] = (int)acc[nb][mb][4 * j + i];
                        }
                    }
                }
        } else {
            if (interior) bf16_epilogue(std::true_type{}, mw, nw);
            else bf16_epilogue(std::false_type{}, mw, nw);
        }
        // The staged u rows are read by every wave before any of them starts
        // the next tile, whose first stage refills that buffer.
        if constexpr (EPI == kEpiLowRank32) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            asm volatile("s_barrier" ::: "memory");
            // the refill deferred from the tile's last stage: the next tile's
            // stage NST - 2, into the buffer that held l2
            load_part(buf(std::integral_constant<int, NST - 2>{}), std::integral_constant<int, 0>{},
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

template <int QT, int EPI>
void launch(const GemmArgs &a, hipStream_t stream) {
    const int tm = (a.M + BM - 1) / BM, tn = (a.N + BN - 1) / BN;
    const int tiles = tm * tn;
    const int grid = tiles < device_cu_count() ? tiles : device_cu_count();
    if (a.K % (BK * NST) == 0) gemm_kernel<QT, EPI, false><<<grid, kThreads, 0, stream>>>(a, tm, tn);
    else gemm_kernel<QT, EPI, true><<<grid, kThreads, 0, stream>>>(a, tm, tn);
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
