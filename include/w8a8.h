/*
 * w8a8.h -- C ABI of the MI355X (gfx950) W8A8 quantized-linear library.
 *
 * What it computes (the pages this follows):
 *  - OneTrainer wiki "Quantization", "Technical" entries of the int W8A8 and
 *    float W8A8 types: weights quantized tensor-wise to int8 or float8 e4m3,
 *    activations quantized token-wise (one scale per row) during training,
 *    and the linear layer's matrix product done in 8 bits.
 *  - bitsandbytes #1401 "LLM.int8() Refactoring: Part 1", "Enhancements": one
 *    fused kernel calibrates the row scale and quantizes; row-major data only,
 *    no layout transforms; calls usable under graph capture.
 *  - OneTrainer PR #1034, "SVDQuant" (and the wiki's SVDQuant entry): a bf16
 *    low-rank branch added to the quantized product of the residual weight.
 *  - entrenar 0.7.8 src/quant/gguf_quant/q8_0.rs: GGUF Q8_0 blocks (32 values,
 *    f16 scale, 34 bytes), Q8_0::quantize and Q8_0::dequantize.
 *  - OneTrainer wiki "Quantization", "Technical" entries of GGUF A8 int and
 *    GGUF A8 float: GGUF weights re-quantized axis-wise (one scale per output
 *    channel) to int8 or float8 e4m3, token-wise activations, 8-bit product.
 *
 * Shared rules
 *  - Absmax scale of a group (a row, a whole tensor, a 32-value block):
 *    s = 1e-10f if absmax < 1e-10f, else absmax / QMAX in f32 (QMAX = 127 for
 *    int8, 448 for e4m3).  int8 code = clamp(round_half_even(f32(x / s)),
 *    -128, 127); e4m3 code = e4m3_rne(clamp(f32(x / s), -448, 448)).
 *  - fp8 is OCP FP8 E4M3FN (bias 7, max finite 448, no infinities).
 *  - bf16 and f16 values travel as uint16_t bit patterns; codes as bytes.
 *  - Row-major only.  X is [M, K] (tokens x in-features), W is [N, K] (the
 *    nn.Linear [out, in] layout), Y is [M, N].
 *  - Inputs are finite (NaN/Inf in inputs give unspecified codes).
 *
 * Ownership and execution
 *  - Every tensor argument is a DEVICE pointer owned by the caller, including
 *    workspaces.  The library never allocates, frees, synchronizes or reads
 *    device memory from the host; it validates arguments on the host,
 *    enqueues kernels on `stream` (NULL = the default stream) and returns.
 *    Calls can therefore be captured into a HIP graph.  No global mutable
 *    state; calls on different streams with disjoint outputs may run
 *    concurrently.
 *  - All pointers must be 16-byte aligned (OneTrainer PR #1034, "Known
 *    issues", reports a misaligned-address failure that 16-byte alignment
 *    fixed).
 *
 * Errors
 *  - Arguments are checked before anything is launched; on an error nothing
 *    is launched and one of the codes below is returned.  Sizes of 0 are a
 *    successful no-op.  A launch failure reported by hipGetLastError()
 *    returns W8A8_ERR_HIP.  No C++ exception crosses this interface.
 */
#ifndef W8A8_H_
#define W8A8_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    W8A8_OK = 0,
    W8A8_ERR_INVALID_ARG = 1, /* null required pointer, negative size, bad enum, r outside [1, 64] */
    W8A8_ERR_SHAPE = 2,       /* a size or stride that the layout rules below forbid */
    W8A8_ERR_ALIGN = 3,       /* a pointer that is not 16-byte aligned */
    W8A8_ERR_UNSUPPORTED = 4, /* a combination the library does not implement */
    W8A8_ERR_HIP = 5,         /* the HIP runtime reported a launch error */
    W8A8_ERR_SCRATCH_LIMIT = 6 /* a call of svdq_linear_noalloc needs more than its fixed scratch */
} w8a8_status;

typedef enum {
    W8A8_INT8 = 0,     /* int8 codes, int32 accumulation */
    W8A8_FP8_E4M3 = 1  /* OCP e4m3 codes, f32 accumulation */
} w8a8_qtype;

/* Human-readable name of a status code (static string). */
const char *w8a8_status_str(w8a8_status status);

/* ------------------------------------------------------------------ weights */

/* Bytes of device workspace w8a8_quant_weight_tensorwise needs for W [N, K]. */
size_t w8a8_weight_workspace_bytes(int64_t N, int64_t K);

/*
 * Tensor-wise weight quantization (wiki "Quantization", int W8A8 / float W8A8
 * "Technical": the weights get one scale for the whole tensor).  One scale
 * for all of W:
 *   w_scale[0] = absmax scale of W;  wq[n, k] = code(W[n, k], w_scale).
 *   w      bf16 [N, K], contiguous.
 *   wq     codes [N, K], contiguous (int8 or e4m3 bytes).
 *   wq_t   optional (NULL to skip): the same codes transposed, [K, N]
 *          contiguous -- the operand layout the input-gradient product
 *          dX = dY . W needs (see w8a8_linear_backward_dx).  Requires N % 16 == 0.
 *   w_scale one f32 (device).
 *   workspace  w8a8_weight_workspace_bytes(N, K) bytes of device scratch
 *          (partial maxima; no clearing needed).
 * Two kernels: per-block partial maxima, then a kernel that re-reduces them
 * (deterministic, no atomics) and writes the codes.
 * Shape rules: N, K >= 0; K % 8 == 0; N, K <= 2^31 and N * K <= 2^40.
 */
w8a8_status w8a8_quant_weight_tensorwise(w8a8_qtype qtype, const uint16_t *w, int64_t N, int64_t K,
                                         void *wq, void *wq_t, float *w_scale, void *workspace,
                                         hipStream_t stream);

/* -------------------------------------------------------------- activations */

/*
 * Row-wise (token-wise) activation quantization -- one kernel that both finds
 * the row scales and quantizes, as bitsandbytes #1401 ("Enhancements") fused
 * them, applied to the W8A8 types of the OneTrainer wiki.  One pass over X:
 *   x_scale[m] = absmax scale of row m;  xq[m, k] = code(X[m, k], x_scale[m]).
 *   x      bf16 [M, ldx]; the first K columns of each row are used.  The
 *          buffer spans M * ldx elements.
 *   xq     codes [M, ldq]; columns K .. ldq-1 are written as zero, so a
 *          caller can pad K up to the 16-multiple the GEMM needs.
 *   x_scale f32 [M].
 * Shape rules: M, K >= 0; K <= 2^30; ldx >= K, ldx % 8 == 0; ldq >= K,
 * ldq % 16 == 0.
 */
w8a8_status w8a8_quant_act_rowwise(w8a8_qtype qtype, const uint16_t *x, int64_t M, int64_t K,
                                   int64_t ldx, void *xq, int64_t ldq, float *x_scale,
                                   hipStream_t stream);

/* --------------------------------------------------------------- the linear */

/*
 * W8A8 linear (wiki "Quantization", int W8A8 / float W8A8 "Technical": the
 * linear layer's matrix product runs in int8 or in float8) with the
 * dequantization fused into the product's epilogue:
 *   acc[m, n] = sum_k xq[m, k] * wq[n, k]   (int32 exact, or f32 for e4m3)
 *   y[m, n]   = bf16(acc[m, n] * x_scale[m] * w_scale[0] + bias[n])
 *   (in f32: acc * f32(x_scale[m] * w_scale[0]) + bias[n] as one fused
 *   multiply-add, rounded once to bf16, nearest even)
 *   xq [M, K] codes, x_scale f32 [M]; wq [N, K] codes, w_scale one f32;
 *   bias bf16 [N] or NULL; y bf16 [M, N].
 * Shape rules: M, N >= 0; K >= 16, K % 16 == 0 (pad K with zero codes: a zero
 * code adds exactly 0); M, N <= 2^30, K <= 2^22.  Any M and N, including
 * ragged tile tails.  The int32
 * sum is exact while |acc| < 2^31: always for codes the quantizers produce
 * (|q| <= 127) when K <= 133143, since 127^2 K < 2^31.
 */
w8a8_status w8a8_linear(w8a8_qtype qtype, const void *xq, const float *x_scale, const void *wq,
                        const float *w_scale, const uint16_t *bias, int64_t M, int64_t N, int64_t K,
                        uint16_t *y, hipStream_t stream);

/*
 * Input gradient of the W8A8 linear with frozen W (the wiki quantizes the
 * activations token-wise in training too): dX = dY . W, from dY quantized row-wise
 * (dyq [M, N], dy_scale f32 [M]) and the transposed weight codes produced by
 * w8a8_quant_weight_tensorwise (wq_t [K, N], w_scale):
 *   dx[m, k] = bf16(sum_n dyq[m, n] * wq_t[k, n] * dy_scale[m] * w_scale[0]).
 * The same product kernel as w8a8_linear with the roles (K <- N, N <- K).
 * Shape rules: M, K >= 0; N >= 16, N % 16 == 0; M, K <= 2^30, N <= 2^22.
 */
w8a8_status w8a8_linear_backward_dx(w8a8_qtype qtype, const void *dyq, const float *dy_scale,
                                    const void *wq_t, const float *w_scale, int64_t M, int64_t N,
                                    int64_t K, uint16_t *dx, hipStream_t stream);

/*
 * Raw int32 accumulators of the int8 product (a test and debugging export):
 *   acc[m, n] = sum_k xq[m, k] * wq[n, k], exact (caller keeps |acc| < 2^31).
 * Same kernel and shape rules as w8a8_linear with W8A8_INT8.
 */
w8a8_status w8a8_gemm_i32(const int8_t *xq, const int8_t *wq, int64_t M, int64_t N, int64_t K,
                          int32_t *acc, hipStream_t stream);

/* ------------------------------------------------------------------ SVDQuant */

/* Bytes of device workspace svdq_linear needs: U = X . L1^T as two bf16
 * halves, hi and lo, [M, roundup(r, 16)] each.  0 if r is outside [1, 64]. */
size_t svdq_workspace_bytes(int64_t M, int64_t r);

/*
 * SVDQuant-style linear (OneTrainer PR #1034 "SVDQuant"; wiki: SVDQuant with
 * bf16 factors, rank 16-32): W ~ L2 . L1 + R with the residual R quantized
 * tensor-wise and a bf16 low-rank pair kept unquantized:
 *   x_scale_out, xq_out = row-wise quantization of X (as w8a8_quant_act_rowwise)
 *   u[m, j]  = sum_k X[m, k] * L1[j, k]          (f32, unrounded to bf16)
 *   y[m, n]  = bf16(acc[m, n] * x_scale[m] * r_scale[0]
 *                   + sum_j u[m, j] * L2[n, j] + bias[n])
 *   x  bf16 [M, K]; rq codes [N, K], r_scale one f32; l1 bf16 [r, K] (down-
 *   projection, nn.Linear layout); l2 bf16 [N, r] (up-projection); bias bf16
 *   [N] or NULL; y bf16 [M, N]; xq_out codes [M, K]; x_scale_out f32 [M];
 *   workspace svdq_workspace_bytes(M, r) bytes.
 * Factor layout: both factors are stored as nn.Linear weights [out, in], the
 * layout of a LoRA pair (down [r, K], up [N, r]); in the matrix-product form
 * y = X A B with A [K, r], B [r, N] that is l1 = A^T and l2 = B^T.  Rows of l1
 * run along K like the rows of X and W, so the down-projection streams them
 * with the same 16-byte loads; rows of l2 hold the r factors of one output
 * column contiguously, which the epilogue reads per column.
 * Launches: for K <= 4096 and r <= 32, two -- one kernel reads X once for
 * both the row-wise quantization and the down-projection (bf16 MFMA, u
 * written as a hi/lo pair of bf16 halves so it keeps ~16 bits), then the
 * 8-bit product whose epilogue adds the up-projection on the bf16 MFMA;
 * otherwise three -- the row-wise act-quant, the down-projection, the
 * product.
 * Shape rules: as w8a8_linear (K % 16 == 0); 1 <= r <= 64, else
 * W8A8_ERR_INVALID_ARG.
 */
w8a8_status svdq_linear(w8a8_qtype qtype, const uint16_t *x, int64_t M, int64_t K, const void *rq,
                        const float *r_scale, const uint16_t *l1, const uint16_t *l2, int64_t r,
                        const uint16_t *bias, int64_t N, uint16_t *y, void *xq_out,
                        float *x_scale_out, void *workspace, hipStream_t stream);

/*
 * svdq_linear without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same launches and results as svdq_linear, with
 * u kept in a fixed array of the library's own device memory,
 * W8A8_SVDQ_NOALLOC_SCRATCH_BYTES (4 MiB) per GPU, held from the library's
 * load on that GPU until the process ends.  Allocates nothing.
 *   Arguments as svdq_linear, without workspace.
 *   Limit: svdq_workspace_bytes(M, r) <= W8A8_SVDQ_NOALLOC_SCRATCH_BYTES,
 *   i.e. M * roundup(r, 16) <= 2^20 (M <= 32768 at r = 32), else
 *   W8A8_ERR_SCRATCH_LIMIT (checked before anything is launched).
 *   `stream` must belong to the current device (else W8A8_ERR_INVALID_ARG).
 * Every call on one GPU uses that GPU's one array: calls that overlap on a
 * GPU (different streams, or host threads) race and give undefined results;
 * calls ordered on one stream are safe.  The array keeps the last call's u,
 * which every call overwrites in full before reading it.
 */
#define W8A8_SVDQ_NOALLOC_SCRATCH_BYTES (4 * 1024 * 1024)
w8a8_status svdq_linear_noalloc(w8a8_qtype qtype, const uint16_t *x, int64_t M, int64_t K, const void *rq,
                                const float *r_scale, const uint16_t *l1, const uint16_t *l2, int64_t r,
                                const uint16_t *bias, int64_t N, uint16_t *y, void *xq_out, float *x_scale_out,
                                hipStream_t stream);

/*
 * SVDQuant weight preparation (OneTrainer PR #1034 "SVDQuant"; wiki SVDQuant:
 * bf16 factors, rank 16-32): the rank-r truncated SVD of W, W_r = U_r S_r V_r^T,
 * stored balanced in the layout svdq_linear takes,
 *   l2 = bf16(U_r S_r^(1/2))  [N, r],   l1 = bf16(S_r^(1/2) V_r^T)  [r, K],
 * and the residual R = bf16(W - l2 . l1) [N, K] (to be quantized with
 * w8a8_quant_weight_tensorwise); sigma f32 [r] = the singular values found.
 * The SVD is computed by randomized subspace iteration (Halko, Martinsson,
 * Tropp 2011) with `iters` power iterations (0..16) in a subspace of
 * s = svdq_prepare_subspace(r) columns, started from the caller's Gaussian
 * test matrix omega bf16 [s, K] (the method's random draw, an input).  The
 * result approximates the exact truncated SVD; the error shrinks with iters
 * and with the gap between sigma_r and sigma_{s+1}.
 *   w bf16 [N, K]; workspace svdq_prepare_workspace_bytes(N, K, r) bytes
 *   (about 2 N K + 8 (N + K) s bytes).
 * Shape rules: 1 <= r <= 64, r <= N, r <= K, N % 8 == K % 8 == 0,
 * N, K < 2^24, N * K <= 2^31; else W8A8_ERR_INVALID_ARG (r, iters) or
 * W8A8_ERR_SHAPE.
 */
int64_t svdq_prepare_subspace(int64_t r);
size_t svdq_prepare_workspace_bytes(int64_t N, int64_t K, int64_t r);
w8a8_status svdq_prepare(const uint16_t *w, int64_t N, int64_t K, int64_t r, const uint16_t *omega, int iters,
                         uint16_t *l1, uint16_t *l2, uint16_t *residual, float *sigma, void *workspace,
                         hipStream_t stream);

/* -------------------------------------------------------------------- Q8_0 */

/* Size in bytes of n values in GGUF Q8_0 blocks: 34 * ceil(n / 32) (struct
 * Q8_0: each block holds 32 values in 34 bytes, a 2-byte scale then 32 codes).
 * Returns 0 for n < 0. */
size_t q8_0_nbytes(int64_t n);

/*
 * Q8_0::quantize: for each block of 32 values (the last one may be partial),
 * s = absmax scale of the block's real values (int8 rule above), codes from
 * the f32 s, the block written as {f16 d = f16_rne(s), int8 qs[32]} in 34
 * bytes (d little-endian first); pad codes of a partial last block are 0.
 *   x f32 [n]; blocks q8_0_nbytes(n) bytes.
 */
w8a8_status q8_0_quantize(const float *x, int64_t n, void *blocks, hipStream_t stream);

/*
 * Q8_0::dequantize with the stored f16 scale: y[i] = f32(qs[i]) * f32(d) of
 * block i / 32 (an exact product).  blocks q8_0_nbytes(n) bytes; y f32 [n].
 */
w8a8_status q8_0_dequantize(const void *blocks, int64_t n, float *y, hipStream_t stream);

/* ---------------------------------------------------------------- Hadamard */

/*
 * Hadamard rotation before quantization (diffusers "SDNQ" overview names it;
 * the definition is the standard one, not the pages'): K is cut into blocks of
 * b = min(1024, largest power of two dividing K) and each block of a row is
 * multiplied by the normalized Sylvester Walsh-Hadamard matrix H_b / sqrt(b),
 * which is orthogonal and symmetric: rotating X and W alike leaves X W^T
 * unchanged.  Evaluated as the fast transform in f32 (stages h = 1, 2, ...,
 * b/2: (x[i], x[i+h]) -> (x[i] + x[i+h], x[i] - x[i+h]) for bit h of i clear),
 * then times c = f32(1 / sqrt(b)); bit-reproducible.
 *
 * w8a8_quant_act_rowwise_hadamard: as w8a8_quant_act_rowwise, on the rotated
 * rows (the shared absmax rule on the f32 rotated values).  K % 16 == 0,
 * 0 < K <= 2^30.
 * w8a8_hadamard_rotate: out bf16 [M, ldo] = the rotated rows of x rounded to
 * bf16 (for the weight, which is then quantized as any weight).  K % 16 == 0,
 * K <= 2^30, ldx >= K, ldo >= K.
 */
w8a8_status w8a8_quant_act_rowwise_hadamard(w8a8_qtype qtype, const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                                            void *xq, int64_t ldq, float *x_scale, hipStream_t stream);
w8a8_status w8a8_hadamard_rotate(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, uint16_t *out, int64_t ldo,
                                 hipStream_t stream);

/* ----------------------------------------------------------------- GGUF A8 */

/*
 * GGUF A8 weight preparation (wiki "Quantization", GGUF A8 int / GGUF A8
 * float, "Technical": weights re-quantized from GGUF to int8 / float8 e4m3
 * axis-wise).  The GGUF weight is Q8_0: row n of W [N, K] is K / 32
 * consecutive 34-byte blocks (as q8_0_quantize lays out N * K values), and
 * its values are the exact dequantization f32(q) * f32(d).  Per row n:
 *   w_scale[n] = absmax scale of the row's values (shared rules, QMAX of qtype)
 *   wq[n, k]   = code of value k (shared rules)
 *   blocks N * (K / 32) * 34 bytes; wq codes [N, K]; w_scale f32 [N].
 * Shape rules: K % 32 == 0 and the block bytes below 2^31, else
 * W8A8_ERR_SHAPE.  K == 0 gives the floor scale 1e-10 for every row.
 */
w8a8_status gguf_a8_requant_q8_0(w8a8_qtype qtype, const void *blocks, int64_t N, int64_t K, void *wq,
                                 float *w_scale, hipStream_t stream);

/*
 * GGUF A8 linear: as w8a8_linear with one weight scale per output channel,
 *   y[m, n] = bf16(acc[m, n] * x_scale[m] * w_scale[n] + bias[n])
 *   xq codes [M, K] (w8a8_quant_act_rowwise), x_scale f32 [M]; wq codes
 *   [N, K] and w_scale f32 [N] (gguf_a8_requant_q8_0); bias bf16 [N] or NULL;
 *   y bf16 [M, N].  Shape rules as w8a8_linear.
 */
w8a8_status gguf_a8_linear(w8a8_qtype qtype, const void *xq, const float *x_scale, const void *wq,
                           const float *w_scale, const uint16_t *bias, int64_t M, int64_t N, int64_t K, uint16_t *y,
                           hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* W8A8_H_ */
