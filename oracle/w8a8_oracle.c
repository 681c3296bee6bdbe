/*
 * w8a8_oracle.c -- plain, slow, obviously-correct CPU oracle for the W8A8
 * quantized-linear path.  TEST INFRASTRUCTURE ONLY: it is linked by the tests,
 * by the smoke check and by the CPU-baseline leg of the benchmark, never by the
 * product library, and it shares no code with the HIP path.
 *
 * Sources (the pages this follows):
 *  - OneTrainer wiki "Quantization", the "Technical" entries of the float W8A8
 *    and int W8A8 types: tensor-wise weight quantization (int8 or float8 e4m3),
 *    activations quantized token-wise, matmul done in 8 bits.
 *  - OneTrainer PR #1034 "New quant types, activation quantization", sections
 *    "W8A8 quant types" and "SVDQuant".
 *  - bitsandbytes #1401 "LLM.int8() Refactoring: Part 1", "Enhancements": a
 *    fused row-wise scale calibration + quantization (absmax over rows).
 *  - entrenar 0.7.8 src/quant/gguf_quant/q8_0.rs: struct Q8_0, Q8_0::quantize
 *    (block absmax, scale = absmax/127 floored at 1e-10, divide, round, clamp
 *    to [-128,127], zero padding of the last block) and Q8_0::dequantize.
 *
 * Readings where the pages leave a step open (each one listed in the design
 * notes of the repository):
 *  - rounding to integer is round-half-to-even (the Q8_0 page's Rust `round`
 *    rounds halves away from zero; the engine's contract fixes RNE);
 *  - the 1e-10 floor of the Q8_0 scale is used for every absmax quantizer;
 *  - fp8 means OCP E4M3FN (max finite 448, no infinities), QMAX = 448, and the
 *    quotient is clamped to [-448, 448] before it is rounded to e4m3;
 *  - Q8_0 codes are computed from the f32 scale; the stored block scale is
 *    f16(scale) (the page keeps f32 scales and converts them to f16 when it
 *    writes the GGUF blocks); dequantize uses the stored f16 scale;
 *  - the dequantized linear output is bf16(acc * sx[m] * sw + bias[n]) with the
 *    right-hand side evaluated in double and rounded to bf16 once;
 *  - the SVDQuant branch adds (X . L1^T) . L2^T, both products in double;
 *  - GGUF A8: the GGUF weight is Q8_0 (the one GGUF format the pages define),
 *    "axis-wise" for the weight means one scale per output channel (row of
 *    W [out, in]), and the row's values are the exact Q8_0 dequantization.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -shared -fPIC.  Every
 * rounding named below happens exactly once; exact sums run in int64 / double.
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include <math.h>

#define ORC_OK 0
#define ORC_ERR 1

/* ------------------------------------------------------------------------- */
/* Number formats.  Each format is decoded by its definition; encoding to it is */
/* the nearest representable value, ties going to the even code, found by a     */
/* binary search over the monotone code space and a comparison with the exact   */
/* midpoint (which double holds exactly for all three formats).                 */
/* ------------------------------------------------------------------------- */

/* bf16: 1 sign, 8 exponent (bias 127), 7 mantissa bits; the top half of f32. */
double orc_bf16_to_f64(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 mantissa bits. */
double orc_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0x1f) v = m ? NAN : INFINITY;
    else if (e == 0) v = ldexp((double)m, -24);            /* subnormal: m * 2^-24 */
    else v = ldexp(1.0 + m / 1024.0, e - 15);
    return sign ? -v : v;
}

/* OCP FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits, no infinities,
 * S.1111.111 is NaN, max finite 448 (0x7E), subnormals 2^-6 * m/8. */
double orc_e4m3_to_f64(uint8_t c) {
    int sign = (c >> 7) & 1;
    int e = (c >> 3) & 0xf;
    int m = c & 7;
    double v;
    if (e == 0xf && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m / 8.0, -6);
    else v = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -v : v;
}

/* Nearest code to |v| among the non-negative codes 0..top, whose values are
 * strictly increasing; `val(top)` may stand for the first value beyond the
 * finite range (an overflow sentinel).  Ties go to the even code. */
static uint32_t nearest_code(double a, uint32_t top, double (*val)(uint32_t)) {
    uint32_t lo = 0, hi = top;
    if (a >= val(top)) return top;
    /* invariant: val(lo) <= a < val(hi) */
    while (hi - lo > 1) {
        uint32_t mid = lo + (hi - lo) / 2;
        if (val(mid) <= a) lo = mid; else hi = mid;
    }
    double vlo = val(lo), vhi = val(hi);
    double midpoint = (vlo + vhi) * 0.5;                 /* exact in double */
    if (a < midpoint) return lo;
    if (a > midpoint) return hi;
    return (lo % 2 == 0) ? lo : hi;
}

/* bf16 codes 0x0000..0x7F7F are finite; 0x7F80 (inf) is treated as the value
 * 2^128 for rounding, which is how IEEE rounding decides overflow. */
static double bf16_code_val(uint32_t c) {
    if (c == 0x7F80u) return ldexp(1.0, 128);
    return orc_bf16_to_f64((uint16_t)c);
}
uint16_t orc_f64_to_bf16(double v) {
    if (isnan(v)) return 0x7FC0;
    uint16_t s = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isinf(a)) return (uint16_t)(s | 0x7F80);
    return (uint16_t)(s | nearest_code(a, 0x7F80u, bf16_code_val));
}
uint16_t orc_f32_to_bf16(float v) { return orc_f64_to_bf16((double)v); }

/* f16 codes 0x0000..0x7BFF are finite; 0x7C00 (inf) stands for 2^16. */
static double f16_code_val(uint32_t c) {
    if (c == 0x7C00u) return 65536.0;
    return orc_f16_to_f64((uint16_t)c);
}
uint16_t orc_f64_to_f16(double v) {
    if (isnan(v)) return 0x7E00;
    uint16_t s = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isinf(a)) return (uint16_t)(s | 0x7C00);
    return (uint16_t)(s | nearest_code(a, 0x7C00u, f16_code_val));
}
uint16_t orc_f32_to_f16(float v) { return orc_f64_to_f16((double)v); }

/* e4m3 codes 0x00..0x7E are finite.  Code 0x7F is NaN; for rounding it stands
 * for 480 (the next value the exponent would give), so a magnitude that rounds
 * above 448 becomes NaN: E4M3FN has no infinity.  The quantizers below clamp to
 * [-448, 448] first, so they never reach that case. */
static double e4m3_code_val(uint32_t c) {
    if (c == 0x7Fu) return 480.0;
    return orc_e4m3_to_f64((uint8_t)c);
}
uint8_t orc_f64_to_e4m3(double v) {
    if (isnan(v)) return 0x7F;
    uint8_t s = signbit(v) ? 0x80 : 0;
    double a = fabs(v);
    if (isinf(a)) return (uint8_t)(s | 0x7F);
    return (uint8_t)(s | nearest_code(a, 0x7Fu, e4m3_code_val));
}
uint8_t orc_f32_to_e4m3(float v) { return orc_f64_to_e4m3((double)v); }

/* ------------------------------------------------------------------------- */
/* Scale and codes (shared rule of every absmax quantizer).                    */
/* ------------------------------------------------------------------------- */

/* entrenar Q8_0::quantize: scale = max_abs / 127, or 1e-10 when max_abs is
 * below 1e-10 (both f32).  QMAX is 127 for int8 and 448 for e4m3. */
float orc_absmax_scale(float amax, float qmax) {
    const float floor_ = 1e-10f;
    if (amax < floor_) return floor_;
    return amax / qmax;                                  /* one f32 rounding */
}

/* Round half to even, written out: |v| < 2^52 here, so v - floor(v) is exact. */
static double round_half_even(double v) {
    double f = floor(v);
    double d = v - f;
    if (d > 0.5) return f + 1.0;
    if (d < 0.5) return f;
    return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

/* int8 code: clamp(rne(fl32(x / s)), -128, 127). */
int8_t orc_code_int8(float x, float s) {
    float q = x / s;                                     /* one f32 rounding */
    double r = round_half_even((double)q);
    if (r < -128.0) r = -128.0;
    if (r > 127.0) r = 127.0;
    return (int8_t)r;
}

/* e4m3 code: e4m3_rne(clamp(fl32(x / s), -448, 448)). */
uint8_t orc_code_e4m3(float x, float s) {
    float q = x / s;
    if (q < -448.0f) q = -448.0f;
    if (q > 448.0f) q = 448.0f;
    return orc_f32_to_e4m3(q);
}

static float bf16_abs_f32(uint16_t b) { return (float)fabs(orc_bf16_to_f64(b)); }

/* ------------------------------------------------------------------------- */
/* Row-wise (token-wise) activation quantization.                              */
/* qtype 0 = int8, 1 = e4m3.  x: bf16 [M, ldx] (first K columns used);        */
/* q: [M, ldq] bytes, columns K..ldq-1 are written as zero; scale: f32 [M].   */
/* ------------------------------------------------------------------------- */
int orc_quant_act_rowwise(int qtype, const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                          uint8_t *q, int64_t ldq, float *scale) {
    if ((qtype != 0 && qtype != 1) || M < 0 || K < 0 || ldx < K || ldq < K) return ORC_ERR;
    const float qmax = qtype == 0 ? 127.0f : 448.0f;
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t *row = x + m * ldx;
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = bf16_abs_f32(row[k]);
            if (a > amax) amax = a;
        }
        float s = orc_absmax_scale(amax, qmax);
        scale[m] = s;
        for (int64_t k = 0; k < K; ++k) {
            float v = (float)orc_bf16_to_f64(row[k]);
            q[m * ldq + k] = qtype == 0 ? (uint8_t)orc_code_int8(v, s) : orc_code_e4m3(v, s);
        }
        for (int64_t k = K; k < ldq; ++k) q[m * ldq + k] = 0;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* Tensor-wise weight quantization: one scale for the whole W [N, K] (bf16).   */
/* q: [N, K] codes; qt (optional): the same codes transposed, [K, N].          */
/* ------------------------------------------------------------------------- */
int orc_quant_weight_tensorwise(int qtype, const uint16_t *w, int64_t N, int64_t K,
                                uint8_t *q, uint8_t *qt, float *scale) {
    if ((qtype != 0 && qtype != 1) || N < 0 || K < 0) return ORC_ERR;
    const float qmax = qtype == 0 ? 127.0f : 448.0f;
    float amax = 0.0f;
    for (int64_t i = 0; i < N * K; ++i) {
        float a = bf16_abs_f32(w[i]);
        if (a > amax) amax = a;
    }
    float s = orc_absmax_scale(amax, qmax);
    *scale = s;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            float v = (float)orc_bf16_to_f64(w[n * K + k]);
            uint8_t c = qtype == 0 ? (uint8_t)orc_code_int8(v, s) : orc_code_e4m3(v, s);
            q[n * K + k] = c;
            if (qt) qt[k * N + n] = c;
        }
    return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* 8-bit products.                                                             */
/* ------------------------------------------------------------------------- */

/* acc[m, n] = sum_k xq[m, k] * wq[n, k] (int8 codes, exact int64 sum).  Returns
 * ORC_ERR if any sum leaves the int32 range. */
int orc_gemm_i32(const int8_t *xq, const int8_t *wq, int64_t M, int64_t N, int64_t K, int32_t *acc) {
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k) s += (int64_t)xq[m * K + k] * (int64_t)wq[n * K + k];
            if (s > INT32_MAX || s < INT32_MIN) return ORC_ERR;
            acc[m * N + n] = (int32_t)s;
        }
    return ORC_OK;
}

/* Exact dot product of two code rows, as a double.  int8: exact integer sum.
 * e4m3: each decoded product is exact in double and so is the running sum:
 * products are multiples of 2^-18 below 448^2 < 2^18, so for K <= 65536 every
 * partial sum is a multiple of 2^-18 below 2^34, which needs 52 bits of
 * mantissa; the result is the exact real sum. */
static double code_dot(int qtype, const uint8_t *a, const uint8_t *b, int64_t K, int64_t stride_b) {
    if (qtype == 0) {
        int64_t s = 0;
        for (int64_t k = 0; k < K; ++k) s += (int64_t)(int8_t)a[k] * (int64_t)(int8_t)b[k * stride_b];
        return (double)s;
    }
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k) s += orc_e4m3_to_f64(a[k]) * orc_e4m3_to_f64(b[k * stride_b]);
    return s;
}

/* Quantized linear: y[m, n] = bf16(acc[m, n] * sx[m] * sw + bias[n]), acc the
 * exact code product over k, evaluated in double and rounded once. bias may be
 * NULL.  xq [M, K], wq [N, K], y bf16 [M, N]. */
int orc_linear(int qtype, const uint8_t *xq, const float *sx, const uint8_t *wq, float sw,
               const uint16_t *bias, int64_t M, int64_t N, int64_t K, uint16_t *y) {
    if ((qtype != 0 && qtype != 1) || M < 0 || N < 0 || K < 0) return ORC_ERR;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = code_dot(qtype, xq + m * K, wq + n * K, K, 1);
            double v = acc * (double)sx[m] * (double)sw;
            if (bias) v += orc_bf16_to_f64(bias[n]);
            y[m * N + n] = orc_f64_to_bf16(v);
        }
    return ORC_OK;
}

/* Input gradient of the quantized linear with frozen W: dX = dY . W, computed
 * from the row-wise quantized dY (dyq [M, N], sdy [M]) and the tensor-wise
 * quantized W (wq [N, K], sw), taken as stored (no transposed copy):
 * dx[m, k] = bf16(sum_n dyq[m, n] * wq[n, k] * sdy[m] * sw). */
int orc_linear_backward_dx(int qtype, const uint8_t *dyq, const float *sdy, const uint8_t *wq,
                           float sw, int64_t M, int64_t N, int64_t K, uint16_t *dx) {
    if ((qtype != 0 && qtype != 1) || M < 0 || N < 0 || K < 0) return ORC_ERR;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) {
            double acc = code_dot(qtype, dyq + m * N, wq + k, N, K);
            dx[m * K + k] = orc_f64_to_bf16(acc * (double)sdy[m] * (double)sw);
        }
    return ORC_OK;
}

/* SVDQuant-style linear: W ~ L2 . L1 + R with a bf16 low-rank pair
 * (l1 [r, K] down-projection, l2 [N, r] up-projection, both stored like
 * nn.Linear weights) and the residual R quantized tensor-wise (rq [N, K], sr).
 * Steps: quantize X row-wise (xq_out, sx_out); acc = codes(X) . codes(R);
 * u[m, j] = sum_k X[m, k] * L1[j, k]; low[m, n] = sum_j u[m, j] * L2[n, j];
 * y = bf16(acc * sx * sr + low + bias), all in double, rounded once. */
int orc_svdq_linear(int qtype, const uint16_t *x, int64_t M, int64_t K, const uint8_t *rq, float sr,
                    const uint16_t *l1, const uint16_t *l2, int64_t r, const uint16_t *bias,
                    int64_t N, uint16_t *y, uint8_t *xq_out, float *sx_out, double *u_work) {
    if ((qtype != 0 && qtype != 1) || M < 0 || N < 0 || K < 0 || r < 0) return ORC_ERR;
    if (orc_quant_act_rowwise(qtype, x, M, K, K, xq_out, K, sx_out) != ORC_OK) return ORC_ERR;
    for (int64_t m = 0; m < M; ++m) {
        double *u = u_work;                              /* [r] for this row */
        for (int64_t j = 0; j < r; ++j) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k) s += orc_bf16_to_f64(x[m * K + k]) * orc_bf16_to_f64(l1[j * K + k]);
            u[j] = s;
        }
        for (int64_t n = 0; n < N; ++n) {
            double acc = code_dot(qtype, xq_out + m * K, rq + n * K, K, 1);
            double low = 0.0;
            for (int64_t j = 0; j < r; ++j) low += u[j] * orc_bf16_to_f64(l2[n * r + j]);
            double v = acc * (double)sx_out[m] * (double)sr + low;
            if (bias) v += orc_bf16_to_f64(bias[n]);
            y[m * N + n] = orc_f64_to_bf16(v);
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* GGUF Q8_0 (entrenar q8_0.rs): 32 values -> 34 bytes, {f16 d; int8 qs[32]}.   */
/* ------------------------------------------------------------------------- */
#define ORC_Q8_0_BLOCK 32
#define ORC_Q8_0_BYTES 34

int64_t orc_q8_0_nbytes(int64_t n) {
    if (n < 0) return -1;
    return ORC_Q8_0_BYTES * ((n + ORC_Q8_0_BLOCK - 1) / ORC_Q8_0_BLOCK);
}

/* Q8_0::quantize, block by block: absmax of the block's real elements, scale
 * with the 1e-10 floor, codes = clamp(rne(x / scale)), pad codes of a partial
 * last block are 0, d = f16(scale) written little-endian before the codes. */
int orc_q8_0_quantize(const float *x, int64_t n, uint8_t *blocks) {
    if (n < 0) return ORC_ERR;
    int64_t nb = (n + ORC_Q8_0_BLOCK - 1) / ORC_Q8_0_BLOCK;
    for (int64_t b = 0; b < nb; ++b) {
        int64_t start = b * ORC_Q8_0_BLOCK;
        int64_t end = start + ORC_Q8_0_BLOCK < n ? start + ORC_Q8_0_BLOCK : n;
        float amax = 0.0f;
        for (int64_t i = start; i < end; ++i) {
            float a = fabsf(x[i]);
            if (a > amax) amax = a;
        }
        float s = orc_absmax_scale(amax, 127.0f);
        uint8_t *blk = blocks + b * ORC_Q8_0_BYTES;
        uint16_t d = orc_f32_to_f16(s);
        blk[0] = (uint8_t)(d & 0xff);
        blk[1] = (uint8_t)(d >> 8);
        for (int64_t i = start; i < start + ORC_Q8_0_BLOCK; ++i)
            blk[2 + (i - start)] = i < end ? (uint8_t)orc_code_int8(x[i], s) : 0;
    }
    return ORC_OK;
}

/* Q8_0::dequantize with the stored f16 scale: y[i] = f32(q[i]) * f32(d[i / 32]);
 * the product of an int8 and an f16 value is exact in f32. */
int orc_q8_0_dequantize(const uint8_t *blocks, int64_t n, float *y) {
    if (n < 0) return ORC_ERR;
    for (int64_t i = 0; i < n; ++i) {
        const uint8_t *blk = blocks + (i / ORC_Q8_0_BLOCK) * ORC_Q8_0_BYTES;
        uint16_t d = (uint16_t)(blk[0] | (blk[1] << 8));
        int8_t q = (int8_t)blk[2 + i % ORC_Q8_0_BLOCK];
        y[i] = (float)((double)q * orc_f16_to_f64(d));
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* GGUF A8 int / GGUF A8 float (OneTrainer wiki "Quantization", "Technical"):  */
/* the weight as stored in the GGUF file is re-quantized axis-wise to int8 or  */
/* e4m3 -- one scale per output channel, i.e. per row n of W [N, K] -- and the */
/* product runs in 8 bits on token-wise quantized activations.  Here the GGUF  */
/* weight is Q8_0: row n is K / 32 consecutive 34-byte blocks (K % 32 == 0).   */
/* ------------------------------------------------------------------------- */

/* Re-quantization of one Q8_0 row per output channel: the row's values are
 * the exact Q8_0 dequantization f32(q) * f32(d); s[n] = absmax scale of the row
 * (1e-10 floor, QMAX 127 or 448); codes as the other quantizers (int8:
 * clamp(rne(v / s)), e4m3: e4m3_rne(clamp(v / s, +-448))).  v_work: f32 [K]. */
int orc_gguf_a8_requant_q8_0(int qtype, const uint8_t *blocks, int64_t N, int64_t K,
                             uint8_t *wq, float *scale, float *v_work) {
    if ((qtype != 0 && qtype != 1) || N < 0 || K < 0 || K % ORC_Q8_0_BLOCK != 0) return ORC_ERR;
    const float qmax = qtype == 0 ? 127.0f : 448.0f;
    const int64_t row_bytes = (K / ORC_Q8_0_BLOCK) * ORC_Q8_0_BYTES;
    for (int64_t n = 0; n < N; ++n) {
        if (orc_q8_0_dequantize(blocks + n * row_bytes, K, v_work) != ORC_OK) return ORC_ERR;
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(v_work[k]);
            if (a > amax) amax = a;
        }
        float s = orc_absmax_scale(amax, qmax);
        scale[n] = s;
        for (int64_t k = 0; k < K; ++k)
            wq[n * K + k] = qtype == 0 ? (uint8_t)orc_code_int8(v_work[k], s) : orc_code_e4m3(v_work[k], s);
    }
    return ORC_OK;
}

/* Quantized linear with a per-output-channel weight scale:
 * y[m, n] = bf16(acc[m, n] * sx[m] * sw[n] + bias[n]), in double, rounded once. */
int orc_linear_axiswise(int qtype, const uint8_t *xq, const float *sx, const uint8_t *wq, const float *sw,
                        const uint16_t *bias, int64_t M, int64_t N, int64_t K, uint16_t *y) {
    if ((qtype != 0 && qtype != 1) || M < 0 || N < 0 || K < 0) return ORC_ERR;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = code_dot(qtype, xq + m * K, wq + n * K, K, 1);
            double v = acc * (double)sx[m] * (double)sw[n];
            if (bias) v += orc_bf16_to_f64(bias[n]);
            y[m * N + n] = orc_f64_to_bf16(v);
        }
    return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* Hadamard rotation before quantization (diffusers "SDNQ" overview: "Hadamard */
/* rotation"; named only there).  Definition used, from outside the pages: the  */
/* input dimension K is split into blocks of b = min(1024, largest power of two */
/* dividing K) and each block is multiplied by the normalized Sylvester         */
/* Walsh-Hadamard matrix H_b / sqrt(b) (orthogonal and symmetric, so rotating   */
/* both X and W leaves X W^T unchanged).  It is evaluated as the fast transform */
/* in f32: stages h = 1, 2, 4, ..., b/2, each replacing the pair (x[i],         */
/* x[i + h]) (i with bit h clear) by (x[i] + x[i + h], x[i] - x[i + h]), then   */
/* every value times c = f32(1 / sqrt(b)); one rounding per operation.         */
/* ------------------------------------------------------------------------- */
int64_t orc_hadamard_block(int64_t K) {
    if (K <= 0) return 0;
    int64_t b = 1;
    while (K % (b * 2) == 0 && b * 2 <= 1024) b *= 2;
    return b;
}

/* out f32 [M, K] = rotated rows of the bf16 x [M, ldx] (first K columns). */
int orc_hadamard_rows_f32(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, float *out) {
    if (M < 0 || K < 0 || ldx < K) return ORC_ERR;
    const int64_t b = orc_hadamard_block(K);
    const float c = (float)(1.0 / sqrt((double)b));
    for (int64_t m = 0; m < M; ++m) {
        float *o = out + m * K;
        for (int64_t k = 0; k < K; ++k) o[k] = (float)orc_bf16_to_f64(x[m * ldx + k]);
        for (int64_t blk = 0; blk < K; blk += b) {
            float *v = o + blk;
            for (int64_t h = 1; h < b; h *= 2)
                for (int64_t i = 0; i < b; ++i)
                    if ((i & h) == 0) {
                        const float a = v[i], d = v[i + h];
                        v[i] = a + d;
                        v[i + h] = a - d;
                    }
            for (int64_t i = 0; i < b; ++i) v[i] = v[i] * c;
        }
    }
    return ORC_OK;
}

/* Row-wise quantization of the rotated rows (the shared absmax rule on the f32
 * rotated values).  work: f32 [K]. */
int orc_quant_act_rowwise_hadamard(int qtype, const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                                   uint8_t *q, int64_t ldq, float *scale, float *work) {
    if ((qtype != 0 && qtype != 1) || M < 0 || K < 0 || ldx < K || ldq < K) return ORC_ERR;
    const float qmax = qtype == 0 ? 127.0f : 448.0f;
    for (int64_t m = 0; m < M; ++m) {
        if (orc_hadamard_rows_f32(x + m * ldx, 1, K, K, work) != ORC_OK) return ORC_ERR;
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(work[k]);
            if (a > amax) amax = a;
        }
        float s = orc_absmax_scale(amax, qmax);
        scale[m] = s;
        for (int64_t k = 0; k < K; ++k)
            q[m * ldq + k] = qtype == 0 ? (uint8_t)orc_code_int8(work[k], s) : orc_code_e4m3(work[k], s);
        for (int64_t k = K; k < ldq; ++k) q[m * ldq + k] = 0;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* Array forms of the scalar conversions above (same arithmetic, one call).    */
/* kind: 0 f32->bf16, 1 f64->bf16, 2 f32->f16, 3 f64->f16, 4 f32->e4m3,        */
/*       5 f64->e4m3, 6 bf16->f64, 7 f16->f64, 8 e4m3->f64.                     */
/* ------------------------------------------------------------------------- */
int orc_convert_array(int kind, const void *in, int64_t n, void *out) {
    if (n < 0) return ORC_ERR;
    for (int64_t i = 0; i < n; ++i) {
        switch (kind) {
        case 0: ((uint16_t *)out)[i] = orc_f32_to_bf16(((const float *)in)[i]); break;
        case 1: ((uint16_t *)out)[i] = orc_f64_to_bf16(((const double *)in)[i]); break;
        case 2: ((uint16_t *)out)[i] = orc_f32_to_f16(((const float *)in)[i]); break;
        case 3: ((uint16_t *)out)[i] = orc_f64_to_f16(((const double *)in)[i]); break;
        case 4: ((uint8_t *)out)[i] = orc_f32_to_e4m3(((const float *)in)[i]); break;
        case 5: ((uint8_t *)out)[i] = orc_f64_to_e4m3(((const double *)in)[i]); break;
        case 6: ((double *)out)[i] = orc_bf16_to_f64(((const uint16_t *)in)[i]); break;
        case 7: ((double *)out)[i] = orc_f16_to_f64(((const uint16_t *)in)[i]); break;
        case 8: ((double *)out)[i] = orc_e4m3_to_f64(((const uint8_t *)in)[i]); break;
        default: return ORC_ERR;
        }
    }
    return ORC_OK;
}
