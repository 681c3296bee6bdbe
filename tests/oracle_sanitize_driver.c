/* Calls every function of the CPU oracle (oracle/w8a8_oracle.c) on small,
 * ragged and degenerate inputs, for a build with the host address and
 * undefined-behaviour sanitizers (tests/test_oracle_sanitizers.py).  Exits 0
 * when every call returns its expected status; the sanitizers abort on any
 * out-of-bounds access or undefined operation. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double orc_bf16_to_f64(uint16_t b);
double orc_f16_to_f64(uint16_t h);
double orc_e4m3_to_f64(uint8_t c);
uint16_t orc_f64_to_bf16(double v);
uint16_t orc_f32_to_bf16(float v);
uint16_t orc_f64_to_f16(double v);
uint16_t orc_f32_to_f16(float v);
uint8_t orc_f64_to_e4m3(double v);
uint8_t orc_f32_to_e4m3(float v);
float orc_absmax_scale(float amax, float qmax);
int8_t orc_code_int8(float x, float s);
uint8_t orc_code_e4m3(float x, float s);
int orc_quant_act_rowwise(int qtype, const uint16_t *x, int64_t M, int64_t K, int64_t ldx, uint8_t *q,
                          int64_t ldq, float *scale);
int orc_quant_weight_tensorwise(int qtype, const uint16_t *w, int64_t N, int64_t K, uint8_t *q, uint8_t *qt,
                                float *scale);
int orc_gemm_i32(const int8_t *xq, const int8_t *wq, int64_t M, int64_t N, int64_t K, int32_t *acc);
int orc_linear(int qtype, const uint8_t *xq, const float *sx, const uint8_t *wq, float sw, const uint16_t *bias,
               int64_t M, int64_t N, int64_t K, uint16_t *y);
int orc_linear_backward_dx(int qtype, const uint8_t *dyq, const float *sdy, const uint8_t *wq, float sw, int64_t M,
                           int64_t N, int64_t K, uint16_t *dx);
int orc_svdq_linear(int qtype, const uint16_t *x, int64_t M, int64_t K, const uint8_t *rq, float sr,
                    const uint16_t *l1, const uint16_t *l2, int64_t r, const uint16_t *bias, int64_t N, uint16_t *y,
                    uint8_t *xq_out, float *sx_out, double *u_work);
int64_t orc_q8_0_nbytes(int64_t n);
int orc_q8_0_quantize(const float *x, int64_t n, uint8_t *blocks);
int orc_q8_0_dequantize(const uint8_t *blocks, int64_t n, float *y);
int orc_gguf_a8_requant_q8_0(int qtype, const uint8_t *blocks, int64_t N, int64_t K, uint8_t *wq, float *scale,
                             float *v_work);
int orc_linear_axiswise(int qtype, const uint8_t *xq, const float *sx, const uint8_t *wq, const float *sw,
                        const uint16_t *bias, int64_t M, int64_t N, int64_t K, uint16_t *y);
int64_t orc_hadamard_block(int64_t K);
int orc_hadamard_rows_f32(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, float *out);
int orc_quant_act_rowwise_hadamard(int qtype, const uint16_t *x, int64_t M, int64_t K, int64_t ldx, uint8_t *q,
                                   int64_t ldq, float *scale, float *work);
int orc_convert_array(int kind, const void *in, int64_t n, void *out);

static int failures = 0;
#define EXPECT(cond)                                                   \
    do {                                                               \
        if (!(cond)) {                                                 \
            fprintf(stderr, "failed: %s (line %d)\n", #cond, __LINE__); \
            ++failures;                                                \
        }                                                              \
    } while (0)

static uint32_t rng_state = 12345u;
static float frand(void) { /* xorshift32, uniform in [-1, 1) */
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 17;
    rng_state ^= rng_state << 5;
    return (float)((double)rng_state / 2147483648.0 - 1.0);
}
static uint16_t *bf16_matrix(int64_t rows, int64_t ld, float scale) {
    uint16_t *p = malloc(sizeof(uint16_t) * (size_t)(rows * ld > 0 ? rows * ld : 1));
    for (int64_t i = 0; i < rows * ld; ++i) p[i] = orc_f32_to_bf16(frand() * scale);
    return p;
}

int main(void) {
    /* formats: every code, and doubles around the edges */
    for (uint32_t c = 0; c < 65536; ++c) {
        double b = orc_bf16_to_f64((uint16_t)c), h = orc_f16_to_f64((uint16_t)c);
        if (!isnan(b)) (void)orc_f64_to_bf16(b);
        if (!isnan(h)) (void)orc_f64_to_f16(h);
    }
    for (uint32_t c = 0; c < 256; ++c) (void)orc_f64_to_e4m3(orc_e4m3_to_f64((uint8_t)c));
    const double edge[] = {0.0, -0.0, 1e-300, -1e-300, 1e300, -1e300, INFINITY, -INFINITY, NAN, 65520.0, 448.0, 464.0};
    for (size_t i = 0; i < sizeof edge / sizeof edge[0]; ++i) {
        (void)orc_f64_to_bf16(edge[i]);
        (void)orc_f64_to_f16(edge[i]);
        (void)orc_f64_to_e4m3(edge[i]);
        (void)orc_f32_to_bf16((float)edge[i]);
    }
    {
        float fin[64];
        double din[64];
        uint16_t u16[64];
        uint8_t u8[64];
        double dout[64];
        for (int i = 0; i < 64; ++i) fin[i] = frand() * 300.0f, din[i] = fin[i], u16[i] = (uint16_t)(i * 997), u8[i] = (uint8_t)(i * 4);
        for (int k = 0; k <= 5; ++k) EXPECT(orc_convert_array(k, k % 2 ? (const void *)din : (const void *)fin, 64, dout) == 0);
        EXPECT(orc_convert_array(6, u16, 64, dout) == 0);
        EXPECT(orc_convert_array(7, u16, 64, dout) == 0);
        EXPECT(orc_convert_array(8, u8, 64, dout) == 0);
        EXPECT(orc_convert_array(9, u8, 64, dout) != 0);
        EXPECT(orc_convert_array(0, fin, -1, dout) != 0);
    }
    EXPECT(orc_absmax_scale(0.0f, 127.0f) == 1e-10f);
    (void)orc_code_int8(1.5f, 1.0f);
    (void)orc_code_e4m3(-1000.0f, 1.0f);

    for (int qt = 0; qt < 2; ++qt) {
        /* act-quant with padded strides and an all-zero row */
        const int64_t M = 5, K = 37, ldx = 40, ldq = 48;
        uint16_t *x = bf16_matrix(M, ldx, 3.0f);
        for (int64_t k = 0; k < ldx; ++k) x[2 * ldx + k] = 0;
        uint8_t *q = malloc((size_t)(M * ldq));
        float *s = malloc(sizeof(float) * M);
        EXPECT(orc_quant_act_rowwise(qt, x, M, K, ldx, q, ldq, s) == 0);
        EXPECT(orc_quant_act_rowwise(qt, x, M, K, K - 1, q, ldq, s) != 0);
        EXPECT(orc_quant_act_rowwise(qt, x, 0, K, ldx, q, ldq, s) == 0);
        float *work = malloc(sizeof(float) * K);
        EXPECT(orc_quant_act_rowwise_hadamard(qt, x, M, 48 > ldx ? 32 : 48, ldx, q, ldq, s, work) == 0);
        free(work);
        free(x), free(q), free(s);

        /* weight quant (+ transposed), products, backward, axis-wise */
        const int64_t N = 7, Kw = 24, Mx = 3;
        uint16_t *w = bf16_matrix(N, Kw, 0.05f);
        uint16_t *xx = bf16_matrix(Mx, Kw, 2.0f);
        uint8_t *wq = malloc((size_t)(N * Kw)), *wqt = malloc((size_t)(N * Kw)), *xq = malloc((size_t)(Mx * Kw));
        float sw, *sx = malloc(sizeof(float) * Mx), *swv = malloc(sizeof(float) * N);
        EXPECT(orc_quant_weight_tensorwise(qt, w, N, Kw, wq, wqt, &sw) == 0);
        EXPECT(orc_quant_weight_tensorwise(qt, w, N, Kw, wq, NULL, &sw) == 0);
        EXPECT(orc_quant_act_rowwise(qt, xx, Mx, Kw, Kw, xq, Kw, sx) == 0);
        uint16_t *bias = bf16_matrix(1, N, 0.1f), *y = malloc(sizeof(uint16_t) * (size_t)(Mx * N));
        uint16_t *dx = malloc(sizeof(uint16_t) * (size_t)(Mx * Kw));
        EXPECT(orc_linear(qt, xq, sx, wq, sw, bias, Mx, N, Kw, y) == 0);
        EXPECT(orc_linear(qt, xq, sx, wq, sw, NULL, Mx, N, Kw, y) == 0);
        for (int64_t n = 0; n < N; ++n) swv[n] = sw * (1.0f + 0.1f * (float)n);
        EXPECT(orc_linear_axiswise(qt, xq, sx, wq, swv, bias, Mx, N, Kw, y) == 0);
        uint8_t *dyq = malloc((size_t)(Mx * N));
        float *sdy = malloc(sizeof(float) * Mx);
        uint16_t *dy = bf16_matrix(Mx, N, 1e-3f);
        EXPECT(orc_quant_act_rowwise(qt, dy, Mx, N, N, dyq, N, sdy) == 0);
        EXPECT(orc_linear_backward_dx(qt, dyq, sdy, wq, sw, Mx, N, Kw, dx) == 0);
        EXPECT(orc_linear(qt, xq, sx, wq, sw, bias, -1, N, Kw, y) != 0);
        if (qt == 0) {
            int32_t *acc = malloc(sizeof(int32_t) * (size_t)(Mx * N));
            EXPECT(orc_gemm_i32((const int8_t *)xq, (const int8_t *)wq, Mx, N, Kw, acc) == 0);
            free(acc);
        }
        /* SVDQuant with r = 5 */
        const int64_t r = 5;
        uint16_t *l1 = bf16_matrix(r, Kw, 0.1f), *l2 = bf16_matrix(N, r, 0.1f);
        double *u = malloc(sizeof(double) * r);
        EXPECT(orc_svdq_linear(qt, xx, Mx, Kw, wq, sw, l1, l2, r, bias, N, y, xq, sx, u) == 0);
        EXPECT(orc_svdq_linear(qt, xx, Mx, Kw, wq, sw, l1, l2, 0, NULL, N, y, xq, sx, u) == 0);
        free(l1), free(l2), free(u);
        free(w), free(xx), free(wq), free(wqt), free(xq), free(sx), free(swv), free(bias), free(y), free(dx);
        free(dyq), free(sdy), free(dy);

        /* GGUF A8: Q8_0 blocks of a [3, 64] weight, re-quantized per row */
        const int64_t Ng = 3, Kg = 64;
        float *vals = malloc(sizeof(float) * (size_t)(Ng * Kg));
        for (int64_t i = 0; i < Ng * Kg; ++i) vals[i] = frand() * 0.1f;
        uint8_t *blocks = malloc((size_t)orc_q8_0_nbytes(Ng * Kg));
        EXPECT(orc_q8_0_quantize(vals, Ng * Kg, blocks) == 0);
        uint8_t *gq = malloc((size_t)(Ng * Kg));
        float *gs = malloc(sizeof(float) * Ng), *vw = malloc(sizeof(float) * Kg);
        EXPECT(orc_gguf_a8_requant_q8_0(qt, blocks, Ng, Kg, gq, gs, vw) == 0);
        EXPECT(orc_gguf_a8_requant_q8_0(qt, blocks, Ng, 48, gq, gs, vw) != 0);
        free(vals), free(blocks), free(gq), free(gs), free(vw);
    }

    /* Q8_0 with partial last blocks and n = 0 */
    const int64_t ns[] = {0, 1, 31, 32, 33, 37, 100};
    for (size_t i = 0; i < sizeof ns / sizeof ns[0]; ++i) {
        const int64_t n = ns[i];
        float *v = malloc(sizeof(float) * (size_t)(n > 0 ? n : 1)), *back = malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
        for (int64_t j = 0; j < n; ++j) v[j] = frand() * 50.0f;
        uint8_t *b = malloc((size_t)(orc_q8_0_nbytes(n) > 0 ? orc_q8_0_nbytes(n) : 1));
        EXPECT(orc_q8_0_quantize(v, n, b) == 0);
        EXPECT(orc_q8_0_dequantize(b, n, back) == 0);
        free(v), free(back), free(b);
    }
    EXPECT(orc_q8_0_nbytes(-1) < 0);

    /* Hadamard rows: b = 16, 1024 and a ragged stride */
    const int64_t Ks[] = {16, 48, 1024, 2080};
    for (size_t i = 0; i < sizeof Ks / sizeof Ks[0]; ++i) {
        const int64_t K = Ks[i], M = 3, ld = K + 8;
        uint16_t *x = bf16_matrix(M, ld, 1.0f);
        float *out = malloc(sizeof(float) * (size_t)(M * K));
        EXPECT(orc_hadamard_block(K) > 0);
        EXPECT(orc_hadamard_rows_f32(x, M, K, ld, out) == 0);
        uint8_t *q = malloc((size_t)(M * K));
        float *s = malloc(sizeof(float) * M), *work = malloc(sizeof(float) * K);
        EXPECT(orc_quant_act_rowwise_hadamard(1, x, M, K, ld, q, K, s, work) == 0);
        free(x), free(out), free(q), free(s), free(work);
    }
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("oracle sanitizer driver: all calls ok\n");
    return 0;
}
