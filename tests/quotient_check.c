/* Host check of the quotient the GPU quantizers compute (CPU only).
 *
 * The kernels form f32(x / s) from r = f32(1 / s) (a correctly rounded
 * division) with one Markstein correction:
 *     q0 = f32(x * r);  e = fma(-q0, s, x);  q = fma(e, r, q0)
 * (Muller et al., Handbook of Floating-Point Arithmetic, "Newton-Raphson-based
 * division"), then restore the sign of x with copysign.  The quantizers'
 * definition divides: code = rne(f32(x / s)) for int8, e4m3_rne(clamp(f32(x /
 * s), +-448)) for e4m3 (entrenar Q8_0::quantize divides each value by the
 * block scale).  This program checks that the corrected quotient equals the
 * IEEE f32 quotient:
 *
 *   mode "bf16": exhaustively, for both QMAX (127 and 448), for every finite
 *     positive bf16 absmax a (scale s = 1e-10 if a < 1e-10 else f32(a / QMAX))
 *     and every bf16 x with |x| <= a, both signs -- the inputs of the
 *     activation and weight quantizers, whose values and absmax are bf16.
 *   mode "f32 <n> <seed>": n random f32 pairs (x, s) with s = f32(a / QMAX)
 *     for a random f32 absmax a >= |x| (Q8_0, GGUF and the Hadamard-rotated
 *     values are f32, not bf16), drawn four ways: x uniform in [-a, a], x with
 *     a random exponent below a's, x a half-way point (k + 1/2) s nudged by
 *     up to 3 ulps, and x = a.
 *
 * In both modes, wherever |x / s| >= 2^-20 the quotient must be the IEEE one
 * bit for bit; below that both must be smaller than 2^-11 in magnitude with
 * the sign of x, so every int8 code (0) and e4m3 code (+-0) they decide is
 * the same.  (For subnormal x the residual e underflows and the last bits of
 * the quotient can differ; those quotients are below 2^-90.)
 *
 * Prints the number of pairs checked and of mismatches, and exits 1 on any
 * mismatch.  Build: gcc -O2 -ffp-contract=off [-fopenmp] (fmaf is the
 * correctly rounded fused multiply-add of C99). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float bits_f32(uint32_t u) {
    float f;
    memcpy(&f, &u, 4);
    return f;
}
static uint32_t f32_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

static float scale_of(float amax, float qmax) { return amax < 1e-10f ? 1e-10f : amax / qmax; }

static float corrected_quotient(float x, float s, float r) {
    float q0 = x * r;
    float e = fmaf(-q0, s, x);
    return copysignf(fmaf(e, r, q0), x);
}

/* The quotient agrees with the IEEE one when it is bit-identical, or, for an
 * IEEE quotient below 2^-20 in magnitude, when both are below 2^-11 with the
 * sign of x (then every int8 code, 0, and e4m3 code, +-0, they decide is the
 * same).  *tiny_diff is set for such a pair whose last bits differ. */
static int agree(float x, float got, float want, int *tiny_diff) {
    if (f32_bits(got) == f32_bits(want)) return 1;
    if (fabsf(want) >= 0x1p-20f) return 0;
    *tiny_diff = 1;
    return fabsf(got) < 0x1p-11f && fabsf(want) < 0x1p-11f && signbit(got) == signbit(x) &&
           signbit(want) == signbit(x);
}

static long long check_bf16(float qmax, long long *pairs, long long *tiny) {
    long long bad = 0, n = 0, nt = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : bad, n, nt)
    for (uint32_t ab = 0x0001; ab <= 0x7F7F; ++ab) {
        const float a = bits_f32(ab << 16);
        const float s = scale_of(a, qmax);
        const float r = 1.0f / s;
        for (uint32_t xb = 0; xb <= ab; ++xb) {
            for (uint32_t sign = 0; sign <= 0x8000; sign += 0x8000) {
                const float x = bits_f32((xb | sign) << 16);
                const float want = x / s;
                const float got = corrected_quotient(x, s, r);
                int td = 0;
                ++n;
                if (!agree(x, got, want, &td)) {
                    if (bad < 5)
                        printf("mismatch qmax %g: x %a s %a got %a want %a\n", qmax, x, s, got, want);
                    ++bad;
                }
                nt += td;
            }
        }
    }
    *pairs += n;
    *tiny += nt;
    return bad;
}

/* splitmix64 (Steele, Lea, Flood 2014) */
static uint64_t sm_state;
static uint64_t next_u64(void) {
    uint64_t z = (sm_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static double unit(void) { return (double)(next_u64() >> 11) * (1.0 / 9007199254740992.0); }

static long long check_f32(long long count, uint64_t seed, long long *pairs, long long *tiny) {
    sm_state = seed;
    long long bad = 0;
    for (long long i = 0; i < count; ++i) {
        const float qmax = (i & 1) ? 448.0f : 127.0f;
        /* absmax: random mantissa, exponent in [-90, 100] (scales stay normal) */
        const int ea = (int)(next_u64() % 191) - 90;
        const float a = ldexpf(1.0f + (float)unit(), ea);
        const float s = scale_of(a, qmax);
        const float r = 1.0f / s;
        float x;
        switch ((i >> 1) & 3) {
            case 0:
                x = (float)((2.0 * unit() - 1.0) * (double)a);
                break;
            case 1:
                x = ldexpf((float)(1.0 + unit()), ea - 1 - (int)(next_u64() % 40));
                if (next_u64() & 1) x = -x;
                break;
            case 2: {
                const int k = (int)(next_u64() % (uint64_t)qmax);
                x = (float)(((double)k + 0.5) * (double)s);
                const int nudge = (int)(next_u64() % 7) - 3;
                for (int j = 0; j < abs(nudge); ++j) x = nextafterf(x, nudge > 0 ? INFINITY : 0.0f);
                if (fabsf(x) > a) x = a;
                if (next_u64() & 1) x = -x;
                break;
            }
            default:
                x = (next_u64() & 1) ? a : -a;
                break;
        }
        const float want = x / s;
        const float got = corrected_quotient(x, s, r);
        int td = 0;
        if (!agree(x, got, want, &td)) {
            if (bad < 5) printf("mismatch qmax %g: x %a s %a got %a want %a\n", qmax, x, s, got, want);
            ++bad;
        }
        *tiny += td;
    }
    *pairs += count;
    return bad;
}

int main(int argc, char **argv) {
    long long pairs = 0, bad = 0, tiny = 0;
    if (argc >= 2 && strcmp(argv[1], "bf16") == 0) {
        bad += check_bf16(127.0f, &pairs, &tiny);
        bad += check_bf16(448.0f, &pairs, &tiny);
    } else if (argc >= 4 && strcmp(argv[1], "f32") == 0) {
        bad += check_f32(atoll(argv[2]), strtoull(argv[3], NULL, 10), &pairs, &tiny);
    } else {
        fprintf(stderr, "usage: %s bf16 | f32 <pairs> <seed>\n", argv[0]);
        return 2;
    }
    printf("pairs %lld mismatches %lld tiny_last_bit_differences %lld\n", pairs, bad, tiny);
    return bad == 0 ? 0 : 1;
}
