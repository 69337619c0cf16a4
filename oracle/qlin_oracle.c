/*
 * qlin_oracle.c -- plain CPU reference for the quantized skinny linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the GPU library includes, links or
 * calls this file; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load it.  It is written for a reader to check by eye, not
 * for speed: straight loops, fp64 where the result is floating point, no
 * blocking, no reordering.  The one concession to run time is an OpenMP
 * "parallel for" over output channels, which does not change any result
 * (every output is computed by one thread, in the same order).
 *
 * Source: "Building a High-Performance and Portable vLLM Linear Backend with
 * Helion", section "Scope" (the three formats) and section "Kernel
 * Implementation" (one product out = a @ b for every schedule, float32
 * accumulator).  Readings of what the pages leave open are listed at each
 * function.
 */
#include "qlin_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define E4M3_MAX 448.0
#define INT8_QMAX 127.0f
#define FP8_QMAX 448.0f
#define GROUP 128

/* ---------------------------------------------------------------- fp8 E4M3 */

/* OCP E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.
 * Exponent field 0 is subnormal: m * 2^-9.  Otherwise (1 + m/8) * 2^(e-7).
 * The pattern with exponent 15 and mantissa 7 is NaN; there is no infinity,
 * so the largest finite magnitude is 1.75 * 2^8 = 448 (code 0x7E). */
double orc_e4m3_decode(uint8_t code) {
    int sign = code >> 7;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -v : v;
}

/* fp32 -> E4M3FN.  Reading of the pages' plain "FP8": saturate to +-448 first,
 * then round to the nearest representable value, ties to the even mantissa;
 * values below the normal range become subnormals (no flush), and the sign is
 * kept, so a negative value that rounds to zero gives 0x80. */
int orc_e4m3_encode(float v, uint8_t *code) {
    if (!isfinite(v)) return -1;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a > E4M3_MAX) a = E4M3_MAX;

    /* binade of a: a in [2^E, 2^(E+1)); below 2^-6 the spacing stays 2^-9 */
    int E = -6;
    if (a >= ldexp(1.0, -6)) {
        int e2;
        frexp(a, &e2);          /* a = f * 2^e2 with f in [0.5, 1) */
        E = e2 - 1;
    }
    double quantum = ldexp(1.0, E - 3);      /* spacing of 3-bit mantissas */
    double r = nearbyint(a / quantum);        /* a / quantum is exact; RNE */
    double val = r * quantum;                 /* exact, <= 448 */

    uint8_t mag;
    if (val == 0.0) {
        mag = 0;
    } else if (val < ldexp(1.0, -6)) {        /* subnormal: m * 2^-9 */
        mag = (uint8_t)(val / ldexp(1.0, -9));
    } else {
        int e2;
        double f = frexp(val, &e2);           /* val = f * 2^e2, f in [0.5,1) */
        int ex = e2 - 1;                      /* val = (2f) * 2^ex */
        int m = (int)((2.0 * f - 1.0) * 8.0); /* exact: 3-bit mantissa */
        mag = (uint8_t)(((ex + 7) << 3) | m);
    }
    *code = sign | mag;
    return 0;
}

int64_t orc_e4m3_encode_array(const float *v, uint8_t *out, int64_t n) {
    int64_t bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        if (orc_e4m3_encode(v[i], &out[i]) != 0) {
            out[i] = 0xFF;
            bad += 1;
        }
    }
    return bad;
}

/* ------------------------------------------------------------ quantization */

static float bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* amax of a run of fp32 values; -1 when one is not finite */
static float absmax(const float *v, int n, int stride, int *bad) {
    float m = 0.0f;
    for (int i = 0; i < n; ++i) {
        float a = fabsf(v[(int64_t)i * stride]);
        if (!isfinite(a)) *bad = 1;
        if (a > m) m = a;
    }
    return m;
}

/* One value -> one code, given its fp32 scale.  Reading: the code is formed
 * from the fp32 IEEE quotient x / s (a correctly rounded division, not a
 * multiplication by 1/s); int8 rounds to nearest even and clamps to
 * [-127, 127]; fp8 goes through the E4M3 rule above.  A zero scale (the
 * whole run was zero) gives the code 0 without dividing. */
static int quantize_one(int fmt, float x, float s, uint8_t *q) {
    if (s == 0.0f) {
        *q = 0;
        return 0;
    }
    float t = x / s;
    if (fmt == ORC_W8A8_INT8) {
        float r = rintf(t);
        if (r > INT8_QMAX) r = INT8_QMAX;
        if (r < -INT8_QMAX) r = -INT8_QMAX;
        *q = (uint8_t)(int8_t)r;
        return 0;
    }
    return orc_e4m3_encode(t, q);
}

static float qmax_of(int fmt) { return fmt == ORC_W8A8_INT8 ? INT8_QMAX : FP8_QMAX; }

/* scale = amax / qmax as one fp32 division (unrounded to powers of two) */
static float scale_of(float amax, int fmt) { return amax == 0.0f ? 0.0f : amax / qmax_of(fmt); }

static int valid_fmt(int fmt) { return fmt == ORC_FP8_DYNAMIC || fmt == ORC_W8A8_INT8 || fmt == ORC_BLOCK_FP8; }

int orc_quant_act(int fmt, int M, int K, const uint16_t *x, uint8_t *q, float *s) {
    if (!valid_fmt(fmt) || M < 0 || K <= 0) return -2;
    if (fmt == ORC_BLOCK_FP8 && K % GROUP != 0) return -2;
    int G = K / GROUP;
    int bad = 0;
    float *row = (float *)malloc(sizeof(float) * (size_t)K);
    if (!row) return -3;
    for (int m = 0; m < M; ++m) {
        for (int k = 0; k < K; ++k) row[k] = bf16_to_f32(x[(int64_t)m * K + k]);
        if (fmt == ORC_BLOCK_FP8) {
            /* one scale per token and 128-wide K group */
            for (int g = 0; g < G; ++g) {
                float sc = scale_of(absmax(row + g * GROUP, GROUP, 1, &bad), fmt);
                s[(int64_t)m * G + g] = sc;
                for (int k = g * GROUP; k < (g + 1) * GROUP; ++k)
                    if (quantize_one(fmt, row[k], sc, &q[(int64_t)m * K + k])) bad = 1;
            }
        } else {
            /* one scale per token */
            float sc = scale_of(absmax(row, K, 1, &bad), fmt);
            s[m] = sc;
            for (int k = 0; k < K; ++k)
                if (quantize_one(fmt, row[k], sc, &q[(int64_t)m * K + k])) bad = 1;
        }
    }
    free(row);
    return bad ? -1 : 0;
}

int orc_quant_weight(int fmt, int N, int K, const float *w, uint8_t *q, float *s) {
    if (!valid_fmt(fmt) || N <= 0 || K <= 0) return -2;
    int bad = 0;
    if (fmt == ORC_BLOCK_FP8) {
        if (N % GROUP != 0 || K % GROUP != 0) return -2;
        int NB = N / GROUP, KB = K / GROUP;
#pragma omp parallel for schedule(static) reduction(| : bad)
        for (int nb = 0; nb < NB; ++nb) {
            for (int kb = 0; kb < KB; ++kb) {
                /* one scale per 128 x 128 block */
                float amax = 0.0f;
                for (int n = nb * GROUP; n < (nb + 1) * GROUP; ++n)
                    amax = fmaxf(amax, absmax(w + (int64_t)n * K + kb * GROUP, GROUP, 1, &bad));
                float sc = scale_of(amax, fmt);
                s[(int64_t)nb * KB + kb] = sc;
                for (int n = nb * GROUP; n < (nb + 1) * GROUP; ++n)
                    for (int k = kb * GROUP; k < (kb + 1) * GROUP; ++k)
                        if (quantize_one(fmt, w[(int64_t)n * K + k], sc, &q[(int64_t)n * K + k])) bad = 1;
            }
        }
    } else {
#pragma omp parallel for schedule(static) reduction(| : bad)
        for (int n = 0; n < N; ++n) {
            /* one scale per output channel (row n of W) */
            float sc = scale_of(absmax(w + (int64_t)n * K, K, 1, &bad), fmt);
            s[n] = sc;
            for (int k = 0; k < K; ++k)
                if (quantize_one(fmt, w[(int64_t)n * K + k], sc, &q[(int64_t)n * K + k])) bad = 1;
        }
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------ accumulation */

static void decode_table(double *t) {
    for (int c = 0; c < 256; ++c) t[c] = orc_e4m3_decode((uint8_t)c);
}

static int64_t dot_int8(const uint8_t *a, const uint8_t *b, int K) {
    int64_t acc = 0;
    for (int k = 0; k < K; ++k) acc += (int64_t)(int8_t)a[k] * (int64_t)(int8_t)b[k];
    return acc;
}

static double dot_fp8(const uint8_t *a, const uint8_t *b, int K, const double *t) {
    double acc = 0.0;
    for (int k = 0; k < K; ++k) acc += t[a[k]] * t[b[k]];
    return acc;
}

int orc_acc_int8(int M, int N, int K, const uint8_t *qa, const uint8_t *qw, int32_t *acc) {
    if (M < 0 || N <= 0 || K <= 0) return -2;
    int overflow = 0;
#pragma omp parallel for schedule(static) reduction(| : overflow)
    for (int n = 0; n < N; ++n) {
        for (int m = 0; m < M; ++m) {
            int64_t v = dot_int8(qa + (int64_t)m * K, qw + (int64_t)n * K, K);
            if (v > INT32_MAX || v < INT32_MIN) overflow = 1;
            acc[(int64_t)m * N + n] = (int32_t)v;
        }
    }
    return overflow ? -4 : 0;
}

int orc_acc_fp8(int M, int N, int K, const uint8_t *qa, const uint8_t *qw, double *acc) {
    if (M < 0 || N <= 0 || K <= 0) return -2;
    double t[256];
    decode_table(t);
#pragma omp parallel for schedule(static)
    for (int n = 0; n < N; ++n)
        for (int m = 0; m < M; ++m)
            acc[(int64_t)m * N + n] = dot_fp8(qa + (int64_t)m * K, qw + (int64_t)n * K, K, t);
    return 0;
}

int orc_acc_fp8_groups(int M, int N, int K, const uint8_t *qa, const uint8_t *qw, double *accg) {
    if (M < 0 || N <= 0 || K <= 0 || K % GROUP != 0) return -2;
    int G = K / GROUP;
    double t[256];
    decode_table(t);
#pragma omp parallel for schedule(static)
    for (int n = 0; n < N; ++n)
        for (int m = 0; m < M; ++m)
            for (int g = 0; g < G; ++g)
                accg[((int64_t)m * N + n) * G + g] =
                    dot_fp8(qa + (int64_t)m * K + g * GROUP, qw + (int64_t)n * K + g * GROUP, GROUP, t);
    return 0;
}

/* ------------------------------------------------------------------ result */

/* One output.  Per-channel formats: acc * sa[m] * sw[n].  Block format: the
 * sum over K-groups g, ascending, of accg * sa[m][g] * sw[n/128][g]. */
static double result_one(int fmt, int m, int n, int N, int K, const uint8_t *qa,
                         const float *sa, const uint8_t *qw, const float *sw,
                         const double *t, int32_t *acc_out, int *overflow) {
    const uint8_t *a = qa + (int64_t)m * K;
    const uint8_t *b = qw + (int64_t)n * K;
    (void)N;
    if (fmt == ORC_W8A8_INT8) {
        int64_t acc = dot_int8(a, b, K);
        if (acc > INT32_MAX || acc < INT32_MIN) *overflow = 1;
        if (acc_out) *acc_out = (int32_t)acc;
        return (double)acc * (double)sa[m] * (double)sw[n];
    }
    if (fmt == ORC_FP8_DYNAMIC)
        return dot_fp8(a, b, K, t) * (double)sa[m] * (double)sw[n];
    int G = K / GROUP;
    double r = 0.0;
    for (int g = 0; g < G; ++g) {
        double accg = dot_fp8(a + g * GROUP, b + g * GROUP, GROUP, t);
        r += accg * (double)sa[(int64_t)m * G + g] * (double)sw[(int64_t)(n / GROUP) * G + g];
    }
    return r;
}

static int gemm_args_ok(int fmt, int M, int N, int K) {
    if (!valid_fmt(fmt) || M < 0 || N <= 0 || K <= 0) return 0;
    if (fmt == ORC_BLOCK_FP8 && (N % GROUP != 0 || K % GROUP != 0)) return 0;
    return 1;
}

int orc_gemm(int fmt, int M, int N, int K, const uint8_t *qa, const float *sa,
             const uint8_t *qw, const float *sw, double *ref, int32_t *acc_i32) {
    if (!gemm_args_ok(fmt, M, N, K)) return -2;
    double t[256];
    decode_table(t);
    int overflow = 0;
#pragma omp parallel for schedule(static) reduction(| : overflow)
    for (int n = 0; n < N; ++n)
        for (int m = 0; m < M; ++m)
            ref[(int64_t)m * N + n] = result_one(fmt, m, n, N, K, qa, sa, qw, sw, t,
                                                 acc_i32 ? &acc_i32[(int64_t)m * N + n] : NULL, &overflow);
    return overflow ? -4 : 0;
}

int orc_gemm_sampled(int fmt, int M, int N, int K, const uint8_t *qa, const float *sa,
                     const uint8_t *qw, const float *sw, int64_t count, const int32_t *ms,
                     const int32_t *ns, double *ref, int32_t *acc_i32) {
    if (!gemm_args_ok(fmt, M, N, K)) return -2;
    for (int64_t i = 0; i < count; ++i)
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N) return -2;
    double t[256];
    decode_table(t);
    int overflow = 0;
#pragma omp parallel for schedule(static) reduction(| : overflow)
    for (int64_t i = 0; i < count; ++i)
        ref[i] = result_one(fmt, ms[i], ns[i], N, K, qa, sa, qw, sw, t,
                            acc_i32 ? &acc_i32[i] : NULL, &overflow);
    return overflow ? -4 : 0;
}

int orc_linear(int fmt, int M, int N, int K, const uint16_t *x, const uint8_t *qw,
               const float *sw, uint8_t *qa, float *sa, double *ref, int32_t *acc_i32) {
    int st = orc_quant_act(fmt, M, K, x, qa, sa);
    if (st != 0) return st;
    return orc_gemm(fmt, M, N, K, qa, sa, qw, sw, ref, acc_i32);
}

/* fp64 -> bfloat16 (8-bit significand), nearest with ties to even, in one
 * step from fp64 (no intermediate fp32 rounding). */
void orc_round_bf16(const double *v, uint16_t *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) {
        double a = v[i];
        if (!isfinite(a) || a == 0.0) {
            float f = (float)a;
            uint32_t u;
            memcpy(&u, &f, sizeof u);
            out[i] = (uint16_t)(u >> 16);
            continue;
        }
        int e2;
        frexp(fabs(a), &e2);
        int E = e2 - 1;
        if (E < -126) E = -126;                 /* bf16 subnormal spacing 2^-133 */
        double quantum = ldexp(1.0, E - 7);
        double r = nearbyint(a / quantum) * quantum;
        float f = (float)r;                     /* exact: r has <= 8 significant bits */
        uint32_t u;
        memcpy(&u, &f, sizeof u);
        out[i] = (uint16_t)(u >> 16);
    }
}

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
