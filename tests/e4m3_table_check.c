/* e4m3_table_check.c -- test infrastructure: a second fp32 -> E4M3FN encoder,
 * written independently of the oracle's, and a parallel sweep that compares
 * a given encoder with it over a range of fp32 bit patterns.
 *
 * The format is the OCP 8-bit floating point E4M3FN ("Building a
 * High-Performance and Portable vLLM Linear Backend with Helion", section
 * "Scope", FP8 formats): 4 exponent bits with bias 7, 3 mantissa bits,
 * subnormals, no infinities, largest finite magnitude 448.
 *
 * This encoder does no binade arithmetic.  It lists the 127 non-negative
 * finite values in code order (which is ascending order), each built as an
 * integer significand times a power of two: code 8e + m is m * 2^-9 for
 * e = 0 and (8 + m) * 2^(e - 10) otherwise.  A value's magnitude is clamped
 * to 448; the nearest table entry is found by binary search; of two equally
 * near entries the even code is taken; the sign bit is copied over (so a
 * negative value that rounds to zero gives 0x80). */
#include <math.h>
#include <stdint.h>
#include <string.h>

typedef int (*encode_fn)(float v, uint8_t *code);

static double table_value(int code) {
    const int e = code >> 3, m = code & 7;
    return e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
}

static uint8_t table_encode(const double *table, float v) {
    double a = fabs((double)v);
    if (a > table[126]) a = table[126];
    int lo = 0, hi = 126;   /* first entry >= a */
    while (lo < hi) {
        const int mid = (lo + hi) / 2;
        if (table[mid] < a) lo = mid + 1;
        else hi = mid;
    }
    int pick = lo;
    if (lo > 0) {
        const double above = table[lo] - a, below = a - table[lo - 1];
        if (below < above || (below == above && (lo - 1) % 2 == 0)) pick = lo - 1;
    }
    return (uint8_t)(pick | (signbit(v) ? 0x80 : 0));
}

/* The table's encoding of n values (for spot checks from the test). */
void table_encode_array(const float *v, uint8_t *out, int64_t n) {
    double table[127];
    for (int c = 0; c < 127; ++c) table[c] = table_value(c);
    for (int64_t i = 0; i < n; ++i) out[i] = table_encode(table, v[i]);
}

/* Compares enc with the table encoder on every finite fp32 bit pattern in
 * [lo, hi).  Returns the number of patterns where they differ (or where enc
 * reports an error) and the lowest such pattern in *first (or 2^32). */
int64_t sweep_mismatches(encode_fn enc, uint64_t lo, uint64_t hi, uint64_t *first) {
    double table[127];
    for (int c = 0; c < 127; ++c) table[c] = table_value(c);
    int64_t bad = 0;
    uint64_t lowest = (uint64_t)1 << 32;
#pragma omp parallel for schedule(static, 1 << 16) reduction(+ : bad) reduction(min : lowest)
    for (int64_t i = (int64_t)lo; i < (int64_t)hi; ++i) {
        const uint32_t bits = (uint32_t)i;
        if (((bits >> 23) & 0xFF) == 0xFF) continue;   /* inf and NaN: outside the domain */
        float v;
        memcpy(&v, &bits, sizeof v);
        uint8_t got = 0;
        if (enc(v, &got) != 0 || got != table_encode(table, v)) {
            bad += 1;
            if ((uint64_t)i < lowest) lowest = (uint64_t)i;
        }
    }
    *first = lowest;
    return bad;
}
