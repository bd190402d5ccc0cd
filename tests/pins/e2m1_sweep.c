/* e2m1_sweep.c -- brute-force check of an E2M1 encoder over fp32 bit
 * patterns (test helper, compiled by tests/test_oracle_codecs.py).
 *
 * For every non-NaN fp32 pattern in [first, first + n): the expected code is
 * the nearest of the eight E2M1 magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}
 * (code = index), found by measuring the distance to each of them in double
 * (exact for fp32 inputs below 2^60; larger ones are past 6 anyway), the
 * even code winning a tie, anything at or beyond 6 (Inf included) taking 6;
 * the sign goes to bit 3.  `enc` is the encoder under test, called with the
 * input widened exactly to double.  Returns the number of patterns where it
 * differs; *first_bad gets the smallest differing offset (-1 if none). */
#include <math.h>
#include <stdint.h>
#include <string.h>

typedef uint8_t (*enc_fn)(double);

static uint8_t brute(double v)
{
    static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    const uint8_t sign = signbit(v) ? 8 : 0;
    const double a = fabs(v);
    if (a >= 6.0)
        return sign | 7;
    int best = 0;
    double bd = a;                       /* distance to magnitude 0 */
    for (int c = 1; c < 8; c++) {
        const double d = fabs(a - mag[c]);
        if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            bd = d;
        }
    }
    return sign | (uint8_t)best;
}

int64_t e2m1_sweep(enc_fn enc, uint64_t first, int64_t n, int64_t *first_bad)
{
    int64_t bad = 0, fb = INT64_MAX;
#pragma omp parallel for schedule(static) reduction(+ : bad) reduction(min : fb)
    for (int64_t i = 0; i < n; i++) {
        const uint32_t u = (uint32_t)(first + (uint64_t)i);
        float f;
        memcpy(&f, &u, 4);
        if (isnan(f))
            continue;
        if (enc((double)f) != brute((double)f)) {
            bad++;
            if (i < fb)
                fb = i;
        }
    }
    *first_bad = bad ? fb : -1;
    return bad;
}
