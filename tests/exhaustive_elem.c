/* Exhaustive accuracy check of the oracle's exp and log spellings against
 * binary64 libm, over all 2^32 binary32 inputs (test helper, built by
 * tests/test_oracle_exhaustive.py).
 *
 * usage: exhaustive_elem <liboracle.so> exp|log
 * Prints one line of JSON: the largest error in units of the last place of
 * the binary64 reference rounded to binary32's grid, how many results are not
 * the nearest binary32 value (error above half a unit), how many miss by more
 * than one unit, special-value mismatches (NaN, infinities, zeros), and the
 * monotonicity breaks between neighbouring inputs with the largest of them in
 * binary32 steps. */
#include <dlfcn.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

typedef float (*unary_fn)(float);

static float bitsf(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

/* binary32 unit in the last place at the magnitude of r (subnormal step below
 * 2^-126; the step of the top binade above it). */
static double ulp32(double r) {
    double a = fabs(r);
    if (a < ldexp(1.0, -126)) return ldexp(1.0, -149);
    int e;
    frexp(a, &e);                 /* a = m * 2^e, m in [0.5, 1) */
    if (e - 1 > 127) e = 128;
    return ldexp(1.0, e - 1 - 23);
}

int main(int argc, char** argv) {
    if (argc != 3) { fprintf(stderr, "usage: %s liboracle.so exp|log\n", argv[0]); return 2; }
    void* h = dlopen(argv[1], RTLD_NOW);
    if (!h) { fprintf(stderr, "dlopen: %s\n", dlerror()); return 2; }
    const int is_exp = strcmp(argv[2], "exp") == 0;
    unary_fn f = (unary_fn)dlsym(h, is_exp ? "orc_exp" : "orc_log");
    if (!f) { fprintf(stderr, "dlsym failed\n"); return 2; }
    const double top = ldexp(1.0, 128) * (1.0 - ldexp(1.0, -25));  /* values at or above round to +inf */
    double max_err = 0.0;
    uint32_t max_at = 0;
    long long not_nearest = 0, over_one = 0, special_bad = 0, mono_bad = 0;
    uint32_t max_break = 0;
    const int64_t NB = 4096, BS = ((int64_t)1 << 32) / NB;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : not_nearest, over_one, special_bad, mono_bad) \
    reduction(max : max_break)
    for (int64_t b = 0; b < NB; ++b) {
        double lmax = 0.0;
        uint32_t lat = 0;
        float prev = 0.0f;
        int have_prev = 0;
        for (int64_t i = b * BS; i < (b + 1) * BS; ++i) {
            const uint32_t u = (uint32_t)i;
            const float x = bitsf(u);
            const float y = f(x);
            /* neighbours in the bit order are neighbours in value on each
             * side of zero: exp rises with u on the positive side and falls on
             * the negative side; log rises on the positive side */
            if (have_prev && !isnan(x) && !isnan(y) && !isnan(prev) && u != 0x80000000u) {
                const int pos = (u >> 31) == 0;
                const int brk = is_exp ? (pos ? (y < prev) : (y > prev)) : (pos && y < prev);
                if (brk) {
                    uint32_t a, c;
                    memcpy(&a, &y, 4);
                    memcpy(&c, &prev, 4);
                    const uint32_t steps = a > c ? a - c : c - a;
                    ++mono_bad;
                    if (steps > max_break) max_break = steps;
                }
            }
            prev = y;
            have_prev = 1;
            if (isnan(x)) { if (!isnan(y)) ++special_bad; continue; }
            double r;
            if (is_exp) {
                r = exp((double)x);
            } else {
                if (x < 0.0f) { if (!isnan(y)) ++special_bad; continue; }
                if (x == 0.0f) { if (!(isinf(y) && y < 0)) ++special_bad; continue; }
                r = log((double)x);
            }
            if (isinf(x)) { if (!(y == (float)r || (isnan(r) && isnan(y)))) ++special_bad; continue; }
            if (isnan(y)) { ++special_bad; continue; }
            double err;
            if (isinf(y)) err = (r >= top) ? 0.0 : (ldexp(1.0, 128) - r) / ulp32(ldexp(1.0, 127));
            else if (r >= top) err = (ldexp(1.0, 128) - (double)y) / ulp32(ldexp(1.0, 127));
            else err = fabs((double)y - r) / ulp32(r);
            if (err > 0.5) ++not_nearest;
            if (err > 1.0) ++over_one;
            if (err > lmax) { lmax = err; lat = u; }
        }
#pragma omp critical
        if (lmax > max_err || (lmax == max_err && lat < max_at)) { max_err = lmax; max_at = lat; }
    }
    printf("{\"fn\": \"%s\", \"inputs\": 4294967296, \"max_ulp\": %.6f, \"max_at\": \"0x%08X\", "
           "\"not_nearest\": %lld, \"over_one_ulp\": %lld, \"special_bad\": %lld, \"monotonic_breaks\": %lld, "
           "\"largest_break_steps\": %u}\n",
           argv[2], max_err, max_at, not_nearest, over_one, special_bad, mono_bad, max_break);
    return 0;
}
