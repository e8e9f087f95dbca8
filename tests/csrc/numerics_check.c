/*
 * Exhaustive checks of the oracle's scalar primitives against independent references.
 * Test code: compiled by the test suite and linked against the oracle library.
 *
 *  - bf16 rounding: every one of the 2^32 binary32 patterns is rounded by the oracle and
 *    by a second formulation that picks the nearer of the two neighbouring BF16 values
 *    with double-precision distances (ties to the even neighbour).
 *  - exp_f / log_f: every binary32 input of the domain is compared with the C library's
 *    double-precision exp/log; the error is measured in units of the binary32 ulp of the
 *    exact value.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

extern uint16_t orc_bf16_rne(float);
extern float orc_exp_f(float);
extern float orc_log_f(float);

static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* Independent RNE to bf16: neighbours lo (truncation) and hi (next bf16 away from zero). */
static uint16_t bf16_ref(float x) {
    uint32_t u; memcpy(&u, &x, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    if ((u & 0x7fffffffu) == 0x7f800000u) return (uint16_t)(u >> 16);
    uint16_t lo = (uint16_t)(u >> 16);
    uint16_t hi = (uint16_t)(lo + 1);
    double dx = fabs((double)x);
    double dlo = fabs((double)u2f((uint32_t)lo << 16));
    double dhi;
    if ((hi & 0x7fffu) == 0x7f80u) dhi = ldexp(1.0, 128);  /* would-be next value: 2^128 */
    else dhi = fabs((double)u2f((uint32_t)hi << 16));
    double a = dx - dlo, b = dhi - dx;
    if (a < b) return lo;
    if (b < a) return hi;
    return (lo & 1u) ? hi : lo;
}

/* Count of mismatching patterns in [start, end). */
uint64_t check_bf16_range(uint64_t start, uint64_t end) {
    uint64_t bad = 0;
#pragma omp parallel for reduction(+:bad) schedule(static)
    for (uint64_t i = start; i < end; ++i) {
        float x = u2f((uint32_t)i);
        if (orc_bf16_rne(x) != bf16_ref(x)) ++bad;
    }
    return bad;
}

static double ulp_of(double v) {
    v = fabs(v);
    if (v < ldexp(1.0, -126)) return ldexp(1.0, -149);
    int e; frexp(v, &e);            /* v = m 2^e, m in [0.5,1) */
    return ldexp(1.0, e - 1 - 23);
}

/* Max error in ulps over binary32 patterns [lo_bits, hi_bits] (same sign). fn 0 exp, 1 log. */
double max_ulp_err(int fn, uint32_t lo_bits, uint32_t hi_bits, uint32_t* worst_bits) {
    double worst = 0.0; uint32_t wb = lo_bits;
#pragma omp parallel
    {
        double lw = 0.0; uint32_t lb = lo_bits;
#pragma omp for schedule(static)
        for (int64_t i = (int64_t)lo_bits; i <= (int64_t)hi_bits; ++i) {
            float x = u2f((uint32_t)i);
            double ref = fn == 0 ? exp((double)x) : log((double)x);
            float y = fn == 0 ? orc_exp_f(x) : orc_log_f(x);
            double err = fabs((double)y - ref) / ulp_of(ref);
            if (err > lw) { lw = err; lb = (uint32_t)i; }
        }
#pragma omp critical
        { if (lw > worst) { worst = lw; wb = lb; } }
    }
    if (worst_bits) *worst_bits = wb;
    return worst;
}
