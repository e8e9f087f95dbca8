/*
 * Exhaustive checks of the oracle's scalar primitives against independent references.
 * Test code: compiled by the test suite and linked against the oracle library.
 *
 *  - bf16 rounding: every one of the 2^32 binary32 patterns is rounded by the oracle and
 *    by a second formulation that picks the nearer of the two neighbouring BF16 values
 *    with double-precision distances (ties to the even neighbour).
 *  - fp16 rounding: every binary32 pattern, against the nearer of the two neighbouring
 *    FP16 grid points computed in double (ties to the even one); fp16 widening: all 2^16
 *    patterns against the format's definition.
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

/* FP16 decoding from the format's definition (sign, 5-bit exponent with bias 15, 10 fraction
 * bits; exponent 0 = subnormal with quantum 2^-24; exponent 31 = inf / NaN). */
static double f16_value(uint16_t h) {
    int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 31) v = m ? NAN : INFINITY;
    else if (e == 0) v = ldexp((double)m, -24);
    else v = ldexp(1.0 + m / 1024.0, e - 15);
    return s ? -v : v;
}

/* Independent RNE to FP16, as a double: the two grid points around |x| (quantum 2^-24 below
 * 2^-14, else 2^(floor(log2 |x|) - 10)), the nearer one, ties to the one with an even
 * multiple of the quantum; above 65504 the next grid point, 65536, stands for infinity. */
static double f16_ref(float x) {
    double ax = fabs((double)x), q;
    if (isinf(ax)) return x;
    if (ax < ldexp(1.0, -14)) q = ldexp(1.0, -24);
    else { int e; frexp(ax, &e); q = ldexp(1.0, e - 1 - 10); }
    double k = floor(ax / q), lo = k * q, hi = lo + q;
    double a = ax - lo, b = hi - ax, r;
    if (a < b) r = lo;
    else if (b < a) r = hi;
    else r = fmod(k, 2.0) == 0.0 ? lo : hi;
    if (r >= 65536.0) r = INFINITY;
    return x < 0 || (x == 0 && signbit(x)) ? -r : r;
}

extern uint16_t orc_f16_rne(float);
extern float orc_f16_up(uint16_t);

/* Count of mismatching patterns in [start, end): the value, the sign of zero, and for NaN the
 * quiet NaN with sign and top payload bits kept. */
uint64_t check_f16_range(uint64_t start, uint64_t end) {
    uint64_t bad = 0;
#pragma omp parallel for reduction(+:bad) schedule(static)
    for (uint64_t i = start; i < end; ++i) {
        float x = u2f((uint32_t)i);
        uint16_t h = orc_f16_rne(x);
        if (isnan(x)) {
            uint16_t want = (uint16_t)(((uint32_t)i >> 16 & 0x8000u) | 0x7e00u | ((uint32_t)i >> 13 & 0x3ffu));
            if (h != want) ++bad;
            continue;
        }
        double got = f16_value(h), want = f16_ref(x);
        if (got != want || !signbit(got) != !signbit(want)) ++bad;
    }
    return bad;
}

/* Widening: all 2^16 FP16 patterns against the definition (NaN must stay NaN with its sign,
 * payload moved to the top of the FP32 fraction). */
uint64_t check_f16_up(void) {
    uint64_t bad = 0;
    for (uint32_t h = 0; h < 65536; ++h) {
        float y = orc_f16_up((uint16_t)h);
        double v = f16_value((uint16_t)h);
        uint32_t u; memcpy(&u, &y, 4);
        if (isnan(v)) {
            if (u != (((h & 0x8000u) << 16) | 0x7f800000u | ((h & 0x3ffu) << 13))) ++bad;
        } else if ((double)y != v || !signbit(y) != !signbit(v)) ++bad;
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
