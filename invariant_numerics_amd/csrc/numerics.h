// numerics.h -- device scalar primitives of the fixed-order path (gfx950).
//
// Every function here is written so that it produces the same binary32 bits as the
// definition stated in its comment: IEEE operations with round-to-nearest-even, explicit
// fused multiply-adds where a single rounding is meant, and nothing else.  The library is
// compiled with -ffp-contract=off (no implicit fma), without fast-math, with subnormals
// kept and with correctly rounded division and square root.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace invnum {

// Pinned constants of the reduction order.
constexpr int KS = 256;       // K-slice width of every dot product
constexpr int CHUNK = 256;    // attention KV chunk (absolute key positions)
constexpr int TV = 1024;      // vocabulary tile of the softmax denominator
constexpr int LW = 64;        // lanes per vocabulary tile (one wavefront)

// exp_f constants: log2(e); ln 2 as a 24-bit head and rounded tail (Cody & Waite 1980);
// range limits ln(2^-126) and ln(2^128); Taylor coefficients 1/k!.
#define INV_LOG2E 0x1.715476p+0f
#define INV_LN2_HI 0x1.62e430p-1f
#define INV_LN2_LO -0x1.05c610p-29f
#define INV_EXP_LO -0x1.5d58a0p+6f
#define INV_EXP_HI 0x1.62e430p+6f
#define INV_IF0 1.0f
#define INV_IF1 1.0f
#define INV_IF2 0x1.000000p-1f
#define INV_IF3 0x1.555556p-3f
#define INV_IF4 0x1.555556p-5f
#define INV_IF5 0x1.111112p-7f
#define INV_IF6 0x1.6c16c2p-10f
#define INV_IF7 0x1.a01a02p-13f
// log_f constants: ln 2 head with 16 significant bits (e * head exact) and its tail;
// atanh-series coefficients 2/(2k+1), k = 1..5 (Abramowitz & Stegun 4.1.27).
#define INV_LN2_HI16 0x1.62e400p-1f
#define INV_LN2_LO16 0x1.7f7d1cp-20f
#define INV_AT1 0x1.555556p-1f
#define INV_AT2 0x1.99999ap-2f
#define INV_AT3 0x1.24924ap-2f
#define INV_AT4 0x1.c71c72p-3f
#define INV_AT5 0x1.745d18p-3f

__device__ __forceinline__ float bits2f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t f2bits(float f) { return __float_as_uint(f); }

// up(): BF16 bits -> FP32, exact.
__device__ __forceinline__ float bf16_up(uint32_t b16) { return __uint_as_float(b16 << 16); }
// Low / high BF16 halves of a 32-bit word holding two consecutive elements.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// bf(): FP32 -> BF16 bits, round to nearest even on the dropped 16 bits; NaN stays quiet NaN.
__device__ __forceinline__ uint32_t bf16_rne(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// FP16 storage rounding: the binary16 value nearest to x (ties to even), returned widened to
// FP32.  binary16 keeps 10 fraction bits between 2^-14 and 65504 and steps of 2^-24 below;
// from 65520 (the tie between 65504 and 2^16, whose even side is 2^16) up the result is inf;
// NaN stays a quiet NaN with its sign and the top 9 payload bits.
__device__ __forceinline__ float f16_round(float x) {
    const uint32_t u = __float_as_uint(x);
    const uint32_t s = u & 0x80000000u, a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return __uint_as_float(s | 0x7fc00000u | (a & 0x007fe000u));
    if (a >= 0x477ff000u) return __uint_as_float(s | 0x7f800000u);      // |x| >= 65520
    if (a < 0x38800000u) {                                               // |x| < 2^-14
        // |x| * 2^24 < 2^10 is exact, rint rounds half to even, * 2^-24 is exact
        const float r = __builtin_rintf(__uint_as_float(a) * 0x1p24f) * 0x1p-24f;
        return __uint_as_float(s | __float_as_uint(r));
    }
    // normal range: round the 13 dropped fraction bits half to even in the FP32 encoding
    // (a carry out of the fraction steps the exponent, which is the next binade's value)
    const uint32_t r = (a + 0x0fffu + ((a >> 13) & 1u)) & ~0x1fffu;
    return __uint_as_float(s | r);
}

// exp_f(x): n = rint(x log2e); r = fma(-n, ln2_hi, x); r = fma(-n, ln2_lo, r);
// p = Taylor degree 7 by fma-Horner from the top; result p * 2^n rounded once.
// x < ln(2^-126) -> +0, x > ln(2^128) -> +inf, NaN -> NaN.
// Written without branches: the polynomial runs on x clamped into [ln(2^-126), ln(2^128)]
// (for x inside it the clamp is the identity, so the arithmetic is exactly the steps above),
// then n lies in [-126, 128] and ldexp(p, n) is p * 2^n with one rounding -- the same value
// as (p * 2) * 2^127 for n = 128.  At the upper clamp point 128 ln2_hi equals the limit, r is
// a tiny positive number, p > 1 and p * 2^128 overflows to +inf: every x at or above the limit
// (+inf included) lands on +inf without a select.  Below the range +0 is selected.
__device__ __forceinline__ float exp_f(float x) {
    const float xc = __builtin_fminf(__builtin_fmaxf(x, INV_EXP_LO), INV_EXP_HI);
    const float t = xc * INV_LOG2E;
    const float n = __builtin_rintf(t);
    float r = __builtin_fmaf(-n, INV_LN2_HI, xc);
    r = __builtin_fmaf(-n, INV_LN2_LO, r);
    float p = INV_IF7;
    p = __builtin_fmaf(p, r, INV_IF6);
    p = __builtin_fmaf(p, r, INV_IF5);
    p = __builtin_fmaf(p, r, INV_IF4);
    p = __builtin_fmaf(p, r, INV_IF3);
    p = __builtin_fmaf(p, r, INV_IF2);
    p = __builtin_fmaf(p, r, INV_IF1);
    p = __builtin_fmaf(p, r, INV_IF0);
    float res = __builtin_ldexpf(p, (int)n);
    res = (x < INV_EXP_LO) ? 0.0f : res;
    return (x != x) ? x + x : res;
}

// log_f(x), x > 0: x = 2^e m, m in (sqrt(1/2), sqrt(2)]; f = m - 1; s = f / (2 + f);
// z = s^2; R = z (2/3 + z (2/5 + z (2/7 + z (2/9 + z 2/11)))); log m = f - s (f - R);
// result = e ln2_hi16 + (f + fma(e, ln2_lo16, -s (f - R))).
__device__ __forceinline__ float log_f(float x) {
    if (x != x) return x + x;
    if (x < 0.0f) return __builtin_nanf("");
    if (x == 0.0f) return -__builtin_inff();
    if (x == __builtin_inff()) return x;
    int e = 0;
    uint32_t u = __float_as_uint(x);
    if (u < 0x00800000u) { x = x * 16777216.0f; u = __float_as_uint(x); e = -24; }
    e += (int)(u >> 23) - 127;
    uint32_t frac = u & 0x007fffffu;
    float m = __uint_as_float(frac | 0x3f800000u);
    if (frac > 0x003504f3u) { m = m * 0.5f; e += 1; }
    float f = m - 1.0f;
    float s = f / (2.0f + f);
    float z = s * s;
    float R = INV_AT5;
    R = __builtin_fmaf(R, z, INV_AT4);
    R = __builtin_fmaf(R, z, INV_AT3);
    R = __builtin_fmaf(R, z, INV_AT2);
    R = __builtin_fmaf(R, z, INV_AT1);
    R = R * z;
    float u2 = s * (f - R);
    float fe = (float)e;
    float t = __builtin_fmaf(fe, INV_LN2_LO16, -u2);
    return fe * INV_LN2_HI16 + (f + t);
}

// Host-side copy of the constant table (same order as the ABI's inv_constants).
static const float kFloatConsts[] = {
    INV_LOG2E, INV_LN2_HI, INV_LN2_LO, INV_EXP_LO, INV_EXP_HI,
    INV_IF0, INV_IF1, INV_IF2, INV_IF3, INV_IF4, INV_IF5, INV_IF6, INV_IF7,
    INV_LN2_HI16, INV_LN2_LO16, INV_AT1, INV_AT2, INV_AT3, INV_AT4, INV_AT5};

// Status codes mirrored from the public header (kept in one place there).
}  // namespace invnum
