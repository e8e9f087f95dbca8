/*
 * oracle.c -- plain CPU oracle for batch-invariant token log-probabilities.
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the benchmark's
 * cpu_baseline leg are the only callers.  The product path (the HIP library and its
 * Python binding) never loads, links or calls this file, and this file includes no
 * header or helper of the product path.
 *
 * What it computes.  The pages describe a method rather than a closed-form result:
 *   - one fixed summation order for every reduction whose order changes the bits
 *     (attention score sums, the softmax denominator, matmul K-sums, the logprob
 *     accumulation) shared by prefill and decode, computed with batch-invariant
 *     operators  [Meituan train/inference bitwise alignment page, "principles" and
 *     "key practices" lists; its FAQ 2 says the fix is the fixed order, not precision];
 *   - full-K accumulation instead of a split reduce  [same page, "key practices", TP];
 *   - LayerCast: weights stored BF16, upcast to FP32 per layer, all matmul and
 *     attention in FP32  ["Give Me FP32 or Give Me Death?" write-up, section 5;
 *     Yuan et al. blog, section 4];
 *   - selective FP32 LM-head recompute when the top-two logit margin is below a
 *     threshold  ["Greedy Decoding Is Not Precision-Invariant", abstract and
 *     "key design" paragraph].
 * The pages fix no tree shape, so one order is pinned here ("canonical reduction
 * order v0") and every function below follows it step by step, one row or one output
 * at a time.  A row's result therefore cannot depend on which other rows are computed
 * beside it.  Threads (OpenMP) split only independent outputs.
 *
 * Arithmetic: IEEE-754 binary32 with round-to-nearest-even and subnormals kept.
 * fmaf() is the single-rounding fused multiply-add.  This file must be compiled with
 * -ffp-contract=off and without any fast-math option, so that a*b+c stays two
 * roundings wherever it is written that way.
 *
 * Pinned constants (reported by orc_constants()):
 *   KS  = 256   contiguous K-slice of every dot product
 *   C   = 256   attention KV chunk (absolute key positions)
 *   TV  = 1024  vocabulary tile of the softmax denominator, LW = 64 lanes per tile
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_KS 256
#define ORC_CHUNK 256
#define ORC_TV 1024
#define ORC_LW 64

/* ------------------------------------------------------------------ bits -- */

static inline uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static inline float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* BF16 = 1 sign, 8 exponent, 7 stored fraction bits (the FP32 write-up, section 10).
 * up(): the 16 BF16 bits are the top half of an FP32 word -- exact. */
float orc_bf16_up(uint16_t b) { return u2f((uint32_t)b << 16); }

/* bf(): FP32 -> BF16, round to nearest, ties to even on the 16 dropped bits.
 * Overflow rounds to infinity; NaN stays a quiet NaN. */
uint16_t orc_bf16_rne(float x) {
    uint32_t u = f2u(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

/* FP16 (IEEE binary16) = 1 sign, 5 exponent (bias 15), 10 stored fraction bits: normals
 * from 2^-14 to 65504, subnormals in steps of 2^-24 (Yuan et al. blog, section 2, the note on
 * mantissa widths: BF16 7 bits, FP16 10, FP32 23).  Used for the FP16-activation setting
 * of the cross-precision comparison ("Greedy Decoding Is Not Precision-Invariant",
 * abstract: one model run in BF16 and in FP16, read here as the activation storage format).
 * f16_up(): exact widening to FP32. */
float orc_f16_up(uint16_t h) {
    uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    uint32_t e = (h >> 10) & 0x1fu, m = h & 0x3ffu;
    if (e == 0x1fu) return u2f(sign | 0x7f800000u | (m << 13));     /* inf, NaN */
    if (e == 0) {                                                   /* zero, subnormal */
        float v = (float)m * 0x1p-24f;                              /* exact: m < 2^10 */
        return sign ? -v : v;
    }
    return u2f(sign | ((e + 112u) << 23) | (m << 13));
}

/* f16(): FP32 -> FP16, round to nearest, ties to even.  Magnitudes from 65520 (the midpoint
 * between 65504 and 2^16, which ties to the even neighbour 2^16) up become infinity; below
 * 2^-14 the result is the nearest multiple of 2^-24 (possibly 2^-14 itself); NaN becomes a
 * quiet NaN keeping the sign and the top 9 payload bits. */
uint16_t orc_f16_rne(float x) {
    uint32_t u = f2u(x);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return (uint16_t)(sign | 0x7e00u | ((a >> 13) & 0x3ffu));
    float ax = u2f(a);
    if (ax >= 65520.0f) return (uint16_t)(sign | 0x7c00u);
    if (ax < 0x1p-14f) {
        /* ax * 2^24 < 2^10 is exact; nearbyintf rounds half to even in the default mode */
        return (uint16_t)(sign | (uint16_t)nearbyintf(ax * 0x1p24f));
    }
    uint32_t h = (((a >> 23) - 112u) << 10) | ((a >> 13) & 0x3ffu);
    uint32_t rest = a & 0x1fffu;                       /* the 13 dropped fraction bits */
    if (rest > 0x1000u || (rest == 0x1000u && (h & 1u))) h += 1u;   /* carry may reach 2^16 */
    return (uint16_t)(sign | h);
}

/* Storage rounding of an activation: fmt 0 keeps FP32, 1 rounds to BF16, 2 to FP16; the
 * result is the rounded value widened back to FP32 (the arithmetic stays FP32). */
static float round_act(float x, int fmt) {
    if (fmt == 1) return orc_bf16_up(orc_bf16_rne(x));
    if (fmt == 2) return orc_f16_up(orc_f16_rne(x));
    return x;
}
void orc_round_act_array(const float* x, int64_t n, int fmt, float* y) {
    for (int64_t i = 0; i < n; ++i) y[i] = round_act(x[i], fmt);
}
static void round_all(float* x, int64_t n, int fmt) {
    if (fmt) for (int64_t i = 0; i < n; ++i) x[i] = round_act(x[i], fmt);
}

/* -------------------------------------------------------- exp_f / log_f -- */
/* Project-defined transcendental functions.  Hardware/libm expf and logf are never
 * used on the compared path because their last bit differs between implementations.
 * The constants are derived here, from their mathematical definitions, by rounding
 * double-precision values to binary32 (they are checked against an exact rational
 * rounding by the test suite). */

static float C_LOG2E, C_LN2_HI, C_LN2_LO, C_EXP_LO, C_EXP_HI;
static float C_INVFACT[8];
static float C_LN2_HI16, C_LN2_LO16, C_ATANH[6];
static int consts_ready = 0;

__attribute__((constructor)) static void init_consts(void) {
    if (consts_ready) return;
    const double ln2 = 0.69314718055994530941723212145817656807550013436026;
    /* Cody & Waite (1980) argument reduction: ln2 split into a 24-bit head and the
     * rounded remainder; with fma the first reduction step is exact. */
    C_LOG2E = (float)(1.0 / ln2);
    C_LN2_HI = (float)ln2;
    C_LN2_LO = (float)(ln2 - (double)C_LN2_HI);
    /* Taylor coefficients of e^r: 1/k!, k = 0..7. */
    double fact = 1.0;
    for (int k = 0; k < 8; ++k) { if (k > 0) fact *= k; C_INVFACT[k] = (float)(1.0 / fact); }
    /* Range limits: below ln(2^-126) the result is pinned to +0; above ln(2^128) to +inf. */
    C_EXP_LO = (float)(-126.0 * ln2);
    C_EXP_HI = (float)(128.0 * ln2);
    /* log: ln2 head with 16 significant bits, so e*head is exact for |e| < 2^8. */
    {
        int ex; double m = frexp(ln2, &ex);          /* ln2 = m * 2^ex, m in [0.5,1) */
        double h = ldexp(nearbyint(ldexp(m, 16)), ex - 16);
        C_LN2_HI16 = (float)h;
        C_LN2_LO16 = (float)(ln2 - h);
    }
    /* atanh series of the logarithm (Abramowitz & Stegun 4.1.27): coefficients 2/(2k+1). */
    for (int k = 1; k <= 5; ++k) C_ATANH[k] = (float)(2.0 / (2.0 * k + 1.0));
    C_ATANH[0] = 0.0f;
    consts_ready = 1;
}

/* exp_f(x):
 *   n = rint(x * log2e)                 (binary32 multiply, round half to even)
 *   r = fma(-n, ln2_hi, x); r = fma(-n, ln2_lo, r)
 *   p = degree-7 Taylor polynomial of e^r, Horner with fma, highest degree first
 *   result = p * 2^n, with 2^n built in the exponent field (n = 128 goes through p*2).
 *   x < ln(2^-126) -> +0; x > ln(2^128) -> +inf.                                      */
float orc_exp_f(float x) {
    init_consts();
    if (x != x) return x + x;
    if (x > C_EXP_HI) return INFINITY;
    if (x < C_EXP_LO) return 0.0f;
    float t = x * C_LOG2E;
    float n = nearbyintf(t);
    float r = fmaf(-n, C_LN2_HI, x);
    r = fmaf(-n, C_LN2_LO, r);
    float p = C_INVFACT[7];
    for (int k = 6; k >= 0; --k) p = fmaf(p, r, C_INVFACT[k]);
    int ni = (int)n;
    if (ni > 127) { p = p * 2.0f; ni -= 1; }
    return p * u2f((uint32_t)(ni + 127) << 23);
}

/* log_f(x), x > 0:
 *   x = 2^e * m with m in (sqrt(1/2), sqrt(2)]  (subnormals scaled by 2^24 first)
 *   f = m - 1 (exact), s = f / (2 + f), z = s*s
 *   R = z*(2/3 + z*(2/5 + z*(2/7 + z*(2/9 + z*2/11))))      (Horner with fma)
 *   log m = 2 atanh(s) = f - s*(f - R)
 *   result = e*ln2_hi16 + (f + fma(e, ln2_lo16, -s*(f - R)))                       */
float orc_log_f(float x) {
    init_consts();
    if (x != x) return x + x;
    if (x < 0.0f) return NAN;
    if (x == 0.0f) return -INFINITY;
    if (x == INFINITY) return x;
    int e = 0;
    uint32_t u = f2u(x);
    if (u < 0x00800000u) { x = x * 16777216.0f; u = f2u(x); e = -24; }
    e += (int)(u >> 23) - 127;
    uint32_t frac = u & 0x007fffffu;
    float m = u2f(frac | 0x3f800000u);            /* m in [1, 2) */
    if (frac > 0x003504f3u) { m = m * 0.5f; e += 1; }  /* m > sqrt(2) -> m/2 */
    float f = m - 1.0f;
    float s = f / (2.0f + f);
    float z = s * s;
    float R = C_ATANH[5];
    for (int k = 4; k >= 1; --k) R = fmaf(R, z, C_ATANH[k]);
    R = R * z;
    float u2 = s * (f - R);
    float fe = (float)e;
    float t = fmaf(fe, C_LN2_LO16, -u2);
    return fe * C_LN2_HI16 + (f + t);
}

/* Constant table, in a fixed order, for comparison with the library's own table. */
int orc_constants(float* out, int cap) {
    init_consts();
    float v[] = {C_LOG2E, C_LN2_HI, C_LN2_LO, C_EXP_LO, C_EXP_HI,
                 C_INVFACT[0], C_INVFACT[1], C_INVFACT[2], C_INVFACT[3],
                 C_INVFACT[4], C_INVFACT[5], C_INVFACT[6], C_INVFACT[7],
                 C_LN2_HI16, C_LN2_LO16,
                 C_ATANH[1], C_ATANH[2], C_ATANH[3], C_ATANH[4], C_ATANH[5]};
    int n = (int)(sizeof v / sizeof v[0]);
    for (int i = 0; i < n && i < cap; ++i) out[i] = v[i];
    return n;
}
int orc_int_constants(int* out, int cap) {
    int v[] = {ORC_KS, ORC_CHUNK, ORC_TV, ORC_LW};
    int n = 4;
    for (int i = 0; i < n && i < cap; ++i) out[i] = v[i];
    return n;
}

/* Vectorised helpers for the tests. */
void orc_exp_f_array(const float* x, float* y, int64_t n) {
    init_consts();
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) y[i] = orc_exp_f(x[i]);
}
void orc_log_f_array(const float* x, float* y, int64_t n) {
    init_consts();
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) y[i] = orc_log_f(x[i]);
}
void orc_bf16_rne_array(const float* x, uint16_t* y, int64_t n) {
    for (int64_t i = 0; i < n; ++i) y[i] = orc_bf16_rne(x[i]);
}

/* Plain binary32 arithmetic for the worked example of non-associativity
 * (FP32 write-up, section 1: 0.1 + 0.2 + (-0.1) in two orders). */
float orc_add_f32(float a, float b) { return a + b; }
uint16_t orc_add_bf16(uint16_t a, uint16_t b) {
    /* The exact sum of two BF16 values whose exponents differ by at most 16 fits in
     * binary32, so rounding the binary32 sum to BF16 is the correctly rounded BF16 sum. */
    return orc_bf16_rne(orc_bf16_up(a) + orc_bf16_up(b));
}

/* ------------------------------------------------------------------ dot -- */
/* dot_KS(x, w, K): the one contraction order used by every matmul-like sum.
 *   for each slice s = [256 s, min(K, 256 (s+1))):  c = +0; c = fma(x_k, w_k, c), k ascending
 *   fold: T = c_0; T = T + c_s for s ascending.
 * The slice width is a constant, independent of the batch, so the same order serves a
 * one-row decode and a 32k-row prefill (full K in one place, no split across workers). */
static float dot_ks_f32(const float* x, const float* w, int64_t K) {
    float T = 0.0f;
    for (int64_t s0 = 0; s0 < K; s0 += ORC_KS) {
        int64_t e = s0 + ORC_KS < K ? s0 + ORC_KS : K;
        float c = 0.0f;
        for (int64_t k = s0; k < e; ++k) c = fmaf(x[k], w[k], c);
        T = (s0 == 0) ? c : T + c;
    }
    return T;
}

/* Same order; the weight operand is BF16 and is upcast (exactly) as it is read. */
static float dot_ks_w16(const float* x, const uint16_t* w, int64_t K) {
    float T = 0.0f;
    for (int64_t s0 = 0; s0 < K; s0 += ORC_KS) {
        int64_t e = s0 + ORC_KS < K ? s0 + ORC_KS : K;
        float c = 0.0f;
        for (int64_t k = s0; k < e; ++k) c = fmaf(x[k], orc_bf16_up(w[k]), c);
        T = (s0 == 0) ? c : T + c;
    }
    return T;
}

float orc_dot_ks(const float* x, const float* w, int64_t K) { return dot_ks_f32(x, w, K); }

/* ----------------------------------------------------------------- GEMM -- */
/* Y[m, n] = dot_KS(X[m, :], up(W[n, :]))   (LayerCast matmul: BF16 storage, FP32 compute).
 * X fp32 [M, K] row stride ldx; W bf16 [N, K] row stride ldw; Y fp32 [M, N] row stride ldy. */
void orc_gemm(const float* X, int64_t M, int64_t K, int64_t ldx,
              const uint16_t* W, int64_t N, int64_t ldw, float* Y, int64_t ldy) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            Y[m * ldy + n] = dot_ks_w16(X + m * ldx, W + n * ldw, K);
}

/* -------------------------------------------------------- GEMM backward -- */
/* Backward of the LayerCast matmul Y = X up(W)^T for an output gradient dY:
 *   dX[m, k] = dot_KS over n of (dY[m, n], up(W[n, k]))   (reduction over the N outputs)
 *   dW[n, k] = dot_KS over m of (dY[m, n], X[m, k])       (reduction over the M tokens)
 * Each is the same slice-then-fold order as the forward, taken along the reduced index, so
 * a gradient's bits do not depend on how the work is split (the Meituan page's principles
 * list: training and inference share one fixed order for every order-sensitive sum).  dW
 * is FP32 (the weights are stored BF16; the optimizer's master copy is not part of this).
 * dY fp32 [M, N] (lddy); X fp32 [M, K] (ldx); W bf16 [N, K] (ldw).  dX or dW may be NULL. */
static float dx_at(const float* dY, int64_t N, int64_t lddy, const uint16_t* W, int64_t ldw,
                   int64_t m, int64_t k, float* a, float* b) {
    for (int64_t n = 0; n < N; ++n) {
        a[n] = dY[m * lddy + n];
        b[n] = orc_bf16_up(W[n * ldw + k]);
    }
    return dot_ks_f32(a, b, N);
}
static float dw_at(const float* dY, int64_t M, int64_t lddy, const float* X, int64_t ldx,
                   int64_t n, int64_t k, float* a, float* b) {
    for (int64_t m = 0; m < M; ++m) {
        a[m] = dY[m * lddy + n];
        b[m] = X[m * ldx + k];
    }
    return dot_ks_f32(a, b, M);
}
void orc_gemm_backward(const float* dY, int64_t M, int64_t N, int64_t lddy,
                       const float* X, int64_t K, int64_t ldx, const uint16_t* W, int64_t ldw,
                       float* dX, int64_t lddx, float* dW, int64_t lddw) {
    int64_t L = M > N ? M : N;
#pragma omp parallel
    {
        float* a = (float*)malloc(sizeof(float) * (size_t)L);
        float* b = (float*)malloc(sizeof(float) * (size_t)L);
        if (dX) {
#pragma omp for collapse(2) schedule(static)
            for (int64_t m = 0; m < M; ++m)
                for (int64_t k = 0; k < K; ++k) dX[m * lddx + k] = dx_at(dY, N, lddy, W, ldw, m, k, a, b);
        }
        if (dW) {
#pragma omp for collapse(2) schedule(static)
            for (int64_t n = 0; n < N; ++n)
                for (int64_t k = 0; k < K; ++k) dW[n * lddw + k] = dw_at(dY, M, lddy, X, ldx, n, k, a, b);
        }
        free(a);
        free(b);
    }
}
/* Sampled outputs of the same definitions: out[i] = dX[rows[i], cols[i]] (which 0) or
 * dW[rows[i], cols[i]] (which 1), for checking full-size results one output at a time. */
void orc_gemm_backward_at(int which, const float* dY, int64_t M, int64_t N, int64_t lddy,
                          const float* X, int64_t K, int64_t ldx, const uint16_t* W, int64_t ldw,
                          const int64_t* rows, const int64_t* cols, int64_t cnt, float* out) {
    (void)K;
    int64_t L = M > N ? M : N;
#pragma omp parallel
    {
        float* a = (float*)malloc(sizeof(float) * (size_t)L);
        float* b = (float*)malloc(sizeof(float) * (size_t)L);
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < cnt; ++i)
            out[i] = which == 0 ? dx_at(dY, N, lddy, W, ldw, rows[i], cols[i], a, b)
                                : dw_at(dY, M, lddy, X, ldx, rows[i], cols[i], a, b);
        free(a);
        free(b);
    }
}

/* -------------------------------------------------------------- RMSNorm -- */
/* ss = dot_KS(x, x, H); r = 1 / sqrt((ss / H) + eps); y_k = (x_k * r) * up(gamma_k). */
void orc_rmsnorm(const float* X, int64_t M, int64_t H, int64_t ldx,
                 const uint16_t* gamma, float eps, float* Y, int64_t ldy) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const float* x = X + m * ldx;
        float ss = dot_ks_f32(x, x, H);
        float r = 1.0f / sqrtf((ss / (float)H) + eps);
        for (int64_t k = 0; k < H; ++k) Y[m * ldy + k] = (x[k] * r) * orc_bf16_up(gamma[k]);
    }
}

/* ----------------------------------------------------------------- RoPE -- */
/* Rotate-half RoPE on one head vector of width D at a position whose cos/sin rows
 * (D/2 entries each) are given:  y_i = x_i c_i - x_{i+D/2} s_i,  y_{i+D/2} = x_i s_i + x_{i+D/2} c_i. */
static void rope_vec(const float* x, const float* cs, const float* sn, int64_t D, float* y) {
    int64_t h = D / 2;
    for (int64_t i = 0; i < h; ++i) {
        float a = x[i], b = x[i + h];
        y[i] = (a * cs[i]) - (b * sn[i]);
        y[i + h] = (a * sn[i]) + (b * cs[i]);
    }
}

/* X [M, nh, D] (row stride ldx) at positions pos[m]; tables [Tmax, D/2]. */
void orc_rope(const float* X, int64_t M, int64_t nh, int64_t D, int64_t ldx,
              const int32_t* pos, const float* cos_t, const float* sin_t,
              float* Y, int64_t ldy) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t h = 0; h < nh; ++h)
            rope_vec(X + m * ldx + h * D, cos_t + (int64_t)pos[m] * (D / 2),
                     sin_t + (int64_t)pos[m] * (D / 2), D, Y + m * ldy + h * D);
}

/* Threads the oracle's parallel loops may use (they split independent outputs only, so the
 * bits do not depend on it); n < 1 restores the OpenMP default.  Returns the new maximum. */
int orc_set_threads(int n) {
    static int deflt = 0;
    if (deflt == 0) deflt = omp_get_max_threads();
    omp_set_num_threads(n >= 1 ? n : deflt);
    return omp_get_max_threads();
}

/* ------------------------------------------------------------ attention -- */
static inline float ld_elem(const void* p, int dt, int64_t i) {
    return dt ? ((const float*)p)[i] : orc_bf16_up(((const uint16_t*)p)[i]);
}

/* One causal attention row: query vector q (already fp32), keys/values of one kv head
 * at absolute positions 0..i, reached through (base, dtype, row stride).
 *   s_j = dot_KS(q, k_j, D) * scale,   j = 0..i
 *   chunks c = 0..floor(i/256) over keys [256c, min(256c+255, i)]   (absolute bounds;
 *   keys after i are not visited at all)
 *   per chunk: m_c = max s_j;  l_c = +0, o_c = +0;
 *              for j ascending: p = exp_f(s_j - m_c); l_c = l_c + p; o_c[d] = fma(p, v_j[d], o_c[d])
 *   merge, starting from chunk 0, c ascending:
 *              m' = max(m, m_c); a = exp_f(m - m'); b = exp_f(m_c - m');
 *              l = l*a + l_c*b;  o[d] = o[d]*a + o_c[d]*b;  m = m'
 *   out[d] = o[d] / l
 * Decode of position i is this same row; prefill computes every row this way. */
static void attention_row(const float* q, const void* Kb, const void* Vb, int dt, int64_t kstride,
                          int64_t i, int64_t D, float scale, float* out,
                          float* s /*[i+1]*/, float* kv /*[D]*/, float* o /*[D]*/, float* oc /*[D]*/) {
    for (int64_t j = 0; j <= i; ++j) {
        for (int64_t d = 0; d < D; ++d) kv[d] = ld_elem(Kb, dt, j * kstride + d);
        s[j] = dot_ks_f32(q, kv, D) * scale;
    }
    float m = 0.0f, l = 0.0f;
    int64_t nch = i / ORC_CHUNK + 1;
    for (int64_t c = 0; c < nch; ++c) {
        int64_t j0 = c * ORC_CHUNK;
        int64_t j1 = (c + 1) * ORC_CHUNK - 1 < i ? (c + 1) * ORC_CHUNK - 1 : i;
        float mc = s[j0];
        for (int64_t j = j0 + 1; j <= j1; ++j) if (s[j] > mc) mc = s[j];
        float lc = 0.0f;
        for (int64_t d = 0; d < D; ++d) oc[d] = 0.0f;
        for (int64_t j = j0; j <= j1; ++j) {
            float p = orc_exp_f(s[j] - mc);
            lc = lc + p;
            for (int64_t d = 0; d < D; ++d) oc[d] = fmaf(p, ld_elem(Vb, dt, j * kstride + d), oc[d]);
        }
        if (c == 0) {
            m = mc; l = lc;
            for (int64_t d = 0; d < D; ++d) o[d] = oc[d];
        } else {
            float mn = (mc > m) ? mc : m;
            float a = orc_exp_f(m - mn), b = orc_exp_f(mc - mn);
            l = (l * a) + (lc * b);
            for (int64_t d = 0; d < D; ++d) o[d] = (o[d] * a) + (oc[d] * b);
            m = mn;
        }
    }
    for (int64_t d = 0; d < D; ++d) out[d] = o[d] / l;
}

/* Causal attention for queries at positions q_start .. q_start+Tq-1 of B sequences.
 * Q [B, Tq, Hq, D]; caches [B, Hkv, Tmax, D] holding keys 0 .. q_start+Tq-1;
 * dt = 0: BF16 Q/K/V (upcast on read), dt = 1: FP32.  O fp32 [B, Tq, Hq, D].
 * Query head h reads kv head floor(h / (Hq/Hkv)). */
void orc_attention(int dt, const void* Q, const void* Kc, const void* Vc,
                   int64_t B, int64_t Tq, int64_t q_start, int64_t Tmax,
                   int64_t Hq, int64_t Hkv, int64_t D, float scale, float* O) {
    int64_t group = Hq / Hkv;
#pragma omp parallel
    {
        float* s = (float*)malloc(sizeof(float) * (size_t)(q_start + Tq));
        float* buf = (float*)malloc(sizeof(float) * (size_t)(4 * D));
#pragma omp for collapse(3) schedule(dynamic, 4)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t t = 0; t < Tq; ++t)
                for (int64_t h = 0; h < Hq; ++h) {
                    float* q = buf + 3 * D;
                    int64_t qo = ((b * Tq + t) * Hq + h) * D;
                    for (int64_t d = 0; d < D; ++d) q[d] = ld_elem(Q, dt, qo + d);
                    int64_t g = h / group;
                    int64_t ko = (b * Hkv + g) * Tmax * D;
                    const void* Kb = dt ? (const void*)((const float*)Kc + ko) : (const void*)((const uint16_t*)Kc + ko);
                    const void* Vb = dt ? (const void*)((const float*)Vc + ko) : (const void*)((const uint16_t*)Vc + ko);
                    attention_row(q, Kb, Vb, dt, D, q_start + t, D, scale, O + qo, s, buf, buf + D, buf + 2 * D);
                }
        free(s);
        free(buf);
    }
}

/* -------------------------------------------------------------- SwiGLU -- */
/* silu(a) = a / (1 + exp_f(-a)); h = silu(g) * u. */
void orc_swiglu(const float* G, const float* U, int64_t M, int64_t F, int64_t ldg, int64_t ldu,
                float* Hout, int64_t ldh) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t f = 0; f < F; ++f) {
            float g = G[m * ldg + f];
            float sg = g / (1.0f + orc_exp_f(-g));
            Hout[m * ldh + f] = sg * U[m * ldu + f];
        }
}

/* --------------------------------------------------------------- LM head -- */
/* One LM-head pass over one row.  a: the row's activation as used by this pass.
 *   z_v = dot_KS(a, up(W_v), K)
 *   top1 = lowest v with the largest z; top2 = lowest v != top1 with the largest of the rest
 *   (values compare with fp ==, so -0 == +0)
 *   M = z_top1; margin = z_top1 - z_top2
 *   S: vocabulary tile u covers v in [1024u, 1024u+1024); lane l (0..63) sums
 *      exp_f(z_v - M) for v = 1024u + 64j + l, j = 0..15 ascending (v < V only), from +0;
 *      then lanes combine pairwise, a_l = a_l + a_{l+w} for l = 0 mod 2w, w = 1,2,...,32;
 *      S_u = a_0; S = S_0, then S = S + S_u for u ascending
 *   lp = (z_target - M) - log_f(S)                                                    */
/* Row statistics of logits z[0..V): top-2 (lowest index first on ties), M = z_top1 and S, the
 * fixed tree of exp_f(z_v - M) (tiles of 1024, 64 lanes, pairwise lane tree, tiles folded in
 * ascending order).
 * NaN logits are unordered, so they never take part in the top-2: top1 is the lowest index
 * of the largest non-NaN logit and top2 the lowest index != top1 of the largest non-NaN
 * logit of the rest.  Where no such index exists the choice falls back to index 0 for top1
 * and to the lowest index != top1 for top2 (a row of NaN logits gives (0, 1)).  Any NaN in
 * the row still reaches S, and through it the logprob. */
static void lmhead_stats(const float* z, int64_t V, float* Mout, float* Sout, int64_t* t1, int64_t* t2) {
    int64_t b1 = -1;
    for (int64_t v = 0; v < V; ++v)
        if (z[v] == z[v] && (b1 < 0 || z[v] > z[b1])) b1 = v;
    if (b1 < 0) b1 = 0;
    int64_t b2 = -1;
    for (int64_t v = 0; v < V; ++v)
        if (v != b1 && z[v] == z[v] && (b2 < 0 || z[v] > z[b2])) b2 = v;
    if (b2 < 0) b2 = (b1 == 0) ? 1 : 0;
    float M = z[b1];
    float S = 0.0f;
    int64_t ntiles = (V + ORC_TV - 1) / ORC_TV;
    for (int64_t u = 0; u < ntiles; ++u) {
        float lane[ORC_LW];
        for (int l = 0; l < ORC_LW; ++l) {
            float acc = 0.0f;
            for (int j = 0; j < ORC_TV / ORC_LW; ++j) {
                int64_t v = u * ORC_TV + (int64_t)j * ORC_LW + l;
                if (v < V) acc = acc + orc_exp_f(z[v] - M);
            }
            lane[l] = acc;
        }
        for (int w = 1; w < ORC_LW; w *= 2)
            for (int l = 0; l < ORC_LW; l += 2 * w) lane[l] = lane[l] + lane[l + w];
        S = (u == 0) ? lane[0] : S + lane[0];
    }
    *Mout = M;
    *Sout = S;
    *t1 = b1;
    *t2 = b2;
}

/* The same row statistics for a caller-supplied logit row (the test suite pins the tile/lane
 * tree of S with it). */
void orc_lmhead_stats(const float* z, int64_t V, float* M, float* S, int32_t* top1, int32_t* top2) {
    int64_t b1, b2;
    lmhead_stats(z, V, M, S, &b1, &b2);
    *top1 = (int32_t)b1;
    *top2 = (int32_t)b2;
}

static void lmhead_pass(const float* a, int64_t K, const uint16_t* W, int64_t ldw, int64_t V,
                        int32_t target, float* z, float* lp, float* margin, int32_t* t1, int32_t* t2) {
#pragma omp parallel for schedule(static) if (!omp_in_parallel())
    for (int64_t v = 0; v < V; ++v) z[v] = dot_ks_w16(a, W + v * ldw, K);
    float M, S;
    int64_t b1, b2;
    lmhead_stats(z, V, &M, &S, &b1, &b2);
    *lp = (z[target] - M) - orc_log_f(S);
    *margin = M - z[b2];
    *t1 = (int32_t)b1;
    *t2 = (int32_t)b2;
}

/* Selective FP32 recompute for one row: pass P on up(bf(h)) (BF16 operands, FP32 sums);
 * when margin_P < tau (strict), pass F on h itself and F's results are returned with flag 1. */
static void lmhead_row(const float* h, int64_t K, const uint16_t* W, int64_t ldw, int64_t V,
                       int32_t target, float tau, float* z, float* aP,
                       float* lp, float* margin, int32_t* t1, int32_t* t2, uint8_t* flag) {
    for (int64_t k = 0; k < K; ++k) aP[k] = orc_bf16_up(orc_bf16_rne(h[k]));
    lmhead_pass(aP, K, W, ldw, V, target, z, lp, margin, t1, t2);
    if (*margin < tau) {
        lmhead_pass(h, K, W, ldw, V, target, z, lp, margin, t1, t2);
        *flag = 1;
    } else {
        *flag = 0;
    }
}

static void lmhead_one(const float* h, int64_t K, const uint16_t* W, int64_t V, int32_t target,
                       float tau, int mode, float* z, float* aP,
                       float* lp, float* margin, int32_t* t1, int32_t* t2, uint8_t* flag) {
    if (mode == 0) {
        lmhead_row(h, K, W, K, V, target, tau, z, aP, lp, margin, t1, t2, flag);
    } else if (mode == 1) {
        for (int64_t k = 0; k < K; ++k) aP[k] = orc_bf16_up(orc_bf16_rne(h[k]));
        lmhead_pass(aP, K, W, K, V, target, z, lp, margin, t1, t2);
        *flag = 0;
    } else {
        lmhead_pass(h, K, W, K, V, target, z, lp, margin, t1, t2);
        *flag = 1;
    }
}

/* mode 0: selective (P, then F when margin_P < tau); mode 1: P only; mode 2: F only.
 * Rows are independent; with fewer rows than threads, each row's logits are split
 * over threads instead (still one output per thread, same order per output). */
void orc_lmhead(const float* Hs, int64_t B, int64_t K, int64_t ldh, const uint16_t* W, int64_t V,
                const int32_t* target, float tau, int mode,
                float* lp, float* margin, int32_t* top1, int32_t* top2, uint8_t* flag) {
    if (B >= (int64_t)omp_get_max_threads()) {
#pragma omp parallel
        {
            float* z = (float*)malloc(sizeof(float) * (size_t)V);
            float* aP = (float*)malloc(sizeof(float) * (size_t)K);
#pragma omp for schedule(dynamic, 1)
            for (int64_t b = 0; b < B; ++b)
                lmhead_one(Hs + b * ldh, K, W, V, target[b], tau, mode, z, aP,
                           lp + b, margin + b, top1 + b, top2 + b, flag + b);
            free(z);
            free(aP);
        }
    } else {
        float* z = (float*)malloc(sizeof(float) * (size_t)V);
        float* aP = (float*)malloc(sizeof(float) * (size_t)K);
        for (int64_t b = 0; b < B; ++b)
            lmhead_one(Hs + b * ldh, K, W, V, target[b], tau, mode, z, aP,
                       lp + b, margin + b, top1 + b, top2 + b, flag + b);
        free(z);
        free(aP);
    }
}

/* ------------------------------------------------------ logit gradient -- */
/* Gradient, with respect to the FP32 logits z = dot_KS(h, up(W_v)), of coef * lp, where lp is
 * the log-probability of the target under the FP32 pass (the pass every row takes with
 * tau = +inf: a trainer's policy-gradient term for one token):
 *   p_v = exp_f(z_v - M) / S        (M and S exactly as the forward computes them)
 *   g_v = coef * ((v == target ? 1 : 0) - p_v)
 * d lp / d z_v = [v == target] - softmax_v, the softmax in the forward's fixed order (Meituan
 * page, "principles": the logprob accumulation is one of the order-sensitive sums, in
 * training as in inference).  Hs fp32 [B, K] (ldh); W bf16 [V, K]; G fp32 [B, V] (ldg);
 * lp (optional) [B] the forward logprob of the same pass. */
void orc_lmhead_logit_grad(const float* Hs, int64_t B, int64_t K, int64_t ldh, const uint16_t* W, int64_t V,
                           const int32_t* target, const float* coef, float* G, int64_t ldg, float* lp) {
    for (int64_t b = 0; b < B; ++b) {
        const float* h = Hs + b * ldh;
        float* z = G + b * ldg;
#pragma omp parallel for schedule(static)
        for (int64_t v = 0; v < V; ++v) z[v] = dot_ks_w16(h, W + v * K, K);
        float M, S;
        int64_t b1, b2;
        lmhead_stats(z, V, &M, &S, &b1, &b2);
        int32_t t = target[b];
        if (lp) lp[b] = (t >= 0 && t < V) ? (z[t] - M) - orc_log_f(S) : NAN;
        for (int64_t v = 0; v < V; ++v) {
            float p = orc_exp_f(z[v] - M) / S;
            float q = (v == t ? 1.0f : 0.0f) - p;
            z[v] = coef[b] * q;
        }
    }
}

/* -------------------------------------------------------------- decoder -- */
/* Llama-shaped decoder on one sequence (the pages' LayerCast setting: BF16 weights,
 * everything computed in FP32, activations and KV cache in FP32):
 *   x_t = up(E[tok_t])
 *   per layer: n = rmsnorm(x, g1); [q|k|v] = n Wqkv^T; q,k = RoPE at position t;
 *              x = x + attn(q, k, v) Wo^T;
 *              n = rmsnorm(x, g2); [g|u] = n W13^T; x = x + (silu(g) * u) W2^T
 *   n = rmsnorm(x, gf); for t = 0..T-1: LM-head row (selective recompute) with target tgt_t.
 * The same decoder with BF16 or FP16 activation storage (act_fmt 1 or 2) is the low-precision
 * body of the cross-precision comparison ("Greedy Decoding Is Not Precision-Invariant",
 * abstract); the weights and the LM head are unchanged.
 * Weight layouts: Wqkv [(Hq+2Hkv)D, H] (q rows, then k rows, then v rows);
 * Wo [H, Hq D]; W13 [2F, H] (gate rows, then up rows); W2 [H, F]; Whead [V, H]. */
void orc_decoder(const int32_t* tok, int64_t T, int64_t H, int64_t Hq, int64_t Hkv, int64_t D,
                 int64_t F, int64_t V, int64_t nlayers,
                 const uint16_t* emb, const uint16_t* const* lw /* nlayers*6 pointers */,
                 const uint16_t* gf, const uint16_t* whead, const float* cos_t, const float* sin_t,
                 float eps, float scale, float tau, int act_fmt,
                 const int32_t* tgt /* [T]: target of every position; all T rows are scored */,
                 float* lp, float* margin, int32_t* top1, int32_t* top2, uint8_t* flag,
                 float* x_out /* optional [T, H]: final normed hidden */) {
    int64_t QD = Hq * D, KD = Hkv * D, NQKV = QD + 2 * KD;
    float* x = (float*)malloc(sizeof(float) * (size_t)(T * H));
    float* n = (float*)malloc(sizeof(float) * (size_t)(T * H));
    float* qkv = (float*)malloc(sizeof(float) * (size_t)(T * NQKV));
    float* q = (float*)malloc(sizeof(float) * (size_t)(T * QD));
    float* kc = (float*)malloc(sizeof(float) * (size_t)(KD * T));
    float* vc = (float*)malloc(sizeof(float) * (size_t)(KD * T));
    float* att = (float*)malloc(sizeof(float) * (size_t)(T * QD));
    float* y = (float*)malloc(sizeof(float) * (size_t)(T * (H > 2 * F ? H : 2 * F)));
    float* hh = (float*)malloc(sizeof(float) * (size_t)(T * F));
    int32_t* pos = (int32_t*)malloc(sizeof(int32_t) * (size_t)T);
    float* ktmp = (float*)malloc(sizeof(float) * (size_t)(T * KD));
    /* act_fmt != 0: every activation tensor an unfused implementation would store between
     * operations is rounded to that format (embedding, each norm output, each projection
     * output, rotated q and k, attention output, the SwiGLU product, each residual sum);
     * each operation still computes in FP32 from the rounded inputs. */
    for (int64_t t = 0; t < T; ++t) pos[t] = (int32_t)t;
    for (int64_t t = 0; t < T; ++t)
        for (int64_t k = 0; k < H; ++k) x[t * H + k] = orc_bf16_up(emb[(int64_t)tok[t] * H + k]);
    round_all(x, T * H, act_fmt);
    for (int64_t L = 0; L < nlayers; ++L) {
        const uint16_t* const* w = lw + 6 * L;
        orc_rmsnorm(x, T, H, H, w[0], eps, n, H);
        round_all(n, T * H, act_fmt);
        orc_gemm(n, T, H, H, w[1], NQKV, H, qkv, NQKV);
        round_all(qkv, T * NQKV, act_fmt);
        orc_rope(qkv, T, Hq, D, NQKV, pos, cos_t, sin_t, q, QD);
        orc_rope(qkv + QD, T, Hkv, D, NQKV, pos, cos_t, sin_t, ktmp, KD);
        round_all(q, T * QD, act_fmt);
        round_all(ktmp, T * KD, act_fmt);
        /* cache layout [Hkv, T, D] for this one sequence */
        for (int64_t t = 0; t < T; ++t)
            for (int64_t g = 0; g < Hkv; ++g)
                for (int64_t d = 0; d < D; ++d) {
                    kc[(g * T + t) * D + d] = ktmp[t * KD + g * D + d];
                    vc[(g * T + t) * D + d] = qkv[t * NQKV + QD + KD + g * D + d];
                }
        orc_attention(1, q, kc, vc, 1, T, 0, T, Hq, Hkv, D, scale, att);
        round_all(att, T * QD, act_fmt);
        orc_gemm(att, T, QD, QD, w[2], H, QD, y, H);
        round_all(y, T * H, act_fmt);
        for (int64_t i = 0; i < T * H; ++i) x[i] = x[i] + y[i];
        round_all(x, T * H, act_fmt);
        orc_rmsnorm(x, T, H, H, w[3], eps, n, H);
        round_all(n, T * H, act_fmt);
        orc_gemm(n, T, H, H, w[4], 2 * F, H, y, 2 * F);
        round_all(y, T * 2 * F, act_fmt);
        orc_swiglu(y, y + F, T, F, 2 * F, 2 * F, hh, F);
        round_all(hh, T * F, act_fmt);
        orc_gemm(hh, T, F, F, w[5], H, F, y, H);
        round_all(y, T * H, act_fmt);
        for (int64_t i = 0; i < T * H; ++i) x[i] = x[i] + y[i];
        round_all(x, T * H, act_fmt);
    }
    orc_rmsnorm(x, T, H, H, gf, eps, n, H);
    round_all(n, T * H, act_fmt);
    if (x_out) memcpy(x_out, n, sizeof(float) * (size_t)(T * H));
    orc_lmhead(n, T, H, H, whead, V, tgt, tau, 0, lp, margin, top1, top2, flag);
    free(x); free(n); free(qkv); free(q); free(kc); free(vc); free(att); free(y); free(hh); free(pos); free(ktmp);
}
