// abi.hip -- extern "C" entry points of libinvnum.so: argument validation, then launches.
// Every check happens before anything is enqueued, so a rejected call leaves the stream
// untouched.  Status codes and argument meaning are documented in include/invnum.h.
#include "invnum.h"
#include "kernels.h"
#include "numerics.h"

#include <stdio.h>
#include <string.h>

using namespace invnum;

namespace {

inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline hipStream_t S(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline int fin(hipError_t e) { return e == hipSuccess ? INV_OK : INV_ERR_LAUNCH; }
constexpr int64_t I32MAX = 2147483647;

}  // namespace

extern "C" {

const char* inv_status_string(int status) {
    switch (status) {
        case INV_OK: return "ok";
        case INV_ERR_NULL: return "null pointer argument";
        case INV_ERR_SHAPE: return "invalid or inconsistent shape";
        case INV_ERR_ALIGN: return "pointer or leading dimension not 16-byte aligned";
        case INV_ERR_DTYPE: return "unknown dtype code";
        case INV_ERR_WORKSPACE: return "workspace missing or too small";
        case INV_ERR_UNSUPPORTED: return "unsupported shape";
        case INV_ERR_LAUNCH: return "kernel launch failed";
        default: return "unknown status";
    }
}

int inv_get_constants(inv_constants* out) {
    if (!out) return INV_ERR_NULL;
    memset(out, 0, sizeof(*out));
    out->ks = KS;
    out->chunk = CHUNK;
    out->vocab_tile = TV;
    out->lanes = LW;
    const int n = (int)(sizeof(kFloatConsts) / sizeof(kFloatConsts[0]));
    out->n_float = n;
    for (int i = 0; i < n; ++i) out->float_consts[i] = kFloatConsts[i];
    return INV_OK;
}

int inv_fixed_order_gemm(const float* X, int64_t M, int64_t K, int64_t ldx, const uint16_t* W,
                         int64_t N, int64_t ldw, const float* R, int64_t ldr, float* Y, int64_t ldy,
                         void* stream) {
    if (!X || !W || !Y) return INV_ERR_NULL;
    if (M < 1 || N < 1 || K < 8 || K % 8 != 0 || M > I32MAX || N > I32MAX || K > I32MAX)
        return INV_ERR_SHAPE;
    if (ldx < K || ldw < K || ldy < N || (R && ldr < N)) return INV_ERR_SHAPE;
    if (!al16(X) || !al16(W) || ldx % 4 || ldw % 8) return INV_ERR_ALIGN;
    if ((reinterpret_cast<uintptr_t>(Y) & 3u) || (R && (reinterpret_cast<uintptr_t>(R) & 3u)))
        return INV_ERR_ALIGN;
    GemmArgs a{X, (int)M, (int)K, ldx, W, (int)N, ldw, R, ldr, Y, ldy, nullptr};
    return fin(launch_gemm(a, S(stream)));
}

int inv_gated_gemm(const float* X, int64_t M, int64_t K, int64_t ldx, const uint16_t* W, int64_t N2,
                   int64_t ldw, float* H, int64_t ldh, void* stream) {
    if (!X || !W || !H) return INV_ERR_NULL;
    if (M < 1 || N2 < 2 || N2 % 2 != 0 || K < 8 || K % 8 != 0 || M > I32MAX || N2 > I32MAX || K > I32MAX)
        return INV_ERR_SHAPE;
    if (ldx < K || ldw < K || ldh < N2 / 2) return INV_ERR_SHAPE;
    if (!al16(X) || !al16(W) || ldx % 4 || ldw % 8) return INV_ERR_ALIGN;
    if (reinterpret_cast<uintptr_t>(H) & 3u) return INV_ERR_ALIGN;
    GemmArgs a{X, (int)M, (int)K, ldx, W, (int)N2, ldw, nullptr, 0, H, ldh, nullptr};
    return fin(launch_gemm(a, S(stream), 2));
}

int inv_rmsnorm(const float* X, int64_t M, int64_t H, int64_t ldx, const uint16_t* gamma, float eps,
                float* Y, int64_t ldy, void* stream) {
    if (!X || !gamma || !Y) return INV_ERR_NULL;
    if (M < 1 || H < 8 || H % 8 != 0 || ldx < H || ldy < H || M > I32MAX) return INV_ERR_SHAPE;
    if (H > 16384) return INV_ERR_UNSUPPORTED;
    if (!al16(X) || !al16(Y) || !al16(gamma) || ldx % 4 || ldy % 4) return INV_ERR_ALIGN;
    return fin(launch_rmsnorm(X, (int)M, (int)H, ldx, gamma, eps, Y, ldy, S(stream)));
}

size_t inv_qkv_rope_kv_append_workspace_bytes(int64_t M, int64_t Hq, int64_t Hkv, int64_t D) {
    if (M < 1 || Hq < 1 || Hkv < 0 || D < 1) return 0;
    if (qkv_rope_fusable(M, D)) return 0;
    return sizeof(float) * (size_t)(M * (Hq + 2 * Hkv) * D);
}

int inv_qkv_rope_kv_append(const float* X, int64_t M, int64_t K, int64_t ldx, const uint16_t* Wqkv, int64_t ldw,
                           int64_t Hq, int64_t Hkv, int64_t D, const int32_t* seq, const int32_t* pos,
                           const float* cos_t, const float* sin_t, int64_t Tmax, int64_t Bcache, float* Qout,
                           float* Kc, float* Vc, void* ws, size_t ws_bytes, void* stream) {
    if (!X || !Wqkv || !seq || !pos || !cos_t || !sin_t || !Qout || !Kc || !Vc) return INV_ERR_NULL;
    if (M < 1 || K < 8 || K % 8 != 0 || Hq < 1 || Hkv < 1 || D < 2 || D % 2 != 0 || Tmax < 1 || Bcache < 1 ||
        ldx < K || ldw < K || M > I32MAX || K > I32MAX || Tmax > I32MAX || Bcache > I32MAX ||
        (Hq + 2 * Hkv) * D > I32MAX)
        return INV_ERR_SHAPE;
    if (!al16(X) || !al16(Wqkv) || ldx % 4 || ldw % 8) return INV_ERR_ALIGN;
    const int64_t N = (Hq + 2 * Hkv) * D;
    const size_t need = inv_qkv_rope_kv_append_workspace_bytes(M, Hq, Hkv, D);
    if (need && (!ws || ws_bytes < need)) return INV_ERR_WORKSPACE;
    if (need && !al16(ws)) return INV_ERR_ALIGN;
    if (!need) {
        GemmArgs a{X, (int)M, (int)K, ldx, Wqkv, (int)N, ldw, nullptr, 0, nullptr, 0, nullptr};
        RopeArgs ra{(int)Hq, (int)Hkv, seq, pos, cos_t, sin_t, (int)Tmax, (int)Bcache, Qout, Kc, Vc};
        return fin(launch_qkv_rope(a, ra, S(stream)));
    }
    float* qkv = reinterpret_cast<float*>(ws);
    GemmArgs a{X, (int)M, (int)K, ldx, Wqkv, (int)N, ldw, nullptr, 0, qkv, N, nullptr};
    if (launch_gemm(a, S(stream), 0) != hipSuccess) return INV_ERR_LAUNCH;
    return fin(launch_rope_kv_append(qkv, (int)M, N, (int)Hq, (int)Hkv, (int)D, seq, pos, cos_t, sin_t, (int)Tmax,
                                     (int)Bcache, Qout, Kc, Vc, INV_F32, S(stream)));
}

// [a, a + an) and [b, b + bn) (bytes) overlap
static bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + bn && pb < pa + an;
}

int inv_rmsnorm_gemm(const float* X, int64_t M, int64_t K, int64_t ldx, const uint16_t* gamma, float eps,
                     const uint16_t* W, int64_t N, int64_t ldw, const float* R, int64_t ldr, float* Y, int64_t ldy,
                     int gated, void* stream) {
    if (!X || !gamma || !W || !Y) return INV_ERR_NULL;
    if (gated != 0 && gated != 1) return INV_ERR_SHAPE;
    if (N < 1 || K < 8 || K % 8 != 0 || M > I32MAX || N > I32MAX || K > I32MAX) return INV_ERR_SHAPE;
    if (gated && (N < 2 || N % 2 != 0 || R)) return INV_ERR_SHAPE;
    const int64_t ny = gated ? N / 2 : N;
    if (M < 1 || ldx < K || ldw < K || ldy < ny || (R && ldr < N)) return INV_ERR_SHAPE;
    if (!gemm_norm_fusable(M) || K > 16384) return INV_ERR_UNSUPPORTED;
    if (!al16(X) || !al16(W) || !al16(gamma) || ldx % 4 || ldw % 8) return INV_ERR_ALIGN;
    if ((reinterpret_cast<uintptr_t>(Y) & 3u) || (R && (reinterpret_cast<uintptr_t>(R) & 3u)))
        return INV_ERR_ALIGN;
    // every workgroup reads the whole rows of X while others already store Y
    if (overlaps(X, sizeof(float) * (size_t)((M - 1) * ldx + K), Y, sizeof(float) * (size_t)((M - 1) * ldy + ny)))
        return INV_ERR_SHAPE;
    GemmArgs a{X, (int)M, (int)K, ldx, W, (int)N, ldw, R, ldr, Y, ldy, nullptr, gamma, eps};
    return fin(launch_gemm(a, S(stream), gated ? 2 : 0));
}

int inv_rmsnorm_qkv_rope_kv_append(const float* X, int64_t M, int64_t K, int64_t ldx, const uint16_t* gamma,
                                   float eps, const uint16_t* Wqkv, int64_t ldw, int64_t Hq, int64_t Hkv, int64_t D,
                                   const int32_t* seq, const int32_t* pos, const float* cos_t, const float* sin_t,
                                   int64_t Tmax, int64_t Bcache, float* Qout, float* Kc, float* Vc, void* stream) {
    if (!X || !gamma || !Wqkv || !seq || !pos || !cos_t || !sin_t || !Qout || !Kc || !Vc) return INV_ERR_NULL;
    if (M < 1 || K < 8 || K % 8 != 0 || Hq < 1 || Hkv < 1 || D < 2 || D % 2 != 0 || Tmax < 1 || Bcache < 1 ||
        ldx < K || ldw < K || M > I32MAX || K > I32MAX || Tmax > I32MAX || Bcache > I32MAX ||
        (Hq + 2 * Hkv) * D > I32MAX)
        return INV_ERR_SHAPE;
    if (!qkv_rope_fusable(M, D) || !gemm_norm_fusable(M) || K > 16384) return INV_ERR_UNSUPPORTED;
    if (!al16(X) || !al16(Wqkv) || !al16(gamma) || ldx % 4 || ldw % 8) return INV_ERR_ALIGN;
    const int64_t N = (Hq + 2 * Hkv) * D;
    // every workgroup reads the whole rows of X while others already store q, k and v
    const size_t xb = sizeof(float) * (size_t)((M - 1) * ldx + K);
    if (overlaps(X, xb, Qout, sizeof(float) * (size_t)(M * Hq * D)) ||
        overlaps(X, xb, Kc, sizeof(float) * (size_t)(Bcache * Hkv * Tmax * D)) ||
        overlaps(X, xb, Vc, sizeof(float) * (size_t)(Bcache * Hkv * Tmax * D)))
        return INV_ERR_SHAPE;
    GemmArgs a{X, (int)M, (int)K, ldx, Wqkv, (int)N, ldw, nullptr, 0, nullptr, 0, nullptr, gamma, eps};
    RopeArgs ra{(int)Hq, (int)Hkv, seq, pos, cos_t, sin_t, (int)Tmax, (int)Bcache, Qout, Kc, Vc};
    return fin(launch_qkv_rope(a, ra, S(stream)));
}

static int check_attn(int dtype, const void* Q, const void* Kc, const void* Vc, const float* O,
                      int64_t B, int64_t Tq, int64_t q_start, int64_t Tmax, int64_t Hq, int64_t Hkv,
                      int64_t D) {
    if (!Q || !Kc || !Vc || !O) return INV_ERR_NULL;
    if (dtype != INV_BF16 && dtype != INV_F32) return INV_ERR_DTYPE;
    if (B < 1 || Tq < 1 || q_start < 0 || Tmax < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 ||
        q_start + Tq > Tmax || B > 65535 || Hq > 65535 || Tmax > I32MAX / 2)
        return INV_ERR_SHAPE;
    if (D != 128 || Hq / Hkv > 16) return INV_ERR_UNSUPPORTED;
    if (!al16(Q) || !al16(Kc) || !al16(Vc) || !al16(O)) return INV_ERR_ALIGN;
    return INV_OK;
}

int inv_attention_prefill(int dtype, const void* Q, const void* Kc, const void* Vc, int64_t B,
                          int64_t Tq, int64_t q_start, int64_t Tmax, int64_t Hq, int64_t Hkv,
                          int64_t D, float scale, float* O, void* stream) {
    int st = check_attn(dtype, Q, Kc, Vc, O, B, Tq, q_start, Tmax, Hq, Hkv, D);
    if (st != INV_OK) return st;
    AttnArgs a{dtype, Q, Kc, Vc, (int)B, (int)Tq, (int)q_start, (int)Tmax, (int)Hq, (int)Hkv, (int)D,
               scale, O};
    return fin(launch_attention_prefill(a, nullptr, 0, S(stream)));
}

size_t inv_attention_prefill_workspace_bytes(int64_t B, int64_t Tq, int64_t q_start, int64_t Hq, int64_t D) {
    if (B < 1 || Tq < 1 || q_start < 0 || Hq < 1 || D != 128) return 0;
    return prefill_split_ws_bytes(B, Tq, q_start, Hq);
}

int inv_attention_prefill_ws(int dtype, const void* Q, const void* Kc, const void* Vc, int64_t B,
                             int64_t Tq, int64_t q_start, int64_t Tmax, int64_t Hq, int64_t Hkv,
                             int64_t D, float scale, float* O, void* ws, size_t ws_bytes, void* stream) {
    int st = check_attn(dtype, Q, Kc, Vc, O, B, Tq, q_start, Tmax, Hq, Hkv, D);
    if (st != INV_OK) return st;
    const size_t need = inv_attention_prefill_workspace_bytes(B, Tq, q_start, Hq, D);
    if (need && (!ws || ws_bytes < need)) return INV_ERR_WORKSPACE;
    if (need && !al16(ws)) return INV_ERR_ALIGN;
    AttnArgs a{dtype, Q, Kc, Vc, (int)B, (int)Tq, (int)q_start, (int)Tmax, (int)Hq, (int)Hkv, (int)D,
               scale, O};
    return fin(launch_attention_prefill(a, need ? reinterpret_cast<float*>(ws) : nullptr, ws_bytes, S(stream)));
}

size_t inv_attention_decode_workspace_bytes(int64_t B, int64_t Tmax, int64_t Hq, int64_t D) {
    if (B < 1 || Tmax < 1 || Hq < 1 || D < 1) return 0;
    const int64_t nch = (Tmax + CHUNK - 1) / CHUNK;
    return sizeof(float) * (size_t)(B * Hq * nch * (D + 2));
}

int inv_attention_decode(int dtype, const void* Q, const void* Kc, const void* Vc, const int32_t* pos,
                         int64_t B, int64_t Tmax, int64_t Hq, int64_t Hkv, int64_t D, float scale,
                         float* O, void* ws, size_t ws_bytes, void* stream) {
    if (!pos) return INV_ERR_NULL;
    int st = check_attn(dtype, Q, Kc, Vc, O, B, 1, 0, Tmax, Hq, Hkv, D);
    if (st != INV_OK) return st;
    if (Tmax > (int64_t)4096 * CHUNK) return INV_ERR_UNSUPPORTED;   // merge keeps <= 4096 chunks
    if (!ws || ws_bytes < inv_attention_decode_workspace_bytes(B, Tmax, Hq, D)) return INV_ERR_WORKSPACE;
    if (!al16(ws)) return INV_ERR_ALIGN;
    AttnArgs a{dtype, Q, Kc, Vc, (int)B, 1, 0, (int)Tmax, (int)Hq, (int)Hkv, (int)D, scale, O};
    return fin(launch_attention_decode(a, pos, reinterpret_cast<float*>(ws), S(stream)));
}

size_t inv_attention_decode_noalloc_max_bytes(void) { return DECODE_SCRATCH_BYTES; }

int inv_attention_decode_noalloc(int dtype, const void* Q, const void* Kc, const void* Vc, const int32_t* pos,
                                 int64_t B, int64_t Tmax, int64_t Hq, int64_t Hkv, int64_t D, float scale,
                                 float* O, void* stream) {
    if (!pos) return INV_ERR_NULL;
    int st = check_attn(dtype, Q, Kc, Vc, O, B, 1, 0, Tmax, Hq, Hkv, D);
    if (st != INV_OK) return st;
    if (Tmax > (int64_t)4096 * CHUNK) return INV_ERR_UNSUPPORTED;
    if (inv_attention_decode_workspace_bytes(B, Tmax, Hq, D) > DECODE_SCRATCH_BYTES) return INV_ERR_WORKSPACE;
    float* ws = nullptr;
    if (decode_scratch(&ws) != hipSuccess) return INV_ERR_LAUNCH;
    AttnArgs a{dtype, Q, Kc, Vc, (int)B, 1, 0, (int)Tmax, (int)Hq, (int)Hkv, (int)D, scale, O};
    return fin(launch_attention_decode(a, pos, ws, S(stream)));
}

size_t inv_lmhead_workspace_bytes(int64_t B, int64_t K, int64_t V) {
    if (B < 1 || K < 1 || V < 1) return 0;
    return lmhead_ws_bytes(B, K, V);
}

int inv_lmhead_logprob_top2(const float* Hs, int64_t B, int64_t K, int64_t ldh, const uint16_t* W,
                            int64_t V, const int32_t* target, float tau, float* logprob, float* margin,
                            int32_t* top1, int32_t* top2, uint8_t* recomputed, void* ws,
                            size_t ws_bytes, void* stream) {
    if (!Hs || !W || !target || !logprob || !margin || !top1 || !top2 || !recomputed)
        return INV_ERR_NULL;
    if (B < 1 || K < 8 || K % 8 != 0 || V < 2 || ldh < K || B > 65535 || K > I32MAX ||
        V > (int64_t)1024 * TV)
        return INV_ERR_SHAPE;
    if (!ws || ws_bytes < inv_lmhead_workspace_bytes(B, K, V)) return INV_ERR_WORKSPACE;
    if (!al16(Hs) || !al16(W) || !al16(ws) || ldh % 4) return INV_ERR_ALIGN;
    LmheadArgs a{Hs, (int)B, (int)K, ldh, W, (int)V, target, tau, logprob, margin, top1, top2,
                 recomputed, ws};
    return fin(launch_lmhead(a, S(stream)));
}

size_t inv_lmhead_logit_grad_workspace_bytes(int64_t B, int64_t K, int64_t V) {
    (void)K;
    if (B < 1 || V < 2) return 0;
    return logit_grad_ws_bytes(B, V);
}

int inv_lmhead_logit_grad(const float* Hs, int64_t B, int64_t K, int64_t ldh, const uint16_t* W, int64_t V,
                          const int32_t* target, const float* coef, float* G, float* logprob, void* ws,
                          size_t ws_bytes, void* stream) {
    if (!Hs || !W || !target || !coef || !G) return INV_ERR_NULL;
    if (B < 1 || K < 8 || K % 8 != 0 || V < 2 || ldh < K || B > 65535 || K > I32MAX || V > (int64_t)1024 * TV ||
        B * V > ((int64_t)1 << 40))
        return INV_ERR_SHAPE;
    if (!ws || ws_bytes < inv_lmhead_logit_grad_workspace_bytes(B, K, V)) return INV_ERR_WORKSPACE;
    if (!al16(Hs) || !al16(W) || !al16(ws) || ldh % 4 || (reinterpret_cast<uintptr_t>(G) & 3u))
        return INV_ERR_ALIGN;
    LogitGradArgs a{Hs, (int)B, (int)K, ldh, W, (int)V, target, coef, G, logprob, ws};
    return fin(launch_logit_grad(a, S(stream)));
}

size_t inv_gemm_backward_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M < 1 || N < 1 || K < 1) return 0;
    return gemm_backward_ws_bytes(M, N, K);
}

int inv_gemm_backward(const float* dY, int64_t M, int64_t N, int64_t lddy, const float* X, int64_t K,
                      int64_t ldx, const uint16_t* W, int64_t ldw, float* dX, int64_t lddx, float* dW,
                      int64_t lddw, void* ws, size_t ws_bytes, void* stream) {
    if (!dY || (dX && !W) || (dW && !X)) return INV_ERR_NULL;
    if (M < 1 || N < 8 || N % 8 != 0 || K < 4 || K % 4 != 0 || lddy < N || M > I32MAX || N > I32MAX ||
        K > I32MAX)
        return INV_ERR_SHAPE;
    if (dX && (ldw < K || lddx < K)) return INV_ERR_SHAPE;
    if (dW && (ldx < K || lddw < K)) return INV_ERR_SHAPE;
    if (!al16(dY) || lddy % 4) return INV_ERR_ALIGN;
    if (dX) {
        if (!ws || ws_bytes < inv_gemm_backward_workspace_bytes(M, N, K)) return INV_ERR_WORKSPACE;
        if ((reinterpret_cast<uintptr_t>(W) & 1u) || (reinterpret_cast<uintptr_t>(ws) & 255u) ||
            (reinterpret_cast<uintptr_t>(dX) & 3u))
            return INV_ERR_ALIGN;
    }
    if (dW && (!al16(X) || ldx % 4 || (reinterpret_cast<uintptr_t>(dW) & 3u))) return INV_ERR_ALIGN;
    if (!dX && !dW) return INV_OK;
    return fin(launch_gemm_backward(dY, (int)M, (int)N, lddy, X, (int)K, ldx, W, ldw, dX, lddx, dW, lddw, ws,
                                    S(stream)));
}

int inv_embed(const int32_t* ids, int64_t M, const uint16_t* table, int64_t vocab, int64_t H, float* X,
              int64_t ldx, void* stream) {
    if (!ids || !table || !X) return INV_ERR_NULL;
    if (M < 1 || vocab < 1 || H < 8 || H % 8 != 0 || ldx < H || M > I32MAX || vocab > I32MAX)
        return INV_ERR_SHAPE;
    if (!al16(table) || !al16(X) || ldx % 4) return INV_ERR_ALIGN;
    return fin(launch_embed(ids, (int)M, table, (int)vocab, (int)H, X, ldx, S(stream)));
}

int inv_rope_kv_append(const float* QKV, int64_t M, int64_t ldqkv, int64_t Hq, int64_t Hkv, int64_t D,
                       const int32_t* seq, const int32_t* pos, const float* cos_t, const float* sin_t,
                       int64_t Tmax, int64_t Bcache, float* Qout, float* Kc, float* Vc, int out_fmt,
                       void* stream) {
    if (!QKV || !seq || !pos || !cos_t || !sin_t || !Qout || !Kc || !Vc) return INV_ERR_NULL;
    if (out_fmt != INV_BF16 && out_fmt != INV_F16 && out_fmt != INV_F32) return INV_ERR_DTYPE;
    if (M < 1 || Hq < 1 || Hkv < 1 || D < 2 || D % 2 != 0 || Tmax < 1 || Bcache < 1 ||
        ldqkv < (Hq + 2 * Hkv) * D || M > I32MAX || Tmax > I32MAX || Bcache > I32MAX)
        return INV_ERR_SHAPE;
    return fin(launch_rope_kv_append(QKV, (int)M, ldqkv, (int)Hq, (int)Hkv, (int)D, seq, pos, cos_t,
                                     sin_t, (int)Tmax, (int)Bcache, Qout, Kc, Vc, out_fmt, S(stream)));
}

int inv_swiglu(const float* G, const float* U, int64_t M, int64_t F, int64_t ldg, int64_t ldu,
               float* Hout, int64_t ldh, void* stream) {
    if (!G || !U || !Hout) return INV_ERR_NULL;
    if (M < 1 || F < 1 || ldg < F || ldu < F || ldh < F || M * F > ((int64_t)1 << 40)) return INV_ERR_SHAPE;
    return fin(launch_swiglu(G, U, (int)M, (int)F, ldg, ldu, Hout, ldh, S(stream)));
}

int inv_add(const float* A, const float* Bm, int64_t M, int64_t N, int64_t lda, int64_t ldb, float* Y,
            int64_t ldy, void* stream) {
    if (!A || !Bm || !Y) return INV_ERR_NULL;
    if (M < 1 || N < 1 || lda < N || ldb < N || ldy < N) return INV_ERR_SHAPE;
    return fin(launch_add(A, Bm, (int)M, (int)N, lda, ldb, Y, ldy, S(stream)));
}

int inv_round_activations(const float* X, int64_t rows, int64_t cols, int64_t ldx, int fmt, float* Y,
                          int64_t ldy, void* stream) {
    if (!X || !Y) return INV_ERR_NULL;
    if (fmt != INV_BF16 && fmt != INV_F16 && fmt != INV_F32) return INV_ERR_DTYPE;
    if (rows < 0 || cols < 0) return INV_ERR_SHAPE;
    if (((uintptr_t)X & 3) || ((uintptr_t)Y & 3)) return INV_ERR_ALIGN;
    if (rows == 0 || cols == 0) return INV_OK;
    if (ldx < cols || ldy < cols) return INV_ERR_SHAPE;
    return fin(launch_round_activations(X, rows, cols, ldx, fmt, Y, ldy, S(stream)));
}

int inv_eval_numerics(int fn, const float* x, float* y, int64_t n, void* stream) {
    if (!x || !y) return INV_ERR_NULL;
    if (fn < 0 || fn > 2) return INV_ERR_DTYPE;
    if (n < 1) return INV_ERR_SHAPE;
    return fin(launch_eval_numerics(fn, x, y, n, S(stream)));
}

int inv_mfma_f32_check(const float* A, const float* B, const float* C, float* D, int64_t ntests,
                       void* stream) {
    if (!A || !B || !C || !D) return INV_ERR_NULL;
    if (ntests < 1) return INV_ERR_SHAPE;
    return fin(launch_mfma_check(A, B, C, D, ntests, S(stream)));
}

int inv_mfma32_f32_check(const float* A, const float* B, const float* C, float* D, int64_t ntests,
                         void* stream) {
    if (!A || !B || !C || !D) return INV_ERR_NULL;
    if (ntests < 1) return INV_ERR_SHAPE;
    return fin(launch_mfma32_check(A, B, C, D, ntests, S(stream)));
}

int inv_mfma_bf16_check(const uint16_t* A, const uint16_t* B, const float* C, float* D, int64_t ntests,
                        void* stream) {
    if (!A || !B || !C || !D) return INV_ERR_NULL;
    if (ntests < 1) return INV_ERR_SHAPE;
    return fin(launch_mfma_bf16_check(A, B, C, D, ntests, S(stream)));
}

int inv_read_stream_probe(const void* src, int64_t bytes, uint32_t* sink, int64_t grid, void* stream) {
    if (!src || !sink) return INV_ERR_NULL;
    if (bytes < 16 || bytes % 16 != 0 || grid < 1 || grid > 65536) return INV_ERR_SHAPE;
    if (!al16(src)) return INV_ERR_ALIGN;
    return fin(launch_read_stream(src, bytes, sink, (int)grid, S(stream)));
}

int inv_mfma_rate_probe(int shape, int64_t iters, int64_t waves_per_cu, float* out, void* stream) {
    if (!out) return INV_ERR_NULL;
    if (shape != 0 && shape != 1) return INV_ERR_DTYPE;
    if (iters < 1 || waves_per_cu < 4 || waves_per_cu > 32 || waves_per_cu % 4 != 0) return INV_ERR_SHAPE;
    return fin(launch_mfma_rate(shape, iters, (int)waves_per_cu, out, S(stream)));
}

int inv_kernel_route(int op, int64_t a, int64_t b, char* name, size_t cap) {
    if (!name || cap == 0) return INV_ERR_NULL;
    if (a < 1 || b < 1) return INV_ERR_SHAPE;
    char buf[96];
    const char* role = "0";
    int64_t M = a, N = b;
    switch (op) {
        case INV_ROUTE_GEMM: break;
        case INV_ROUTE_GATED_GEMM: role = "2"; break;
        case INV_ROUTE_LMHEAD_GEMM: role = "1"; M = lmhead_projection_rows(a, 1.0f); break;
        case INV_ROUTE_ATTN_PREFILL: {
            const int nw = attention_prefill_waves(1, b, a);
            snprintf(buf, sizeof(buf), "attn_prefill_kernel<DT,%d,%d>", nw, nw == 8 ? 64 : 32);
            snprintf(name, cap, "%s", buf);
            return INV_OK;
        }
        default: return INV_ERR_DTYPE;
    }
    // the template name with its ROLE argument filled in; a split-off tail adds its GEMV
    auto fill = [&](char* out, size_t n, int64_t rows) {
        const char* t = gemm_route_name(gemm_route(rows, N));
        const char* r = strstr(t, "ROLE");
        if (r) snprintf(out, n, "%.*s%s%s", (int)(r - t), t, role, r + 4);
        else snprintf(out, n, "%s", t);
    };
    const int64_t tail = gemm_tail_rows(M, nullptr);
    fill(buf, sizeof(buf), M - tail);
    if (tail) {
        char tb[64];
        fill(tb, sizeof(tb), tail);
        snprintf(name, cap, "%s+%s", buf, tb);
    } else {
        snprintf(name, cap, "%s", buf);
    }
    return INV_OK;
}

}  // extern "C"
