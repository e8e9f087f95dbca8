/*
 * invnum.h -- C ABI of libinvnum.so: batch-invariant, fixed-reduction-order kernels for
 * token log-probabilities on AMD Instinct MI355X (gfx950).
 *
 * The operations follow the pages on invariant numerics:
 *   - every reduction whose order changes the bits (matmul K-sums, attention score sums,
 *     the softmax denominator, the logprob accumulation) runs in ONE fixed order that
 *     prefill and decode share  [Meituan bitwise train/inference alignment page,
 *     "principles" and "key practices" lists];
 *   - full-K accumulation, never a split reduce  [same page, "key practices", TP item];
 *   - LayerCast: weights stored BF16 and upcast to FP32 per layer, all matmul and
 *     attention arithmetic in FP32  ["Give Me FP32 or Give Me Death?" write-up,
 *     section 5; Yuan et al. blog, section 4];
 *   - selective FP32 LM-head recompute when the top-two logit margin falls below a
 *     threshold  ["Greedy Decoding Is Not Precision-Invariant", abstract].
 *
 * The pinned order ("canonical reduction order v0"), used by every entry point:
 *   dot_KS(x, w, K): contiguous K-slices of 256; per slice c = +0, c = fma(x_k, w_k, c)
 *     for k ascending; then T = c_0, T = T + c_s for s ascending.
 *   attention: scores dot_KS(q, k_j, D) * scale; keys in absolute chunks of 256; per
 *     chunk m_c = max, l_c and o_c summed for j ascending with p = exp_f(s_j - m_c);
 *     chunks merged left to right from chunk 0; out = o / l.
 *   LM head: tiles of 1024 vocabulary entries, 64 lanes per tile summing 16 entries each,
 *     a pairwise lane tree, tiles folded left to right; lp = (z_t - M) - log_f(S).
 *   exp_f / log_f are the library's own functions (Cody-Waite reduction + degree-7 Taylor;
 *     atanh series), identical on every device and on the CPU check.
 * A row's output bits depend only on that row's inputs and these constants: never on the
 * batch size, the row's position in the batch, the grid, the stream or the CU count.
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers (e.g. torch tensors' data_ptr()), row-major,
 *     with the leading dimensions given.  BF16 tensors are passed as uint16_t bit patterns.
 *     Pointers must be 16-byte aligned and leading dimensions multiples of 4 elements (FP32)
 *     or 8 elements (BF16); otherwise INV_ERR_ALIGN.
 *   - The caller owns all memory.  The library never allocates and keeps no pointer after
 *     the call returns.  Scratch memory comes from a caller-supplied workspace whose size
 *     is given by the matching *_workspace_bytes() query.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously; there is no host synchronisation inside any call.  Outputs are valid
 *     once the stream has completed the enqueued work.
 *   - Return value: INV_OK (0) or a negative status.  On any validation error nothing is
 *     enqueued.  A launch failure returns INV_ERR_LAUNCH.  Calls are stateless and
 *     re-entrant; calls on different streams must not write the same outputs/workspace.
 */
#ifndef INVNUM_H
#define INVNUM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum inv_status {
    INV_OK = 0,
    INV_ERR_NULL = -1,        /* a required pointer is NULL */
    INV_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
    INV_ERR_ALIGN = -3,       /* pointer or leading dimension not aligned as required */
    INV_ERR_DTYPE = -4,       /* unknown dtype code */
    INV_ERR_WORKSPACE = -5,   /* workspace missing or smaller than the query returned */
    INV_ERR_UNSUPPORTED = -6, /* valid but unsupported shape (e.g. head dim != 128) */
    INV_ERR_LAUNCH = -7       /* the HIP runtime rejected a launch */
};

enum inv_dtype { INV_BF16 = 0, INV_F32 = 1, INV_F16 = 2 };

#define INV_MAX_FLOAT_CONSTS 32

typedef struct inv_constants {
    int32_t ks;            /* K-slice width of dot_KS: 256 */
    int32_t chunk;         /* attention KV chunk: 256 */
    int32_t vocab_tile;    /* LM-head vocabulary tile: 1024 */
    int32_t lanes;         /* lanes of the vocabulary tree: 64 */
    int32_t n_float;       /* number of valid entries in float_consts */
    /* exp_f / log_f constants in a fixed order: log2e, ln2_hi, ln2_lo, exp lower limit,
     * exp upper limit, 1/k! for k = 0..7, ln2_hi16, ln2_lo16, 2/(2k+1) for k = 1..5 */
    float float_consts[INV_MAX_FLOAT_CONSTS];
} inv_constants;

/* Text for a status code (static storage). */
const char* inv_status_string(int status);

/* The pinned constants of the reduction order.  Host-only; no device is touched. */
int inv_get_constants(inv_constants* out);

/* ------------------------------------------------------------------------------------ *
 * inv_fixed_order_gemm -- LayerCast matmul with the fixed K order.
 *   Y[m, n] = dot_KS(X[m, :], up(W[n, :]), K)        (+ R[m, n] when R != NULL)
 * X: FP32 [M, K] (row stride ldx).  W: BF16 [N, K] (nn.Linear layout, row stride ldw),
 * upcast exactly (bits << 16) as it is read.  Y: FP32 [M, N] (row stride ldy).
 * R: optional FP32 residual [M, N] (row stride ldr) added after the full dot as
 * Y = R + dot (one rounding; the same bits as a separate inv_add).  R may equal Y.
 * Sizes: M >= 1, N >= 1, K >= 8 and K % 8 == 0.  X and W follow the 16-byte rule above;
 * Y and R need only 4-byte alignment (any ldy, ldr >= N).  Each output is owned by one workgroup
 * (no split-K, no atomics); launch geometry depends on M but the order never does.
 * Sources: Meituan page, "key practices" (full-K, batch-invariant operators); FP32
 * write-up section 5 (LayerCast).
 * ------------------------------------------------------------------------------------ */
int inv_fixed_order_gemm(const float* X, int64_t M, int64_t K, int64_t ldx,
                         const uint16_t* W, int64_t N, int64_t ldw,
                         const float* R, int64_t ldr,
                         float* Y, int64_t ldy, void* stream);

/* ------------------------------------------------------------------------------------ *
 * inv_gated_gemm -- SwiGLU of a gate/up projection pair in one call:
 *   H[m, i] = silu(dot_KS(X[m, :], up(W[2i, :]), K)) * dot_KS(X[m, :], up(W[2i+1, :]), K)
 * with silu(a) = a / (1 + exp_f(-a)): bit for bit inv_fixed_order_gemm(X, W) followed by
 * inv_swiglu on its even (gate) and odd (up) columns, without the intermediate.
 * W: BF16 [N2, K] with the gate and up rows interleaved (row 2i = gate i, row 2i+1 = up i);
 * N2 even.  H: FP32 [M, N2/2] (row stride ldh >= N2/2, 4-byte aligned, must not overlap X).
 * X, M, K, ldx, ldw as inv_fixed_order_gemm.
 * Sources: FP32 write-up section 5 (LayerCast); Meituan page, "key practices"
 * (batch-invariant operators).
 * ------------------------------------------------------------------------------------ */
int inv_gated_gemm(const float* X, int64_t M, int64_t K, int64_t ldx,
                   const uint16_t* W, int64_t N2, int64_t ldw,
                   float* H, int64_t ldh, void* stream);

/* ------------------------------------------------------------------------------------ *
 * inv_rmsnorm -- ss = dot_KS(x, x, H); r = 1 / sqrt((ss / H) + eps); y_k = (x_k * r) * up(g_k)
 * X: FP32 [M, H] (ldx); gamma: BF16 [H]; Y: FP32 [M, H] (ldy), may alias X when ldy == ldx.
 * Division and square root are IEEE correctly rounded.  H >= 8, H % 8 == 0.
 * ------------------------------------------------------------------------------------ */
int inv_rmsnorm(const float* X, int64_t M, int64_t H, int64_t ldx, const uint16_t* gamma,
                float eps, float* Y, int64_t ldy, void* stream);

/* ------------------------------------------------------------------------------------ *
 * inv_attention_prefill -- causal attention for queries at positions q_start..q_start+Tq-1.
 * dtype: INV_BF16 (Q, caches BF16, upcast on load) or INV_F32.
 * Q: [B, Tq, Hq, D]; Kc, Vc: [B, Hkv, Tmax, D] already holding keys/values of positions
 * 0..q_start+Tq-1; O: FP32 [B, Tq, Hq, D].  Query head h reads kv head h / (Hq / Hkv).
 * Per row: the chunked order in the header comment, with the merge folded as chunks are
 * produced -- the same bits as inv_attention_decode for that row.
 * Constraints: D == 128 (else INV_ERR_UNSUPPORTED), Hq % Hkv == 0, q_start + Tq <= Tmax.
 * Sources: Meituan page, "principles" (attention score sums, softmax denominator) and
 * "key practices" (DCP: the forward replays decode's accumulation path).
 * ------------------------------------------------------------------------------------ */
int inv_attention_prefill(int dtype, const void* Q, const void* Kc, const void* Vc,
                          int64_t B, int64_t Tq, int64_t q_start, int64_t Tmax,
                          int64_t Hq, int64_t Hkv, int64_t D, float scale,
                          float* O, void* stream);

/* inv_attention_prefill_ws -- the same results as inv_attention_prefill, bit for bit, with a
 * caller-supplied workspace that lets small grids (64-row blocks giving fewer than two
 * workgroups per compute unit, e.g. 8 heads x 2048 rows) spread the long rows' chunks over more
 * workgroups: each chunk's (m_c, l_c, o_c) is stored and then folded in ascending chunk order
 * with the decode merge's arithmetic -- the order the single-task loop folds them in.
 * inv_attention_prefill_workspace_bytes returns the bytes needed (0: this shape runs as one
 * task per block and ws may be null).  ws: device memory, 16-byte aligned, owned by the caller,
 * contents on entry ignored.  Status as inv_attention_prefill, plus INV_ERR_WORKSPACE when a
 * nonzero size is needed and ws is null or ws_bytes is smaller, INV_ERR_ALIGN.
 * Sources: Meituan page, "key practices" (the decode accumulation path; fixed KV chunks). */
size_t inv_attention_prefill_workspace_bytes(int64_t B, int64_t Tq, int64_t q_start, int64_t Hq,
                                             int64_t D);
int inv_attention_prefill_ws(int dtype, const void* Q, const void* Kc, const void* Vc,
                             int64_t B, int64_t Tq, int64_t q_start, int64_t Tmax,
                             int64_t Hq, int64_t Hkv, int64_t D, float scale,
                             float* O, void* ws, size_t ws_bytes, void* stream);

/* Workspace for inv_attention_decode: B * Hq * ceil(Tmax/256) * (D + 2) floats. */
size_t inv_attention_decode_workspace_bytes(int64_t B, int64_t Tmax, int64_t Hq, int64_t D);

/* ------------------------------------------------------------------------------------ *
 * inv_attention_decode -- one query per sequence, at position pos[b] (keys 0..pos[b]).
 * Q: [B, Hq, D] (dtype as above); caches [B, Hkv, Tmax, D]; pos: INT32 [B] on the device,
 * 0 <= pos[b] < Tmax (rows may differ; a row with pos outside that range gets NaN and its
 * cache is not read).  O: FP32 [B, Hq, D].
 * One workgroup per (b, kv head, chunk) writes the chunk partial (m_c, l_c, o_c) into the
 * workspace; a second kernel folds them per (b, q head) in ascending chunk order.
 * Tmax <= 1,048,576 (4096 chunks), else INV_ERR_UNSUPPORTED.
 * ------------------------------------------------------------------------------------ */
int inv_attention_decode(int dtype, const void* Q, const void* Kc, const void* Vc,
                         const int32_t* pos, int64_t B, int64_t Tmax,
                         int64_t Hq, int64_t Hkv, int64_t D, float scale,
                         float* O, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------
 * inv_attention_decode_noalloc -- for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation, arguments and bits as inv_attention_decode, without the workspace
 * arguments.  The chunk partials go to a device array the library owns, of
 * inv_attention_decode_noalloc_max_bytes() bytes (32 MiB) on each GPU, held until the
 * process ends; nothing is allocated, here or by any routine it calls.
 *   Limit: inv_attention_decode_workspace_bytes(B, Tmax, Hq, D) must not exceed that size
 *   (e.g. B <= 15 rows of 32 query heads at Tmax = 32768), else INV_ERR_WORKSPACE and
 *   nothing is enqueued.
 *   Every call on one GPU shares the array: calls that overlap on the same GPU (other
 *   streams, other host threads) race and must be ordered by the caller.  Nothing needs
 *   clearing between calls: every partial the call reads it has written itself.
 * Other status codes as inv_attention_decode; INV_ERR_LAUNCH also when the array's device
 * address cannot be obtained.
 * ------------------------------------------------------------------------------------ */
size_t inv_attention_decode_noalloc_max_bytes(void);
int inv_attention_decode_noalloc(int dtype, const void* Q, const void* Kc, const void* Vc, const int32_t* pos,
                                 int64_t B, int64_t Tmax, int64_t Hq, int64_t Hkv, int64_t D, float scale,
                                 float* O, void* stream);

/* Workspace for inv_lmhead_logprob_top2. */
size_t inv_lmhead_workspace_bytes(int64_t B, int64_t K, int64_t V);

/* ------------------------------------------------------------------------------------ *
 * inv_lmhead_logprob_top2 -- log-softmax at the target, top-2 and margin, with selective
 * FP32 recompute.
 *   P pass: a = up(bf(h)) (BF16 operands, FP32 sums); z_v = dot_KS(a, up(W_v), K);
 *           top1 = lowest index of the maximum, top2 = lowest other index of the maximum
 *           of the rest; M = z_top1; margin = z_top1 - z_top2; S as in the header comment;
 *           lp = (z_target - M) - log_f(S).
 *   Rows with margin_P < tau (strict) are compacted on the device and redone with a = h
 *   (F pass); their outputs are F's and recomputed[b] = 1.  tau = +inf recomputes every
 *   row; tau = 0 recomputes none.  For B <= 32 the F-pass logits of every row are computed
 *   in the same sweep over W as the P ones (the weights are read once), and only the flagged
 *   rows' are used; the results are the same bits either way.
 * Hs: FP32 [B, K] (ldh); W: BF16 [V, K] (row stride K); target: INT32 [B] (device),
 * 0 <= t < V (a row whose target is outside that range gets logprob NaN).
 * Outputs (device, [B]): logprob, margin (FP32), top1, top2 (INT32), recomputed (UINT8).
 * V >= 2, K >= 8, K % 8 == 0.
 * Sources: "Greedy Decoding Is Not Precision-Invariant", abstract and "key design"
 * paragraph (margin-triggered FP32 LM-head recompute); Meituan page, "principles"
 * (logprob accumulation is one of the order-sensitive sums).
 * ------------------------------------------------------------------------------------ */
int inv_lmhead_logprob_top2(const float* Hs, int64_t B, int64_t K, int64_t ldh,
                            const uint16_t* W, int64_t V, const int32_t* target, float tau,
                            float* logprob, float* margin, int32_t* top1, int32_t* top2,
                            uint8_t* recomputed, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------ *
 * inv_lmhead_logit_grad -- gradient of coef[b] * lp_b with respect to the logits of the FP32
 * pass (z_v = dot_KS(h, up(W_v)); the pass every row takes with tau = +inf), lp_b the
 * log-probability of target[b] -- one token's policy-gradient term:
 *   p_v = exp_f(z_v - M) / S     (M = z_top1 and S the fixed tree, exactly as the forward)
 *   G[b, v] = coef[b] * ([v == target[b]] - p_v)
 * Together with inv_gemm_backward on G (dX: the hidden-state gradient, a sum over the V
 * logits; dW: the head's weight gradient, a sum over tokens) this is the LM-head backward of
 * a policy-gradient step, every sum in a fixed order.
 * Hs: FP32 [B, K] (ldh); W: BF16 [V, K] (row stride K); target: INT32 [B]; coef: FP32 [B]
 * (device).  G: FP32 [B, V], row stride V (also holds the logits while they are reduced).
 * logprob: FP32 [B] or NULL.  A target outside [0, V) gives logprob NaN and no +1 term.
 * Sizes as inv_lmhead_logprob_top2; ws: inv_lmhead_logit_grad_workspace_bytes(B, K, V).
 * Sources: Meituan page, "principles" (the logprob accumulation is order-sensitive in
 * training as in inference); "Greedy Decoding Is Not Precision-Invariant", abstract (the
 * FP32 LM head).
 * ------------------------------------------------------------------------------------ */
size_t inv_lmhead_logit_grad_workspace_bytes(int64_t B, int64_t K, int64_t V);
int inv_lmhead_logit_grad(const float* Hs, int64_t B, int64_t K, int64_t ldh, const uint16_t* W, int64_t V,
                          const int32_t* target, const float* coef, float* G, float* logprob,
                          void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------ *
 * inv_gemm_backward -- fixed-order backward of Y = X up(W)^T (inv_fixed_order_gemm) for an
 * output gradient dY:
 *   dX[m, k] = dot_KS over n of (dY[m, n], up(W[n, k]))   (sum over the N outputs)
 *   dW[n, k] = dot_KS over m of (dY[m, n], X[m, k])       (sum over the M tokens)
 * each in the forward's order along the reduced index (256-wide slices of in-order fused
 * multiply-adds from +0, folded left to right), so a gradient's bits do not depend on the
 * batch or on how the work is launched.  dW is FP32.
 * dY: FP32 [M, N] (lddy); X: FP32 [M, K] (ldx); W: BF16 [N, K] (ldw); dX: FP32 [M, K] (lddx);
 * dW: FP32 [N, K] (lddw).  dX or dW may be NULL to skip it (X is not read when dW is NULL,
 * W and the workspace are not used when dX is NULL).
 * Sizes: M >= 1, N >= 8 with N % 8 == 0, K >= 4 with K % 4 == 0; dY and X 16-byte aligned
 * with lddy, ldx multiples of 4; W 2-byte aligned (any ldw >= K); dX and dW 4-byte aligned.
 * Errors: INV_ERR_NULL, INV_ERR_SHAPE, INV_ERR_ALIGN, INV_ERR_WORKSPACE.  ws: at least
 * inv_gemm_backward_workspace_bytes(M, N, K) bytes, 256-byte aligned (holds W transposed).
 * Sources: Meituan page, "principles" (training and inference share one fixed order for the
 * order-sensitive sums; the matmul reduce is one of them) and "key practices" (full-K
 * accumulation, batch-invariant operators).
 * ------------------------------------------------------------------------------------ */
size_t inv_gemm_backward_workspace_bytes(int64_t M, int64_t N, int64_t K);
int inv_gemm_backward(const float* dY, int64_t M, int64_t N, int64_t lddy,
                      const float* X, int64_t K, int64_t ldx,
                      const uint16_t* W, int64_t ldw,
                      float* dX, int64_t lddx, float* dW, int64_t lddw,
                      void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- decoder helpers --- *
 * Elementwise steps of a Llama-shaped decoder (no reductions, so no order to pin).
 * ------------------------------------------------------------------------------------ */

/* X[m, :] = up(table[ids[m], :]).  table BF16 [Vocab, H]; ids INT32 [M] (device).
 * An id outside [0, Vocab) is not read; its row is filled with NaN. */
int inv_embed(const int32_t* ids, int64_t M, const uint16_t* table, int64_t vocab, int64_t H,
              float* X, int64_t ldx, void* stream);

/* Rotate-half RoPE on the q and k parts of a fused projection, and cache append.
 * QKV: FP32 [M, (Hq + 2 Hkv) D] (ldqkv) laid out [q heads | k heads | v heads].
 * Row m belongs to sequence seq[m] at position pos[m] (INT32, device).
 * cos_t, sin_t: FP32 [Tmax, D/2].  For pairs (i, i + D/2):
 *   y_i = (x_i c_i) - (x_{i+D/2} s_i);  y_{i+D/2} = (x_i s_i) + (x_{i+D/2} c_i)   (no fma)
 * Qout: FP32 [M, Hq, D]; Kc, Vc: FP32 [Bcache, Hkv, Tmax, D] receive rotated k and v at
 * [seq[m], g, pos[m], :].  D even.  Rows whose seq/pos fall outside the cache are skipped
 * (nothing written for them).  out_fmt: INV_F32 stores the values as computed; INV_BF16 or
 * INV_F16 stores every written value (q, k, v) rounded to that format, exactly as
 * inv_round_activations would (low-precision activation storage). */
int inv_rope_kv_append(const float* QKV, int64_t M, int64_t ldqkv, int64_t Hq, int64_t Hkv,
                       int64_t D, const int32_t* seq, const int32_t* pos,
                       const float* cos_t, const float* sin_t, int64_t Tmax, int64_t Bcache,
                       float* Qout, float* Kc, float* Vc, int out_fmt, void* stream);

/* Hout[m, f] = silu(G[m, f]) * U[m, f], silu(a) = a / (1 + exp_f(-a)). */
int inv_swiglu(const float* G, const float* U, int64_t M, int64_t F, int64_t ldg, int64_t ldu,
               float* Hout, int64_t ldh, void* stream);

/* Y[m, n] = A[m, n] + Bm[m, n]. */
int inv_add(const float* A, const float* Bm, int64_t M, int64_t N, int64_t lda, int64_t ldb,
            float* Y, int64_t ldy, void* stream);

/* ------------------------------------------------------------------------------------ *
 * inv_round_activations -- storage rounding of FP32 activations:
 *   Y[r, c] = widen(round_fmt(X[r, c]))  for r < rows, c < cols,
 * fmt INV_BF16: the nearest BF16 value (ties to even, overflow to inf, NaN kept quiet);
 * fmt INV_F16: the nearest IEEE binary16 value (ties to even; 10 fraction bits from 2^-14 to
 * 65504, multiples of 2^-24 below, inf from 65520 up, NaN kept quiet with its sign and top 9
 * payload bits); fmt INV_F32: a copy.  The rounded value is returned widened to FP32, so the
 * following operation keeps computing in FP32 on the stored (rounded) value.
 * This is the low-precision activation storage of the cross-precision comparison: the same
 * model with BF16 or with FP16 activations ("Greedy Decoding Is Not Precision-Invariant",
 * abstract); the format widths follow the Yuan et al. blog, section 2 (mantissa bits).
 * X, Y: FP32 device pointers, 4-byte aligned, row strides ldx, ldy >= cols (elements).
 * Y == X with ldy == ldx rounds in place; any other overlap is not allowed.
 * rows == 0 or cols == 0 enqueues nothing and returns INV_OK.  Errors: INV_ERR_NULL,
 * INV_ERR_SHAPE (negative size, stride < cols), INV_ERR_ALIGN, INV_ERR_DTYPE (other fmt).
 * ------------------------------------------------------------------------------------ */
int inv_round_activations(const float* X, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                          float* Y, int64_t ldy, void* stream);

/* Diagnostic: y[i] = exp_f(x[i]) (fn 0), log_f(x[i]) (fn 1) or up(bf(x[i])) (fn 2) on the
 * device, for checking the library's scalar primitives against the CPU check. */
int inv_eval_numerics(int fn, const float* x, float* y, int64_t n, void* stream);

/* Diagnostic: runs one v_mfma_f32_16x16x4_f32 per test.  Test t reads A [16 x 4],
 * B [4 x 16] and C [16 x 16] (row-major FP32, at A + 64 t, B + 64 t, C + 256 t) and writes
 * D = C + A B (at D + 256 t) exactly as the instruction rounds it.  The matrix-core path of
 * attention relies on this instruction being the same arithmetic as four fused multiply-adds
 * in k order (k = 0, 1, 2, 3), i.e. a sequential fma chain; the test suite checks that
 * property against the CPU reference through this entry point. */
int inv_mfma_f32_check(const float* A, const float* B, const float* C, float* D, int64_t ntests,
                       void* stream);

/* Diagnostic: runs one v_mfma_f32_32x32x2_f32 per test.  Test t reads A [32 x 2], B [2 x 32]
 * and C [32 x 32] (row-major FP32, at A + 64 t, B + 64 t, C + 1024 t) and writes D = C + A B
 * (at D + 1024 t) exactly as the instruction rounds it.  The matrix-core path of
 * fixed_order_gemm (and of the LM head's vocabulary projection) relies on this instruction
 * being two fused multiply-adds in k order (k = 0, then 1), i.e. the slice chain of dot_KS;
 * the test suite checks that property against the CPU reference through this entry point.
 * Status: INV_ERR_NULL for a null pointer, INV_ERR_SHAPE for ntests < 1. */
int inv_mfma32_f32_check(const float* A, const float* B, const float* C, float* D, int64_t ntests,
                         void* stream);

/* Diagnostic: runs one v_mfma_f32_16x16x32_bf16 per test, in lane form.  Test t supplies,
 * for each lane l = 0..63 of one wavefront, the lane's 8 A operands and 8 B operands (BF16
 * bit patterns at A + 8 (64 t + l) and B + 8 (64 t + l)) and its 4 FP32 accumulator values
 * (C + 4 (64 t + l)); the lane's 4 results are written to D + 4 (64 t + l).  Which matrix
 * element each lane register holds is left to the caller (the test suite pins it with
 * small-integer operands, where every summation order gives the exact result).  Used to
 * test candidate models of the instruction's accumulation ("Greedy Decoding Is Not
 * Precision-Invariant", abstract: a BF16 LM head) against the CPU before any use; the
 * library's BF16 pass does not use this instruction.  Status: INV_ERR_NULL for a null
 * pointer, INV_ERR_SHAPE for ntests < 1. */
int inv_mfma_bf16_check(const uint16_t* A, const uint16_t* B, const float* C, float* D, int64_t ntests,
                        void* stream);

/* Diagnostic (measurement, not part of the method): reads `bytes` (a multiple of 16) at src
 * with 16-byte loads from `grid` workgroups of 256 threads and writes one checksum per
 * workgroup to sink[grid] (so the loads are kept).  Timed by the benchmarks for the practical
 * HBM read rate of a plain stream, the ceiling the memory-bound kernels are compared with.
 * Status: INV_ERR_NULL, INV_ERR_SHAPE (bytes, grid out of range), INV_ERR_ALIGN. */
int inv_read_stream_probe(const void* src, int64_t bytes, uint32_t* sink, int64_t grid, void* stream);

/* Diagnostic (measurement): every one of 256 x waves_per_cu / 4 workgroups of four wavefronts
 * issues `iters` rounds of 8 independent FP32 matrix instructions (shape 0:
 * v_mfma_f32_16x16x4_f32, shape 1: v_mfma_f32_32x32x2_f32) on register operands and writes its
 * accumulators to out[grid * 256].  Flops per launch = grid * 4 * iters * 8 * 2048 (shape 0)
 * or * 4096 (shape 1); timed by the benchmarks for the instruction rates at 1-8 wavefronts
 * per SIMD.  Status: INV_ERR_NULL, INV_ERR_DTYPE (shape), INV_ERR_SHAPE (iters < 1,
 * waves_per_cu not a multiple of 4 in 4..32). */
int inv_mfma_rate_probe(int shape, int64_t iters, int64_t waves_per_cu, float* out, void* stream);

/* ------------------------------------------------------------------------------------
 * inv_qkv_rope_kv_append -- the QKV projection of a decoder layer followed by the RoPE
 * rotation and the KV-cache append: bit for bit inv_fixed_order_gemm(X, Wqkv) and then
 * inv_rope_kv_append (FP32 output format) on its output.  Wqkv is [(Hq + 2 Hkv) D, K] BF16,
 * q rows | k rows | v rows, as for those calls.  For one to four rows with D = 128 both run
 * as one GEMV launch: the weight rows of each rotated head are visited in rotate-half pairs
 * (d, d + 64), whose two outputs are folded by neighbouring threads that rotate and store
 * them (no change to any sum: the rows are only read in another order); otherwise the
 * projection goes to the workspace (inv_qkv_rope_kv_append_workspace_bytes, 0 when fused)
 * and the rotation kernel follows.  Arguments and layouts as for inv_fixed_order_gemm and
 * inv_rope_kv_append: X [M, K] FP32 (ldx), seq/pos [M] int32 (rows outside the cache are
 * skipped), tables [Tmax, D/2] FP32, Qout [M, Hq, D], caches [Bcache, Hkv, Tmax, D] FP32.
 * Errors: INV_ERR_NULL, INV_ERR_SHAPE, INV_ERR_ALIGN, INV_ERR_WORKSPACE, INV_ERR_LAUNCH.
 * ------------------------------------------------------------------------------------ */
size_t inv_qkv_rope_kv_append_workspace_bytes(int64_t M, int64_t Hq, int64_t Hkv, int64_t D);
int inv_qkv_rope_kv_append(const float* X, int64_t M, int64_t K, int64_t ldx, const uint16_t* Wqkv, int64_t ldw,
                           int64_t Hq, int64_t Hkv, int64_t D, const int32_t* seq, const int32_t* pos,
                           const float* cos_t, const float* sin_t, int64_t Tmax, int64_t Bcache, float* Qout,
                           float* Kc, float* Vc, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------
 * inv_rmsnorm_gemm -- a projection of RMSNorm-ed rows, for one to four rows (decode):
 *   bit for bit inv_rmsnorm(X, gamma, eps) followed by inv_fixed_order_gemm (gated = 0, with
 *   the optional residual R) or inv_gated_gemm (gated = 1: W interleaved gate/up rows, N even,
 *   Y [M, N/2], R must be NULL) on the normalised rows, without storing them: each workgroup of
 *   the GEMV computes r = 1 / sqrt((dot_KS(x, x, K) / K) + eps) of every row itself, in the
 *   RMSNorm's order, and stages (x_k * r) * up(g_k) as the operand.  One launch instead of two;
 *   the rows' norms are computed one after another, so it pays for a single row.
 * X: FP32 [M, K] (ldx), the norm's input; gamma: BF16 [K], 16-byte aligned.  W, N, ldw, R,
 * ldr, Y, ldy as inv_fixed_order_gemm / inv_gated_gemm; R may equal Y, but Y must not overlap X
 * (every workgroup reads the whole rows of X while others store Y).  K <= 16384.
 * Errors: INV_ERR_NULL, INV_ERR_SHAPE (also for Y overlapping X), INV_ERR_ALIGN,
 * INV_ERR_UNSUPPORTED (M outside 1..4, or K > 16384), INV_ERR_LAUNCH.
 * Sources: Meituan page, "key practices" (batch-invariant RMSNorm and GEMM operators); FP32
 * write-up section 5 (LayerCast).
 * ------------------------------------------------------------------------------------ */
int inv_rmsnorm_gemm(const float* X, int64_t M, int64_t K, int64_t ldx, const uint16_t* gamma, float eps,
                     const uint16_t* W, int64_t N, int64_t ldw, const float* R, int64_t ldr,
                     float* Y, int64_t ldy, int gated, void* stream);

/* ------------------------------------------------------------------------------------
 * inv_rmsnorm_qkv_rope_kv_append -- inv_qkv_rope_kv_append of the RMSNorm-ed rows: bit for
 * bit inv_rmsnorm(X, gamma, eps) and then inv_qkv_rope_kv_append on its output, in one GEMV
 * launch whose workgroups compute the norm themselves (as inv_rmsnorm_gemm).  For one to four
 * rows with D = 128 only (INV_ERR_UNSUPPORTED otherwise; K <= 16384); needs no workspace.
 * Arguments as inv_qkv_rope_kv_append, plus gamma (BF16 [K], 16-byte aligned) and eps; X must
 * not overlap Qout or the caches (INV_ERR_SHAPE).
 * Errors: INV_ERR_NULL, INV_ERR_SHAPE, INV_ERR_ALIGN, INV_ERR_UNSUPPORTED, INV_ERR_LAUNCH.
 * Sources: Meituan page, "key practices" (batch-invariant operators; decode replays the same
 * accumulation path as prefill).
 * ------------------------------------------------------------------------------------ */
int inv_rmsnorm_qkv_rope_kv_append(const float* X, int64_t M, int64_t K, int64_t ldx, const uint16_t* gamma,
                                   float eps, const uint16_t* Wqkv, int64_t ldw, int64_t Hq, int64_t Hkv,
                                   int64_t D, const int32_t* seq, const int32_t* pos, const float* cos_t,
                                   const float* sin_t, int64_t Tmax, int64_t Bcache, float* Qout, float* Kc,
                                   float* Vc, void* stream);

/* ------------------------------------------------------------------------------------
 * inv_kernel_route -- host-only query (enqueues nothing, touches no device): the name of
 * the kernel instantiation that a call with these sizes launches, written as a
 * NUL-terminated string into name[0 .. cap-1] (truncated to fit).  The choice is launch
 * geometry only: every route computes the same bits, which the test suite checks across
 * sizes and against the CPU check.  Used by the tests and the benchmark to state which
 * kernels a check covers.
 *   op INV_ROUTE_GEMM:         inv_fixed_order_gemm with M = a activation rows, N = b
 *                              weight rows (K does not change the route);
 *   op INV_ROUTE_GATED_GEMM:   inv_gated_gemm with M = a, N2 = b;
 *   op INV_ROUTE_LMHEAD_GEMM:  the vocabulary projection inside inv_lmhead_logprob_top2
 *                              for B = a rows, V = b entries and tau > 0 (up to 32 rows
 *                              the primary and FP32 operand rows share one projection of
 *                              2B rows; with tau <= 0 it is the route of a rows);
 *   op INV_ROUTE_ATTN_PREFILL: inv_attention_prefill with B * Hq = a and Tq = b.
 * Returns INV_OK, INV_ERR_NULL (name NULL or cap 0), INV_ERR_DTYPE (unknown op) or
 * INV_ERR_SHAPE (a or b < 1).
 * ------------------------------------------------------------------------------------ */
enum inv_route_op {
    INV_ROUTE_GEMM = 0, INV_ROUTE_GATED_GEMM = 1, INV_ROUTE_LMHEAD_GEMM = 2, INV_ROUTE_ATTN_PREFILL = 3
};
int inv_kernel_route(int op, int64_t a, int64_t b, char* name, size_t cap);

#ifdef __cplusplus
}
#endif

#endif /* INVNUM_H */
