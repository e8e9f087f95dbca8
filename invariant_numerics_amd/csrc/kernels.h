// kernels.h -- host-side launchers of the library's kernels (internal to libinvnum.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace invnum {

struct GemmArgs {
    const float* X; int M; int K; int64_t ldx;
    const uint16_t* W; int N; int64_t ldw;
    const float* R; int64_t ldr;
    float* Y; int64_t ldy;
    const int* Mdev;  // optional: device-side row count (<= M); rows beyond it are skipped
};
// role 0: activation projections; role 1: the LM head's vocabulary projection; role 2: gated
// projection (W rows interleaved gate/up, Y[m][i] = silu(gate) * up, N even, R unused)
hipError_t launch_gemm(const GemmArgs& a, hipStream_t st, int role = 0);
int64_t gemm_skinny_max_k();

hipError_t launch_rmsnorm(const float* X, int M, int H, int64_t ldx, const uint16_t* g, float eps,
                          float* Y, int64_t ldy, hipStream_t st);

struct AttnArgs {
    int dtype;  // 0 bf16, 1 f32
    const void* Q; const void* Kc; const void* Vc;
    int B, Tq, q_start, Tmax, Hq, Hkv, D;
    float scale;
    float* O;
};
hipError_t launch_attention_prefill(const AttnArgs& a, hipStream_t st);
hipError_t launch_attention_decode(const AttnArgs& a, const int32_t* pos, float* ws,
                                   hipStream_t st);

struct LmheadArgs {
    const float* Hs; int B; int K; int64_t ldh;
    const uint16_t* W; int V;
    const int32_t* target; float tau;
    float* logprob; float* margin; int32_t* top1; int32_t* top2; uint8_t* recomputed;
    void* ws;
};
size_t lmhead_ws_bytes(int64_t B, int64_t K, int64_t V);
struct LogitGradArgs {
    const float* Hs; int B; int K; int64_t ldh;
    const uint16_t* W; int V;
    const int32_t* target; const float* coef;
    float* G; float* logprob;
    void* ws;
};
size_t logit_grad_ws_bytes(int64_t B, int64_t V);
hipError_t launch_logit_grad(const LogitGradArgs& a, hipStream_t st);
size_t gemm_backward_ws_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_backward(const float* dY, int M, int N, int64_t lddy, const float* X, int K, int64_t ldx,
                                const uint16_t* W, int64_t ldw, float* dX, int64_t lddx, float* dW,
                                int64_t lddw, void* ws, hipStream_t st);
hipError_t launch_lmhead(const LmheadArgs& a, hipStream_t st);

hipError_t launch_embed(const int32_t* ids, int M, const uint16_t* table, int vocab, int H, float* X,
                        int64_t ldx, hipStream_t st);
hipError_t launch_rope_kv_append(const float* QKV, int M, int64_t ldqkv, int Hq, int Hkv, int D,
                                 const int32_t* seq, const int32_t* pos, const float* cos_t,
                                 const float* sin_t, int Tmax, int Bcache, float* Qout, float* Kc,
                                 float* Vc, int out_fmt, hipStream_t st);
hipError_t launch_swiglu(const float* G, const float* U, int M, int F, int64_t ldg, int64_t ldu,
                         float* Hout, int64_t ldh, hipStream_t st);
hipError_t launch_add(const float* A, const float* B, int M, int N, int64_t lda, int64_t ldb,
                      float* Y, int64_t ldy, hipStream_t st);
hipError_t launch_round_activations(const float* X, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                                    float* Y, int64_t ldy, hipStream_t st);
hipError_t launch_eval_numerics(int fn, const float* x, float* y, int64_t n, hipStream_t st);
hipError_t launch_mfma_check(const float* A, const float* B, const float* C, float* D, int64_t ntest,
                             hipStream_t st);
hipError_t launch_mfma32_check(const float* A, const float* B, const float* C, float* D, int64_t ntest,
                               hipStream_t st);

}  // namespace invnum
