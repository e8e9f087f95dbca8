// kernels.h -- host-side launchers of the library's kernels (internal to libinvnum.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace invnum {

// RoPE and KV-append targets of the fused QKV projection (role 3): rotary head dim 128
struct RopeArgs {
    int Hq, Hkv;
    const int32_t* seq; const int32_t* pos;
    const float* cos_t; const float* sin_t;   // [Tmax, 64]
    int Tmax, Bcache;
    float* Qout; float* Kc; float* Vc;
};

struct GemmArgs {
    const float* X; int M; int K; int64_t ldx;
    const uint16_t* W; int N; int64_t ldw;
    const float* R; int64_t ldr;
    float* Y; int64_t ldy;
    const int* Mdev;  // optional: device-side row count (<= M); rows beyond it are skipped
    // optional RMSNorm of the activation rows (gains G, BF16 [K]) applied as they are staged;
    // only the slice-parallel GEMV routes (M <= 4) take it
    const uint16_t* G = nullptr;
    float eps = 0.0f;
};
// role 0: activation projections; role 1: the LM head's vocabulary projection; role 2: gated
// projection (W rows interleaved gate/up, Y[m][i] = silu(gate) * up, N even, R unused)
hipError_t launch_gemm(const GemmArgs& a, hipStream_t st, int role = 0);
// the same sums on 64 x 64 tiles whatever M is (for a device-side row count far below M: only
// the tile rows holding live rows do any work)
hipError_t launch_gemm_tiles64(const GemmArgs& a, hipStream_t st, int role);
// the kernel a GEMM of M activation rows and N weight rows runs on (every role routes alike)
enum GemmRoute : int {
    GR_SKINNY_M1_R4, GR_SKINNY_M1_R16, GR_SKINNY_M2_R4, GR_SKINNY_M2_R16, GR_SKINNY_M4_R16,
    GR_GEMV16_WN1, GR_GEMV16_WN1_W8, GR_GEMV16_WN2, GR_GEMV16_WN4, GR_GEMV32_WN1, GR_GEMV32_WN2, GR_GEMV32_WN4,
    GR_GEMV32_G16, GR_GEMV64_G32, GR_GEMV64_G16, GR_SMALL32, GR_TILE64, GR_TILE64x128, GR_TILE128x256
};
GemmRoute gemm_route(int64_t M, int64_t N);
// rows split off to the skinny GEMV after the tiled part (0: none)
int64_t gemm_tail_rows(int64_t M, const int* Mdev);
const char* gemm_route_name(GemmRoute r);   // kernel template with ROLE left symbolic
// QKV projection of up to four rows (head dim 128) with RoPE and the KV append done by the
// VALU GEMV's epilogue (role 3); the caller runs the projection and rope_kv_append otherwise
bool qkv_rope_fusable(int64_t M, int64_t D);
// the RMSNorm of the activation rows runs in the GEMV's prologue for up to this many rows
bool gemm_norm_fusable(int64_t M);
hipError_t launch_qkv_rope(const GemmArgs& a, const RopeArgs& ra, hipStream_t st);

hipError_t launch_rmsnorm(const float* X, int M, int H, int64_t ldx, const uint16_t* g, float eps,
                          float* Y, int64_t ldy, hipStream_t st);

struct AttnArgs {
    int dtype;  // 0 bf16, 1 f32
    const void* Q; const void* Kc; const void* Vc;
    int B, Tq, q_start, Tmax, Hq, Hkv, D;
    float scale;
    float* O;
};
// ws (may be null): partials of the split path for small grids, used when ws_bytes is at least
// prefill_split_ws_bytes(); otherwise the single-task kernel runs.  Same bits either way.
hipError_t launch_attention_prefill(const AttnArgs& a, float* ws, size_t ws_bytes, hipStream_t st);
size_t prefill_split_ws_bytes(int64_t B, int64_t Tq, int64_t q_start, int64_t Hq);
// 8 (128-row workgroups) or 4 (64-row workgroups): wavefronts per prefill workgroup
int attention_prefill_waves(int64_t B, int64_t Tq, int64_t Hq);
hipError_t launch_attention_decode(const AttnArgs& a, const int32_t* pos, float* ws,
                                   hipStream_t st);
// size of the library-owned partials array of the allocation-free decode entry point, and its
// device address on the current GPU
constexpr size_t DECODE_SCRATCH_BYTES = (size_t)32 << 20;
hipError_t decode_scratch(float** out);

struct LmheadArgs {
    const float* Hs; int B; int K; int64_t ldh;
    const uint16_t* W; int V;
    const int32_t* target; float tau;
    float* logprob; float* margin; int32_t* top1; int32_t* top2; uint8_t* recomputed;
    void* ws;
};
size_t lmhead_ws_bytes(int64_t B, int64_t K, int64_t V);
// activation rows of the vocabulary projection for B rows at threshold tau
int64_t lmhead_projection_rows(int64_t B, float tau);
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
hipError_t launch_read_stream(const void* src, int64_t bytes, uint32_t* sink, int grid, hipStream_t st);
hipError_t launch_mfma_rate(int shape, int64_t iters, int waves_per_cu, float* out, hipStream_t st);
hipError_t launch_mfma_bf16_check(const uint16_t* A, const uint16_t* B, const float* C, float* D, int64_t ntest,
                                  hipStream_t st);

}  // namespace invnum
