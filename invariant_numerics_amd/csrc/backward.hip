// backward.hip -- fixed-order backward of the LayerCast matmul Y = X up(W)^T.
//
//   dX[m, k] = dot_KS over n of (dY[m, n], up(W[n, k]))   (sum over the N outputs)
//   dW[n, k] = dot_KS over m of (dY[m, n], X[m, k])       (sum over the M tokens)
//
// Both sums follow the forward's order along the reduced index: 256-wide slices, each an
// in-order fused multiply-add chain from +0, folded left to right.  dX is the forward GEMM
// applied to the transposed weights (W^T is BF16 [K, N], so the forward kernels compute
// exactly the chain above); dW has both operands in FP32 and its own matrix-core kernel,
// which reads dY and X in their natural [M, *] layouts.
#include "invnum.h"
#include "numerics.h"
#include "kernels.h"

namespace invnum {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Wt[k, n] = W[n, k] (BF16 bits), 64 x 64 tiles through LDS.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ W, int N, int K,
                                                             int64_t ldw, uint16_t* __restrict__ Wt,
                                                             int64_t ldt) {
    __shared__ uint16_t t[64][66];
    const int nkt = (K + 63) / 64;
    const int n0 = (blockIdx.x / nkt) * 64, k0 = (blockIdx.x % nkt) * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int r = ty; r < 64; r += 4) {
        const int n = n0 + r, k = k0 + tx;
        if (n < N && k < K) t[r][tx] = W[(int64_t)n * ldw + k];
    }
    __syncthreads();
    for (int r = ty; r < 64; r += 4) {
        const int k = k0 + r, n = n0 + tx;
        if (k < K && n < N) Wt[(int64_t)k * ldt + n] = t[tx][r];
    }
}

// dW on the FP32 matrix cores (v_mfma_f32_32x32x2_f32: per step, k = 2s then 2s + 1 as two
// fused multiply-adds in that order -- the measured property the forward GEMM relies on).
// Here the instruction's reduction index is the token m: A operand = dY^T (row n, column m),
// B operand = X (row m, column k), so a step advances every output by tokens 2s and 2s + 1.
// Workgroup: 2 x WGK wavefronts over a 128 x 64 WGK output tile, each wavefront 64 x 64
// (2 x 2 tiles of 32 x 32).  Tokens stream in stages of 32 rows of dY and X (row segments,
// coalesced), double-buffered in LDS in their natural layout; lane (h, c) reads column c of
// rows 2s + h.  With HALF the next stage's LDS stores are issued halfway through the
// current stage's steps.  After every 256 tokens the slice accumulator is folded into the
// total.  (Measured at 16384 tokens: 2 x 2 wavefronts with HALF 117-120 TFLOP/s; without
// HALF 114-118; 2 x 4 wavefronts 118.)
// Tokens past M load as dY = -0 and X = +0: fma(-0, +0, c) = c for every c, signed zeros
// included, so a partial stage leaves every chain exactly as the sequential sum would.
constexpr int TN_BM = 32;           // tokens per stage

template <int WGK, bool HALF>
__global__ __launch_bounds__(128 * WGK) void gemm_tn_kernel(const float* __restrict__ A, int M, int N, int64_t lda,
                                                            const float* __restrict__ B, int K, int64_t ldb,
                                                            float* __restrict__ C, int64_t ldc) {
    constexpr int NT = 128 * WGK;               // 2 x WGK wavefronts
    constexpr int TNN = 128, TNK = 64 * WGK;     // output tile: rows n, columns k
    constexpr int LDA = TNN + 4, LDB = TNK + 4;
    constexpr int AU = TN_BM * TNN / 4 / NT;     // float4 loads of dY per thread per stage
    constexpr int BU = TN_BM * TNK / 4 / NT;     // float4 loads of X per thread per stage
    __shared__ __attribute__((aligned(16))) float As[2][TN_BM][LDA];
    __shared__ __attribute__((aligned(16))) float Bs[2][TN_BM][LDB];
    const int nKt = (K + TNK - 1) / TNK;
    const int n0 = (blockIdx.x / nKt) * TNN, k0 = (blockIdx.x % nKt) * TNK;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int h = lane >> 5, c = lane & 31;
    const int wn0 = (wv / WGK) * 64, wk0 = (wv % WGK) * 64;
    float4 ar[AU], br[BU];
    auto load = [&](int m0) {
#pragma unroll
        for (int i = 0; i < AU; ++i) {
            const int q = tid + NT * i;
            const int row = q / (TNN / 4), c4 = (q % (TNN / 4)) * 4;
            const int m = m0 + row;
            ar[i] = make_float4(-0.f, -0.f, -0.f, -0.f);
            if (m < M && n0 + c4 < N) ar[i] = *reinterpret_cast<const float4*>(A + (int64_t)m * lda + n0 + c4);
        }
#pragma unroll
        for (int i = 0; i < BU; ++i) {
            const int q = tid + NT * i;
            const int row = q / (TNK / 4), c4 = (q % (TNK / 4)) * 4;
            const int m = m0 + row;
            br[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (m < M && k0 + c4 < K) br[i] = *reinterpret_cast<const float4*>(B + (int64_t)m * ldb + k0 + c4);
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < AU; ++i) {
            const int q = tid + NT * i;
            *reinterpret_cast<float4*>(&As[buf][q / (TNN / 4)][(q % (TNN / 4)) * 4]) = ar[i];
        }
#pragma unroll
        for (int i = 0; i < BU; ++i) {
            const int q = tid + NT * i;
            *reinterpret_cast<float4*>(&Bs[buf][q / (TNK / 4)][(q % (TNK / 4)) * 4]) = br[i];
        }
    };
    f32x16 acc[2][2], T[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) { acc[i][j][v] = 0.0f; T[i][j][v] = 0.0f; }
    const int nst = (M + TN_BM - 1) / TN_BM;
    constexpr int SPS = KS / TN_BM;              // stages per slice
    auto steps = [&](int buf, int s0, int s1) {
#pragma unroll 4
        for (int s = s0; s < s1; ++s) {
            float a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) a[i] = As[buf][2 * s + h][wn0 + 32 * i + c];
#pragma unroll
            for (int j = 0; j < 2; ++j) b[j] = Bs[buf][2 * s + h][wk0 + 32 * j + c];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    };
    load(0);
    store(0);
    __syncthreads();
    for (int st = 0; st < nst; ++st) {
        const int buf = st & 1;
        if (st + 1 < nst) load((st + 1) * TN_BM);
        if constexpr (HALF) {
            // the next stage's stores go out halfway through this stage's steps
            steps(buf, 0, TN_BM / 4);
            if (st + 1 < nst) store(buf ^ 1);
            steps(buf, TN_BM / 4, TN_BM / 2);
        } else {
            steps(buf, 0, TN_BM / 2);
        }
        if (st % SPS == SPS - 1 || st == nst - 1) {
            const bool first = st < SPS;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        T[i][j][v] = first ? acc[i][j][v] : T[i][j][v] + acc[i][j][v];
                        acc[i][j][v] = 0.0f;
                    }
        }
        if constexpr (!HALF) {
            if (st + 1 < nst) store(buf ^ 1);
        }
        __syncthreads();
    }
    // register v of lane (h, c) in tile (i, j): row n = 8 (v / 4) + 4 h + v % 4, column k = c
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int n = n0 + wn0 + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
            if (n >= N) continue;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int k = k0 + wk0 + 32 * j + c;
                if (k < K) C[(int64_t)n * ldc + k] = T[i][j][v];
            }
        }
}

template <int WGK, bool HALF>
hipError_t launch_tn(const float* dY, int M, int N, int64_t lddy, const float* X, int K, int64_t ldx, float* dW,
                     int64_t lddw, hipStream_t st) {
    const int tiles = ((N + 127) / 128) * ((K + 64 * WGK - 1) / (64 * WGK));
    hipLaunchKernelGGL((gemm_tn_kernel<WGK, HALF>), dim3(tiles), dim3(128 * WGK), 0, st, dY, M, N, lddy, X, K, ldx,
                       dW, lddw);
    return hipGetLastError();
}

inline size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t gemm_backward_ws_bytes(int64_t M, int64_t N, int64_t K) {
    (void)M;
    return align_up(sizeof(uint16_t) * (size_t)N * (size_t)K);
}

hipError_t launch_gemm_backward(const float* dY, int M, int N, int64_t lddy, const float* X, int K, int64_t ldx,
                                const uint16_t* W, int64_t ldw, float* dX, int64_t lddx, float* dW,
                                int64_t lddw, void* ws, hipStream_t st) {
    hipError_t e;
    if (dX) {
        uint16_t* Wt = reinterpret_cast<uint16_t*>(ws);
        const int tiles = ((N + 63) / 64) * ((K + 63) / 64);
        hipLaunchKernelGGL(transpose_bf16_kernel, dim3(tiles), dim3(256), 0, st, W, N, K, ldw, Wt, (int64_t)N);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        // dX[m, k] = dot_KS over n of (dY[m, n], up(Wt[k, n])): the forward GEMM with K' = N
        GemmArgs ga{dY, M, N, lddy, Wt, K, (int64_t)N, nullptr, 0, dX, lddx, nullptr};
        if ((e = launch_gemm(ga, st, 0)) != hipSuccess) return e;
    }
    if (dW) {
        if ((e = launch_tn<2, true>(dY, M, N, lddy, X, K, ldx, dW, lddw, st)) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace invnum
