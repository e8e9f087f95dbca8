// elementwise.hip -- RMSNorm (one fixed-order reduction per row) and the decoder's
// elementwise steps (embedding gather, RoPE + KV-cache append, SwiGLU, residual add, storage
// rounding of activations to BF16 / FP16).
#include "invnum.h"
#include "numerics.h"
#include "kernels.h"

namespace invnum {

namespace {

// RMSNorm: one 256-thread workgroup per row.  The row is staged in LDS with coalesced
// 16-byte loads (up to 4 per thread in flight, together with the gains they will meet);
// thread s then runs the slice chain ss_s = fma(x_k, x_k, ss_s) over k in slice s
// (ascending); thread 0 folds the slices in order and evaluates r = 1 / sqrt(ss / H + eps);
// finally every thread writes y_k = (x_k * r) * up(g_k).  In LDS each 256-float slice is
// followed by 4 floats of padding (x_k at k + 4 (k / 256)), so the chain threads' reads fall on
// different banks, and each chain reads 64 elements ahead of its fused multiply-adds.
constexpr int RN_T = 256;     // threads per row
constexpr int RN_U = 4;       // float4 per thread per batch
constexpr int RN_PAD = 4;     // floats of padding after each slice in LDS
constexpr int RN_CH = 16;     // float4 read ahead by a chain thread
__device__ __forceinline__ int rn_at(int k) { return k + RN_PAD * (k / KS); }

__global__ __launch_bounds__(RN_T) void rmsnorm_kernel(const float* __restrict__ X, int H, int64_t ldx,
                                                       const uint16_t* __restrict__ g, float eps,
                                                       float* __restrict__ Y, int64_t ldy) {
    extern __shared__ float lds[];  // [H + 4 S] padded row, then [S] slice partials, then r
    const int S = (H + KS - 1) / KS;
    float* xs = lds;
    float* part = lds + H + RN_PAD * S;
    const int row = blockIdx.x;
    const int tid = threadIdx.x;
    const float* x = X + (int64_t)row * ldx;
    for (int i0 = tid * 4; i0 < H; i0 += RN_U * RN_T * 4) {
        float4 v[RN_U];
#pragma unroll
        for (int u = 0; u < RN_U; ++u) {
            const int i = i0 + u * RN_T * 4;
            v[u] = *reinterpret_cast<const float4*>(x + (i < H ? i : 0));
        }
#pragma unroll
        for (int u = 0; u < RN_U; ++u) {
            const int i = i0 + u * RN_T * 4;
            if (i < H) *reinterpret_cast<float4*>(xs + rn_at(i)) = v[u];
        }
    }
    // the first batch of gains is requested before the reduction and used after it
    uint2 g0[RN_U];
#pragma unroll
    for (int u = 0; u < RN_U; ++u) {
        const int i = tid * 4 + u * RN_T * 4;
        g0[u] = *reinterpret_cast<const uint2*>(g + (i < H ? i : 0));
    }
    __syncthreads();
    for (int s = tid; s < S; s += RN_T) {
        const int n = min(KS, H - s * KS);       // a multiple of 8
        const float* sx = xs + s * (KS + RN_PAD);
        float c = 0.0f;
        for (int kb = 0; kb < n; kb += 4 * RN_CH) {
            float4 v[RN_CH];
#pragma unroll
            for (int u = 0; u < RN_CH; ++u) v[u] = *reinterpret_cast<const float4*>(sx + min(kb + 4 * u, n - 4));
#pragma unroll
            for (int u = 0; u < RN_CH; ++u) {
                if (kb + 4 * u < n) {
                    c = __builtin_fmaf(v[u].x, v[u].x, c);
                    c = __builtin_fmaf(v[u].y, v[u].y, c);
                    c = __builtin_fmaf(v[u].z, v[u].z, c);
                    c = __builtin_fmaf(v[u].w, v[u].w, c);
                }
            }
        }
        part[s] = c;
    }
    __syncthreads();
    if (tid == 0) {
        float T = part[0];
        for (int s = 1; s < S; ++s) T = T + part[s];
        part[S] = 1.0f / __builtin_sqrtf((T / (float)H) + eps);
    }
    __syncthreads();
    const float r = part[S];
    float* y = Y + (int64_t)row * ldy;
    for (int i0 = tid * 4; i0 < H; i0 += RN_U * RN_T * 4) {
        uint2 gg[RN_U];
#pragma unroll
        for (int u = 0; u < RN_U; ++u) {
            const int i = i0 + u * RN_T * 4;
            gg[u] = (i0 == tid * 4) ? g0[u] : *reinterpret_cast<const uint2*>(g + (i < H ? i : 0));
        }
#pragma unroll
        for (int u = 0; u < RN_U; ++u) {
            const int i = i0 + u * RN_T * 4;
            if (i < H) {
                const float4 v = *reinterpret_cast<const float4*>(xs + rn_at(i));
                float4 o;
                o.x = (v.x * r) * bf16_lo(gg[u].x);
                o.y = (v.y * r) * bf16_hi(gg[u].x);
                o.z = (v.z * r) * bf16_lo(gg[u].y);
                o.w = (v.w * r) * bf16_hi(gg[u].y);
                *reinterpret_cast<float4*>(y + i) = o;
            }
        }
    }
}

__global__ void embed_kernel(const int32_t* __restrict__ ids, int M, const uint16_t* __restrict__ table,
                             int vocab, int H, float* __restrict__ X, int64_t ldx) {
    const int64_t n4 = (int64_t)M * (H / 4);
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int m = (int)(i / (H / 4));
        const int k = (int)(i % (H / 4)) * 4;
        const int id = ids[m];
        float4 o;
        if (id >= 0 && id < vocab) {
            const uint2 w = *reinterpret_cast<const uint2*>(table + (int64_t)id * H + k);
            o = make_float4(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y));
        } else {
            const float nan = __builtin_nanf("");
            o = make_float4(nan, nan, nan, nan);   // out-of-range id: poisoned row
        }
        *reinterpret_cast<float4*>(X + (int64_t)m * ldx + k) = o;
    }
}

// Storage rounding of one value to the activation format FMT (INV_F32: unchanged).
template <int FMT>
__device__ __forceinline__ float store_round(float v) {
    if (FMT == INV_BF16) return bf16_up(bf16_rne(v));
    if (FMT == INV_F16) return f16_round(v);
    return v;
}

// One thread per (row, head, pair i < D/2).  Heads 0..Hq-1 are q heads (written to Qout),
// Hq..Hq+Hkv-1 are k heads (rotated into Kc), the last Hkv are v heads (copied into Vc).
// Every value written is rounded to the activation format FMT.
template <int FMT>
__global__ void rope_kv_kernel(const float* __restrict__ QKV, int M, int64_t ldqkv, int Hq, int Hkv,
                               int D, const int32_t* __restrict__ seq, const int32_t* __restrict__ pos,
                               const float* __restrict__ cos_t, const float* __restrict__ sin_t,
                               int Tmax, int Bcache, float* __restrict__ Qout, float* __restrict__ Kc,
                               float* __restrict__ Vc) {
    const int half = D / 2;
    const int nh = Hq + 2 * Hkv;
    const int64_t total = (int64_t)M * nh * half;
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int i = (int)(t % half);
        const int h = (int)((t / half) % nh);
        const int m = (int)(t / ((int64_t)half * nh));
        const float* x = QKV + (int64_t)m * ldqkv + (int64_t)h * D;
        const int p = pos[m];
        const int sq = seq[m];
        if (p < 0 || p >= Tmax || sq < 0 || sq >= Bcache) continue;   // row outside the cache
        if (h < Hq + Hkv) {
            const float c = cos_t[(int64_t)p * half + i];
            const float s = sin_t[(int64_t)p * half + i];
            const float a = x[i], b = x[i + half];
            const float y0 = store_round<FMT>((a * c) - (b * s));
            const float y1 = store_round<FMT>((a * s) + (b * c));
            if (h < Hq) {
                float* q = Qout + ((int64_t)m * Hq + h) * D;
                q[i] = y0;
                q[i + half] = y1;
            } else {
                const int gk = h - Hq;
                float* k = Kc + (((int64_t)sq * Hkv + gk) * Tmax + p) * D;
                k[i] = y0;
                k[i + half] = y1;
            }
        } else {
            const int gv = h - Hq - Hkv;
            float* v = Vc + (((int64_t)sq * Hkv + gv) * Tmax + p) * D;
            v[i] = store_round<FMT>(x[i]);
            v[i + half] = store_round<FMT>(x[i + half]);
        }
    }
}

__global__ void swiglu_kernel(const float* __restrict__ G, const float* __restrict__ U, int M, int F,
                              int64_t ldg, int64_t ldu, float* __restrict__ Hout, int64_t ldh) {
    const int64_t total = (int64_t)M * F;
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int m = (int)(t / F), f = (int)(t % F);
        const float g = G[(int64_t)m * ldg + f];
        const float sg = g / (1.0f + exp_f(-g));
        Hout[(int64_t)m * ldh + f] = sg * U[(int64_t)m * ldu + f];
    }
}

__global__ void add_kernel(const float* __restrict__ A, const float* __restrict__ B, int M, int N,
                           int64_t lda, int64_t ldb, float* __restrict__ Y, int64_t ldy) {
    const int64_t total = (int64_t)M * N;
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int m = (int)(t / N), n = (int)(t % N);
        Y[(int64_t)m * ldy + n] = A[(int64_t)m * lda + n] + B[(int64_t)m * ldb + n];
    }
}

// Storage rounding of FP32 activations (fmt INV_BF16, INV_F16, or INV_F32 = copy), 2-D with
// row strides.  In place when Y == X (each element is read before its own write).  VEC: rows
// of whole float4s with 16-byte aligned base pointers and strides.
template <int FMT, bool VEC>
__global__ void round_act_kernel(const float* X, int64_t rows, int64_t cols, int64_t ldx, float* Y,
                                 int64_t ldy) {
    const int64_t cw = VEC ? cols / 4 : cols;
    const int64_t total = rows * cw;
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t m = t / cw, c = t % cw;
        if (VEC) {
            float4 v = *(const float4*)(X + m * ldx + 4 * c);
            v.x = store_round<FMT>(v.x);
            v.y = store_round<FMT>(v.y);
            v.z = store_round<FMT>(v.z);
            v.w = store_round<FMT>(v.w);
            *(float4*)(Y + m * ldy + 4 * c) = v;
        } else {
            Y[m * ldy + c] = store_round<FMT>(X[m * ldx + c]);
        }
    }
}

__global__ void eval_numerics_kernel(int fn, const float* __restrict__ x, float* __restrict__ y,
                                     int64_t n) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const float v = x[i];
        y[i] = fn == 0 ? exp_f(v) : fn == 1 ? log_f(v) : bf16_up(bf16_rne(v));
    }
}

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// One v_mfma_f32_16x16x4_f32 per test: test t supplies A [16 x 4], B [4 x 16], C [16 x 16]
// (row-major) and receives D = C + A B as the instruction computes it.
__global__ __launch_bounds__(64) void mfma_check_kernel(const float* __restrict__ A,
                                                        const float* __restrict__ B,
                                                        const float* __restrict__ C,
                                                        float* __restrict__ D, int64_t ntest) {
    const int l = threadIdx.x, g = l >> 4, r = l & 15;
    for (int64_t t = blockIdx.x; t < ntest; t += gridDim.x) {
        const float a = A[t * 64 + r * 4 + g];      // A[r][g]
        const float b = B[t * 64 + g * 16 + r];     // B[g][r]
        f32x4_t c;
        for (int v = 0; v < 4; ++v) c[v] = C[t * 256 + (4 * g + v) * 16 + r];
        const f32x4_t d = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
        for (int v = 0; v < 4; ++v) D[t * 256 + (4 * g + v) * 16 + r] = d[v];
    }
}

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// One v_mfma_f32_32x32x2_f32 per test: test t supplies A [32 x 2], B [2 x 32], C [32 x 32]
// (row-major) and receives D = C + A B as the instruction computes it.  Lane l supplies
// A[l % 32][l / 32] and B[l / 32][l % 32]; register v of lane l is the element at row
// 8 (v / 4) + 4 (l / 32) + (v % 4), column l % 32.
__global__ __launch_bounds__(64) void mfma32_check_kernel(const float* __restrict__ A,
                                                          const float* __restrict__ B,
                                                          const float* __restrict__ C,
                                                          float* __restrict__ D, int64_t ntest) {
    const int l = threadIdx.x, h = l >> 5, c = l & 31;
    for (int64_t t = blockIdx.x; t < ntest; t += gridDim.x) {
        const float a = A[t * 64 + c * 2 + h];      // A[c][h]
        const float b = B[t * 64 + h * 32 + c];     // B[h][c]
        f32x16_t acc;
        for (int v = 0; v < 16; ++v) acc[v] = C[t * 1024 + (8 * (v >> 2) + 4 * h + (v & 3)) * 32 + c];
        const f32x16_t d = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
        for (int v = 0; v < 16; ++v) D[t * 1024 + (8 * (v >> 2) + 4 * h + (v & 3)) * 32 + c] = d[v];
    }
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// One v_mfma_f32_16x16x32_bf16 per test, in lane form: test t supplies for each lane l of the
// wavefront its 8 A operands (BF16 bits, A + (64 t + l) * 8), its 8 B operands (same layout in
// B) and its 4 accumulator values (C + (64 t + l) * 4), and receives the lane's 4 results at
// D + (64 t + l) * 4.  The mapping of matrix elements to lanes is left to the caller.
__global__ __launch_bounds__(64) void mfma_bf16_check_kernel(const uint16_t* __restrict__ A,
                                                             const uint16_t* __restrict__ B,
                                                             const float* __restrict__ C,
                                                             float* __restrict__ D, int64_t ntest) {
    const int l = threadIdx.x;
    for (int64_t t = blockIdx.x; t < ntest; t += gridDim.x) {
        const int64_t o = t * 64 + l;
        bf16x8_t a, b;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[i] = __builtin_bit_cast(__bf16, A[o * 8 + i]);
            b[i] = __builtin_bit_cast(__bf16, B[o * 8 + i]);
        }
        f32x4_t c;
#pragma unroll
        for (int v = 0; v < 4; ++v) c[v] = C[o * 4 + v];
        const f32x4_t d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 4; ++v) D[o * 4 + v] = d[v];
    }
}

// Read-stream probe: every thread reads 16-byte units of src (grid-stride over n16 units,
// four in flight) and adds their bits into a per-workgroup checksum, so the loads cannot be
// dropped; the practical HBM read rate of a plain streaming kernel.
__global__ __launch_bounds__(256) void read_stream_kernel(const uint4* __restrict__ src, int64_t n16,
                                                         uint32_t* __restrict__ sink) {
    __shared__ uint32_t acc[4];
    uint32_t x = 0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        x += a.x ^ a.y ^ a.z ^ a.w;
        x += b.x ^ b.y ^ b.z ^ b.w;
        x += c.x ^ c.y ^ c.z ^ c.w;
        x += d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < n16; i += stride) { const uint4 a = src[i]; x += a.x ^ a.y ^ a.z ^ a.w; }
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    if ((threadIdx.x & 63) == 0) acc[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = acc[0] + acc[1] + acc[2] + acc[3];
}

// Matrix-core rate probe: each wavefront issues `iters` rounds of 8 independent FP32 matrix
// instructions (shape 0: 16x16x4, shape 1: 32x32x2) on register operands, with no memory
// traffic, and stores its accumulators once so the work is kept.
template <int SHAPE>
__global__ __launch_bounds__(256) void mfma_rate_kernel(int64_t iters, float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const float a = 1.0f + lane * 1e-3f, b = 1.0f - lane * 1e-3f;
    if constexpr (SHAPE == 0) {
        f32x4_t acc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[j], 0, 0, 0);
        }
        float t = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) t += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
        out[blockIdx.x * (int64_t)blockDim.x + threadIdx.x] = t;
    } else {
        f32x16_t acc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[j][v] = 0.0f;
        for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[j], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(b, a, acc[j], 0, 0, 0);
        }
        float t = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) t += acc[j][v];
        out[blockIdx.x * (int64_t)blockDim.x + threadIdx.x] = t;
    }
}

inline int grid_for(int64_t work, int block) {
    int64_t g = (work + block - 1) / block;
    if (g > 65536) g = 65536;
    if (g < 1) g = 1;
    return (int)g;
}

}  // namespace

hipError_t launch_rmsnorm(const float* X, int M, int H, int64_t ldx, const uint16_t* g, float eps,
                          float* Y, int64_t ldy, hipStream_t st) {
    const int S = (H + KS - 1) / KS;
    const size_t lds = sizeof(float) * ((size_t)H + RN_PAD * S + S + 1);
    hipLaunchKernelGGL(rmsnorm_kernel, dim3(M), dim3(RN_T), lds, st, X, H, ldx, g, eps, Y, ldy);
    return hipGetLastError();
}

hipError_t launch_embed(const int32_t* ids, int M, const uint16_t* table, int vocab, int H, float* X,
                        int64_t ldx, hipStream_t st) {
    hipLaunchKernelGGL(embed_kernel, dim3(grid_for((int64_t)M * H / 4, 256)), dim3(256), 0, st,
                       ids, M, table, vocab, H, X, ldx);
    return hipGetLastError();
}

hipError_t launch_rope_kv_append(const float* QKV, int M, int64_t ldqkv, int Hq, int Hkv, int D,
                                 const int32_t* seq, const int32_t* pos, const float* cos_t,
                                 const float* sin_t, int Tmax, int Bcache, float* Qout, float* Kc,
                                 float* Vc, int out_fmt, hipStream_t st) {
    const int64_t work = (int64_t)M * (Hq + 2 * Hkv) * (D / 2);
    const dim3 grid(grid_for(work, 256)), block(256);
    if (out_fmt == INV_BF16)
        hipLaunchKernelGGL(rope_kv_kernel<INV_BF16>, grid, block, 0, st, QKV, M, ldqkv, Hq, Hkv, D, seq,
                           pos, cos_t, sin_t, Tmax, Bcache, Qout, Kc, Vc);
    else if (out_fmt == INV_F16)
        hipLaunchKernelGGL(rope_kv_kernel<INV_F16>, grid, block, 0, st, QKV, M, ldqkv, Hq, Hkv, D, seq,
                           pos, cos_t, sin_t, Tmax, Bcache, Qout, Kc, Vc);
    else
        hipLaunchKernelGGL(rope_kv_kernel<INV_F32>, grid, block, 0, st, QKV, M, ldqkv, Hq, Hkv, D, seq,
                           pos, cos_t, sin_t, Tmax, Bcache, Qout, Kc, Vc);
    return hipGetLastError();
}

hipError_t launch_swiglu(const float* G, const float* U, int M, int F, int64_t ldg, int64_t ldu,
                         float* Hout, int64_t ldh, hipStream_t st) {
    hipLaunchKernelGGL(swiglu_kernel, dim3(grid_for((int64_t)M * F, 256)), dim3(256), 0, st, G, U,
                       M, F, ldg, ldu, Hout, ldh);
    return hipGetLastError();
}

hipError_t launch_add(const float* A, const float* B, int M, int N, int64_t lda, int64_t ldb,
                      float* Y, int64_t ldy, hipStream_t st) {
    hipLaunchKernelGGL(add_kernel, dim3(grid_for((int64_t)M * N, 256)), dim3(256), 0, st, A, B, M,
                       N, lda, ldb, Y, ldy);
    return hipGetLastError();
}

template <int FMT>
static hipError_t launch_round_fmt(const float* X, int64_t rows, int64_t cols, int64_t ldx, float* Y,
                                   int64_t ldy, hipStream_t st) {
    const bool vec = cols % 4 == 0 && ldx % 4 == 0 && ldy % 4 == 0 &&
                     ((uintptr_t)X & 15) == 0 && ((uintptr_t)Y & 15) == 0;
    if (vec)
        hipLaunchKernelGGL((round_act_kernel<FMT, true>), dim3(grid_for(rows * (cols / 4), 256)),
                           dim3(256), 0, st, X, rows, cols, ldx, Y, ldy);
    else
        hipLaunchKernelGGL((round_act_kernel<FMT, false>), dim3(grid_for(rows * cols, 256)), dim3(256),
                           0, st, X, rows, cols, ldx, Y, ldy);
    return hipGetLastError();
}

hipError_t launch_round_activations(const float* X, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                                    float* Y, int64_t ldy, hipStream_t st) {
    if (fmt == INV_BF16) return launch_round_fmt<INV_BF16>(X, rows, cols, ldx, Y, ldy, st);
    if (fmt == INV_F16) return launch_round_fmt<INV_F16>(X, rows, cols, ldx, Y, ldy, st);
    return launch_round_fmt<INV_F32>(X, rows, cols, ldx, Y, ldy, st);
}

hipError_t launch_eval_numerics(int fn, const float* x, float* y, int64_t n, hipStream_t st) {
    hipLaunchKernelGGL(eval_numerics_kernel, dim3(grid_for(n, 256)), dim3(256), 0, st, fn, x, y, n);
    return hipGetLastError();
}

hipError_t launch_mfma_check(const float* A, const float* B, const float* C, float* D, int64_t ntest,
                             hipStream_t st) {
    const int grid = (int)(ntest < 4096 ? ntest : 4096);
    hipLaunchKernelGGL(mfma_check_kernel, dim3(grid), dim3(64), 0, st, A, B, C, D, ntest);
    return hipGetLastError();
}

hipError_t launch_mfma32_check(const float* A, const float* B, const float* C, float* D, int64_t ntest,
                               hipStream_t st) {
    const int grid = (int)(ntest < 4096 ? ntest : 4096);
    hipLaunchKernelGGL(mfma32_check_kernel, dim3(grid), dim3(64), 0, st, A, B, C, D, ntest);
    return hipGetLastError();
}

hipError_t launch_mfma_bf16_check(const uint16_t* A, const uint16_t* B, const float* C, float* D, int64_t ntest,
                                  hipStream_t st) {
    const int grid = (int)(ntest < 4096 ? ntest : 4096);
    hipLaunchKernelGGL(mfma_bf16_check_kernel, dim3(grid), dim3(64), 0, st, A, B, C, D, ntest);
    return hipGetLastError();
}

hipError_t launch_read_stream(const void* src, int64_t bytes, uint32_t* sink, int grid, hipStream_t st) {
    hipLaunchKernelGGL(read_stream_kernel, dim3(grid), dim3(256), 0, st, reinterpret_cast<const uint4*>(src),
                       bytes / 16, sink);
    return hipGetLastError();
}

hipError_t launch_mfma_rate(int shape, int64_t iters, int waves_per_cu, float* out, hipStream_t st) {
    // 256 CUs x waves_per_cu wavefronts in workgroups of 4 (one per SIMD)
    const int grid = 256 * waves_per_cu / 4;
    if (shape == 0)
        hipLaunchKernelGGL(mfma_rate_kernel<0>, dim3(grid), dim3(256), 0, st, iters, out);
    else
        hipLaunchKernelGGL(mfma_rate_kernel<1>, dim3(grid), dim3(256), 0, st, iters, out);
    return hipGetLastError();
}

}  // namespace invnum
