// gemm.hip -- LayerCast matmul Y = X . up(W)^T with the fixed K order dot_KS.
//
// Order of every output (never depends on M, the grid or the kernel variant):
//   K is cut into contiguous slices of 256; within a slice c = +0 then c = fma(x_k, w_k, c)
//   for k ascending; the slices are folded T = c_0, T = T + c_s for s ascending.
// Two kernels implement it:
//   * gemm_mfma: a workgroup owns a BM x BN output tile and walks K in 32-wide LDS tiles
//     (8 per slice) on the FP32 matrix cores, keeping two registers per output (the slice
//     accumulator and the folded total T).  Used when M > 16.
//   * gemm_skinny: for M <= 16 the work per output row is too small to fill the chip,
//     so a workgroup owns 16 weight rows and all M activation rows; each thread owns one
//     (weight row, slice) pair, keeps one accumulator per activation row, and the slice
//     partials are folded in slice order through LDS by one thread per output.
// BF16 weights are upcast (bits << 16, exact) as they are loaded.
#include "numerics.h"
#include "kernels.h"

namespace invnum {

namespace {

constexpr int BK = 32;  // K tile; divides KS, so slice ends fall on tile ends

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Position of k (0..31) inside a tile row of LDS: lane group g of an MFMA reads
// k = g, g+4, ..., g+28 (one per 4-wide MFMA step) as 8 contiguous floats.
__device__ __forceinline__ int kpos(int k) { return (k & 3) * 8 + (k >> 2); }

// Register-tiled GEMM on the FP32 matrix cores.  v_mfma_f32_16x16x4_f32 advances every
// output of a 16x16 tile by k = 4s, 4s+1, 4s+2, 4s+3 as four fused multiply-adds in that
// order (each rounded once) -- the same arithmetic as the sequential fma chain of a slice,
// so issuing the steps s in ascending order reproduces dot_KS bit for bit.  (This is a
// measured property of the gfx950 instruction, checked by the test suite against the
// CPU reference through inv_mfma_f32_check.)
// Workgroup: 256 threads = 4 wavefronts in a 2 x 2 grid over a BM x BN output tile; each
// wavefront owns (BM/2) x (BN/2) outputs = TI x TJ MFMA tiles.  Per output two registers:
// the slice accumulator (MFMA C/D) and the folded total T.
// ROLE only separates instantiations: 0 = activation projections, 1 = the vocabulary
// projection of the LM head, so each can carry its own tile choice and profiles attribute
// their time separately.
template <int BM, int BN, int ROLE>
__global__ __launch_bounds__(256) void gemm_mfma_kernel(
    const float* __restrict__ X, int M, int K, int64_t ldx,
    const uint16_t* __restrict__ W, int N, int64_t ldw,
    const float* __restrict__ R, int64_t ldr,
    float* __restrict__ Y, int64_t ldy, const int* __restrict__ Mdev) {
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int TI = WM / 16, TJ = WN / 16;
    constexpr int LDT = BK + 4;                    // padded LDS row (floats)
    constexpr int XV = BM * (BK / 4) / 256;        // float4 loads of X per thread per tile
    constexpr int WV = BN * (BK / 8) / 256;        // 16-byte loads of W per thread per tile
    static_assert(XV >= 1 && WV >= 1 && TI >= 1 && TJ >= 1, "tile too small");
    __shared__ float As[2][BM][LDT];
    __shared__ float Bs[2][BN][LDT];

    if (Mdev) M = min(M, *Mdev);
    const int m0 = blockIdx.y * BM;
    const int n0 = blockIdx.x * BN;
    if (m0 >= M) return;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int g = lane >> 4, r = lane & 15;
    const int wm0 = (wv >> 1) * WM, wn0 = (wv & 1) * WN;

    float4 xr[XV];
    uint4 wr[WV];
    auto load_tile = [&](int k0) {
#pragma unroll
        for (int i = 0; i < XV; ++i) {
            const int idx = tid + i * 256;
            const int row = idx / (BK / 4), q = idx % (BK / 4);
            const int gm = m0 + row, gk = k0 + 4 * q;
            const bool in = gm < M && gk < K;   // outside: read a valid element, use zeros
            const float4 t = *reinterpret_cast<const float4*>(X + (int64_t)min(gm, M - 1) * ldx + min(gk, K - 4));
            xr[i] = in ? t : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int i = 0; i < WV; ++i) {
            const int idx = tid + i * 256;
            const int row = idx / (BK / 8), o = idx % (BK / 8);
            const int gn = n0 + row, gk = k0 + 8 * o;
            const bool in = gn < N && gk < K;
            const uint4 t = *reinterpret_cast<const uint4*>(W + (int64_t)min(gn, N - 1) * ldw + min(gk, K - 8));
            wr[i] = in ? t : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < XV; ++i) {
            const int idx = tid + i * 256;
            const int row = idx / (BK / 4), q = idx % (BK / 4);
            float* d = As[buf][row];
            d[kpos(4 * q + 0)] = xr[i].x;
            d[kpos(4 * q + 1)] = xr[i].y;
            d[kpos(4 * q + 2)] = xr[i].z;
            d[kpos(4 * q + 3)] = xr[i].w;
        }
#pragma unroll
        for (int i = 0; i < WV; ++i) {
            const int idx = tid + i * 256;
            const int row = idx / (BK / 8), o = idx % (BK / 8);
            float* d = Bs[buf][row];
            d[kpos(8 * o + 0)] = bf16_lo(wr[i].x);
            d[kpos(8 * o + 1)] = bf16_hi(wr[i].x);
            d[kpos(8 * o + 2)] = bf16_lo(wr[i].y);
            d[kpos(8 * o + 3)] = bf16_hi(wr[i].y);
            d[kpos(8 * o + 4)] = bf16_lo(wr[i].z);
            d[kpos(8 * o + 5)] = bf16_hi(wr[i].z);
            d[kpos(8 * o + 6)] = bf16_lo(wr[i].w);
            d[kpos(8 * o + 7)] = bf16_hi(wr[i].w);
        }
    };

    f32x4 acc[TI][TJ], T[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) { acc[i][j][v] = 0.0f; T[i][j][v] = 0.0f; }

    const int nt = (K + BK - 1) / BK;
    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int t = 0; t < nt; ++t) {
        const int buf = t & 1;
        if (t + 1 < nt) load_tile((t + 1) * BK);
        float a[TI][8], b[TJ][8];
#pragma unroll
        for (int i = 0; i < TI; ++i) {
            const float4* src = reinterpret_cast<const float4*>(&As[buf][wm0 + i * 16 + r][g * 8]);
            const float4 lo = src[0], hi = src[1];
            a[i][0] = lo.x; a[i][1] = lo.y; a[i][2] = lo.z; a[i][3] = lo.w;
            a[i][4] = hi.x; a[i][5] = hi.y; a[i][6] = hi.z; a[i][7] = hi.w;
        }
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            const float4* src = reinterpret_cast<const float4*>(&Bs[buf][wn0 + j * 16 + r][g * 8]);
            const float4 lo = src[0], hi = src[1];
            b[j][0] = lo.x; b[j][1] = lo.y; b[j][2] = lo.z; b[j][3] = lo.w;
            b[j][4] = hi.x; b[j][5] = hi.y; b[j][6] = hi.z; b[j][7] = hi.w;
        }
        const int kend = min(BK, K - t * BK);
        if (kend == BK) {
#pragma unroll
            for (int s = 0; s < BK / 4; ++s)
#pragma unroll
                for (int i = 0; i < TI; ++i)
#pragma unroll
                    for (int j = 0; j < TJ; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i][s], b[j][s], acc[i][j], 0, 0, 0);
        } else {
            // partial last tile: only the k-steps below K (zero padding is never multiplied in)
#pragma unroll
            for (int s = 0; s < BK / 4; ++s) {
                if (4 * s < kend) {
#pragma unroll
                    for (int i = 0; i < TI; ++i)
#pragma unroll
                        for (int j = 0; j < TJ; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i][s], b[j][s], acc[i][j], 0, 0, 0);
                }
            }
        }
        const int kdone = t * BK + kend;
        if (kdone % KS == 0 || kdone == K) {
            const bool first = kdone <= KS;
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int j = 0; j < TJ; ++j)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        T[i][j][v] = first ? acc[i][j][v] : T[i][j][v] + acc[i][j][v];
                        acc[i][j][v] = 0.0f;
                    }
        }
        if (t + 1 < nt) store_tile(buf ^ 1);
        __syncthreads();
    }

    // lane (g, r) holds rows 4g..4g+3, column r of each 16 x 16 tile
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int gm = m0 + wm0 + i * 16 + 4 * g + v;
            if (gm >= M) continue;
#pragma unroll
            for (int j = 0; j < TJ; ++j) {
                const int gn = n0 + wn0 + j * 16 + r;
                if (gn >= N) continue;
                float y = T[i][j][v];
                if (R) y = R[(int64_t)gm * ldr + gn] + y;
                Y[(int64_t)gm * ldy + gn] = y;
            }
        }
}

// ---------------------------------------------------------------- skinny --
constexpr int SK_ROWS = 16;   // weight rows per workgroup
constexpr int SK_LANES = 16;  // slice lanes per weight row

template <int MB, int ROLE>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(
    const float* __restrict__ X, int M, int K, int64_t ldx,
    const uint16_t* __restrict__ W, int N, int64_t ldw,
    const float* __restrict__ R, int64_t ldr,
    float* __restrict__ Y, int64_t ldy, const int* __restrict__ Mdev) {
    extern __shared__ float part[];  // [S][MB][SK_ROWS]
    if (Mdev) M = min(M, *Mdev);
    if (M <= 0) return;
    const int S = (K + KS - 1) / KS;
    const int tid = threadIdx.x;
    const int nl = tid % SK_ROWS;
    const int sl = tid / SK_ROWS;
    const int n = blockIdx.x * SK_ROWS + nl;
    const bool nvalid = n < N;
    const uint16_t* wrow = W + (int64_t)(nvalid ? n : 0) * ldw;

    for (int s = sl; s < S; s += SK_LANES) {
        float c[MB];
#pragma unroll
        for (int m = 0; m < MB; ++m) c[m] = 0.0f;
        const int k0 = s * KS;
        const int k1 = min(K, k0 + KS);
        if (nvalid) {
            for (int k = k0; k < k1; k += 8) {
                const uint4 w8 = *reinterpret_cast<const uint4*>(wrow + k);
                const float w[8] = {bf16_lo(w8.x), bf16_hi(w8.x), bf16_lo(w8.y), bf16_hi(w8.y),
                                    bf16_lo(w8.z), bf16_hi(w8.z), bf16_lo(w8.w), bf16_hi(w8.w)};
#pragma unroll
                for (int m = 0; m < MB; ++m) {
                    if (m < M) {
                        const float* xr = X + (int64_t)m * ldx + k;
                        const float4 xa = *reinterpret_cast<const float4*>(xr);
                        const float4 xb = *reinterpret_cast<const float4*>(xr + 4);
                        c[m] = __builtin_fmaf(xa.x, w[0], c[m]);
                        c[m] = __builtin_fmaf(xa.y, w[1], c[m]);
                        c[m] = __builtin_fmaf(xa.z, w[2], c[m]);
                        c[m] = __builtin_fmaf(xa.w, w[3], c[m]);
                        c[m] = __builtin_fmaf(xb.x, w[4], c[m]);
                        c[m] = __builtin_fmaf(xb.y, w[5], c[m]);
                        c[m] = __builtin_fmaf(xb.z, w[6], c[m]);
                        c[m] = __builtin_fmaf(xb.w, w[7], c[m]);
                    }
                }
            }
        }
#pragma unroll
        for (int m = 0; m < MB; ++m) part[(s * MB + m) * SK_ROWS + nl] = c[m];
    }
    __syncthreads();
    // fold: one thread per (m, weight row), slices ascending
    for (int o = tid; o < MB * SK_ROWS; o += 256) {
        const int m = o / SK_ROWS, r = o % SK_ROWS;
        const int gn = blockIdx.x * SK_ROWS + r;
        if (m >= M || gn >= N) continue;
        float T = part[(0 * MB + m) * SK_ROWS + r];
        for (int s = 1; s < S; ++s) T = T + part[(s * MB + m) * SK_ROWS + r];
        if (R) T = R[(int64_t)m * ldr + gn] + T;
        Y[(int64_t)m * ldy + gn] = T;
    }
}

template <int BM, int BN, int ROLE>
hipError_t launch_tiled(const GemmArgs& a, hipStream_t st) {
    dim3 grid((a.N + BN - 1) / BN, (a.M + BM - 1) / BM);
    hipLaunchKernelGGL((gemm_mfma_kernel<BM, BN, ROLE>), grid, dim3(256), 0, st,
                       a.X, a.M, a.K, a.ldx, a.W, a.N, a.ldw, a.R, a.ldr, a.Y, a.ldy, a.Mdev);
    return hipGetLastError();
}

template <int MB, int ROLE>
hipError_t launch_skinny(const GemmArgs& a, hipStream_t st) {
    const int S = (a.K + KS - 1) / KS;
    const size_t lds = sizeof(float) * (size_t)S * MB * SK_ROWS;
    dim3 grid((a.N + SK_ROWS - 1) / SK_ROWS);
    hipLaunchKernelGGL((gemm_skinny_kernel<MB, ROLE>), grid, dim3(256), lds, st,
                       a.X, a.M, a.K, a.ldx, a.W, a.N, a.ldw, a.R, a.ldr, a.Y, a.ldy, a.Mdev);
    return hipGetLastError();
}

}  // namespace

int64_t gemm_skinny_max_k() {
    // LDS partials: S * 16 * 16 floats must fit in 64 KiB of dynamic LDS.
    return (int64_t)KS * (65536 / (int)(sizeof(float) * 16 * SK_ROWS));
}

template <int ROLE>
hipError_t launch_role(const GemmArgs& a, hipStream_t st) {
    // M is an upper bound when Mdev is set (rows beyond *Mdev are skipped on the device).
    if (a.M <= 16 && a.K <= gemm_skinny_max_k()) {
        if (a.M <= 1) return launch_skinny<1, ROLE>(a, st);
        if (a.M <= 2) return launch_skinny<2, ROLE>(a, st);
        if (a.M <= 4) return launch_skinny<4, ROLE>(a, st);
        if (a.M <= 8) return launch_skinny<8, ROLE>(a, st);
        return launch_skinny<16, ROLE>(a, st);
    }
    if (a.M <= 64) return launch_tiled<64, 64, ROLE>(a, st);
    return launch_tiled<128, 128, ROLE>(a, st);
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st, int role) {
    return role == 1 ? launch_role<1>(a, st) : launch_role<0>(a, st);
}


}  // namespace invnum
