// gemm.hip -- LayerCast matmul Y = X . up(W)^T with the fixed K order dot_KS.
//
// Order of every output (never depends on M, the grid or the kernel variant):
//   K is cut into contiguous slices of 256; within a slice c = +0 then c = fma(x_k, w_k, c)
//   for k ascending; the slices are folded T = c_0, T = T + c_s for s ascending.
// Two kernels implement it:
//   * gemm_tiled: a workgroup owns a BM x BN output tile; each thread owns TM x TN outputs
//     and walks K in 32-wide LDS tiles (8 per slice) keeping two registers per output
//     (the slice accumulator c and the folded total T).  Used when M is large.
//   * gemm_skinny: for M <= 16 the work per output row is too small to fill the chip,
//     so a workgroup owns 16 weight rows and all M activation rows; each thread owns one
//     (weight row, slice) pair, keeps one accumulator per activation row, and the slice
//     partials are folded in slice order through LDS by one thread per output.
// BF16 weights are upcast (bits << 16, exact) as they are loaded.
#include "numerics.h"
#include "kernels.h"

namespace invnum {

namespace {

constexpr int BK = 32;  // K tile of gemm_tiled; divides KS, so slice ends fall on tile ends

// ROLE only separates instantiations: 0 = activation projections, 1 = the vocabulary
// projection of the LM head (N up to 128256), so each can carry its own tile choice and
// profiles attribute their time separately.
template <int BM, int BN, int TM, int TN, int ROLE>
__global__ __launch_bounds__(256) void gemm_tiled_kernel(
    const float* __restrict__ X, int M, int K, int64_t ldx,
    const uint16_t* __restrict__ W, int N, int64_t ldw,
    const float* __restrict__ R, int64_t ldr,
    float* __restrict__ Y, int64_t ldy, const int* __restrict__ Mdev) {
    constexpr int NTX = BN / TN;
    constexpr int NTY = BM / TM;
    static_assert(NTX * NTY == 256, "256 threads");
    constexpr int PADA = 4, PADB = 4;
    constexpr int XV = BM * (BK / 4) / 256;  // float4 loads of X per thread per tile
    constexpr int WV = BN * (BK / 8) / 256;  // 16-byte loads of W per thread per tile
    static_assert(XV >= 1 && WV >= 1, "tile too small");
    __shared__ float As[2][BK][BM + PADA];
    __shared__ float Bs[2][BK][BN + PADB];

    if (Mdev) M = min(M, *Mdev);
    const int m0 = blockIdx.y * BM;
    const int n0 = blockIdx.x * BN;
    if (m0 >= M) return;
    const int tid = threadIdx.x;
    const int tx = tid % NTX, ty = tid / NTX;

    float4 xr[XV];
    uint4 wr[WV];
    auto load_tile = [&](int k0) {
#pragma unroll
        for (int i = 0; i < XV; ++i) {
            const int idx = tid + i * 256;
            const int r = idx / (BK / 4), q = idx % (BK / 4);
            const int gm = m0 + r, gk = k0 + 4 * q;
            if (gm < M && gk < K)
                xr[i] = *reinterpret_cast<const float4*>(X + (int64_t)gm * ldx + gk);
            else
                xr[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int i = 0; i < WV; ++i) {
            const int idx = tid + i * 256;
            const int r = idx / (BK / 8), o = idx % (BK / 8);
            const int gn = n0 + r, gk = k0 + 8 * o;
            if (gn < N && gk < K)
                wr[i] = *reinterpret_cast<const uint4*>(W + (int64_t)gn * ldw + gk);
            else
                wr[i] = make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < XV; ++i) {
            const int idx = tid + i * 256;
            const int r = idx / (BK / 4), q = idx % (BK / 4);
            As[buf][4 * q + 0][r] = xr[i].x;
            As[buf][4 * q + 1][r] = xr[i].y;
            As[buf][4 * q + 2][r] = xr[i].z;
            As[buf][4 * q + 3][r] = xr[i].w;
        }
#pragma unroll
        for (int i = 0; i < WV; ++i) {
            const int idx = tid + i * 256;
            const int r = idx / (BK / 8), o = idx % (BK / 8);
            Bs[buf][8 * o + 0][r] = bf16_lo(wr[i].x);
            Bs[buf][8 * o + 1][r] = bf16_hi(wr[i].x);
            Bs[buf][8 * o + 2][r] = bf16_lo(wr[i].y);
            Bs[buf][8 * o + 3][r] = bf16_hi(wr[i].y);
            Bs[buf][8 * o + 4][r] = bf16_lo(wr[i].z);
            Bs[buf][8 * o + 5][r] = bf16_hi(wr[i].z);
            Bs[buf][8 * o + 6][r] = bf16_lo(wr[i].w);
            Bs[buf][8 * o + 7][r] = bf16_hi(wr[i].w);
        }
    };

    float c[TM][TN], T[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) { c[i][j] = 0.0f; T[i][j] = 0.0f; }

    auto step = [&](int buf, int kk) {
        float a[TM], b[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) a[i] = As[buf][kk][ty * TM + i];
#pragma unroll
        for (int j = 0; j < TN; ++j) b[j] = Bs[buf][kk][tx * TN + j];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) c[i][j] = __builtin_fmaf(a[i], b[j], c[i][j]);
    };

    const int nt = (K + BK - 1) / BK;
    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int t = 0; t < nt; ++t) {
        const int buf = t & 1;
        if (t + 1 < nt) load_tile((t + 1) * BK);
        const int kend = min(BK, K - t * BK);
        if (kend == BK) {
#pragma unroll
            for (int kk = 0; kk < BK; ++kk) step(buf, kk);
        } else {
            for (int kk = 0; kk < kend; ++kk) step(buf, kk);
        }
        const int kdone = t * BK + kend;
        if (kdone % KS == 0 || kdone == K) {
            const bool first = kdone <= KS;
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    T[i][j] = first ? c[i][j] : T[i][j] + c[i][j];
                    c[i][j] = 0.0f;
                }
        }
        if (t + 1 < nt) store_tile(buf ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int gm = m0 + ty * TM + i;
        if (gm >= M) continue;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int gn = n0 + tx * TN + j;
            if (gn >= N) continue;
            float y = T[i][j];
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

template <int BM, int BN, int TM, int TN, int ROLE>
hipError_t launch_tiled(const GemmArgs& a, hipStream_t st) {
    dim3 grid((a.N + BN - 1) / BN, (a.M + BM - 1) / BM);
    hipLaunchKernelGGL((gemm_tiled_kernel<BM, BN, TM, TN, ROLE>), grid, dim3(256), 0, st,
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
    if (a.M <= 64) return launch_tiled<64, 64, 4, 4, ROLE>(a, st);
    return launch_tiled<128, 128, 8, 8, ROLE>(a, st);
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st, int role) {
    return role == 1 ? launch_role<1>(a, st) : launch_role<0>(a, st);
}


}  // namespace invnum
