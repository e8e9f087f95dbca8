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
//     so a workgroup owns 16 (or 4) weight rows and all M activation rows; each thread owns one
//     (weight row, slice) pair, keeps one accumulator per activation row, and the slice
//     partials are folded in slice order through LDS by one thread per output.
// BF16 weights are upcast (bits << 16, exact) as they are loaded.
#include "numerics.h"
#include "kernels.h"

namespace invnum {

namespace {

constexpr int BK = 32;  // K tile; divides KS, so slice ends fall on tile ends

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

// Position of k (0..31) inside a tile row of LDS: the lane half h of an MFMA reads
// k = h, h+2, ..., h+30 (one per 2-wide MFMA step) as 16 contiguous floats.
__device__ __forceinline__ int kpos(int k) { return (k & 1) * 16 + (k >> 1); }

// Register-tiled GEMM on the FP32 matrix cores.  v_mfma_f32_32x32x2_f32 advances every
// output of a 32x32 tile by k = 2s, then k = 2s+1, as two fused multiply-adds in that order
// (each rounded once) -- the same arithmetic as the sequential fma chain of a slice, so
// issuing the steps s in ascending order reproduces dot_KS bit for bit.  (This is a measured
// property of the gfx950 instruction, checked by the test suite against the CPU reference
// through inv_mfma_f32_check.)  The 32x32 form is used rather than the 16x16x4 one because
// a single wavefront per SIMD keeps the matrix pipe nearly full with it; with the 16x16
// form it issues a quarter of its cycles idle.
// Operands: lane l (half h = l / 32, c = l % 32) supplies A[row c][k = 2s + h] and
// B[k = 2s + h][column c]; result register v of lane l is the output at row
// 8 (v / 4) + 4 h + (v % 4), column c.
// Workgroup: WGM x WGN wavefronts over a BM x BN output tile; each wavefront owns
// (BM/WGM) x (BN/WGN) outputs = TI x TJ MFMA tiles.  Per output two registers: the slice
// accumulator (MFMA C/D) and the folded total T.  The large tile runs 8 wavefronts of
// 64 x 64 outputs, two per SIMD, so one wavefront's LDS waits and barrier are covered by
// the other's matrix work.
// ROLE: 0 = activation projections, 1 = the vocabulary projection of the LM head (separate
// instantiations, so each carries its own tile order and profiles attribute their time
// separately), 2 = a gated projection: weight rows interleaved as (gate i, up i) and the
// epilogue writes silu(gate) * up, the SwiGLU of the two outputs, instead of both.
template <int BM, int BN, int WGM, int WGN, int ROLE>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_mfma_kernel(
    const float* __restrict__ X, int M, int K, int64_t ldx,
    const uint16_t* __restrict__ W, int N, int64_t ldw,
    const float* __restrict__ R, int64_t ldr,
    float* __restrict__ Y, int64_t ldy, const int* __restrict__ Mdev) {
    const int gridM = M;                           // the row count the grid was sized for
    constexpr int NT = 64 * WGM * WGN;              // threads
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int TI = WM / 32, TJ = WN / 32;
    constexpr int LDT = BK + 4;                    // padded LDS row (floats)
    constexpr int XV = BM * (BK / 4) / NT;         // float4 loads of X per thread per tile
    constexpr int WV = BN * (BK / 8) / NT;         // 16-byte loads of W per thread per tile
    static_assert(XV >= 1 && WV >= 1 && TI >= 1 && TJ >= 1, "tile too small");
    __shared__ float As[2][BM][LDT];
    __shared__ float Bs[2][BN][LDT];

    if (Mdev) M = min(M, *Mdev);
    int m0, n0;
    {
        // 1-D grid over the nMt x nNt output tiles.  The mapping decides only which workgroup
        // owns a tile, never the order inside a dot.
        const int nMt = (gridM + BM - 1) / BM, nNt = (N + BN - 1) / BN;
        const int L = blockIdx.x;
        if constexpr (ROLE != 1) {
            // Consecutive workgroup ids go to the 8 XCDs in turn, so id L is given tile u from
            // a contiguous range per XCD (a bijection of [0, T)); within it tiles are walked in
            // groups of GM tile rows, column by column, so the ~32 workgroups an XCD runs at
            // once share GM activation and ~32/GM weight tiles in its L2.
            constexpr int NXCD = 8, GM = 4;
            const int T = nMt * nNt;
            const int xcd = L % NXCD, q = L / NXCD;
            const int u = xcd * (T / NXCD) + min(xcd, T % NXCD) + q;
            const int grp = u / (GM * nNt);
            const int mf = grp * GM;
            const int gsz = min(nMt - mf, GM);
            const int within = u - grp * GM * nNt;
            m0 = (mf + within % gsz) * BM;
            n0 = (within / gsz) * BN;
        } else {
            // vocabulary projection: columns fastest.  Its recompute pass has a device-side
            // row count (trailing tile rows exit at once), and this order keeps the live tiles
            // spread over every XCD.
            m0 = (L / nNt) * BM;
            n0 = (L % nNt) * BN;
        }
    }
    if (m0 >= M) return;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int h = lane >> 5, c = lane & 31;
    const int wm0 = (wv / WGN) * WM, wn0 = (wv % WGN) * WN;

    // Per-thread source rows (clamped into range) and their last in-range k offsets are
    // computed once; a tile's loads add its k0, clamped to those offsets.
    // Loads read clamped, in-range addresses with no zero fill: rows past M or N reach only
    // outputs that are never stored, and columns past K only the k-steps a partial last tile
    // skips.  One branch-free path, into native vector registers, so nothing waits on a
    // load before the LDS store that needs it.
    f32x4v xr[XV];
    u32x4v wr[WV];
    const float* xp[XV];
    const uint16_t* wp[WV];
    int xlim[XV], wlim[WV];
#pragma unroll
    for (int i = 0; i < XV; ++i) {
        const int idx = tid + i * NT;
        const int row = idx / (BK / 4), q = idx % (BK / 4);
        xp[i] = X + (int64_t)min(m0 + row, M - 1) * ldx + 4 * q;
        xlim[i] = K - 4 - 4 * q;
    }
#pragma unroll
    for (int i = 0; i < WV; ++i) {
        const int idx = tid + i * NT;
        const int row = idx / (BK / 8), o = idx % (BK / 8);
        wp[i] = W + (int64_t)min(n0 + row, N - 1) * ldw + 8 * o;
        wlim[i] = K - 8 - 8 * o;
    }
    const bool interior = (m0 + BM <= M) && (n0 + BN <= N);
    auto load_tile = [&](int k0) {
#pragma unroll
        for (int i = 0; i < XV; ++i) xr[i] = *reinterpret_cast<const f32x4v*>(xp[i] + min(k0, xlim[i]));
#pragma unroll
        for (int i = 0; i < WV; ++i) wr[i] = *reinterpret_cast<const u32x4v*>(wp[i] + min(k0, wlim[i]));
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < XV; ++i) {
            const int idx = tid + i * NT;
            const int row = idx / (BK / 4), q = idx % (BK / 4);
            // k = 4q + {0, 2} and 4q + {1, 3} land on adjacent positions
            float* d = As[buf][row];
            *reinterpret_cast<float2*>(d + kpos(4 * q)) = make_float2(xr[i].x, xr[i].z);
            *reinterpret_cast<float2*>(d + kpos(4 * q + 1)) = make_float2(xr[i].y, xr[i].w);
        }
#pragma unroll
        for (int i = 0; i < WV; ++i) {
            const int idx = tid + i * NT;
            const int row = idx / (BK / 8), o = idx % (BK / 8);
            // the even k of the 8 (low halves) and the odd k (high halves) are 4 adjacent
            // positions each
            float* d = Bs[buf][row];
            *reinterpret_cast<float4*>(d + kpos(8 * o)) =
                make_float4(bf16_lo(wr[i].x), bf16_lo(wr[i].y), bf16_lo(wr[i].z), bf16_lo(wr[i].w));
            *reinterpret_cast<float4*>(d + kpos(8 * o + 1)) =
                make_float4(bf16_hi(wr[i].x), bf16_hi(wr[i].y), bf16_hi(wr[i].z), bf16_hi(wr[i].w));
        }
    };

    f32x16 acc[TI][TJ], T[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) { acc[i][j][v] = 0.0f; T[i][j][v] = 0.0f; }

    const int ntf = K / BK;                        // full tiles
    const int nt = (K + BK - 1) / BK;              // plus a partial last tile when K % BK != 0
    const int nslices = (K + KS - 1) / KS;
    constexpr int NS = BK / 2;                     // MFMA k-steps per tile
    // Full tiles run in four groups of four k-steps.  The operands of a group sit in one of
    // two register sets; the LDS reads of the next group go out while the current group's
    // matrix instructions run, and the first group of the next tile is read right after the
    // barrier, so no group waits for LDS and the barrier sits between queued matrix work.
    constexpr int GS = 4, NG = NS / GS;            // k-steps per group, groups per tile
    static_assert(NG == 4, "four groups per tile");
    float ga[2][TI][GS], gb[2][TJ][GS];
    auto read_group = [&](int buf, int g, float (&fa)[TI][GS], float (&fb)[TJ][GS]) {
#pragma unroll
        for (int i = 0; i < TI; ++i) {
            const float4 v = *reinterpret_cast<const float4*>(&As[buf][wm0 + i * 32 + c][h * 16 + GS * g]);
            fa[i][0] = v.x; fa[i][1] = v.y; fa[i][2] = v.z; fa[i][3] = v.w;
        }
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            const float4 v = *reinterpret_cast<const float4*>(&Bs[buf][wn0 + j * 32 + c][h * 16 + GS * g]);
            fb[j][0] = v.x; fb[j][1] = v.y; fb[j][2] = v.z; fb[j][3] = v.w;
        }
    };
    auto group = [&](const float (&fa)[TI][GS], const float (&fb)[TJ][GS]) {
#pragma unroll
        for (int s = 0; s < GS; ++s)
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int j = 0; j < TJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i][s], fb[j][s], acc[i][j], 0, 0, 0);
    };
    load_tile(0);
    store_tile(0);
    load_tile(BK);
    __syncthreads();
    read_group(0, 0, ga[0], gb[0]);
    // slice by slice (KS / BK tiles each), so the fold T = T + acc runs once per slice; the
    // loop body sees full tiles only (a partial tile can only be the very last one)
    int t = 0;
    for (int sl = 0; sl < nslices; ++sl) {
        const int tend = min(ntf, t + KS / BK);
        for (; t < tend; ++t) {
            const int buf = t & 1;
            // group 0 (read during the previous tile), reading group 1.  The scheduling
            // barriers keep each group's LDS reads ahead of the previous group's matrix
            // instructions (left alone, the compiler sinks them to just before their use).
            read_group(buf, 1, ga[1], gb[1]);
            __builtin_amdgcn_sched_barrier(0);
            group(ga[0], gb[0]);
            __builtin_amdgcn_sched_barrier(0);
            // group 1, reading group 2; the next tile (in registers since the previous
            // tile) goes to the other LDS buffer, and the loads of the tile after it are
            // issued into the freed registers: a whole tile of matrix work to arrive
            // (past the last tile the stored values are never read).  The staging
            // instructions are spread between the matrix instructions, so they issue while
            // the matrix pipe works.
            read_group(buf, 2, ga[0], gb[0]);
            __builtin_amdgcn_sched_barrier(0);
            store_tile(buf ^ 1);
            load_tile((t + 2) * BK);
            group(ga[1], gb[1]);
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one matrix instruction
                __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // three VALU
                __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // one LDS store
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // one global load
            }
            __builtin_amdgcn_sched_barrier(0);
            // group 2, reading group 3
            read_group(buf, 3, ga[1], gb[1]);
            __builtin_amdgcn_sched_barrier(0);
            group(ga[0], gb[0]);
            __builtin_amdgcn_sched_barrier(0);
            // every wavefront's reads of this tile are issued and the next tile is stored
            __syncthreads();
            // group 3, reading group 0 of the next tile (past the last tile: unused values
            // from inside the buffer)
            read_group(buf ^ 1, 0, ga[0], gb[0]);
            __builtin_amdgcn_sched_barrier(0);
            group(ga[1], gb[1]);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (t == ntf && ntf < nt && sl == nslices - 1) {
            // partial last tile: only the k-steps below K (zero padding is never multiplied in)
            const int kend = K - t * BK;
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                read_group(t & 1, g, ga[1], gb[1]);
#pragma unroll
                for (int s = 0; s < GS; ++s)
                    if (2 * (GS * g + s) < kend)
#pragma unroll
                        for (int i = 0; i < TI; ++i)
#pragma unroll
                            for (int j = 0; j < TJ; ++j)
                                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(ga[1][i][s], gb[1][j][s], acc[i][j],
                                                                                0, 0, 0);
            }
            ++t;
        }
        // the slice is complete: fold it into T in slice order, restart the accumulator
        if (sl == 0) {
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int j = 0; j < TJ; ++j) T[i][j] = acc[i][j];
        } else {
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int j = 0; j < TJ; ++j)
#pragma unroll
                    for (int v = 0; v < 16; ++v) T[i][j][v] = T[i][j][v] + acc[i][j][v];
        }
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    }

    // register v of lane (h, c) holds row 8 (v / 4) + 4 h + (v % 4), column c of each 32 x 32 tile
    if constexpr (ROLE == 2) {
        // gated projection: columns 2i (gate) and 2i + 1 (up) sit in lanes c and c + 1 (c
        // even).  Of the rows of registers v and v + 1 (v even) the even lane finishes the
        // first and the odd lane the second, so each lane evaluates half the
        // H[m][i] = silu(gate) * up, silu(a) = a / (1 + exp_f(-a))
        const int odd = c & 1;
        const int gc = (n0 + wn0 + (c & ~1)) >> 1;          // output column of lane pair, tile 0
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int vp = 0; vp < 16; vp += 2) {
                const int gm = m0 + wm0 + i * 32 + 8 * (vp >> 2) + 4 * h + (vp & 3) + odd;
#pragma unroll
                for (int j = 0; j < TJ; ++j) {
                    const float a0 = T[i][j][vp], a1 = T[i][j][vp + 1];
                    const float x0 = __shfl_xor(a0, 1), x1 = __shfl_xor(a1, 1);
                    const float gate = odd ? x1 : a0;
                    const float up = odd ? a1 : x0;
                    const int gn = n0 + wn0 + j * 32 + (c & ~1);
                    if (interior || (gm < M && gn < N))
                        Y[(int64_t)gm * ldy + gc + j * 16] = (gate / (1.0f + exp_f(-gate))) * up;
                }
            }
        return;
    }
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int gm = m0 + wm0 + i * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
            if (!interior && gm >= M) continue;
            float* yrow = Y + (int64_t)gm * ldy + n0 + wn0 + c;
            const float* rrow = R ? R + (int64_t)gm * ldr + n0 + wn0 + c : nullptr;
#pragma unroll
            for (int j = 0; j < TJ; ++j) {
                if (!interior && n0 + wn0 + j * 32 + c >= N) continue;
                float y = T[i][j][v];
                if (rrow) y = rrow[j * 32] + y;
                yrow[j * 32] = y;
            }
        }
}

// ----------------------------------------------------------------- small --
// 16 < M <= 64: 32 x 32 tiles, one 16 x 16 tile per wavefront on
// v_mfma_f32_16x16x4_f32 (four fused multiply-adds in k order per step; the same measured
// property as the 32x32x2 form, checked through inv_mfma_f32_check), so M = 64, N = 4096
// gives 256 workgroups of 4 wavefronts instead of 64.  K walks the same 32-wide LDS tiles
// and 256-slices with one fold per slice; inside a tile row k sits at (k % 4) * 8 + k / 4,
// so lane group g reads its 8 operands (k = g, g + 4, ..., g + 28) as two 16-byte reads.
// Tile u of a contiguous range per XCD is (row u % nMt, column u / nMt): the tile rows that
// share a weight tile run on one XCD.
__device__ __forceinline__ int kpos16(int k) { return (k & 3) * 8 + (k >> 2); }

template <int ROLE>
__global__ __launch_bounds__(256) void gemm_small_kernel(
    const float* __restrict__ X, int M, int K, int64_t ldx,
    const uint16_t* __restrict__ W, int N, int64_t ldw,
    const float* __restrict__ R, int64_t ldr,
    float* __restrict__ Y, int64_t ldy, const int* __restrict__ Mdev) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    constexpr int TS = 32, LDT = BK + 4;
    __shared__ __attribute__((aligned(16))) float As[2][TS][LDT];
    __shared__ __attribute__((aligned(16))) float Bs[2][TS][LDT];
    const int gridM = M;
    if (Mdev) M = min(M, *Mdev);
    int m0, n0;
    {
        const int nMt = (gridM + TS - 1) / TS, nNt = (N + TS - 1) / TS;
        const int T = nMt * nNt, L = blockIdx.x;
        constexpr int NXCD = 8;
        const int xcd = L % NXCD, q = L / NXCD;
        const int u = xcd * (T / NXCD) + min(xcd, T % NXCD) + q;
        m0 = (u % nMt) * TS;
        n0 = (u / nMt) * TS;
    }
    if (m0 >= M) return;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int g = lane >> 4, r = lane & 15;
    const int wm0 = (wv >> 1) * 16, wn0 = (wv & 1) * 16;
    // staging: thread t carries X row t / 8, k = 4 (t % 8) .. + 3 and, for t < 128, W row
    // t / 4, k = 8 (t % 4) .. + 7; rows past M or N read row M - 1 or N - 1 and k past K reads
    // inside the row: those values only reach outputs that are never stored or k-steps that
    // are never issued
    const int xrow = tid >> 3, xq = tid & 7;
    const int wrw = (tid >> 2) & 31, wo = tid & 3;
    const bool wl = tid < 128;
    const float* xp = X + (int64_t)min(m0 + xrow, M - 1) * ldx + 4 * xq;
    const uint16_t* wp = W + (int64_t)min(n0 + wrw, N - 1) * ldw + 8 * wo;
    float4 xr;
    uint4 wr = make_uint4(0u, 0u, 0u, 0u);
    auto load_tile = [&](int k0) {
        xr = *reinterpret_cast<const float4*>(xp + min(k0, K - 4 - 4 * xq));
        if (wl) wr = *reinterpret_cast<const uint4*>(wp + min(k0, K - 8 - 8 * wo));
    };
    auto store_tile = [&](int buf) {
        float* d = As[buf][xrow];
        d[kpos16(4 * xq + 0)] = xr.x;
        d[kpos16(4 * xq + 1)] = xr.y;
        d[kpos16(4 * xq + 2)] = xr.z;
        d[kpos16(4 * xq + 3)] = xr.w;
        if (wl) {
            float* e = Bs[buf][wrw];
            e[kpos16(8 * wo + 0)] = bf16_lo(wr.x);
            e[kpos16(8 * wo + 1)] = bf16_hi(wr.x);
            e[kpos16(8 * wo + 2)] = bf16_lo(wr.y);
            e[kpos16(8 * wo + 3)] = bf16_hi(wr.y);
            e[kpos16(8 * wo + 4)] = bf16_lo(wr.z);
            e[kpos16(8 * wo + 5)] = bf16_hi(wr.z);
            e[kpos16(8 * wo + 6)] = bf16_lo(wr.w);
            e[kpos16(8 * wo + 7)] = bf16_hi(wr.w);
        }
    };
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f}, T = f32x4{0.f, 0.f, 0.f, 0.f};
    float a[8], b[8];
    auto read_frags = [&](int buf) {
        const float4* sa = reinterpret_cast<const float4*>(&As[buf][wm0 + r][g * 8]);
        const float4* sb = reinterpret_cast<const float4*>(&Bs[buf][wn0 + r][g * 8]);
        const float4 a0 = sa[0], a1 = sa[1], b0 = sb[0], b1 = sb[1];
        a[0] = a0.x; a[1] = a0.y; a[2] = a0.z; a[3] = a0.w; a[4] = a1.x; a[5] = a1.y; a[6] = a1.z; a[7] = a1.w;
        b[0] = b0.x; b[1] = b0.y; b[2] = b0.z; b[3] = b0.w; b[4] = b1.x; b[5] = b1.y; b[6] = b1.z; b[7] = b1.w;
    };
    const int ntf = K / BK, nt = (K + BK - 1) / BK, nslices = (K + KS - 1) / KS;
    load_tile(0);
    store_tile(0);
    __syncthreads();
    int t = 0;
    for (int sl = 0; sl < nslices; ++sl) {
        const int tend = min(ntf, t + KS / BK);
        for (; t < tend; ++t) {
            const int buf = t & 1;
            if (t + 1 < nt) load_tile((t + 1) * BK);
            read_frags(buf);
#pragma unroll
            for (int s = 0; s < BK / 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
            if (t + 1 < nt) store_tile(buf ^ 1);
            __syncthreads();
        }
        if (t == ntf && ntf < nt && sl == nslices - 1) {
            // partial last tile: only the k-steps below K
            const int kend = K - t * BK;
            read_frags(t & 1);
#pragma unroll
            for (int s = 0; s < BK / 4; ++s)
                if (4 * s < kend) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
            ++t;
        }
        if (sl == 0) {
            T = acc;
        } else {
#pragma unroll
            for (int v = 0; v < 4; ++v) T[v] = T[v] + acc[v];
        }
        acc = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // lane (g, r) holds rows 4g .. 4g + 3, column r of the wavefront's 16 x 16 tile
    if constexpr (ROLE == 2) {
        // gated: columns 2i (gate) and 2i + 1 (up) sit in lanes r and r + 1 (r even); the even
        // lane finishes rows 4g and 4g + 2, the odd lane rows 4g + 1 and 4g + 3
        const int odd = r & 1;
        const int gc = (n0 + wn0 + (r & ~1)) >> 1;
#pragma unroll
        for (int vp = 0; vp < 4; vp += 2) {
            const float a0 = T[vp], a1 = T[vp + 1];
            const float x0 = __shfl_xor(a0, 1), x1 = __shfl_xor(a1, 1);
            const float gate = odd ? x1 : a0;
            const float up = odd ? a1 : x0;
            const int gm = m0 + wm0 + 4 * g + vp + odd;
            if (gm < M && n0 + wn0 + (r & ~1) < N) Y[(int64_t)gm * ldy + gc] = (gate / (1.0f + exp_f(-gate))) * up;
        }
        return;
    }
    const int gn = n0 + wn0 + r;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int gm = m0 + wm0 + 4 * g + v;
        if (gm < M && gn < N) {
            float y = T[v];
            if (R) y = R[(int64_t)gm * ldr + gn] + y;
            Y[(int64_t)gm * ldy + gn] = y;
        }
    }
}

// 32 x 32 tiles when the 64 x 64 grid would have fewer than SMALL_BELOW tiles (two per CU;
// one per CU for M <= 64)
constexpr int64_t SMALL_BELOW = 512;

template <int ROLE>
hipError_t launch_small(const GemmArgs& a, hipStream_t st) {
    dim3 grid(((a.M + 31) / 32) * ((a.N + 31) / 32));
    hipLaunchKernelGGL((gemm_small_kernel<ROLE>), grid, dim3(256), 0, st,
                       a.X, a.M, a.K, a.ldx, a.W, a.N, a.ldw, a.R, a.ldr, a.Y, a.ldy, a.Mdev);
    return hipGetLastError();
}

// ------------------------------------------------------------------ gemv16 --
// 5 <= M <= 16 MT: MT tiles of 16 activation rows (rows past M are never stored).  Matrix
// cores (v_mfma_f32_16x16x4_f32, four in-order fused multiply-adds per step) with the
// activation rows as the A operand and 16 weight rows per wavefront as B, so every weight
// element is read from LDS once per use (and serves all MT row tiles) and the activation
// chunk once per wavefront.
// Workgroup: 4 wavefronts = WN along the weight rows x WK = 4 / WN along K: with WK > 1 the
// wavefronts of a round take consecutive slices (round r, wavefront wk: slice r * WK + wk)
// and their slice partials meet in LDS, where one wavefront folds them in ascending slice
// order into the running total -- the same fold as everywhere else.  Each slice walks
// CH-wide chunks staged through LDS (double buffered): the weight tile as BF16 in the order
// lane group g reads it (k = 4 s + g for s = 0..CH/4-1: CH/2 contiguous bytes), the
// activation tile as FP32 in the same order.  Measured: 64-wide chunks are best or equal on
// every decoder shape (128-wide ones halve the workgroups a CU holds at N >= 12288).
// With a grid of several rows (blockIdx.y) each grid row takes its own group of 16 MT
// activation rows: more and lighter workgroups, so a CU holds several and one's staging and
// barriers run under another's matrix work (every output's sum is unchanged).
template <int WN, int PD, int CH, int ROLE, int MT, int NW>
__global__ __launch_bounds__(64 * NW) void gemm_gemv16_kernel(
    const float* __restrict__ X, int M, int K, int64_t ldx,
    const uint16_t* __restrict__ W, int N, int64_t ldw,
    const float* __restrict__ R, int64_t ldr,
    float* __restrict__ Y, int64_t ldy, const int* __restrict__ Mdev) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    constexpr int NT = 64 * NW;                  // threads
    constexpr int WK = NW / WN;
    constexpr int BN = 16 * WN;
    constexpr int NSTEP = CH / 4;                // matrix steps per chunk
    constexpr int WSEG = CH * 2 + 16;            // bytes per (weight row, slice) segment (+ pad)
    constexpr int XSEG = CH + 4;                 // floats per (activation row, slice) segment (+ pad)
    constexpr int WUN = BN * WK * CH / 8 / NT;   // 16-byte weight loads per thread and chunk
    constexpr int MR = 16 * MT;                  // activation rows (MT row tiles of 16)
    constexpr int XU = MR * WK * CH / 4 / NT;    // activation float4 per thread and chunk
    static_assert(BN * WK * CH % (8 * NT) == 0 && MR * WK * CH % (4 * NT) == 0, "tile / thread split");
    __shared__ __attribute__((aligned(16))) unsigned char Wl[2][BN * WK * WSEG];
    __shared__ __attribute__((aligned(16))) float Xl[2][MR * WK * XSEG];
    __shared__ __attribute__((aligned(16))) float part[WK > 1 ? WK * WN * MT * 64 * 4 : 4];
    if (Mdev) M = min(M, *Mdev);
    if (gridDim.y > 1) {
        // row group blockIdx.y: activation rows 16 MT y .. 16 MT y + 16 MT - 1
        const int my = blockIdx.y * 16 * MT;
        X += (int64_t)my * ldx;
        Y += (int64_t)my * ldy;
        if (R) R += (int64_t)my * ldr;
        M = min(M - my, 16 * MT);
    }
    if (M <= 0) return;
    const int n0 = blockIdx.x * BN;
    const int S = (K + KS - 1) / KS;
    const int nrounds = (S + WK - 1) / WK;
    const int nit = nrounds * (KS / CH);
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int g = lane >> 4, r = lane & 15;
    const int wn = wv % WN, wk = wv / WN;

    // Which (slice of the round, row) a staging unit belongs to.  A weight unit is the CH/8
    // lanes that read one CH-wide row segment (16 bytes each, contiguous in memory), an
    // activation unit the CH/4 lanes of one row segment.  The units of one 64-lane store
    // instruction go to rows whose LDS segments start in different banks: rows RSW (weights)
    // or RSX (activations) apart, so the 4-byte scatter stores below are conflict free
    // (64-wide chunks: weight rows 2 x 144 bytes and activation rows 4 x 272 bytes apart; 32-wide:
    // 1 x 80 and 2 x 144).  Any bijection would do: the mapping only decides which thread
    // moves which element.
    static_assert(CH == 64 || CH == 32, "chunk width");
    constexpr int UW = 512 / CH, RSW = 16 / UW;  // weight units per instruction, row step
    constexpr int UX = 256 / CH, RSX = 16 / UX;  // activation units per instruction, row step
    auto wunit = [&](int rest, int& sk, int& rr) {
        sk = rest / BN;
        rr = RSW * (rest % UW) + (rest / UW) % RSW + 16 * ((rest / 16) % WN);
    };
    auto xunit = [&](int rest, int& sk, int& m) {
        sk = rest / MR;
        m = RSX * (rest % UX) + (rest / UX) % RSX + 16 * ((rest / 16) % MT);
    };
    // PD chunks in flight in registers
    uint4 wr[PD][WUN];
    float4 xr[PD][XU];
    // global -> registers for chunk `it` (round it / (KS / CH), chunk it % (KS / CH) of each
    // of its slices).  Every load is issued, unconditionally, from an address clamped into the
    // operand, so the compiler waits for the oldest chunk only (a load under a branch makes it
    // wait for every load in flight).  Units past N, K or M then hold other elements of the
    // operand; none of them reaches a stored output: a weight row past N feeds only its own
    // (unstored) column, an activation row past M only its own (unstored) row, and k past K
    // only matrix steps that are never issued.
    auto load = [&](int it, uint4 (&wq)[WUN], float4 (&xq)[XU]) {
        const int rd = it / (KS / CH), c = it % (KS / CH);
#pragma unroll
        for (int i = 0; i < WUN; ++i) {
            const int q = tid + NT * i;
            const int c8 = q % (CH / 8);
            int sk, rr;
            wunit(q / (CH / 8), sk, rr);
            const int k = (rd * WK + sk) * KS + c * CH + 8 * c8;
            wq[i] = *reinterpret_cast<const uint4*>(W + (int64_t)min(n0 + rr, N - 1) * ldw + min(k, K - 8));
        }
#pragma unroll
        for (int j = 0; j < XU; ++j) {
            const int u = tid + NT * j;
            const int q4 = u % (CH / 4);
            int sk, m;
            xunit(u / (CH / 4), sk, m);
            const int k = (rd * WK + sk) * KS + c * CH + 4 * q4;
            xq[j] = *reinterpret_cast<const float4*>(X + (int64_t)min(m, M - 1) * ldx + min(k, K - 4));
        }
    };
    // registers -> LDS in the read order: element k = 8 c8 + e of a weight chunk goes to
    // lane group g = e % 4, step s = 2 c8 + e / 4; element k = 4 q4 + e of an activation chunk
    // to g = e, s = q4
    auto store = [&](int buf, const uint4 (&wq)[WUN], const float4 (&xq)[XU]) {
#pragma unroll
        for (int i = 0; i < WUN; ++i) {
            const int q = tid + NT * i;
            const int c8 = q % (CH / 8);
            int sk, rr;
            wunit(q / (CH / 8), sk, rr);
            // segments slice-major (sk, row): the 16 rows a lane group reads are WSEG apart,
            // which spreads a 16-lane quarter's 16-byte reads over all 64 banks
            unsigned char* seg = &Wl[buf][(sk * BN + rr) * WSEG + c8 * 4];
            const uint4 v = wq[i];
            *reinterpret_cast<uint32_t*>(seg + 0 * (CH / 2)) = (v.x & 0xffffu) | (v.z << 16);
            *reinterpret_cast<uint32_t*>(seg + 1 * (CH / 2)) = (v.x >> 16) | (v.z & 0xffff0000u);
            *reinterpret_cast<uint32_t*>(seg + 2 * (CH / 2)) = (v.y & 0xffffu) | (v.w << 16);
            *reinterpret_cast<uint32_t*>(seg + 3 * (CH / 2)) = (v.y >> 16) | (v.w & 0xffff0000u);
        }
#pragma unroll
        for (int j = 0; j < XU; ++j) {
            const int u = tid + NT * j;
            const int q4 = u % (CH / 4);
            int sk, m;
            xunit(u / (CH / 4), sk, m);
            float* seg = &Xl[buf][(sk * MR + m) * XSEG + q4];
            seg[0 * NSTEP] = xq[j].x;
            seg[1 * NSTEP] = xq[j].y;
            seg[2 * NSTEP] = xq[j].z;
            seg[3 * NSTEP] = xq[j].w;
        }
    };

    f32x4 acc[MT], T[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) { acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f}; T[mt] = acc[mt]; }
    const unsigned char* wseg0 = &Wl[0][(wk * BN + wn * 16 + r) * WSEG + g * (CH / 2)];
    const float* xseg0 = &Xl[0][(wk * MR + r) * XSEG + g * NSTEP];
    auto compute = [&](int it) {
        const int buf = it & 1;
        const int rd = it / (KS / CH), c = it % (KS / CH);
        const int sl = rd * WK + wk;
        const int kvalid = sl < S ? min(CH, K - (sl * KS + c * CH)) : 0;
        const uint4* wp = reinterpret_cast<const uint4*>(wseg0 + buf * (BN * WK * WSEG));
        const float* xb = xseg0 + buf * (MR * WK * XSEG);
        uint32_t wv8[NSTEP / 2];
        float a[MT][NSTEP];
#pragma unroll
        for (int q = 0; q < NSTEP / 8; ++q) {
            const uint4 w = wp[q];
            wv8[4 * q] = w.x; wv8[4 * q + 1] = w.y; wv8[4 * q + 2] = w.z; wv8[4 * q + 3] = w.w;
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const float4* xp = reinterpret_cast<const float4*>(xb + mt * 16 * XSEG);
#pragma unroll
            for (int q = 0; q < NSTEP / 4; ++q) {
                const float4 x = xp[q];
                a[mt][4 * q] = x.x; a[mt][4 * q + 1] = x.y; a[mt][4 * q + 2] = x.z; a[mt][4 * q + 3] = x.w;
            }
        }
        if (kvalid == CH) {
#pragma unroll
            for (int st = 0; st < NSTEP; ++st) {
                const float b = (st & 1) ? bf16_hi(wv8[st >> 1]) : bf16_lo(wv8[st >> 1]);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[mt][st], b, acc[mt], 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int st = 0; st < NSTEP; ++st) {
                const float b = (st & 1) ? bf16_hi(wv8[st >> 1]) : bf16_lo(wv8[st >> 1]);
                if (4 * st < kvalid) {
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[mt][st], b, acc[mt], 0, 0, 0);
                }
            }
        }
        if (c == KS / CH - 1) {
            // end of a round: every wavefront holds the slice sum of slice rd * WK + wk
            if constexpr (WK == 1) {
                if (sl < S) {
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        if (sl == 0) {
                            T[mt] = acc[mt];
                        } else {
#pragma unroll
                            for (int v = 0; v < 4; ++v) T[mt][v] = T[mt][v] + acc[mt][v];
                        }
                    }
                }
            } else {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    *reinterpret_cast<f32x4*>(&part[(((wk * WN + wn) * MT + mt) * 64 + lane) * 4]) = acc[mt];
                __syncthreads();
                if (wk == 0) {
                    for (int j = 0; j < WK; ++j) {
                        const int sj = rd * WK + j;
                        if (sj >= S) break;
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) {
                            const f32x4 pj = *reinterpret_cast<const f32x4*>(&part[(((j * WN + wn) * MT + mt) * 64 + lane) * 4]);
                            if (sj == 0) {
                                T[mt] = pj;
                            } else {
#pragma unroll
                                for (int v = 0; v < 4; ++v) T[mt][v] = T[mt][v] + pj[v];
                            }
                        }
                    }
                }
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };

    // chunk it sits in register slot it % PD from its load until its store into LDS buffer
    // it % 2; chunk it + PD is requested as soon as slot it % PD has been stored
#pragma unroll
    for (int d = 0; d < PD; ++d)
        if (d < nit) load(d, wr[d], xr[d]);
    store(0, wr[0], xr[0]);
    __syncthreads();
    for (int it0 = 0; it0 < nit; it0 += PD) {
#pragma unroll
        for (int d = 0; d < PD; ++d) {
            const int it = it0 + d;
            if (it < nit) {
                if (it + PD < nit) load(it + PD, wr[d], xr[d]);
                compute(it);
                if (it + 1 < nit) store((it + 1) & 1, wr[(d + 1) % PD], xr[(d + 1) % PD]);
                __syncthreads();
            }
        }
    }
    if (wk != 0) return;
    // lane (g, r) holds rows 4g .. 4g + 3, column r of the wavefront's 16 weight rows
    if constexpr (ROLE == 2) {
        const int odd = r & 1;
        const int gc = (n0 + wn * 16 + (r & ~1)) >> 1;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int vp = 0; vp < 4; vp += 2) {
                const float a0 = T[mt][vp], a1 = T[mt][vp + 1];
                const float x0 = __shfl_xor(a0, 1), x1 = __shfl_xor(a1, 1);
                const float gate = odd ? x1 : a0;
                const float up = odd ? a1 : x0;
                const int gm = 16 * mt + 4 * g + vp + odd;
                if (gm < M && n0 + wn * 16 + (r & ~1) < N) Y[(int64_t)gm * ldy + gc] = (gate / (1.0f + exp_f(-gate))) * up;
            }
        return;
    }
    const int gn = n0 + wn * 16 + r;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int gm = 16 * mt + 4 * g + v;
            if (gm < M && gn < N) {
                float y = T[mt][v];
                if (R) y = R[(int64_t)gm * ldr + gn] + y;
                Y[(int64_t)gm * ldy + gn] = y;
            }
        }
}

// groups > 1: the rows are cut into groups of 16 MT, one grid row (blockIdx.y) per group
template <int WN, int PD, int CH, int ROLE, int MT = 1, int NW = 4>
hipError_t launch_gemv16(const GemmArgs& a, hipStream_t st, int groups = 1) {
    dim3 grid((a.N + 16 * WN - 1) / (16 * WN), groups);
    hipLaunchKernelGGL((gemm_gemv16_kernel<WN, PD, CH, ROLE, MT, NW>), grid, dim3(64 * NW), 0, st,
                       a.X, a.M, a.K, a.ldx, a.W, a.N, a.ldw, a.R, a.ldr, a.Y, a.ldy, a.Mdev);
    return hipGetLastError();
}

// ---------------------------------------------------------------- skinny --
// M <= 4.  A workgroup owns ROWS weight rows (16, or 4 when the grid would otherwise be
// too coarse to balance the CUs) and every activation row; thread (slice lane sl, row nl)
// computes the chain of slice s = group + sl for all M rows, keeping one accumulator per
// activation row.  Slices are processed in groups of 16; within a group the weights stream
// in 4 phases of 64 elements per slice:
//   * load: ROWS rows x 16 slices x 128 bytes, each 128-byte segment read by 8 consecutive
//     lanes (coalesced), into registers DEPTH phases ahead, then into LDS; the activation
//     phase tile X[m][slice][64] is staged the same way and read as a broadcast;
//   * compute: each thread runs its slice chain over the phase's 64 elements in order.
//     The 16 lanes of an LDS pass hold 16 consecutive slices of one weight row: weight
//     segments are 144 bytes apart and activation rows 272 bytes apart, so both 16-byte
//     reads spread over all banks.  Each weight row's 16 segments, and each activation row's
//     16 slices, are followed by two unused ones, so rows sit 32 bytes apart in the bank
//     order: the matrix-instruction form, whose lanes of one pass read four weight rows or
//     four activation rows of two slices, then reads without bank conflicts too (3-5% faster
//     at M = 4, unchanged at M = 1-2).
// After each group the 16 new slice partials of every output are folded, in slice order,
// into that output's running total by the thread that owns it.
constexpr int SK_LANES = 16;  // slices per group
constexpr int PH = 64;        // elements per slice per phase
constexpr int WSEG = PH * 2 + 16;   // padded bytes per (row, slice) segment in LDS
constexpr int XLD = PH + 4;         // padded floats per (m, slice) activation segment
constexpr int RD = 128;             // rotary head dim of the fused QKV projection

// ROLE 3 (QKV projection with RoPE and KV append): weight row of logical output o.  Within
// each rotated (q or k) head the outputs run over the rotate-half pairs, (d = 0, d = 64),
// (1, 65), ..., so a pair's two outputs sit on adjacent folding threads; value rows keep
// their order.
__device__ __forceinline__ int qkv_row(int o, int rot) {
    if (o >= rot) return o;
    const int j = o & (RD - 1), pr = j >> 1;
    return (o & ~(RD - 1)) + ((j & 1) ? pr + RD / 2 : pr);
}

// NRM: the activation rows are RMSNorm inputs.  Before its first phase every workgroup
// computes each row's r = 1 / sqrt(dot_KS(x, x) / K + eps) itself (the rows are staged 16
// slices at a time in LDS, thread s runs slice s's chain x_k * x_k in k order, one thread per
// row folds the slices in order) and the activation tiles are stored into LDS as
// (x_k * r) * up(g_k) -- the arithmetic of rmsnorm_kernel, so the products see the bits the
// separate RMSNorm would have stored, without its launch or its output.  The first weight
// phases are requested before this prologue, so it runs under their latency.
constexpr int NRM_SL = KS + 4;      // padded floats per slice of a staged norm row
template <int MB, int ROLE, int ROWS, int MX = 0, int NRM = 0>
__global__ __launch_bounds__(ROWS * SK_LANES) void gemm_skinny_kernel(
    const float* __restrict__ X, int M, int K, int64_t ldx,
    const uint16_t* __restrict__ W, int N, int64_t ldw,
    const float* __restrict__ R, int64_t ldr,
    float* __restrict__ Y, int64_t ldy, const int* __restrict__ Mdev, RopeArgs ra,
    const uint16_t* __restrict__ G, float eps) {
    constexpr int NT = ROWS * SK_LANES;          // threads
    constexpr int XU = SK_LANES * (PH / 4) / NT; // activation float4 per thread, row and phase
    constexpr int WL_BYTES = ROWS * (SK_LANES + 2) * WSEG;
    constexpr int XL_BYTES = MB * (SK_LANES + 2) * XLD * 4;
    constexpr int NRM_BYTES = NRM ? SK_LANES * NRM_SL * 4 : 0;
    constexpr int SMEM = WL_BYTES + XL_BYTES > NRM_BYTES ? WL_BYTES + XL_BYTES : NRM_BYTES;
    // the weight and activation tiles; the norm prologue's staged row shares their space
    __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
    unsigned char* const Wl = smem;
    float (*const Xl)[SK_LANES + 2][XLD] = reinterpret_cast<float (*)[SK_LANES + 2][XLD]>(smem + WL_BYTES);
    __shared__ float part[SK_LANES][MB][ROWS];
    __shared__ float nrm[NRM ? MB * (SK_LANES + 1) : 1];
    if (Mdev) M = min(M, *Mdev);
    if (M <= 0) return;
    const int S = (K + KS - 1) / KS;
    const int tid = threadIdx.x;
    // MX: the chains run on v_mfma_f32_4x4x1_16b_f32 -- block b of a wavefront is slice
    // group + b, lane 4 b + j supplies weight row 4 w + j (w: wavefront) and activation row j
    // (plus 4 g for the g-th group of four rows), and gets the four rows' accumulators of its
    // weight row.  One instruction is one fma per (row, weight row, slice), the chain's step.
    static_assert(MX == 0 || (MB % 4 == 0 && ROWS % 4 == 0), "matrix GEMV: 4-row groups");
    const int sl = MX ? (tid & 63) >> 2 : tid % SK_LANES;
    const int nl = MX ? ((tid >> 6) << 2) + (tid & 3) : tid / SK_LANES;
    const int n0 = blockIdx.x * ROWS;
    const int rot = ROLE == 3 ? (ra.Hq + ra.Hkv) * RD : 0;     // rotated outputs (ROLE 3)

    // load duty: 8 x 16 bytes of weights and MB * XU x 16 bytes of activations per thread and
    // phase; DEPTH phases are in flight in registers (two when the activation tile is small).
    // The loads read clamped, in-range addresses with no zero fill: what lands past N, M or K
    // reaches no stored output (the chains stop at K, rows past N or M are not written), and
    // with no per-element condition around a load the compiler no longer turns the zero fill
    // into a branch that makes each LDS store wait for every load in flight.  The buffers
    // are native vectors (copies of the struct types were kept in scratch memory), and a
    // scheduling barrier keeps the loads ahead of the phase's compute.
    constexpr int DEPTH = MB * XU <= 4 ? 2 : 1;
    constexpr int GU = NRM ? XU : 1;             // gain pairs per thread and phase (NRM)
    u32x4v wpre[DEPTH][8];
    f32x4v xpre[DEPTH][MB * XU];
    uint2 gpre[DEPTH][GU];
    auto load = [&](int stg, u32x4v (&wp)[8], f32x4v (&xp)[MB * XU], uint2 (&gp)[GU]) {
        const int sg = (stg / (KS / PH)) * SK_LANES;
        const int p = stg % (KS / PH);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int q = tid + NT * i;           // 16-byte unit index in the phase tile
            const int seg = q >> 3, c8 = q & 7;   // segment (row, slice) and chunk in it
            const int rn = seg >> 4, ss = seg & 15;
            const int k = (sg + ss) * KS + p * PH + 8 * c8;
            int wrow = min(n0 + rn, N - 1);
            if constexpr (ROLE == 3) wrow = qkv_row(wrow, rot);
            wp[i] = *reinterpret_cast<const u32x4v*>(W + (int64_t)wrow * ldw + min(k, K - 8));
        }
#pragma unroll
        for (int m = 0; m < MB; ++m) {
#pragma unroll
            for (int j = 0; j < XU; ++j) {
                const int u = tid + NT * j;
                const int ss = u >> 4, c4 = u & 15;          // 16 slices x 16 float4
                const int k = (sg + ss) * KS + p * PH + 4 * c4;
                xp[m * XU + j] = *reinterpret_cast<const f32x4v*>(X + (int64_t)min(m, M - 1) * ldx + min(k, K - 4));
            }
        }
        if constexpr (NRM) {
#pragma unroll
            for (int j = 0; j < XU; ++j) {
                const int u = tid + NT * j;
                const int k = (sg + (u >> 4)) * KS + p * PH + 4 * (u & 15);
                gp[j] = *reinterpret_cast<const uint2*>(G + min(k, K - 4));
            }
        }
    };
    float rn[MB];                                // r of each row (NRM)
    auto store = [&](const u32x4v (&wp)[8], const f32x4v (&xp)[MB * XU], const uint2 (&gp)[GU]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int q = tid + NT * i;
            const int seg = q >> 3, c8 = q & 7;
            *reinterpret_cast<u32x4v*>(&Wl[((seg >> 4) * (SK_LANES + 2) + (seg & 15)) * WSEG + c8 * 16]) = wp[i];
        }
#pragma unroll
        for (int m = 0; m < MB; ++m) {
#pragma unroll
            for (int j = 0; j < XU; ++j) {
                const int u = tid + NT * j;
                f32x4v v = xp[m * XU + j];
                if constexpr (NRM) {
                    const float r = rn[m];
                    v.x = (v.x * r) * bf16_lo(gp[j].x);
                    v.y = (v.y * r) * bf16_hi(gp[j].x);
                    v.z = (v.z * r) * bf16_lo(gp[j].y);
                    v.w = (v.w * r) * bf16_hi(gp[j].y);
                }
                *reinterpret_cast<f32x4v*>(&Xl[m][u >> 4][(u & 15) * 4]) = v;
            }
        }
    };

    const int ngroups = (S + SK_LANES - 1) / SK_LANES;
    const int nstages = ngroups * (KS / PH);
    const bool folder = tid < MB * ROWS;
    const int fm = tid / ROWS, fr = tid % ROWS;   // output folded by this thread
    float T = 0.0f;
    float c[MB];
    constexpr int NG = MX ? MB / 4 : 1;
    f32x4v cm[NG];
    // one phase: its tile is in LDS; every thread advances its slice chain over it
    auto compute = [&](int st) {
        const int sg = (st / (KS / PH)) * SK_LANES;
        const int p = st % (KS / PH);
        if (p == 0) {
#pragma unroll
            for (int m = 0; m < MB; ++m) c[m] = 0.0f;
#pragma unroll
            for (int g = 0; g < NG; ++g) cm[g] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
        }
        const int s = sg + sl;
        const int kb = s * KS + p * PH;                       // first k of this phase
        const int nk = min(PH, K - kb);                       // elements of this phase (<= 0: none)
        const unsigned char* wseg = &Wl[(nl * (SK_LANES + 2) + sl) * WSEG];
        if constexpr (MX != 0) {
            // A lane past its chain's end feeds 0 * 0: the accumulator, never -0 (it starts
            // at +0 and an exact zero sum rounds to +0), is unchanged.
            const int mi = tid & 3;
            const bool full = (sg + SK_LANES - 1) * KS + (p + 1) * PH <= K;
#pragma unroll
            for (int j = 0; j < PH / 8; ++j) {
                const uint4 w8 = *reinterpret_cast<const uint4*>(wseg + 16 * j);
                float w[8] = {bf16_lo(w8.x), bf16_hi(w8.x), bf16_lo(w8.y), bf16_hi(w8.y),
                              bf16_lo(w8.z), bf16_hi(w8.z), bf16_lo(w8.w), bf16_hi(w8.w)};
                float x[NG][8];
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    const float4 xa = *reinterpret_cast<const float4*>(&Xl[4 * g + mi][sl][8 * j]);
                    const float4 xb = *reinterpret_cast<const float4*>(&Xl[4 * g + mi][sl][8 * j + 4]);
                    x[g][0] = xa.x; x[g][1] = xa.y; x[g][2] = xa.z; x[g][3] = xa.w;
                    x[g][4] = xb.x; x[g][5] = xb.y; x[g][6] = xb.z; x[g][7] = xb.w;
                }
                if (!full) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const bool ok = 8 * j + e < nk;
                        w[e] = ok ? w[e] : 0.0f;
#pragma unroll
                        for (int g = 0; g < NG; ++g) x[g][e] = ok ? x[g][e] : 0.0f;
                    }
                }
#pragma unroll
                for (int e = 0; e < 8; ++e)
#pragma unroll
                    for (int g = 0; g < NG; ++g)
                        cm[g] = __builtin_amdgcn_mfma_f32_4x4x1f32(x[g][e], w[e], cm[g], 0, 0, 0);
            }
            if (p == KS / PH - 1) {
#pragma unroll
                for (int g = 0; g < NG; ++g)
#pragma unroll
                    for (int i = 0; i < 4; ++i) c[4 * g + i] = cm[g][i];
            }
        } else if (nk == PH) {
#pragma unroll
            for (int j = 0; j < PH / 8; ++j) {
                const uint4 w8 = *reinterpret_cast<const uint4*>(wseg + 16 * j);
                const float w[8] = {bf16_lo(w8.x), bf16_hi(w8.x), bf16_lo(w8.y), bf16_hi(w8.y),
                                    bf16_lo(w8.z), bf16_hi(w8.z), bf16_lo(w8.w), bf16_hi(w8.w)};
#pragma unroll
                for (int m = 0; m < MB; ++m) {
                    const float4 xa = *reinterpret_cast<const float4*>(&Xl[m][sl][8 * j]);
                    const float4 xb = *reinterpret_cast<const float4*>(&Xl[m][sl][8 * j + 4]);
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
        } else {
            for (int j = 0; j < nk / 8; ++j) {
                const uint4 w8 = *reinterpret_cast<const uint4*>(wseg + 16 * j);
                const float w[8] = {bf16_lo(w8.x), bf16_hi(w8.x), bf16_lo(w8.y), bf16_hi(w8.y),
                                    bf16_lo(w8.z), bf16_hi(w8.z), bf16_lo(w8.w), bf16_hi(w8.w)};
#pragma unroll
                for (int m = 0; m < MB; ++m) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) c[m] = __builtin_fmaf(Xl[m][sl][8 * j + e], w[e], c[m]);
                }
            }
        }
        if (p == KS / PH - 1) {
#pragma unroll
            for (int m = 0; m < MB; ++m) part[sl][m][nl] = c[m];
            __syncthreads();
            if (folder) {
                for (int j = 0; j < SK_LANES; ++j) {
                    const int sj = sg + j;
                    if (sj < S) T = (sj == 0) ? part[j][fm][fr] : T + part[j][fm][fr];
                }
            }
        }
    };
    // the norm's row loads (per thread NU float4 of a 16-slice group, in batches of NB)
    constexpr int NU = SK_LANES * KS / 4 / NT;
    constexpr int NB = NU < 8 ? NU : 8;
    // with 256 threads and one row the first group is requested ahead of the weights (loads
    // complete in order, so behind them it would wait for the whole first weight burst)
    constexpr bool XFIRST = NRM && NU <= 4 && MB == 1;
    f32x4v xv0[XFIRST ? NU : 1];
    if constexpr (XFIRST) {
        const int kn0 = min(SK_LANES * KS, K);
#pragma unroll
        for (int u = 0; u < NU; ++u) xv0[u] = *reinterpret_cast<const f32x4v*>(X + min(4 * (tid + NT * u), kn0 - 4));
    }
    // phase st lives in register buffer st % DEPTH from its load until its store
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
        if (d < nstages) load(d, wpre[d], xpre[d], gpre[d]);
    if constexpr (NRM) {
        // r of each activation row, in the order of rmsnorm_kernel
        float* xs = reinterpret_cast<float*>(smem);
        for (int m = 0; m < M; ++m) {
            const float* x = X + (int64_t)m * ldx;
            float T = 0.0f;                          // thread 0: the row's running fold
            for (int s0 = 0; s0 < S; s0 += SK_LANES) {
                const int k0 = s0 * KS, kn = min(SK_LANES * KS, K - k0);
                __syncthreads();       // the previous group's chains are done with xs
#pragma unroll
                for (int u0 = 0; u0 < NU; u0 += NB) {
                    f32x4v v[NB];
                    if (XFIRST && m == 0 && s0 == 0) {
#pragma unroll
                        for (int u = 0; u < NB; ++u) v[u] = xv0[XFIRST ? u0 + u : 0];
                    } else {
#pragma unroll
                        for (int u = 0; u < NB; ++u)
                            v[u] = *reinterpret_cast<const f32x4v*>(x + k0 + min(4 * (tid + NT * (u0 + u)), kn - 4));
                    }
                    // stores at the clamped index too: a clamped load holds the elements of that
                    // index, so a unit past the row rewrites them with their own values
#pragma unroll
                    for (int u = 0; u < NB; ++u) {
                        const int i = min(4 * (tid + NT * (u0 + u)), kn - 4);
                        *reinterpret_cast<f32x4v*>(&xs[(i / KS) * NRM_SL + i % KS]) = v[u];
                    }
                }
                __syncthreads();
                if (tid < SK_LANES && s0 + tid < S) {
                    const int n = min(KS, K - (s0 + tid) * KS);   // a multiple of 8
                    const float* sx = xs + tid * NRM_SL;
                    float c = 0.0f;
                    // 8 float4 read ahead of the chain's fused multiply-adds
                    for (int kb = 0; kb < n; kb += 32) {
                        f32x4v r4[8];
#pragma unroll
                        for (int u = 0; u < 8; ++u) r4[u] = *reinterpret_cast<const f32x4v*>(sx + min(kb + 4 * u, n - 4));
#pragma unroll
                        for (int u = 0; u < 8; ++u) {
                            if (kb + 4 * u < n) {
                                c = __builtin_fmaf(r4[u].x, r4[u].x, c);
                                c = __builtin_fmaf(r4[u].y, r4[u].y, c);
                                c = __builtin_fmaf(r4[u].z, r4[u].z, c);
                                c = __builtin_fmaf(r4[u].w, r4[u].w, c);
                            }
                        }
                    }
                    nrm[m * (SK_LANES + 1) + tid] = c;
                }
                __syncthreads();
                if (tid == 0) {
                    for (int j = 0; j < SK_LANES && s0 + j < S; ++j) {
                        const float c = nrm[m * (SK_LANES + 1) + j];
                        T = (s0 + j == 0) ? c : T + c;
                    }
                    if (s0 + SK_LANES >= S)
                        nrm[m * (SK_LANES + 1) + SK_LANES] = 1.0f / __builtin_sqrtf((T / (float)K) + eps);
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < MB; ++m) rn[m] = nrm[min(m, M - 1) * (SK_LANES + 1) + SK_LANES];
    }
    for (int st = 0; st < nstages; st += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            if (st + d < nstages) {
                __syncthreads();       // everyone is done with the previous phase's LDS data
                store(wpre[d], xpre[d], gpre[d]);
                __syncthreads();
                if (st + d + DEPTH < nstages) load(st + d + DEPTH, wpre[d], xpre[d], gpre[d]);
                __builtin_amdgcn_sched_barrier(0);
                compute(st + d);
            }
        }
    }
    if constexpr (ROLE == 2) {
        // gated projection: weight rows 2i (gate) and 2i + 1 (up) are folded by threads fr and
        // fr + 1 (adjacent lanes; ROWS is even); the even one writes silu(gate) * up
        const float u = __shfl_down(T, 1);
        if (folder && (fr & 1) == 0) {
            const int gn = n0 + fr;
            if (fm < M && gn < N) Y[(int64_t)fm * ldy + (gn >> 1)] = (T / (1.0f + exp_f(-T))) * u;
        }
    } else if constexpr (ROLE == 3) {
        // RoPE and KV append: a rotate-half pair (x_i, x_{i+64}) sits on threads fr, fr ^ 1;
        // y_i = x_i c - x_{i+64} s and y_{i+64} = x_i s + x_{i+64} c, each product rounded, as
        // the standalone RoPE kernel computes them.  q goes to Qout [M, Hq, 128], rotated k and
        // plain v into the caches at (seq[m], pos[m]); a row outside the cache is skipped.
        const float other = __shfl_xor(T, 1);
        const int o = n0 + fr;
        if (folder && fm < M && o < N) {
            const int p = ra.pos[fm], sq = ra.seq[fm];
            if (p >= 0 && p < ra.Tmax && sq >= 0 && sq < ra.Bcache) {
                const int head = o / RD;
                if (o < rot) {
                    const int j = o & (RD - 1), i = j >> 1, hi = j & 1;
                    const float a = hi ? other : T, b = hi ? T : other;
                    const float cs = ra.cos_t[(int64_t)p * (RD / 2) + i];
                    const float sn = ra.sin_t[(int64_t)p * (RD / 2) + i];
                    const float y = hi ? (a * sn) + (b * cs) : (a * cs) - (b * sn);
                    const int d = hi ? i + RD / 2 : i;
                    if (head < ra.Hq)
                        ra.Qout[((int64_t)fm * ra.Hq + head) * RD + d] = y;
                    else
                        ra.Kc[(((int64_t)sq * ra.Hkv + head - ra.Hq) * ra.Tmax + p) * RD + d] = y;
                } else {
                    const int gv = head - ra.Hq - ra.Hkv, d = o & (RD - 1);
                    ra.Vc[(((int64_t)sq * ra.Hkv + gv) * ra.Tmax + p) * RD + d] = T;
                }
            }
        }
    } else if (folder) {
        const int gn = n0 + fr;
        if (fm < M && gn < N) {
            float y = T;
            if (R) y = R[(int64_t)fm * ldr + gn] + y;
            Y[(int64_t)fm * ldy + gn] = y;
        }
    }
}

template <int BM, int BN, int WGM, int WGN, int ROLE>
hipError_t launch_tiled(const GemmArgs& a, hipStream_t st) {
    dim3 grid(((a.N + BN - 1) / BN) * ((a.M + BM - 1) / BM));
    hipLaunchKernelGGL((gemm_mfma_kernel<BM, BN, WGM, WGN, ROLE>), grid, dim3(64 * WGM * WGN), 0, st,
                       a.X, a.M, a.K, a.ldx, a.W, a.N, a.ldw, a.R, a.ldr, a.Y, a.ldy, a.Mdev);
    return hipGetLastError();
}

template <int MB, int ROLE, int ROWS, int MX = 0>
hipError_t launch_skinny(const GemmArgs& a, hipStream_t st, const RopeArgs& ra = RopeArgs{}) {
    dim3 grid((a.N + ROWS - 1) / ROWS);
    if (a.G) {
        hipLaunchKernelGGL((gemm_skinny_kernel<MB, ROLE, ROWS, MX, 1>), grid, dim3(ROWS * SK_LANES), 0, st,
                           a.X, a.M, a.K, a.ldx, a.W, a.N, a.ldw, a.R, a.ldr, a.Y, a.ldy, a.Mdev, ra, a.G,
                           a.eps);
    } else {
        hipLaunchKernelGGL((gemm_skinny_kernel<MB, ROLE, ROWS, MX>), grid, dim3(ROWS * SK_LANES), 0, st,
                           a.X, a.M, a.K, a.ldx, a.W, a.N, a.ldw, a.R, a.ldr, a.Y, a.ldy, a.Mdev, ra, nullptr,
                           0.0f);
    }
    return hipGetLastError();
}

}  // namespace

// Kernel choice for M rows and N weight rows (launch geometry only: the order of every
// output's sum is the same on every route, which the tests check across M).
//   M <= 4: the slice-parallel GEMV (16-row workgroups, or 4-row ones for N < 16384 and M <= 2
//     so the small projections still spread evenly over the CUs), its chains on the VALU for
//     M <= 2 and on 4x4x1 matrix instructions for M = 3-4 (8-12% faster there, equal bits);
//   5 <= M <= 16: the matrix-core GEMV with one 16-row tile (the VALU GEMV's per-row
//     accumulators and LDS reads make it slower from 5 rows on); weight rows per workgroup:
//     64 from N = 65536 (four wavefronts along the rows, two along K: 4-10% faster on the
//     128256-row vocabulary than one along K), 32 from 12288 (two along the rows, two along K), else 16 with the slices split over four wavefronts, or over eight for
//     N = 2048..4096, where there are only N / 16 workgroups (12-18% faster at N = 4096 for
//     K = 4096 and 14336, slower at N = 6144);
//   17 <= M <= 32: the same with two row tiles (measured faster than the 32 x 32 tiles, or
//     equal, at every decoder shape), except for 4096 < N < 12288, where the rows run as two
//     grid rows of one 16-row tile (N = 6144: 46 -> 35 us at M = 24-32, cold weights);
//   33 <= M <= 64 with N of 1024 to 8192: grid rows of 32 activation rows (two row tiles,
//     32-wide chunks) above 48 rows from N = 3072, else of 16 rows (one tile); one workgroup
//     with four row tiles took 41 us at every N of 1024-4096 and K = 4096 (its chunk loop, not
//     the weight stream, set the time), row groups 35 us at N = 4096 (108 against 134 us at
//     K = 14336) and 17-22 us at N = 1024-2048; at N = 6144 and 8192 they beat the 32 x 32
//     tiles (79 -> 53-59 us, 82 -> 69 us), from N = 14336 the tiles are faster;
//   other M: 32 x 32 tiles while the 64 x 64 grid would have fewer than SMALL_BELOW (512)
//     tiles, two per CU (256 for M <= 64) (M = 128 / 257 at N = 4096: 1.36 / 1.29x faster
//     than 64 x 64, and the same for the down projection; equal or slower from 512 tiles on);
//   M > 64 otherwise: 128 x 256 when that gives at least one workgroup per CU, else 64 x 64
//     (e.g. M = 512, N = 4096: 64 large tiles, 512 small ones, 3x faster).
GemmRoute gemm_route(int64_t M, int64_t N) {
    if (M <= 1) return N < 16 * 1024 ? GR_SKINNY_M1_R4 : GR_SKINNY_M1_R16;
    if (M <= 2) return N < 16 * 1024 ? GR_SKINNY_M2_R4 : GR_SKINNY_M2_R16;
    if (M <= 4) return GR_SKINNY_M4_R16;
    if (M <= 16) {
        if (N >= 65536) return GR_GEMV16_WN4;
        if (N >= 12288) return GR_GEMV16_WN2;
        return (N >= 2048 && N <= 4096) ? GR_GEMV16_WN1_W8 : GR_GEMV16_WN1;
    }
    if (M <= 32) {
        if (N >= 65536) return GR_GEMV32_WN4;
        if (N >= 12288) return GR_GEMV32_WN2;
        return N > 4096 ? GR_GEMV32_G16 : GR_GEMV32_WN1;
    }
    if (M <= 64 && N >= 1024 && N <= 8192) return (M > 48 && N >= 3072) ? GR_GEMV64_G32 : GR_GEMV64_G16;
    const int64_t big = ((M + 127) / 128) * ((N + 255) / 256);
    const int64_t mid = ((M + 63) / 64) * ((N + 63) / 64);
    if (M <= 64) return mid < SMALL_BELOW / 2 ? GR_SMALL32 : GR_TILE64;
    // 64 < M (measured on the decoder's weight shapes, cold weights): 32 x 32 tiles while the
    // 64 x 64 grid has fewer than 256 tiles and N is moderate; the 128 x 256 tile (one workgroup
    // per CU) when its tiles fill whole waves of 256 (the last one at least 90% full) or there
    // are four waves or more; otherwise 64 x 128 tiles of eight wavefronts, or 64 x 64 ones when
    // the 64 x 128 grid has fewer than 192 tiles, or for large N where M is just past a
    // multiple of 64 or between 256 and 512 rows.  (Rows just past a multiple of 64 are
    // usually split off to the skinny GEMV first: gemm_tail_rows.)
    if (mid < SMALL_BELOW / 2 && N <= 8192) return GR_SMALL32;
    if (big >= 4 * 256 || (big >= 230 && (big % 256 == 0 || big % 256 >= 230))) return GR_TILE128x256;
    const int64_t mtail = M % 64;
    const int64_t w8 = ((M + 63) / 64) * ((N + 127) / 128);
    if (w8 < 192 || (N > 8192 && ((mtail > 0 && mtail <= 16) || (M > 256 && M <= 512)))) return GR_TILE64;
    return GR_TILE64x128;
}

const char* gemm_route_name(GemmRoute r) {
    switch (r) {
        case GR_SKINNY_M1_R4: return "gemm_skinny_kernel<1,ROLE,4>";
        case GR_SKINNY_M1_R16: return "gemm_skinny_kernel<1,ROLE,16>";
        case GR_SKINNY_M2_R4: return "gemm_skinny_kernel<2,ROLE,4>";
        case GR_SKINNY_M2_R16: return "gemm_skinny_kernel<2,ROLE,16>";
        case GR_SKINNY_M4_R16: return "gemm_skinny_kernel<4,ROLE,16,1>";
        case GR_GEMV16_WN1: return "gemm_gemv16_kernel<1,2,64,ROLE,1,4>";
        case GR_GEMV16_WN1_W8: return "gemm_gemv16_kernel<1,2,64,ROLE,1,8>";
        case GR_GEMV16_WN2: return "gemm_gemv16_kernel<2,2,64,ROLE,1,4>";
        case GR_GEMV16_WN4: return "gemm_gemv16_kernel<4,2,64,ROLE,1,8>";
        case GR_GEMV32_WN1: return "gemm_gemv16_kernel<1,2,64,ROLE,2,4>";
        case GR_GEMV32_WN2: return "gemm_gemv16_kernel<2,2,64,ROLE,2,4>";
        case GR_GEMV32_WN4: return "gemm_gemv16_kernel<4,2,64,ROLE,2,4>";
        case GR_GEMV32_G16: return "gemm_gemv16_kernel<1,2,64,ROLE,1,4> by 16-row groups";
        case GR_GEMV64_G32: return "gemm_gemv16_kernel<1,2,32,ROLE,2,4> by 32-row groups";
        case GR_GEMV64_G16: return "gemm_gemv16_kernel<1,2,64,ROLE,1,4> by 16-row groups";
        case GR_SMALL32: return "gemm_small_kernel<ROLE>";
        case GR_TILE64: return "gemm_mfma_kernel<64,64,2,2,ROLE>";
        case GR_TILE64x128: return "gemm_mfma_kernel<64,128,2,4,ROLE>";
        case GR_TILE128x256: return "gemm_mfma_kernel<128,256,2,4,ROLE>";
        default: return "unknown";
    }
}

template <int ROLE>
hipError_t launch_role(const GemmArgs& a, hipStream_t st) {
    // M is an upper bound when Mdev is set (rows beyond *Mdev are skipped on the device)
    switch (gemm_route(a.M, a.N)) {
        case GR_SKINNY_M1_R4: return launch_skinny<1, ROLE, 4>(a, st);
        case GR_SKINNY_M1_R16: return launch_skinny<1, ROLE, 16>(a, st);
        case GR_SKINNY_M2_R4: return launch_skinny<2, ROLE, 4>(a, st);
        case GR_SKINNY_M2_R16: return launch_skinny<2, ROLE, 16>(a, st);
        case GR_SKINNY_M4_R16: return launch_skinny<4, ROLE, 16, 1>(a, st);
        case GR_GEMV16_WN1: return launch_gemv16<1, 2, 64, ROLE>(a, st);
        case GR_GEMV16_WN1_W8: return launch_gemv16<1, 2, 64, ROLE, 1, 8>(a, st);
        case GR_GEMV16_WN2: return launch_gemv16<2, 2, 64, ROLE>(a, st);
        case GR_GEMV16_WN4: return launch_gemv16<4, 2, 64, ROLE, 1, 8>(a, st);
        case GR_GEMV32_WN1: return launch_gemv16<1, 2, 64, ROLE, 2>(a, st);
        case GR_GEMV32_WN2: return launch_gemv16<2, 2, 64, ROLE, 2>(a, st);
        case GR_GEMV32_WN4: return launch_gemv16<4, 2, 64, ROLE, 2>(a, st);
        case GR_GEMV32_G16: return launch_gemv16<1, 2, 64, ROLE, 1>(a, st, (int)((a.M + 15) / 16));
        case GR_GEMV64_G32: return launch_gemv16<1, 2, 32, ROLE, 2>(a, st, (int)((a.M + 31) / 32));
        case GR_GEMV64_G16: return launch_gemv16<1, 2, 64, ROLE, 1>(a, st, (int)((a.M + 15) / 16));
        case GR_SMALL32: return launch_small<ROLE>(a, st);
        case GR_TILE64: return launch_tiled<64, 64, 2, 2, ROLE>(a, st);
        case GR_TILE64x128: return launch_tiled<64, 128, 2, 4, ROLE>(a, st);
        case GR_TILE128x256: return launch_tiled<128, 256, 2, 4, ROLE>(a, st);
        default: return hipErrorInvalidValue;
    }
}

bool qkv_rope_fusable(int64_t M, int64_t D) { return M >= 1 && M <= 4 && D == RD; }

bool gemm_norm_fusable(int64_t M) { return M >= 1 && M <= 4; }

// the QKV projection of up to four rows with RoPE and the KV append in the VALU GEMV's epilogue
// (same weight rows per workgroup as the plain projection of these sizes)
hipError_t launch_qkv_rope(const GemmArgs& a, const RopeArgs& ra, hipStream_t st) {
    if (!qkv_rope_fusable(a.M, RD)) return hipErrorInvalidValue;
    switch (gemm_route(a.M, a.N)) {
        case GR_SKINNY_M1_R4: return launch_skinny<1, 3, 4>(a, st, ra);
        case GR_SKINNY_M1_R16: return launch_skinny<1, 3, 16>(a, st, ra);
        case GR_SKINNY_M2_R4: return launch_skinny<2, 3, 4>(a, st, ra);
        case GR_SKINNY_M2_R16: return launch_skinny<2, 3, 16>(a, st, ra);
        case GR_SKINNY_M4_R16: return launch_skinny<4, 3, 16, 1>(a, st, ra);
        default: return hipErrorInvalidValue;
    }
}

// Rows past a multiple of 64 that would leave the last tile row nearly empty: M = 64 q + r
// with r <= 4 and 64 q >= 128 runs as the tiled GEMM on the first 64 q rows and the skinny
// GEMV on the last r (every output's order is per output, so the bits are the same).  Not for
// a device-side row count.
int64_t gemm_tail_rows(int64_t M, const int* Mdev) {
    const int64_t r = M % 64;
    return (!Mdev && M - r >= 128 && r >= 1 && r <= 4) ? r : 0;
}

hipError_t launch_gemm_tiles64(const GemmArgs& a, hipStream_t st, int role) {
    if (role == 2) return launch_tiled<64, 64, 2, 2, 2>(a, st);
    return role == 1 ? launch_tiled<64, 64, 2, 2, 1>(a, st) : launch_tiled<64, 64, 2, 2, 0>(a, st);
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st, int role) {
    // a normalised operand only on the slice-parallel GEMV, whose prologue computes the norm
    if (a.G && (!gemm_norm_fusable(a.M) || gemm_route(a.M, a.N) > GR_SKINNY_M4_R16))
        return hipErrorInvalidValue;
    const int64_t tail = gemm_tail_rows(a.M, a.Mdev);
    if (tail) {
        GemmArgs head = a, rest = a;
        head.M = (int)(a.M - tail);
        rest.M = (int)tail;
        rest.X = a.X + (int64_t)head.M * a.ldx;
        rest.Y = a.Y + (int64_t)head.M * a.ldy;
        if (a.R) rest.R = a.R + (int64_t)head.M * a.ldr;
        hipError_t e = launch_gemm(head, st, role);
        if (e != hipSuccess) return e;
        return launch_gemm(rest, st, role);
    }
    if (role == 2) return launch_role<2>(a, st);
    return role == 1 ? launch_role<1>(a, st) : launch_role<0>(a, st);
}


}  // namespace invnum
