// lmhead.hip -- LM head: logits, log-softmax at the target, top-2 and margin, with
// selective FP32 recompute of the rows whose top-two logit margin is below tau.
//
// Sequence on one stream, no host synchronisation:
//   1. a_P = up(bf(h))                          (BF16 operands of the primary pass)
//   2. z = fixed-order GEMM(a_P, W)             (FP32 sums, dot_KS order)
//   3. row reduce (three kernels spread over rows x vocabulary groups): top-2, M = z_top1,
//      S, lp, margin; outputs with recomputed = (margin < tau)
//   4. compaction: flagged rows' indices (ascending) and a device-side count; their h
//      rows are gathered into a dense buffer
//   5. z = fixed-order GEMM(h_F, W) on the first `count` rows (count read on the device)
//   6. row reduce of those rows; results overwrite the flagged rows' outputs.
// Up to LM_FUSED_MAX_B rows, the FP32 logits of every row are computed by the same GEMM as
// the primary ones (operand rows a_P | h, so the weights stream from memory once), and one
// row reduce runs over all 2B logit rows; its last kernel writes, per row, the primary
// result or, when the primary margin is below tau, the FP32 one.  A GEMM row and a reduced
// row depend on nothing but their own operand row, so these are the same bits as the
// separate pass (steps 4-6 disappear).  With tau <= 0 no row can be flagged (margins are
// >= 0 or NaN), and steps 4-6 are skipped.
//
// Row reduce order (identical for both passes):
//   top1 = lowest index of the maximum; top2 = lowest index != top1 of the maximum of the
//   rest (fp compare, so -0 == +0) -- a total order, so any reduction tree finds them;
//   S: tile u = entries [1024u, 1024u + 1024); lane l sums exp_f(z_v - M) for
//   v = 1024u + 64j + l, j = 0..15 ascending (v < V), from +0; lanes combine pairwise
//   a_l = a_l + a_{l+w}, w = 1, 2, ..., 32; S_u = a_0; S = S_0, S = S + S_u ascending;
//   lp = (z_target - M) - log_f(S).
#include "numerics.h"
#include "kernels.h"

namespace invnum {

namespace {

constexpr int RED_THREADS = 256;   // 4 wavefronts: one per vocabulary tile of a group

struct Top2 {
    float v1; int i1; float v2; int i2;
};

// (value desc, index asc): does (va, ia) come before (vb, ib)?
__device__ __forceinline__ bool before(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

__device__ __forceinline__ void top2_push(Top2& t, float v, int i) {
    if (before(v, i, t.v1, t.i1)) { t.v2 = t.v1; t.i2 = t.i1; t.v1 = v; t.i1 = i; }
    else if (before(v, i, t.v2, t.i2)) { t.v2 = v; t.i2 = i; }
}

__device__ __forceinline__ void top2_merge(Top2& t, const Top2& o) {
    top2_push(t, o.v1, o.i1);
    top2_push(t, o.v2, o.i2);
}

// Row reduction in three kernels, so a few rows still spread over the whole chip:
//   top2_kernel   grid (groups of TOPG tiles, rows): each workgroup's top-2 of its entries,
//                 all requested before the first comparison (order free: a total order on
//                 (value desc, index asc));
//   tiles_kernel  grid (groups of 4 tiles, rows): merges the row's partial top-2 pairs (again
//                 order free) to get M = z_top1, then one wavefront per tile of its group sums
//                 exp_f(z - M) in the pinned lane order and combines the 64 lanes pairwise ->
//                 S_u; the first workgroup of a row stores the merged top-2 for the last kernel;
//   final_kernel  one thread per row: S = S_0, S = S + S_u ascending; lp; margin; flags.
// mode 0: rows 0..gridDim.y-1 as they are (output row = row); mode 1: F pass over the first
// *count rows of the compacted list (output row = idx[row]).
constexpr int GROUP = 4;                 // tiles per workgroup of the tiles kernel
constexpr int LM_FUSED_MAX_B = 32;       // batch sizes whose FP32 logits share the primary GEMM

__device__ __forceinline__ const float* zrow(const float* z, int V, int row) {
    return z + (int64_t)row * V;
}
constexpr int TOPG = 4;                  // tiles per workgroup of the top-2 kernel
constexpr int TOPE = TOPG * TV / RED_THREADS;   // entries per thread of the top-2 kernel

__global__ __launch_bounds__(RED_THREADS) void lmhead_top2_kernel(
    const float* __restrict__ z, int V, int mode, const int32_t* __restrict__ count,
    Top2* __restrict__ part) {
    __shared__ Top2 wtop[RED_THREADS / 64];
    const int u = blockIdx.x, row = blockIdx.y, ntop = gridDim.x;
    if (mode != 0 && row >= *count) return;
    const float* zr = zrow(z, V, row);
    const int tid = threadIdx.x, lane = tid % 64, w = tid / 64;
    float zv[TOPE];
#pragma unroll
    for (int e = 0; e < TOPE; ++e) zv[e] = zr[min(u * TOPG * TV + e * RED_THREADS + tid, V - 1)];
    Top2 t = {-__builtin_inff(), 0x7fffffff, -__builtin_inff(), 0x7fffffff};
#pragma unroll
    for (int e = 0; e < TOPE; ++e) {
        const int v = u * TOPG * TV + e * RED_THREADS + tid;
        if (v < V) top2_push(t, zv[e], v);
    }
    for (int off = 32; off >= 1; off >>= 1) {
        Top2 o;
        o.v1 = __shfl_xor(t.v1, off); o.i1 = __shfl_xor(t.i1, off);
        o.v2 = __shfl_xor(t.v2, off); o.i2 = __shfl_xor(t.i2, off);
        top2_merge(t, o);
    }
    if (lane == 0) wtop[w] = t;
    __syncthreads();
    if (tid == 0) {
        t = wtop[0];
        for (int k = 1; k < RED_THREADS / 64; ++k) top2_merge(t, wtop[k]);
        part[(int64_t)row * ntop + u] = t;
    }
}

// The row's top-2 from its partials, computed by a whole wavefront: each lane merges up to two
// partial pairs per round (both requested before either merge), then the lanes merge in a
// shuffle tree (the merge is order free, so the result is the serial one's); every lane
// returns it.  Values that compare with nothing (NaN logits) leave the sentinel index in
// place; such an index is replaced by the scan's starting choice (top1 = 0, top2 = the lowest
// index != top1), so no index >= V ever reaches a load.
__device__ __forceinline__ Top2 merged_top2_wave(const Top2* __restrict__ part, int row, int ngrp, int V,
                                                 int lane) {
    const Top2* pr = part + (int64_t)row * ngrp;
    Top2 t = {-__builtin_inff(), 0x7fffffff, -__builtin_inff(), 0x7fffffff};
    for (int k = lane; k < ngrp; k += 128) {
        const bool two = k + 64 < ngrp;
        const Top2 q0 = pr[k];
        const Top2 q1 = pr[two ? k + 64 : k];
        top2_merge(t, q0);
        if (two) top2_merge(t, q1);
    }
    for (int off = 32; off >= 1; off >>= 1) {
        Top2 o;
        o.v1 = __shfl_xor(t.v1, off); o.i1 = __shfl_xor(t.i1, off);
        o.v2 = __shfl_xor(t.v2, off); o.i2 = __shfl_xor(t.i2, off);
        top2_merge(t, o);
    }
    if (t.i1 < 0 || t.i1 >= V) t.i1 = 0;
    if (t.i2 < 0 || t.i2 >= V || t.i2 == t.i1) t.i2 = (t.i1 == 0) ? 1 : 0;
    return t;
}

__global__ __launch_bounds__(RED_THREADS) void lmhead_tiles_kernel(
    const float* __restrict__ z, int V, int mode, const int32_t* __restrict__ count,
    const Top2* __restrict__ part, int ntop, Top2* __restrict__ rowtop, float* __restrict__ tileS) {
    const int grp = blockIdx.x, row = blockIdx.y;
    if (mode != 0 && row >= *count) return;
    const float* zr = zrow(z, V, row);
    const int lane = threadIdx.x % 64, w = threadIdx.x / 64;
    const Top2 t = merged_top2_wave(part, row, ntop, V, lane);
    if (grp == 0 && threadIdx.x == 0) rowtop[row] = t;   // the row's top-2 for the final kernels
    const float M = zr[t.i1];
    const int ntiles = (V + TV - 1) / TV;
    const int u = grp * GROUP + w;                       // this wavefront's tile
    if (u >= ntiles) return;
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < TV / LW; ++j) {
        const int v = u * TV + j * LW + lane;
        if (v < V) acc = acc + exp_f(zr[v] - M);
    }
    // pairwise lane tree: a_l + a_{l+w} for w = 1, 2, 4, ..., 32
#pragma unroll
    for (int s = 1; s < LW; s <<= 1) acc = acc + __shfl_down(acc, s);
    if (lane == 0) tileS[(int64_t)row * ntiles + u] = acc;
}

// S = S_0, S = S + S_u for the tiles in ascending order; the tile sums are loaded 16 at a
// time ahead of the adds
__device__ __forceinline__ float fold_tiles(const float* __restrict__ ts, int ntiles) {
    float S = ts[0];
    int u = 1;
    for (; u + 16 <= ntiles; u += 16) {
        float q[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) q[e] = ts[u + e];
#pragma unroll
        for (int e = 0; e < 16; ++e) S = S + q[e];
    }
    for (; u < ntiles; ++u) S = S + ts[u];
    return S;
}

struct RowOut {
    float lp, mg; int t1, t2;
};

// lp, margin and the top-2 of reduced row `row` (its logits, top-2 and tile sums)
__device__ __forceinline__ RowOut row_result(const float* __restrict__ z, int V, int row, int tg,
                                             const Top2* __restrict__ rowtop,
                                             const float* __restrict__ tileS) {
    const float* zr = zrow(z, V, row);
    const Top2 t = rowtop[row];
    const float M = zr[t.i1];
    const int ntiles = (V + TV - 1) / TV;
    const float S = fold_tiles(tileS + (int64_t)row * ntiles, ntiles);
    RowOut r;
    r.lp = (tg >= 0 && tg < V) ? (zr[tg] - M) - log_f(S) : __builtin_nanf("");
    r.mg = M - zr[t.i2];
    r.t1 = t.i1;
    r.t2 = t.i2;
    return r;
}

// mode 0: output row = reduced row, flag = (margin < tau); mode 1: reduced row `row` is the F
// pass of compacted row idx[row] (flag 1)
__global__ void lmhead_final_kernel(
    const float* __restrict__ z, int V, int B, const int32_t* __restrict__ target, float tau, int mode,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ count,
    const Top2* __restrict__ rowtop, const float* __restrict__ tileS,
    float* __restrict__ logprob, float* __restrict__ margin, int32_t* __restrict__ top1,
    int32_t* __restrict__ top2, uint8_t* __restrict__ recomputed) {
    const int row = blockIdx.x * blockDim.x + threadIdx.x;
    if (row >= B) return;
    if (mode != 0 && row >= *count) return;
    const int orow = mode != 0 ? idx[row] : row;
    const RowOut r = row_result(z, V, row, target[orow], rowtop, tileS);
    logprob[orow] = r.lp;
    margin[orow] = r.mg;
    top1[orow] = r.t1;
    top2[orow] = r.t2;
    recomputed[orow] = (uint8_t)(mode != 0 ? 1 : (r.mg < tau ? 1 : 0));
}

// Rows 0..B-1 are the primary pass and rows B..2B-1 the FP32 pass of the same hidden states:
// output row b takes the FP32 result when the primary margin is below tau (strict; NaN never).
// One workgroup of two wavefronts per output row: wavefront 0 finishes row b, wavefront 1 row
// B + b.  Each stages its row's tile sums in LDS (all requested at once) and lets one lane fold
// them in ascending order.
constexpr int SEL_MAXT = 1024;           // tiles per row held in LDS (V <= 1024 tiles)

__global__ __launch_bounds__(128) void lmhead_final_select_kernel(
    const float* __restrict__ z, int V, int B, const int32_t* __restrict__ target, float tau,
    const Top2* __restrict__ rowtop, const float* __restrict__ tileS,
    float* __restrict__ logprob, float* __restrict__ margin, int32_t* __restrict__ top1,
    int32_t* __restrict__ top2, uint8_t* __restrict__ recomputed) {
    __shared__ __attribute__((aligned(16))) float ts[2][SEL_MAXT];
    __shared__ RowOut res[2];
    const int b = blockIdx.x, w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row = w == 0 ? b : B + b;
    const int tg = target[b];
    const int ntiles = (V + TV - 1) / TV;
    const float* tr = tileS + (int64_t)row * ntiles;
    for (int u = lane; u < ntiles; u += 64) ts[w][u] = tr[u];
    for (int u = ntiles + lane; u < ((ntiles + 3) & ~3); u += 64) ts[w][u] = 0.0f;   // last float4's padding
    __syncthreads();
    if (lane == 0) {
        const Top2 t = rowtop[row];
        const float* zr = zrow(z, V, row);
        const float M = zr[t.i1];
        const float z2 = zr[t.i2];
        const float zt = (tg >= 0 && tg < V) ? zr[tg] : 0.0f;
        float S = ts[w][0];
        int u = 1;
        for (; u < 4 && u < ntiles; ++u) S = S + ts[w][u];
        for (; u + 4 <= ntiles; u += 4) {
            const float4 q = *reinterpret_cast<const float4*>(&ts[w][u]);
            S = S + q.x; S = S + q.y; S = S + q.z; S = S + q.w;
        }
        for (; u < ntiles; ++u) S = S + ts[w][u];
        RowOut r;
        r.lp = (tg >= 0 && tg < V) ? (zt - M) - log_f(S) : __builtin_nanf("");
        r.mg = M - z2;
        r.t1 = t.i1;
        r.t2 = t.i2;
        res[w] = r;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const bool flag = res[0].mg < tau;
        const RowOut r = flag ? res[1] : res[0];
        logprob[b] = r.lp;
        margin[b] = r.mg;
        top1[b] = r.t1;
        top2[b] = r.t2;
        recomputed[b] = (uint8_t)(flag ? 1 : 0);
    }
}

// Logit gradient, step 1: per row M = z_top1 and S (the forward's fold), and the logprob.
__global__ void lmhead_rowstats_kernel(const float* __restrict__ z, int V, int B, const int32_t* __restrict__ target,
                                       const Top2* __restrict__ rowtop, const float* __restrict__ tileS,
                                       float* __restrict__ stats, float* __restrict__ logprob) {
    const int row = blockIdx.x * blockDim.x + threadIdx.x;
    if (row >= B) return;
    const float* zr = z + (int64_t)row * V;
    const Top2 t = rowtop[row];
    const float M = zr[t.i1];
    const int ntiles = (V + TV - 1) / TV;
    const float S = fold_tiles(tileS + (int64_t)row * ntiles, ntiles);
    stats[2 * row] = M;
    stats[2 * row + 1] = S;
    if (logprob) {
        const int tg = target[row];
        logprob[row] = (tg >= 0 && tg < V) ? (zr[tg] - M) - log_f(S) : __builtin_nanf("");
    }
}

// Logit gradient, step 2, in place over the logits: p = exp_f(z - M) / S (one rounded
// division), g = coef * ([v == target] - p).
__global__ void logit_grad_kernel(float* __restrict__ G, int V, const int32_t* __restrict__ target,
                                  const float* __restrict__ coef, const float* __restrict__ stats) {
    const int row = blockIdx.y;
    const float M = stats[2 * row], S = stats[2 * row + 1], c = coef[row];
    const int tg = target[row];
    float* gr = G + (int64_t)row * V;
    for (int v = blockIdx.x * blockDim.x + threadIdx.x; v < V; v += gridDim.x * blockDim.x) {
        const float p = exp_f(gr[v] - M) / S;
        const float q = (v == tg ? 1.0f : 0.0f) - p;
        gr[v] = c * q;
    }
}

// a_P[b, k] = up(bf(h[b, k])); with `both`, also A[B + b, k] = h[b, k] (the FP32 operands)
__global__ void round_bf16_kernel(const float* __restrict__ H, int B, int K, int64_t ldh, int both,
                                  float* __restrict__ A) {
    const int64_t n4 = (int64_t)B * (K / 4);
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int b = (int)(i / (K / 4)), k = (int)(i % (K / 4)) * 4;
        const float4 v = *reinterpret_cast<const float4*>(H + (int64_t)b * ldh + k);
        float4 o;
        o.x = bf16_up(bf16_rne(v.x)); o.y = bf16_up(bf16_rne(v.y));
        o.z = bf16_up(bf16_rne(v.z)); o.w = bf16_up(bf16_rne(v.w));
        *reinterpret_cast<float4*>(A + (int64_t)b * K + k) = o;
        if (both) *reinterpret_cast<float4*>(A + (int64_t)(B + b) * K + k) = v;
    }
}

// Rows of the FP32 pass given to a GEMV of their own when the batch is small (see launch_lmhead).
constexpr int LM_FHEAD = 32;
constexpr int LM_FHEAD_MAX_B = 512;

// Single workgroup: ascending list of rows flagged by the P pass, and their count; count[1] is
// the count past the first LM_FHEAD rows (0 when there are no more).
// Every thread keeps its own copy of the running base; the per-wavefront counts are
// rewritten by each wavefront in every round, between two barriers.
__global__ __launch_bounds__(1024) void compact_kernel(const uint8_t* __restrict__ flag, int B,
                                                       int32_t* __restrict__ idx,
                                                       int32_t* __restrict__ count) {
    __shared__ int32_t wsum[16];
    const int tid = threadIdx.x, lane = tid % 64, w = tid / 64;
    int base = 0;
    for (int b0 = 0; b0 < B; b0 += 1024) {
        const int b = b0 + tid;
        const int f = (b < B && flag[b]) ? 1 : 0;
        const unsigned long long bal = __ballot(f);
        const int before_me = __popcll(bal & ((1ull << lane) - 1ull));
        if (lane == 0) wsum[w] = __popcll(bal);
        __syncthreads();
        int off = base, tot = 0;
        for (int k = 0; k < 16; ++k) {
            if (k < w) off += wsum[k];
            tot += wsum[k];
        }
        if (f) idx[off + before_me] = b;
        base += tot;
        __syncthreads();
    }
    if (tid == 0) {
        count[0] = base;
        count[1] = base > LM_FHEAD ? base - LM_FHEAD : 0;
    }
}

// Gather the flagged rows of h (fp32) into a dense [count, K] buffer.
__global__ void gather_rows_kernel(const float* __restrict__ H, int K, int64_t ldh,
                                   const int32_t* __restrict__ idx, const int32_t* __restrict__ count,
                                   float* __restrict__ A) {
    const int r = blockIdx.x;
    if (r >= *count) return;
    const float* src = H + (int64_t)idx[r] * ldh;
    float* dst = A + (int64_t)r * K;
    for (int k = threadIdx.x * 4; k < K; k += blockDim.x * 4)
        *reinterpret_cast<float4*>(dst + k) = *reinterpret_cast<const float4*>(src + k);
}

inline size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
    size_t a, z, idx, count, part, rowtop, tiles, total;
};
WsLayout ws_layout(int64_t B, int64_t K, int64_t V) {
    WsLayout L;
    const int64_t ntiles = (V + TV - 1) / TV;
    const int64_t zrows = B <= LM_FUSED_MAX_B ? 2 * B : B;     // P rows, then F rows when fused
    size_t off = 0;
    L.a = off; off = align_up(off + sizeof(float) * (size_t)zrows * K);
    L.z = off; off = align_up(off + sizeof(float) * (size_t)zrows * V);
    L.idx = off; off = align_up(off + sizeof(int32_t) * (size_t)B);
    L.count = off; off = align_up(off + 2 * sizeof(int32_t));   // the count, and the count past LM_FHEAD
    L.part = off; off = align_up(off + sizeof(Top2) * (size_t)zrows * ((ntiles + TOPG - 1) / TOPG));
    L.rowtop = off; off = align_up(off + sizeof(Top2) * (size_t)zrows);
    L.tiles = off; off = align_up(off + sizeof(float) * (size_t)zrows * ntiles);
    L.total = off;
    return L;
}

// top-2 partials and tile sums of `rows` logit rows (mode 0: all of them; mode 1: the first
// *count, the compacted F rows)
hipError_t launch_row_stats(const float* Z, int V, int rows, int mode, const int32_t* count, Top2* part, Top2* rowtop,
                            float* tiles, hipStream_t st) {
    const int ntiles = (V + TV - 1) / TV;
    const int ntop = (ntiles + TOPG - 1) / TOPG;
    hipLaunchKernelGGL(lmhead_top2_kernel, dim3(ntop, rows), dim3(RED_THREADS), 0, st, Z, V, mode, count, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lmhead_tiles_kernel, dim3((ntiles + GROUP - 1) / GROUP, rows), dim3(RED_THREADS), 0, st, Z,
                       V, mode, count, part, ntop, rowtop, tiles);
    return hipGetLastError();
}

hipError_t launch_reduce(const LmheadArgs& a, int mode, const float* Z, const int32_t* idx,
                         const int32_t* count, Top2* part, Top2* rowtop, float* tiles, hipStream_t st) {
    hipError_t e = launch_row_stats(Z, a.V, a.B, mode, count, part, rowtop, tiles, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lmhead_final_kernel, dim3((a.B + 63) / 64), dim3(64), 0, st, Z, a.V, a.B, a.target,
                       a.tau, mode, idx, count, rowtop, tiles, a.logprob, a.margin, a.top1, a.top2,
                       a.recomputed);
    return hipGetLastError();
}

struct GradWs {
    size_t part, rowtop, tiles, stats, total;
};
GradWs grad_ws_layout(int64_t B, int64_t V) {
    GradWs L;
    const int64_t ntiles = (V + TV - 1) / TV;
    size_t off = 0;
    L.part = off; off = align_up(off + sizeof(Top2) * (size_t)B * ((ntiles + TOPG - 1) / TOPG));
    L.rowtop = off; off = align_up(off + sizeof(Top2) * (size_t)B);
    L.tiles = off; off = align_up(off + sizeof(float) * (size_t)B * ntiles);
    L.stats = off; off = align_up(off + sizeof(float) * 2 * (size_t)B);
    L.total = off;
    return L;
}

}  // namespace

size_t lmhead_ws_bytes(int64_t B, int64_t K, int64_t V) { return ws_layout(B, K, V).total; }

int64_t lmhead_projection_rows(int64_t B, float tau) {
    return (tau > 0.0f && B <= LM_FUSED_MAX_B) ? 2 * B : B;
}

size_t logit_grad_ws_bytes(int64_t B, int64_t V) { return grad_ws_layout(B, V).total; }

// Logit gradient of coef * lp on the FP32 pass: logits into G (the vocabulary GEMM on h
// itself), the forward's row reductions (mode 0 of the top-2 and tile kernels), row
// statistics, then the gradient in place.
hipError_t launch_logit_grad(const LogitGradArgs& a, hipStream_t st) {
    const GradWs L = grad_ws_layout(a.B, a.V);
    char* ws = reinterpret_cast<char*>(a.ws);
    Top2* part = reinterpret_cast<Top2*>(ws + L.part);
    Top2* rowtop = reinterpret_cast<Top2*>(ws + L.rowtop);
    float* tiles = reinterpret_cast<float*>(ws + L.tiles);
    float* stats = reinterpret_cast<float*>(ws + L.stats);
    hipError_t e;
    GemmArgs ga{a.Hs, a.B, a.K, a.ldh, a.W, a.V, (int64_t)a.K, nullptr, 0, a.G, (int64_t)a.V, nullptr};
    if ((e = launch_gemm(ga, st, 1)) != hipSuccess) return e;
    if ((e = launch_row_stats(a.G, a.V, a.B, 0, nullptr, part, rowtop, tiles, st)) != hipSuccess) return e;
    hipLaunchKernelGGL(lmhead_rowstats_kernel, dim3((a.B + 63) / 64), dim3(64), 0, st, a.G, a.V, a.B, a.target,
                       rowtop, tiles, stats, a.logprob);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int gx = (a.V + 1023) / 1024;
    hipLaunchKernelGGL(logit_grad_kernel, dim3(gx < 64 ? gx : 64, a.B), dim3(256), 0, st, a.G, a.V, a.target, a.coef,
                       stats);
    return hipGetLastError();
}

hipError_t launch_lmhead(const LmheadArgs& a, hipStream_t st) {
    const WsLayout L = ws_layout(a.B, a.K, a.V);
    char* ws = reinterpret_cast<char*>(a.ws);
    float* A = reinterpret_cast<float*>(ws + L.a);
    float* Z = reinterpret_cast<float*>(ws + L.z);
    int32_t* idx = reinterpret_cast<int32_t*>(ws + L.idx);
    int32_t* count = reinterpret_cast<int32_t*>(ws + L.count);
    Top2* part = reinterpret_cast<Top2*>(ws + L.part);
    Top2* rowtop = reinterpret_cast<Top2*>(ws + L.rowtop);
    float* tiles = reinterpret_cast<float*>(ws + L.tiles);
    hipError_t e;

    // margins are >= 0 (or NaN), so tau <= 0 (or NaN) flags no row: no recompute machinery
    const bool recompute = a.tau > 0.0f;
    const bool fused = recompute && a.B <= LM_FUSED_MAX_B;
    int64_t n4 = (int64_t)a.B * (a.K / 4);
    int g = (int)((n4 + 255) / 256);
    if (g > 65536) g = 65536;
    hipLaunchKernelGGL(round_bf16_kernel, dim3(g), dim3(256), 0, st, a.Hs, a.B, a.K, a.ldh, fused ? 1 : 0, A);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    const int rows = fused ? 2 * a.B : a.B;
    GemmArgs ga{A, rows, a.K, (int64_t)a.K, a.W, a.V, (int64_t)a.K, nullptr, 0, Z, (int64_t)a.V, nullptr};
    if ((e = launch_gemm(ga, st, 1)) != hipSuccess) return e;

    if (fused) {
        // both passes' rows in one reduce; the last kernel picks each row's pass
        if ((e = launch_row_stats(Z, a.V, 2 * a.B, 0, nullptr, part, rowtop, tiles, st)) != hipSuccess) return e;
        hipLaunchKernelGGL(lmhead_final_select_kernel, dim3(a.B), dim3(128), 0, st, Z, a.V, a.B,
                           a.target, a.tau, rowtop, tiles, a.logprob, a.margin, a.top1, a.top2,
                           a.recomputed);
        return hipGetLastError();
    }
    if ((e = launch_reduce(a, 0, Z, nullptr, nullptr, part, rowtop, tiles, st)) != hipSuccess) return e;
    if (!recompute) return hipSuccess;

    hipLaunchKernelGGL(compact_kernel, dim3(1), dim3(1024), 0, st, a.recomputed, a.B, idx, count);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(gather_rows_kernel, dim3(a.B), dim3(256), 0, st, a.Hs, a.K, a.ldh, idx, count, A);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    // The FP32 pass runs over the `count` compacted rows, a number known on the device only, so
    // its launch covers B rows and the rows past the count exit.  A tile row with any live row
    // runs whole, and with the usual handful of flagged rows in a batch of 33-512 that is the
    // first tile row of a full-size GEMM (128 rows from B = 128 on).  So the first LM_FHEAD rows
    // go to the GEMV of their own size, and the rest (count - LM_FHEAD live rows, count[1]) to
    // 64 x 64 tiles, which exit at once when no row is left.  With tau = +inf every row is
    // flagged and the pass runs as one GEMM of B rows.  Every row's sums are the same on every
    // route.
    if (a.B > LM_FHEAD && a.B <= LM_FHEAD_MAX_B && a.tau != __builtin_inff()) {
        GemmArgs gh{A, LM_FHEAD, a.K, (int64_t)a.K, a.W, a.V, (int64_t)a.K, nullptr, 0, Z, (int64_t)a.V, count};
        if ((e = launch_gemm(gh, st, 1)) != hipSuccess) return e;
        GemmArgs gr{A + (int64_t)LM_FHEAD * a.K, a.B - LM_FHEAD, a.K, (int64_t)a.K, a.W, a.V, (int64_t)a.K,
                    nullptr, 0, Z + (int64_t)LM_FHEAD * a.V, (int64_t)a.V, count + 1};
        if ((e = launch_gemm_tiles64(gr, st, 1)) != hipSuccess) return e;
    } else {
        GemmArgs gf{A, a.B, a.K, (int64_t)a.K, a.W, a.V, (int64_t)a.K, nullptr, 0, Z, (int64_t)a.V, count};
        if ((e = launch_gemm(gf, st, 1)) != hipSuccess) return e;
    }

    return launch_reduce(a, 1, Z, idx, count, part, rowtop, tiles, st);
}

}  // namespace invnum
