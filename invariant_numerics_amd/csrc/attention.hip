// attention.hip -- causal attention with fixed KV chunks and one merge order shared by
// prefill and decode.
//
// Per query row (b, h, i), keys of kv head g = h / (Hq / Hkv):
//   s_j = dot_KS(q, k_j, 128) * scale                (one sequential fma chain over d)
//   chunks c = 0 .. floor(i / 256), keys [256c, min(256c + 255, i)]; keys after i are never
//   visited; per chunk m_c = max s_j; p_j = exp_f(s_j - m_c); l_c = l_c + p_j and
//   o_c[d] = fma(p_j, v_j[d], o_c[d]) for j ascending, from +0;
//   merge left to right starting from chunk 0: m' = max(m, m_c), a = exp_f(m - m'),
//   b = exp_f(m_c - m'), l = l*a + l_c*b, o = o*a + o_c*b (no fma), m = m';
//   out = o / l.
// Prefill folds chunk c into the running state as soon as it is computed; decode computes
// all chunk partials in parallel (one workgroup per chunk) and folds them in a second
// kernel in the same ascending order, so both produce the same bits for the same row.
#include "numerics.h"
#include "kernels.h"

namespace invnum {

namespace {

constexpr int D = 128;
constexpr int BQ = 64;    // query rows per prefill workgroup
constexpr int SUB = 32;   // keys staged per LDS sub-block
constexpr int SPAD = 4;

template <int DT>
__device__ __forceinline__ void load_row4(const void* base, int64_t off, float* dst) {
    // 4 consecutive elements at element offset `off` (multiple of 4) -> fp32
    if (DT == 1) {
        const float4 v = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + off);
        dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
    } else {
        const uint2 v = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + off);
        dst[0] = bf16_lo(v.x); dst[1] = bf16_hi(v.x); dst[2] = bf16_lo(v.y); dst[3] = bf16_hi(v.y);
    }
}

// ------------------------------------------------------------------ prefill --
// Workgroup: 256 threads, BQ = 64 query rows of one (b, h).  Thread t works on row t / 4:
// for scores it owns keys (t % 4) * 8 .. +8 of each 32-key sub-block, for the PV sum it
// owns head dims (t % 4) * 32 .. +32.
template <int DT>
__global__ __launch_bounds__(256) void attn_prefill_kernel(
    const void* __restrict__ Q, const void* __restrict__ Kc, const void* __restrict__ Vc,
    int Tq, int q_start, int Tmax, int Hq, int Hkv, float scale, float* __restrict__ O) {
    __shared__ float Qs[BQ][D + SPAD];
    __shared__ float KVs[SUB][D + SPAD];
    __shared__ float Ss[BQ][CHUNK + SPAD];

    const int tid = threadIdx.x;
    const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int g = h / (Hq / Hkv);
    const int r0 = qb * BQ;
    const int nrows = min(BQ, Tq - r0);
    const int imax = q_start + r0 + nrows - 1;          // last absolute query position
    const int64_t kvbase = ((int64_t)b * Hkv + g) * Tmax * D;

    // stage the query rows
    for (int e = tid; e < BQ * (D / 4); e += 256) {
        const int r = e / (D / 4), d4 = (e % (D / 4)) * 4;
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        if (r < nrows) load_row4<DT>(Q, (((int64_t)b * Tq + r0 + r) * Hq + h) * D + d4, v);
        Qs[r][d4 + 0] = v[0]; Qs[r][d4 + 1] = v[1]; Qs[r][d4 + 2] = v[2]; Qs[r][d4 + 3] = v[3];
    }

    const int r = tid / 4;            // this thread's row
    const int q4 = tid % 4;
    const int i = q_start + r0 + r;   // its absolute position
    const bool rvalid = r < nrows;
    float o[32], oc[32];
    float m = 0.0f, l = 0.0f;
#pragma unroll
    for (int u = 0; u < 32; ++u) o[u] = 0.0f;

    const int clast = imax / CHUNK;
    for (int c = 0; c <= clast; ++c) {
        const int kbase = c * CHUNK;
        const int kend = min(kbase + CHUNK, imax + 1);   // keys needed by some row
        // ---- scores for this chunk
        for (int kb = kbase; kb < kend; kb += SUB) {
            __syncthreads();
            for (int e = tid; e < SUB * (D / 4); e += 256) {
                const int jj = e / (D / 4), d4 = (e % (D / 4)) * 4;
                float v[4] = {0.f, 0.f, 0.f, 0.f};
                if (kb + jj < kend) load_row4<DT>(Kc, kvbase + (int64_t)(kb + jj) * D + d4, v);
                KVs[jj][d4 + 0] = v[0]; KVs[jj][d4 + 1] = v[1];
                KVs[jj][d4 + 2] = v[2]; KVs[jj][d4 + 3] = v[3];
            }
            __syncthreads();
            float acc[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) acc[u] = 0.0f;
            for (int d = 0; d < D; d += 4) {
                const float4 qv = *reinterpret_cast<const float4*>(&Qs[r][d]);
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const float4 kv = *reinterpret_cast<const float4*>(&KVs[q4 * 8 + u][d]);
                    acc[u] = __builtin_fmaf(qv.x, kv.x, acc[u]);
                    acc[u] = __builtin_fmaf(qv.y, kv.y, acc[u]);
                    acc[u] = __builtin_fmaf(qv.z, kv.z, acc[u]);
                    acc[u] = __builtin_fmaf(qv.w, kv.w, acc[u]);
                }
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) Ss[r][kb - kbase + q4 * 8 + u] = acc[u] * scale;
        }
        __syncthreads();
        // ---- chunk max and probabilities for this row (4 threads per row)
        const int jlast = min(kbase + CHUNK - 1, i);     // last key of this chunk for row i
        const bool nonempty = rvalid && jlast >= kbase;
        float mc = -__builtin_inff();
        if (nonempty) {
            for (int j = kbase + q4; j <= jlast; j += 4) {
                const float s = Ss[r][j - kbase];
                mc = (s > mc) ? s : mc;
            }
        }
        // combine the 4 partial maxima of the row (lanes 4r..4r+3 of the wavefront)
        {
            float o1 = __shfl_xor(mc, 1);
            mc = (o1 > mc) ? o1 : mc;
            float o2 = __shfl_xor(mc, 2);
            mc = (o2 > mc) ? o2 : mc;
        }
        __syncthreads();
        if (nonempty) {
            for (int j = kbase + q4; j <= jlast; j += 4) {
                const float s = Ss[r][j - kbase];
                Ss[r][j - kbase] = exp_f(s - mc);
            }
        }
        // ---- PV and l_c, j ascending; this thread owns dims q4*32 .. +32
        float lc = 0.0f;
#pragma unroll
        for (int u = 0; u < 32; ++u) oc[u] = 0.0f;
        for (int kb = kbase; kb < kend; kb += SUB) {
            __syncthreads();
            for (int e = tid; e < SUB * (D / 4); e += 256) {
                const int jj = e / (D / 4), d4 = (e % (D / 4)) * 4;
                float v[4] = {0.f, 0.f, 0.f, 0.f};
                if (kb + jj < kend) load_row4<DT>(Vc, kvbase + (int64_t)(kb + jj) * D + d4, v);
                KVs[jj][d4 + 0] = v[0]; KVs[jj][d4 + 1] = v[1];
                KVs[jj][d4 + 2] = v[2]; KVs[jj][d4 + 3] = v[3];
            }
            __syncthreads();
            if (nonempty) {
                const int jstop = min(kb + SUB - 1, jlast);
                for (int j = kb; j <= jstop; ++j) {
                    const float p = Ss[r][j - kbase];
                    lc = lc + p;
                    const float* vr = &KVs[j - kb][q4 * 32];
#pragma unroll
                    for (int u = 0; u < 32; u += 4) {
                        const float4 vv = *reinterpret_cast<const float4*>(vr + u);
                        oc[u + 0] = __builtin_fmaf(p, vv.x, oc[u + 0]);
                        oc[u + 1] = __builtin_fmaf(p, vv.y, oc[u + 1]);
                        oc[u + 2] = __builtin_fmaf(p, vv.z, oc[u + 2]);
                        oc[u + 3] = __builtin_fmaf(p, vv.w, oc[u + 3]);
                    }
                }
            }
        }
        // ---- merge into the running state
        if (nonempty) {
            if (c == 0) {
                m = mc; l = lc;
#pragma unroll
                for (int u = 0; u < 32; ++u) o[u] = oc[u];
            } else {
                const float mn = (mc > m) ? mc : m;
                const float a = exp_f(m - mn), bb = exp_f(mc - mn);
                l = (l * a) + (lc * bb);
#pragma unroll
                for (int u = 0; u < 32; ++u) o[u] = (o[u] * a) + (oc[u] * bb);
                m = mn;
            }
        }
    }
    if (rvalid) {
        float* out = O + (((int64_t)b * Tq + r0 + r) * Hq + h) * D + q4 * 32;
#pragma unroll
        for (int u = 0; u < 32; u += 4) {
            float4 v;
            v.x = o[u + 0] / l; v.y = o[u + 1] / l; v.z = o[u + 2] / l; v.w = o[u + 3] / l;
            *reinterpret_cast<float4*>(out + u) = v;
        }
    }
}

// ------------------------------------------------------------------- decode --
// Workgroup: one (b, kv head g, chunk c); 256 threads, one key per thread for the scores;
// the G = Hq / Hkv query heads that share kv head g are done together.
constexpr int GMAX = 16;

template <int DT>
__global__ __launch_bounds__(256) void attn_decode_partial_kernel(
    const void* __restrict__ Q, const void* __restrict__ Kc, const void* __restrict__ Vc,
    const int32_t* __restrict__ pos, int Tmax, int Hq, int Hkv, float scale, int nchunks,
    float* __restrict__ ws) {
    __shared__ float Qs[GMAX][D];
    __shared__ float Ps[GMAX][CHUNK];
    __shared__ float Ms[GMAX];
    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int G = Hq / Hkv;
    const int p = pos[b];
    if (p < 0 || p >= Tmax) return;             // invalid position: the merge writes NaN
    const int kbase = c * CHUNK;
    if (kbase > p) return;                      // empty chunk: never folded
    const int jlast = min(kbase + CHUNK - 1, p);
    const int tid = threadIdx.x;
    const int64_t kvbase = ((int64_t)b * Hkv + g) * Tmax * D;

    for (int e = tid; e < G * (D / 4); e += 256) {
        const int hh = e / (D / 4), d4 = (e % (D / 4)) * 4;
        float v[4];
        load_row4<DT>(Q, ((int64_t)b * Hq + g * G + hh) * D + d4, v);
        Qs[hh][d4 + 0] = v[0]; Qs[hh][d4 + 1] = v[1]; Qs[hh][d4 + 2] = v[2]; Qs[hh][d4 + 3] = v[3];
    }
    __syncthreads();
    const int j = kbase + tid;
    if (j <= jlast) {
        float acc[GMAX];
#pragma unroll
        for (int hh = 0; hh < GMAX; ++hh) acc[hh] = 0.0f;
        for (int d = 0; d < D; d += 4) {
            float kv[4];
            load_row4<DT>(Kc, kvbase + (int64_t)j * D + d, kv);
#pragma unroll
            for (int hh = 0; hh < GMAX; ++hh) {
                if (hh < G) {
                    acc[hh] = __builtin_fmaf(Qs[hh][d + 0], kv[0], acc[hh]);
                    acc[hh] = __builtin_fmaf(Qs[hh][d + 1], kv[1], acc[hh]);
                    acc[hh] = __builtin_fmaf(Qs[hh][d + 2], kv[2], acc[hh]);
                    acc[hh] = __builtin_fmaf(Qs[hh][d + 3], kv[3], acc[hh]);
                }
            }
        }
#pragma unroll
        for (int hh = 0; hh < GMAX; ++hh)
            if (hh < G) Ps[hh][tid] = acc[hh] * scale;
    }
    __syncthreads();
    // chunk max per head: wavefront w reduces head w, w+4, ...
    const int lane = tid % 64, w = tid / 64;
    const int nk = jlast - kbase + 1;
    for (int hh = w; hh < G; hh += 4) {
        float mc = -__builtin_inff();
        for (int jj = lane; jj < nk; jj += 64) { const float s = Ps[hh][jj]; mc = (s > mc) ? s : mc; }
        for (int off = 32; off >= 1; off >>= 1) { const float t = __shfl_xor(mc, off); mc = (t > mc) ? t : mc; }
        if (lane == 0) Ms[hh] = mc;
    }
    __syncthreads();
    for (int e = tid; e < G * nk; e += 256) {
        const int hh = e / nk, jj = e % nk;
        Ps[hh][jj] = exp_f(Ps[hh][jj] - Ms[hh]);
    }
    __syncthreads();
    // o_c[d] and l_c, keys ascending; thread owns (head, d) pairs
    const int D2 = D + 2;
    for (int e = tid; e < G * D; e += 256) {
        const int hh = e / D, d = e % D;
        float oc = 0.0f, lc = 0.0f;
        for (int jj = 0; jj < nk; ++jj) {
            const float pj = Ps[hh][jj];
            float v;
            if (DT == 1) v = reinterpret_cast<const float*>(Vc)[kvbase + (int64_t)(kbase + jj) * D + d];
            else v = bf16_up(reinterpret_cast<const uint16_t*>(Vc)[kvbase + (int64_t)(kbase + jj) * D + d]);
            oc = __builtin_fmaf(pj, v, oc);
            lc = lc + pj;
        }
        float* dst = ws + (((int64_t)b * Hq + g * G + hh) * nchunks + c) * D2;
        dst[2 + d] = oc;
        if (d == 0) { dst[0] = Ms[hh]; dst[1] = lc; }
    }
}

__global__ __launch_bounds__(128) void attn_decode_merge_kernel(const int32_t* __restrict__ pos,
                                                                int Hq, int Tmax, int nchunks,
                                                                const float* __restrict__ ws,
                                                                float* __restrict__ O) {
    const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
    const int p = pos[b];
    if (p < 0 || p >= Tmax) {
        O[((int64_t)b * Hq + h) * D + d] = __builtin_nanf("");
        return;
    }
    const int nc = p / CHUNK + 1;
    const int D2 = D + 2;
    const float* src = ws + ((int64_t)b * Hq + h) * nchunks * D2;
    float m = src[0], l = src[1], o = src[2 + d];
    for (int c = 1; c < nc; ++c) {
        const float* s = src + (int64_t)c * D2;
        const float mc = s[0], lc = s[1], oc = s[2 + d];
        const float mn = (mc > m) ? mc : m;
        const float a = exp_f(m - mn), bb = exp_f(mc - mn);
        l = (l * a) + (lc * bb);
        o = (o * a) + (oc * bb);
        m = mn;
    }
    O[((int64_t)b * Hq + h) * D + d] = o / l;
}

}  // namespace

hipError_t launch_attention_prefill(const AttnArgs& a, hipStream_t st) {
    dim3 grid((a.Tq + BQ - 1) / BQ, a.Hq, a.B);
    if (a.dtype == 1)
        hipLaunchKernelGGL(attn_prefill_kernel<1>, grid, dim3(256), 0, st, a.Q, a.Kc, a.Vc, a.Tq,
                           a.q_start, a.Tmax, a.Hq, a.Hkv, a.scale, a.O);
    else
        hipLaunchKernelGGL(attn_prefill_kernel<0>, grid, dim3(256), 0, st, a.Q, a.Kc, a.Vc, a.Tq,
                           a.q_start, a.Tmax, a.Hq, a.Hkv, a.scale, a.O);
    return hipGetLastError();
}

hipError_t launch_attention_decode(const AttnArgs& a, const int32_t* pos, float* ws, hipStream_t st) {
    const int nchunks = (a.Tmax + CHUNK - 1) / CHUNK;
    dim3 grid(nchunks, a.Hkv, a.B);
    if (a.dtype == 1)
        hipLaunchKernelGGL(attn_decode_partial_kernel<1>, grid, dim3(256), 0, st, a.Q, a.Kc, a.Vc,
                           pos, a.Tmax, a.Hq, a.Hkv, a.scale, nchunks, ws);
    else
        hipLaunchKernelGGL(attn_decode_partial_kernel<0>, grid, dim3(256), 0, st, a.Q, a.Kc, a.Vc,
                           pos, a.Tmax, a.Hq, a.Hkv, a.scale, nchunks, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_decode_merge_kernel, dim3(a.Hq, a.B), dim3(D), 0, st, pos, a.Hq, a.Tmax,
                       nchunks, ws, a.O);
    return hipGetLastError();
}

}  // namespace invnum
