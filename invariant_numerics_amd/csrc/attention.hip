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
// Matrix-core prefill.  v_mfma_f32_16x16x4_f32 advances each output of a 16 x 16 tile by
// four fused multiply-adds in k order, so both contractions keep their sequential order:
// the scores over d = 0..127 and the PV sums over keys in ascending j.
// Workgroup: 256 threads = 4 wavefronts over BQ = 64 consecutive query rows of one (b, h);
// wavefront w owns rows 16w .. 16w + 15.  Per 256-key chunk:
//   1. scores: K staged through LDS in 64-key sub-blocks; 16 key tiles x 32 MFMA steps, all
//      256 scores of the chunk kept in registers (lane (g, r) holds rows 4g..4g+3 of key
//      column r of every key tile);
//   2. chunk max over the row's keys <= i (16-lane shuffles), p = exp_f(s - m_c);
//   3. PV: p re-laid out through LDS, V staged row-major; MFMA over keys below the first
//      multiple-of-4 boundary that every row of the wavefront can see; l_c runs on the same
//      instruction with an all-ones operand (fma(p, 1, l) = l + p, one rounding); the keys
//      from there to each row's own i (at most 19) continue on the VALU, ascending, so
//      masked keys are skipped rather than added as zeros;
//   4. merge into the running (m, l, o) exactly as the decode merge kernel does.
constexpr int SB = 64;          // keys per LDS sub-block
constexpr int KPAD = 4;

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float rowmax16(float x) {
    // maximum over the 16 lanes sharing lane >> 4 (max is order independent)
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
        const float y = __shfl_xor(x, off);
        x = (y > x) ? y : x;
    }
    return x;
}

template <int DT>
__device__ __forceinline__ void load4(const void* base, int64_t off, float* v) {
    if (DT == 1) {
        const float4 t = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + off);
        v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    } else {
        const uint2 t = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + off);
        v[0] = bf16_lo(t.x); v[1] = bf16_hi(t.x); v[2] = bf16_lo(t.y); v[3] = bf16_hi(t.y);
    }
}

// Global -> register -> LDS staging of one 64-key sub-block of K or V (fp32 in LDS).
// Thread t carries 8 groups of 4 consecutive d of rows (e / 32) for e = t + 256 i.
template <int DT>
struct Stage {
    float4 v[8];
    // rows at or beyond kend are read from row kend - 1 (always valid) and replaced by zeros
    __device__ __forceinline__ void load(const void* base, int64_t kvbase, int kb, int kend, int tid) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int e = tid + 256 * i;
            const int jj = e >> 5, d4 = (e & 31) * 4;
            const bool in = kb + jj < kend;
            const int row = in ? kb + jj : kend - 1;
            float t[4];
            load4<DT>(base, kvbase + (int64_t)row * D + d4, t);
            v[i] = in ? make_float4(t[0], t[1], t[2], t[3]) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    // K layout: row jj, d permuted (d % 4) * 32 + d / 4 (a lane's 32 operands contiguous)
    __device__ __forceinline__ void store_k(float* KV, int tid) const {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int e = tid + 256 * i;
            const int jj = e >> 5, q = e & 31;
            float* dst = KV + jj * (D + KPAD) + q;
            dst[0] = v[i].x; dst[32] = v[i].y; dst[64] = v[i].z; dst[96] = v[i].w;
        }
    }
    // V layout: row-major [key][d]
    __device__ __forceinline__ void store_v(float* KV, int tid) const {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int e = tid + 256 * i;
            const int jj = e >> 5, d4 = (e & 31) * 4;
            *reinterpret_cast<float4*>(KV + jj * (D + KPAD) + d4) = v[i];
        }
    }
};

template <int DT>
__global__ __launch_bounds__(256) void attn_prefill_kernel(
    const void* __restrict__ Q, const void* __restrict__ Kc, const void* __restrict__ Vc,
    int Tq, int q_start, int Tmax, int Hq, int Hkv, float scale, float* __restrict__ O) {
    // two K/V sub-block buffers; per-wavefront p of the whole chunk
    // [16 rows][4 sub-blocks x 64 keys, keys permuted (j % 4) * 16 + j / 4 inside each]
    __shared__ float KV[2][SB * (D + KPAD)];
    __shared__ float Ps[4][16][CHUNK + KPAD];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, r = lane & 15;
    const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int kvh = h / (Hq / Hkv);
    const int r0 = qb * BQ;
    const int nrows = min(BQ, Tq - r0);
    const int imax = q_start + r0 + nrows - 1;          // last valid absolute row of the block
    const int64_t kvbase = ((int64_t)b * Hkv + kvh) * Tmax * D;
    const int wrow0 = r0 + 16 * w;                      // first row (relative) of this wavefront
    const int i0 = q_start + wrow0;                     // its absolute position
    int irow[4];                                        // the lane's output rows, clamped
#pragma unroll
    for (int v = 0; v < 4; ++v) irow[v] = min(i0 + 4 * g + v, imax);

    // Q fragments: lane (g, r) supplies Q[row r][d = 4s + g], s = 0..31
    float qf[32];
    {
        const int qrow = min(wrow0 + r, Tq - 1);
        const int64_t qoff = (((int64_t)b * Tq + qrow) * Hq + h) * D;
#pragma unroll
        for (int s = 0; s < 32; ++s) {
            const int d = 4 * s + g;
            qf[s] = DT == 1 ? reinterpret_cast<const float*>(Q)[qoff + d]
                            : bf16_up(reinterpret_cast<const uint16_t*>(Q)[qoff + d]);
        }
    }

    f32x4 o[8];
    float m[4], l[4];
#pragma unroll
    for (int t = 0; t < 8; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int v = 0; v < 4; ++v) { m[v] = 0.0f; l[v] = 0.0f; }

    const int clast = imax / CHUNK;
    Stage<DT> st;
    int buf = 0;
    // prologue: chunk 0, K sub-block 0
    st.load(Kc, kvbase, 0, min(CHUNK, imax + 1), tid);
    st.store_k(KV[0], tid);
    __syncthreads();

    for (int c = 0; c <= clast; ++c) {
        const int kbase = c * CHUNK;
        const int kend = min(kbase + CHUNK, imax + 1);         // keys some row of the block needs
        const int nsb = (kend - kbase + SB - 1) / SB;          // active sub-blocks (1..4)
        const int nkend = min(kbase + 2 * CHUNK, imax + 1);    // next chunk's key bound
        // ------------------------------------------------------ 1. scores (stages K_0..K_nsb-1)
        f32x4 S[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) S[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sb = 0; sb < CHUNK / SB; ++sb) {
            if (sb < nsb) {
                // prefetch the next stage: K_{sb+1}, or V_0 of this chunk
                if (sb + 1 < nsb) st.load(Kc, kvbase, kbase + (sb + 1) * SB, kend, tid);
                else st.load(Vc, kvbase, kbase, kend, tid);
                const float* kvb = KV[buf];
                if (kbase + sb * SB <= i0 + 15) {
                    f32x4 acc[SB / 16];
#pragma unroll
                    for (int kt = 0; kt < SB / 16; ++kt) acc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s4 = 0; s4 < 8; ++s4) {
                        float4 kk[SB / 16];
#pragma unroll
                        for (int kt = 0; kt < SB / 16; ++kt)
                            kk[kt] = *reinterpret_cast<const float4*>(kvb + (kt * 16 + r) * (D + KPAD) + g * 32 + 4 * s4);
#pragma unroll
                        for (int kt = 0; kt < SB / 16; ++kt)
                            acc[kt] = __builtin_amdgcn_mfma_f32_16x16x4f32(qf[4 * s4 + 0], kk[kt].x, acc[kt], 0, 0, 0);
#pragma unroll
                        for (int kt = 0; kt < SB / 16; ++kt)
                            acc[kt] = __builtin_amdgcn_mfma_f32_16x16x4f32(qf[4 * s4 + 1], kk[kt].y, acc[kt], 0, 0, 0);
#pragma unroll
                        for (int kt = 0; kt < SB / 16; ++kt)
                            acc[kt] = __builtin_amdgcn_mfma_f32_16x16x4f32(qf[4 * s4 + 2], kk[kt].z, acc[kt], 0, 0, 0);
#pragma unroll
                        for (int kt = 0; kt < SB / 16; ++kt)
                            acc[kt] = __builtin_amdgcn_mfma_f32_16x16x4f32(qf[4 * s4 + 3], kk[kt].w, acc[kt], 0, 0, 0);
                    }
#pragma unroll
                    for (int kt = 0; kt < SB / 16; ++kt) S[sb * 4 + kt] = acc[kt];
                }
                if (sb + 1 < nsb) st.store_k(KV[buf ^ 1], tid);
                else st.store_v(KV[buf ^ 1], tid);
                __syncthreads();
                buf ^= 1;
            }
        }
        // ------------------------------------------------------ 2. chunk max and p
        float mc[4];
        bool ne[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            ne[v] = irow[v] >= kbase;
            float x = -__builtin_inff();
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const int j = kbase + t * 16 + r;
                const float sv = S[t][v] * scale;
                S[t][v] = sv;
                if (j <= irow[v]) x = (sv > x) ? sv : x;
            }
            mc[v] = rowmax16(x);
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int jj = (t & 3) * 16 + r;                   // key inside its sub-block
            const int pj = (t >> 2) * SB + (jj & 3) * 16 + (jj >> 2);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int j = kbase + t * 16 + r;
                Ps[w][4 * g + v][pj] = (j <= irow[v]) ? exp_f(S[t][v] - mc[v]) : 0.0f;
            }
        }
        __syncthreads();
        // ------------------------------------------------------ 3. PV and l (stages V_0..)
        // keys [kbase, jv) go through the matrix cores for every row of the wavefront
        const int jspan = min(i0, kend) - kbase;
        const int jv = kbase + ((jspan > 0 ? jspan : 0) & ~3);
        f32x4 oc[8];
        f32x4 lc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 8; ++t) oc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sb = 0; sb < CHUNK / SB; ++sb) {
            if (sb < nsb) {
                const int kb = kbase + sb * SB;
                // prefetch: V_{sb+1}, or the next chunk's K_0
                const bool more = sb + 1 < nsb;
                if (more) st.load(Vc, kvbase, kb + SB, kend, tid);
                else if (c < clast) st.load(Kc, kvbase, kbase + CHUNK, nkend, tid);
                const float* kvb = KV[buf];
                const int nsteps = max(0, min(SB, jv - kb)) >> 2;
                const float* prow = &Ps[w][r][sb * SB + g * 16];
                for (int s = 0; s < nsteps; ++s) {
                    const float a = prow[s];
                    const float* vr = kvb + (4 * s + g) * (D + KPAD) + r;
#pragma unroll
                    for (int t = 0; t < 8; ++t)
                        oc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, vr[t * 16], oc[t], 0, 0, 0);
                    lc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, 1.0f, lc, 0, 0, 0);
                }
                // VALU continuation for keys [max(kb, jv), row's own i], ascending
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int j1 = min(kb + SB, irow[v] + 1);
                    for (int j = max(kb, jv); j < j1; ++j) {
                        const int jj = j - kb;
                        const float pv = Ps[w][4 * g + v][sb * SB + (jj & 3) * 16 + (jj >> 2)];
                        lc[v] = lc[v] + pv;
#pragma unroll
                        for (int t = 0; t < 8; ++t)
                            oc[t][v] = __builtin_fmaf(pv, kvb[jj * (D + KPAD) + t * 16 + r], oc[t][v]);
                    }
                }
                if (more) st.store_v(KV[buf ^ 1], tid);
                else if (c < clast) st.store_k(KV[buf ^ 1], tid);
                __syncthreads();
                buf ^= 1;
            }
        }
        // ------------------------------------------------------ 4. merge
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            if (!ne[v]) continue;
            if (c == 0) {
                m[v] = mc[v];
                l[v] = lc[v];
#pragma unroll
                for (int t = 0; t < 8; ++t) o[t][v] = oc[t][v];
            } else {
                const float mn = (mc[v] > m[v]) ? mc[v] : m[v];
                const float al = exp_f(m[v] - mn), be = exp_f(mc[v] - mn);
                l[v] = (l[v] * al) + (lc[v] * be);
#pragma unroll
                for (int t = 0; t < 8; ++t) o[t][v] = (o[t][v] * al) + (oc[t][v] * be);
                m[v] = mn;
            }
        }
    }
    // ------------------------------------------------------------------ output
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int rel = wrow0 + 4 * g + v;
        if (rel >= r0 + nrows) continue;
        float* out = O + (((int64_t)b * Tq + rel) * Hq + h) * D;
#pragma unroll
        for (int t = 0; t < 8; ++t) out[t * 16 + r] = o[t][v] / l[v];
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
