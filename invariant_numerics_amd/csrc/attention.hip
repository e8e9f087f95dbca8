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

#include <algorithm>
#include <mutex>
#include <type_traits>

namespace invnum {

namespace {

constexpr int D = 128;

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
//
// Workgroup: NW wavefronts (8, or 4 when the grid would be small) over BQ = 16 NW consecutive
// query rows of one (b, h); wavefront w owns rows 16 w .. 16 w + 15 outright (scores of every
// key, every d of the output), so no partial state is exchanged between wavefronts and all of
// them share each K/V sub-block staged in LDS.  Per 256-key chunk:
//   1. scores S^T = K Q^T on the matrix cores: A = K tile (lane (g, r) supplies key
//      16t + pi(r), d = 4s + g, with pi(i) = 4 (i % 4) + i / 4), B = Q^T (lane (g, r) supplies
//      row r, d = 4s + g, held in registers); lane (g, r) receives in register v the score of
//      row r with key 16t + 4v + g.  K streams through double-buffered LDS in SB-key
//      sub-blocks (64 or 32 keys: SB / 16 key tiles each);
//   2. m_c = the maximum of the row's visible scores (lanes of a row exchange theirs);
//      p = exp_f(s - m_c) in place;
//   3. PV: O^T = V^T P^T over all keys of the chunk in ascending order, output tile t
//      (t = 0..7) taking d = 8i + t: step s covers keys 4s .. 4s + 3, lane (g, r) supplies
//      V[key 4s + g][8r .. 8r + 7] (two 16-byte LDS reads for the eight tiles) and, as B, its
//      own p of key 4s + g, and accumulates o[row r][d = 32g + 8v + t].  The l-sum runs on
//      the same instruction with an all-ones A operand, fma(1, p, l) = l + p, one rounding per
//      key.  The matrix cores take the keys below the first multiple-of-4 boundary that every
//      row of the wavefront sees; the rest of the causal triangle (at most 19 keys per row)
//      continues on the VALU in ascending j, with those p passed through a small per-wavefront
//      LDS buffer, so masked keys are skipped rather than added as zeros;
//   4. merge into the running (m, l, o) with the formulas of the decode merge kernel.
// Blocks are issued heaviest first (the last rows see the most keys), and consecutive
// workgroup ids cycle over the kv heads so the workgroups running together on one XCD (ids
// are dealt to the 8 XCDs in turn) share one kv head's K/V in its L2.
constexpr int KLD = D + 4;      // LDS row: K with d permuted ((d % 4) * 32 + d / 4), V row-major
constexpr int TW = 20;          // keys of the causal tail buffer (at most 19 are used)
constexpr int TLD = TW + 1;     // its padded row

typedef float f32x4 __attribute__((ext_vector_type(4)));

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

// Global -> register -> LDS staging of one SBK-key sub-block of K or V (fp32 in LDS) by NT
// threads.  Thread t carries SV groups of 4 consecutive d of rows (e / 32), e = t + NT i, as
// loaded (4 floats, or 4 BF16 values in two words, upcast only at the LDS store, which halves
// the registers the BF16 staging holds).  Rows at or beyond kend are read from row kend - 1
// (always valid) and replaced by zeros (zero bits are +0 in both formats).
template <int DT>
struct StageRaw { typedef float4 type; };
template <>
struct StageRaw<0> { typedef uint2 type; };

template <int DT, int NT, int SBK>
struct Stage {
    static constexpr int SV = SBK * (D / 4) / NT;
    typedef typename StageRaw<DT>::type raw_t;
    raw_t v[SV];
    __device__ __forceinline__ static raw_t fetch(const void* base, int64_t off) {
        if constexpr (DT == 1) return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + off);
        else return *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + off);
    }
    __device__ __forceinline__ static float4 up(const raw_t& t) {
        if constexpr (DT == 1) return t;
        else return make_float4(bf16_lo(t.x), bf16_hi(t.x), bf16_lo(t.y), bf16_hi(t.y));
    }
    __device__ __forceinline__ void load(const void* base, int64_t kvbase, int kb, int kend, int tid) {
        if (kb + SBK <= kend) {
            // whole sub-block in range: row (tid >> 5) + (NT / 32) i, column 4 (tid & 31)
            const int64_t off = kvbase + (int64_t)(kb + (tid >> 5)) * D + (tid & 31) * 4;
#pragma unroll
            for (int i = 0; i < SV; ++i) v[i] = fetch(base, off + (int64_t)((NT / 32) * i) * D);
            return;
        }
#pragma unroll
        for (int i = 0; i < SV; ++i) {
            const int e = tid + NT * i;
            const int jj = e >> 5, d4 = (e & 31) * 4;
            const bool in = kb + jj < kend;
            const int row = in ? kb + jj : kend - 1;
            const raw_t t = fetch(base, kvbase + (int64_t)row * D + d4);
            v[i] = in ? t : raw_t{};
        }
    }
    __device__ __forceinline__ void store_k(float* KV, int tid) const {
#pragma unroll
        for (int i = 0; i < SV; ++i) {
            const int e = tid + NT * i;
            const int jj = e >> 5, q = e & 31;
            float* dst = KV + jj * KLD + q;
            const float4 x = up(v[i]);
            dst[0] = x.x; dst[32] = x.y; dst[64] = x.z; dst[96] = x.w;
        }
    }
    __device__ __forceinline__ void store_v(float* KV, int tid) const {
#pragma unroll
        for (int i = 0; i < SV; ++i) {
            const int e = tid + NT * i;
            const int jj = e >> 5, d4 = (e & 31) * 4;
            *reinterpret_cast<float4*>(KV + jj * KLD + d4) = up(v[i]);
        }
    }
};

// Task split (SPLIT = true, small grids): a row block whose rows see more than R chunks is cut
// into tasks of at most R consecutive chunks, so more workgroups share its keys.  A task of a
// cut block stores each chunk's (m_c, l_c, o_c) per row -- the values the running merge would
// fold next -- into the partials array, and attn_prefill_merge_kernel folds them in ascending
// chunk order afterwards: the same two-rounding merge as in the single-task loop, so the same
// bits.  Blocks with at most R chunks run whole, as without the split.
struct PrefillSplit {
    int R;          // chunks per task (0: no split)
    int r_split;    // first row of the first cut block (rows >= r_split are folded by the merge)
    int nch;        // chunk dimension of the partials array
    float* ws;      // partials [B][Tq - r_split][Hq][nch][D + 2]
};

template <int DT, int NW, int SB, bool SPLIT>
__global__ __launch_bounds__(64 * NW, 2) void attn_prefill_kernel(
    const void* __restrict__ Q, const void* __restrict__ Kc, const void* __restrict__ Vc,
    int B, int Tq, int q_start, int Tmax, int Hq, int Hkv, float scale, float* __restrict__ O,
    PrefillSplit sp) {
    constexpr int BQ = 16 * NW;                 // query rows per workgroup
    constexpr int KT = SB / 16;                 // key tiles per sub-block
    __shared__ __attribute__((aligned(16))) float KV[2][SB * KLD];
    __shared__ float Tail[NW][16][TLD];

    const int tid = threadIdx.x;
    // the wavefront index is uniform in a wavefront: in a scalar register, everything derived
    // from it (rows, causal bounds) takes scalar branches
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, r = lane & 15;
    const int pr = 4 * (r & 3) + (r >> 2);             // pi(r)
    int qb, h, b, c0 = 0, c1 = 0;
    bool cut = false;                                   // this block's chunks go to several tasks
    {
        // workgroup id -> (row block, head, sequence): row blocks from the last (heaviest) down;
        // within one row block, consecutive ids take q heads h = (u % Hkv) G + u / Hkv, i.e. they
        // cycle over the kv heads
        const int nqb = (Tq + BQ - 1) / BQ, HB = Hq * B;
        const int L = blockIdx.x, u = L % HB, G = Hq / Hkv;
        if constexpr (SPLIT) {
            // task j = L / HB: the blocks' tasks listed from the last block down, each block's
            // chunk ranges [t R, (t + 1) R) in order
            int j = L / HB;
            qb = nqb - 1;
            for (; qb > 0; --qb) {
                const int n = (q_start + min(Tq, (qb + 1) * BQ) - 1) / CHUNK + 1;
                const int nt = (n + sp.R - 1) / sp.R;
                if (j < nt) break;
                j -= nt;
            }
            const int n = (q_start + min(Tq, (qb + 1) * BQ) - 1) / CHUNK + 1;
            cut = n > sp.R;
            c0 = j * sp.R;
            c1 = min(n, c0 + sp.R);
        } else {
            qb = nqb - 1 - L / HB;
        }
        b = u / Hq;
        const int hh = u % Hq;
        h = (hh % Hkv) * G + hh / Hkv;
    }
    const int kvh = h / (Hq / Hkv);
    const int r0 = qb * BQ;
    const int nrows = min(BQ, Tq - r0);
    const int imax = q_start + r0 + nrows - 1;          // last valid absolute row of the block
    if constexpr (!SPLIT) c1 = imax / CHUNK + 1;
    const int64_t kvbase = ((int64_t)b * Hkv + kvh) * Tmax * D;
    const int wrow0 = r0 + 16 * w;                      // first row (relative) of the wavefront
    const int i0 = q_start + wrow0;                     // its absolute position
    const int irow = min(i0 + r, imax);                 // the lane's row, clamped

    // Q^T operand: lane (g, r) supplies Q[row r][d = 4s + g], s = 0..31
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
    float m = 0.0f, l = 0.0f;
#pragma unroll
    for (int t = 0; t < 8; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    Stage<DT, 64 * NW, SB> st;
    int buf = 0;
    st.load(Kc, kvbase, c0 * CHUNK, min(c0 * CHUNK + CHUNK, imax + 1), tid);
    st.store_k(KV[0], tid);
    __syncthreads();
    float* tail = &Tail[w][r][0];

    // One chunk.  FAST: every row of the workgroup sees all 256 keys of the chunk and all four
    // sub-blocks are in range -- the common case -- so no guard, mask or causal tail is needed
    // and the body is straight-line; otherwise every step checks its bounds.
    auto chunk = [&](const int c, auto fast_tag) {
        constexpr bool FAST = decltype(fast_tag)::value;
        const int kbase = c * CHUNK;
        const int kend = min(kbase + CHUNK, imax + 1);         // keys some row of the block needs
        const int nsb = FAST ? CHUNK / SB : (kend - kbase + SB - 1) / SB;   // active sub-blocks
        const int nkend = min(kbase + 2 * CHUNK, imax + 1);    // next chunk's key bound
        // ------------------------------------------------------ 1. scores
        // S[t] is key tile t of the chunk
        f32x4 S[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) S[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sb = 0; sb < CHUNK / SB; ++sb) {
            if (FAST || sb < nsb) {
                if (sb + 1 < nsb) st.load(Kc, kvbase, kbase + (sb + 1) * SB, kend, tid);
                else st.load(Vc, kvbase, kbase, kend, tid);
                // keep the loads here, ahead of this sub-block's matrix-core work: left to itself
                // the scheduler sinks them next to their LDS stores, where their whole latency
                // is waited out
                __builtin_amdgcn_sched_barrier(0);
                const float* kvb = KV[buf];
                if (FAST || kbase + sb * SB <= i0 + 15) {
#pragma unroll
                    for (int s4 = 0; s4 < 8; ++s4) {
                        float4 kk[KT];
#pragma unroll
                        for (int e = 0; e < KT; ++e)
                            kk[e] = *reinterpret_cast<const float4*>(kvb + (e * 16 + pr) * KLD + g * 32 + 4 * s4);
#pragma unroll
                        for (int e = 0; e < KT; ++e)
                            S[sb * KT + e] = __builtin_amdgcn_mfma_f32_16x16x4f32(kk[e].x, qf[4 * s4 + 0], S[sb * KT + e], 0, 0, 0);
#pragma unroll
                        for (int e = 0; e < KT; ++e)
                            S[sb * KT + e] = __builtin_amdgcn_mfma_f32_16x16x4f32(kk[e].y, qf[4 * s4 + 1], S[sb * KT + e], 0, 0, 0);
#pragma unroll
                        for (int e = 0; e < KT; ++e)
                            S[sb * KT + e] = __builtin_amdgcn_mfma_f32_16x16x4f32(kk[e].z, qf[4 * s4 + 2], S[sb * KT + e], 0, 0, 0);
#pragma unroll
                        for (int e = 0; e < KT; ++e)
                            S[sb * KT + e] = __builtin_amdgcn_mfma_f32_16x16x4f32(kk[e].w, qf[4 * s4 + 3], S[sb * KT + e], 0, 0, 0);
                    }
                }
                if (sb + 1 < nsb) st.store_k(KV[buf ^ 1], tid);
                else st.store_v(KV[buf ^ 1], tid);
                __syncthreads();
                buf ^= 1;
            }
        }
        // ------------------------------------------------------ 2. chunk max and p
        // m_c = max of the row's visible scores.  NaN scores are passed over (as the
        // sequential compare-and-keep does); which zero a tie between +0 and -0 keeps cannot
        // change any result, since every p and merge factor built from a zero difference is
        // exp_f(+-0) = 1.  So the hardware maximum serves, in any grouping.
        const bool ne = irow >= kbase;
        const bool full = FAST || kbase + CHUNK <= i0;         // every row sees the whole chunk
        float mh = -__builtin_inff();
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            if (FAST || t < KT * nsb) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int j = kbase + 16 * t + 4 * v + g;
                    const float sv = S[t][v] * scale;
                    S[t][v] = sv;
                    if (full || j <= irow) mh = __builtin_fmaxf(mh, sv);
                }
            }
        }
        mh = __builtin_fmaxf(mh, __shfl_xor(mh, 16));
        const float mc = __builtin_fmaxf(mh, __shfl_xor(mh, 32));
        const int jspan = min(i0, kend) - kbase;
        const int jv = FAST ? kbase + CHUNK : kbase + ((jspan > 0 ? jspan : 0) & ~3);   // MFMA keys: [kbase, jv)
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            if (FAST || t < KT * nsb) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int j = kbase + 16 * t + 4 * v + g;
                    const float pv = (full || j <= irow) ? exp_f(S[t][v] - mc) : 0.0f;
                    S[t][v] = pv;
                    // the causal tail's p (keys jv .. jv + 18), read back in key order by the
                    // lanes of the row; the buffer belongs to this wavefront alone
                    if (!FAST && j >= jv && j < jv + TW) tail[j - jv] = pv;
                }
            }
        }
        // ------------------------------------------------------ 3. PV and l
        f32x4 oc[8];
        f32x4 lc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 8; ++t) oc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sb = 0; sb < CHUNK / SB; ++sb) {
            if (FAST || sb < nsb) {
                const int kb = kbase + sb * SB;
                const bool more = sb + 1 < nsb;
                // after the last V sub-block comes the next chunk's first K sub-block (past the
                // last chunk every row is out of range: the stage clamps and stores zeros)
                if (more) st.load(Vc, kvbase, kb + SB, kend, tid);
                else st.load(Kc, kvbase, kbase + CHUNK, nkend, tid);
                __builtin_amdgcn_sched_barrier(0);     // as in the scores
                const float* kvb = KV[buf];
                const float* vop = kvb + g * KLD + 8 * r;       // + 4 s KLD at step s
                const int nmk = min(SB, jv - kb);               // keys of this sub-block on MFMA
#pragma unroll
                for (int s = 0; s < SB / 4; ++s) {
                    if (FAST || 4 * s < nmk) {
                        const float bp = S[sb * KT + (s >> 2)][s & 3];
                        const float4 va = *reinterpret_cast<const float4*>(vop + 4 * s * KLD);
                        const float4 vb = *reinterpret_cast<const float4*>(vop + 4 * s * KLD + 4);
                        oc[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(va.x, bp, oc[0], 0, 0, 0);
                        oc[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(va.y, bp, oc[1], 0, 0, 0);
                        oc[2] = __builtin_amdgcn_mfma_f32_16x16x4f32(va.z, bp, oc[2], 0, 0, 0);
                        oc[3] = __builtin_amdgcn_mfma_f32_16x16x4f32(va.w, bp, oc[3], 0, 0, 0);
                        oc[4] = __builtin_amdgcn_mfma_f32_16x16x4f32(vb.x, bp, oc[4], 0, 0, 0);
                        oc[5] = __builtin_amdgcn_mfma_f32_16x16x4f32(vb.y, bp, oc[5], 0, 0, 0);
                        oc[6] = __builtin_amdgcn_mfma_f32_16x16x4f32(vb.z, bp, oc[6], 0, 0, 0);
                        oc[7] = __builtin_amdgcn_mfma_f32_16x16x4f32(vb.w, bp, oc[7], 0, 0, 0);
                        lc = __builtin_amdgcn_mfma_f32_16x16x4f32(1.0f, bp, lc, 0, 0, 0);
                    }
                }
                if (!FAST) {
                    // VALU continuation for keys [max(kb, jv), i], ascending (row r)
                    const int j1 = min(kb + SB, irow + 1);
                    for (int j = max(kb, jv); j < j1; ++j) {
                        const float pv = tail[j - jv];
                        const float* vr = kvb + (j - kb) * KLD + 32 * g;    // d = 32g + 8v + t
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const float4 x0 = *reinterpret_cast<const float4*>(vr + 8 * v);
                            const float4 x1 = *reinterpret_cast<const float4*>(vr + 8 * v + 4);
                            oc[0][v] = __builtin_fmaf(pv, x0.x, oc[0][v]);
                            oc[1][v] = __builtin_fmaf(pv, x0.y, oc[1][v]);
                            oc[2][v] = __builtin_fmaf(pv, x0.z, oc[2][v]);
                            oc[3][v] = __builtin_fmaf(pv, x0.w, oc[3][v]);
                            oc[4][v] = __builtin_fmaf(pv, x1.x, oc[4][v]);
                            oc[5][v] = __builtin_fmaf(pv, x1.y, oc[5][v]);
                            oc[6][v] = __builtin_fmaf(pv, x1.z, oc[6][v]);
                            oc[7][v] = __builtin_fmaf(pv, x1.w, oc[7][v]);
                        }
                        lc[0] = lc[0] + pv;
                    }
                }
                if (more) st.store_v(KV[buf ^ 1], tid);
                else st.store_k(KV[buf ^ 1], tid);
                __syncthreads();
                buf ^= 1;
            }
        }
        // ------------------------------------------------------ 4. merge
        if (SPLIT && cut) {
            // the chunk's partial for the merge kernel: (m_c, l_c, o_c[d]) of the lane's row
            const int rel = wrow0 + r;
            if (ne && rel < r0 + nrows) {
                float* dst = sp.ws + ((((int64_t)b * (Tq - sp.r_split) + (rel - sp.r_split)) * Hq + h) * sp.nch + c) * (D + 2);
                if (g == 0) { dst[0] = mc; dst[1] = lc[0]; }
#pragma unroll
                for (int v = 0; v < 4; ++v)
#pragma unroll
                    for (int t = 0; t < 8; t += 2)
                        *reinterpret_cast<float2*>(dst + 2 + 32 * g + 8 * v + t) = make_float2(oc[t][v], oc[t + 1][v]);
            }
            return;
        }
        if (ne) {
            if (c == 0) {
                m = mc;
                l = lc[0];
#pragma unroll
                for (int t = 0; t < 8; ++t) o[t] = oc[t];
            } else {
                const float mn = (mc > m) ? mc : m;
                const float al = exp_f(m - mn), be = exp_f(mc - mn);
                l = (l * al) + (lc[0] * be);
#pragma unroll
                for (int t = 0; t < 8; ++t)
#pragma unroll
                    for (int v = 0; v < 4; ++v) o[t][v] = (o[t][v] * al) + (oc[t][v] * be);
                m = mn;
            }
        }
    };
    for (int c = c0; c < c1; ++c) {
        // the fast path needs the whole workgroup to agree: its first rows see the whole chunk
        // (every later row does too) and the chunk ends inside the block's range
        const bool wg_fast = (c + 1) * CHUNK <= q_start + r0 && (c + 1) * CHUNK <= imax + 1;
        if (wg_fast) chunk(c, std::integral_constant<bool, true>());
        else chunk(c, std::integral_constant<bool, false>());
    }
    if (SPLIT && cut) return;                           // the merge kernel writes these rows
    // ------------------------------------------------------------------ output
    const int rel = wrow0 + r;
    if (rel < r0 + nrows) {
        float* out = O + (((int64_t)b * Tq + rel) * Hq + h) * D + 32 * g;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float4 y0, y1;
            y0.x = o[0][v] / l; y0.y = o[1][v] / l; y0.z = o[2][v] / l; y0.w = o[3][v] / l;
            y1.x = o[4][v] / l; y1.y = o[5][v] / l; y1.z = o[6][v] / l; y1.w = o[7][v] / l;
            *reinterpret_cast<float4*>(out + 8 * v) = y0;
            *reinterpret_cast<float4*>(out + 8 * v + 4) = y1;
        }
    }
}

// ------------------------------------------------------------------- decode --
// attn_decode_partial_kernel: one workgroup per (b, kv head g, chunk c), the G = Hq / Hkv
// query heads of g together (G <= GT, the template bound).  Thread j owns key j of the chunk
// for the scores: s_j = dot_KS(q, k_j, 128) * scale runs its chain over d ascending with one
// accumulator per head.  K streams through LDS in four 32-wide d slices of all 256 keys (row
// segments of 128 bytes, rows padded to 33 floats so each thread's row walk is bank-conflict
// free); the chain simply continues from one slice to the next.  Then per head m_c = max,
// p_j = exp_f(s_j - m_c), and V streams through LDS in 64-key blocks while thread (head, d)
// runs o_c[d] = fma(p_j, v_j[d], o_c[d]) and l_c = l_c + p_j for j ascending.  Every stage
// is prefetched into registers one stage ahead; about 40 KB of LDS for G = 4 lets four
// workgroups share a CU, so loads of one overlap the arithmetic of another.
// attn_decode_merge_kernel: per (b, q head), folds the chunk partials in ascending order,
// m' = max(m, m_c), a = exp_f(m - m'), b = exp_f(m_c - m'), l = l a + l_c b, o = o a + o_c b.
// The running maximum is a parallel prefix scan (max is exact, so any grouping gives the
// sequential values) and every chunk's (a, b) pair is then evaluated in parallel -- the same
// values the sequential loop computes -- so the 128 threads (one per d) only run the fold.
constexpr int GMAX = 16;
constexpr int KSL = 32;               // d per K stage
constexpr int KSLD = KSL + 1;         // padded K stage row
constexpr int NKST = D / KSL;         // K stages
constexpr int VKEYS = 64;             // keys per V stage
constexpr int DBUF = CHUNK * KSLD;    // stage buffer (floats); >= VKEYS * D

template <int DT, int GT>
__global__ __launch_bounds__(256) void attn_decode_partial_kernel(
    const void* __restrict__ Q, const void* __restrict__ Kc, const void* __restrict__ Vc,
    const int32_t* __restrict__ pos, int Tmax, int Hq, int Hkv, float scale, int nchunks,
    float* __restrict__ ws) {
    __shared__ __attribute__((aligned(16))) float Buf[DBUF];
    __shared__ __attribute__((aligned(16))) float Qs[GT][D];
    __shared__ __attribute__((aligned(16))) float Ps[GT][CHUNK];
    __shared__ float Ms[GT];
    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int G = Hq / Hkv;
    const int p = pos[b];
    if (p < 0 || p >= Tmax) return;             // invalid position: the merge writes NaN
    const int kbase = c * CHUNK;
    if (kbase > p) return;                      // empty chunk: never folded
    const int nk = min(CHUNK, p + 1 - kbase);   // keys of this chunk for this row
    const int nvs = (nk + VKEYS - 1) / VKEYS;   // V stages needed
    const int nst = NKST + nvs;
    const int tid = threadIdx.x;
    const int64_t kvbase = ((int64_t)b * Hkv + g) * Tmax * D;

    for (int e = tid; e < G * (D / 4); e += 256) {
        const int hh = e / (D / 4), d4 = (e % (D / 4)) * 4;
        float v[4];
        load4<DT>(Q, ((int64_t)b * Hq + g * G + hh) * D + d4, v);
        *reinterpret_cast<float4*>(&Qs[hh][d4]) = make_float4(v[0], v[1], v[2], v[3]);
    }
    // stage st < NKST: d slice [32 st, 32 st + 32) of keys 0..255 (rows past nk repeat row
    // nk - 1, a valid row whose values are never used); stage NKST + v: keys [64 v, 64 v + 64)
    float pre[8][4];
    auto load_stage = [&](int st) {
        if (st < NKST) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int q = tid + 256 * i, row = q >> 3, c4 = q & 7;
                load4<DT>(Kc, kvbase + (int64_t)(kbase + min(row, nk - 1)) * D + st * KSL + 4 * c4, pre[i]);
            }
        } else {
            const int j0 = (st - NKST) * VKEYS;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int q = tid + 256 * i, row = q >> 5, c4 = q & 31;
                load4<DT>(Vc, kvbase + (int64_t)(kbase + min(j0 + row, nk - 1)) * D + 4 * c4, pre[i]);
            }
        }
    };
    auto store_stage = [&](int st) {
        if (st < NKST) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int q = tid + 256 * i, row = q >> 3, c4 = q & 7;
                float* dst = Buf + row * KSLD + 4 * c4;
                dst[0] = pre[i][0]; dst[1] = pre[i][1]; dst[2] = pre[i][2]; dst[3] = pre[i][3];
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int q = tid + 256 * i, row = q >> 5, c4 = q & 31;
                *reinterpret_cast<float4*>(Buf + row * D + 4 * c4) =
                    make_float4(pre[i][0], pre[i][1], pre[i][2], pre[i][3]);
            }
        }
    };

    // ---- scores: thread tid owns key tid
    float acc[GT];
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) acc[hh] = 0.0f;
    load_stage(0);
    for (int st = 0; st < NKST; ++st) {
        __syncthreads();
        store_stage(st);
        __syncthreads();
        load_stage(st + 1);                     // the next K slice, or the first V block
        const float* kr = Buf + tid * KSLD;
#pragma unroll
        for (int dd = 0; dd < KSL; dd += 4) {
            const float k0 = kr[dd], k1 = kr[dd + 1], k2 = kr[dd + 2], k3 = kr[dd + 3];
#pragma unroll
            for (int hh = 0; hh < GT; ++hh) {
                if (hh < G) {
                    const float4 qv = *reinterpret_cast<const float4*>(&Qs[hh][st * KSL + dd]);
                    float a = acc[hh];
                    a = __builtin_fmaf(qv.x, k0, a);
                    a = __builtin_fmaf(qv.y, k1, a);
                    a = __builtin_fmaf(qv.z, k2, a);
                    a = __builtin_fmaf(qv.w, k3, a);
                    acc[hh] = a;
                }
            }
        }
    }
    if (tid < nk) {
#pragma unroll
        for (int hh = 0; hh < GT; ++hh)
            if (hh < G) Ps[hh][tid] = acc[hh] * scale;
    }
    __syncthreads();
    // ---- chunk max per head (wavefront w reduces heads w, w + 4, ...), then p
    const int lane = tid % 64, w = tid / 64;
    for (int hh = w; hh < G; hh += 4) {
        float mc = -__builtin_inff();
        for (int jj = lane; jj < nk; jj += 64) { const float sv = Ps[hh][jj]; mc = (sv > mc) ? sv : mc; }
        for (int off = 32; off >= 1; off >>= 1) { const float t = __shfl_xor(mc, off); mc = (t > mc) ? t : mc; }
        if (lane == 0) Ms[hh] = mc;
    }
    __syncthreads();
    if (tid < nk) {
#pragma unroll
        for (int hh = 0; hh < GT; ++hh)
            if (hh < G) Ps[hh][tid] = exp_f(Ps[hh][tid] - Ms[hh]);
    }
    // ---- o_c[d] and l_c, keys ascending; thread owns d = tid % D of heads tid / D + 2u
    constexpr int NO = GT >= 2 ? GT / 2 : 1;
    const int d = tid % D, hb = tid / D;
    float oc[NO], lc[NO];
#pragma unroll
    for (int u = 0; u < NO; ++u) { oc[u] = 0.0f; lc[u] = 0.0f; }
    for (int st = NKST; st < nst; ++st) {
        __syncthreads();
        store_stage(st);
        __syncthreads();
        if (st + 1 < nst) load_stage(st + 1);
        const int j0 = (st - NKST) * VKEYS;
        const int n = min(VKEYS, nk - j0);
        if (n == VKEYS) {
#pragma unroll 4
            for (int jj = 0; jj < VKEYS; jj += 4) {
                const float v0 = Buf[(jj + 0) * D + d], v1 = Buf[(jj + 1) * D + d];
                const float v2 = Buf[(jj + 2) * D + d], v3 = Buf[(jj + 3) * D + d];
#pragma unroll
                for (int u = 0; u < NO; ++u) {
                    const int hh = hb + 2 * u;
                    if (hh < G) {
                        const float4 pv = *reinterpret_cast<const float4*>(&Ps[hh][j0 + jj]);
                        float o = oc[u], l = lc[u];
                        o = __builtin_fmaf(pv.x, v0, o); l = l + pv.x;
                        o = __builtin_fmaf(pv.y, v1, o); l = l + pv.y;
                        o = __builtin_fmaf(pv.z, v2, o); l = l + pv.z;
                        o = __builtin_fmaf(pv.w, v3, o); l = l + pv.w;
                        oc[u] = o; lc[u] = l;
                    }
                }
            }
        } else {
            for (int jj = 0; jj < n; ++jj) {
                const float v = Buf[jj * D + d];
#pragma unroll
                for (int u = 0; u < NO; ++u) {
                    const int hh = hb + 2 * u;
                    if (hh < G) {
                        const float pj = Ps[hh][j0 + jj];
                        oc[u] = __builtin_fmaf(pj, v, oc[u]);
                        lc[u] = lc[u] + pj;
                    }
                }
            }
        }
    }
    const int D2 = D + 2;
#pragma unroll
    for (int u = 0; u < NO; ++u) {
        const int hh = hb + 2 * u;
        if (hh < G) {
            float* dst = ws + (((int64_t)b * Hq + g * G + hh) * nchunks + c) * D2;
            dst[2 + d] = oc[u];
            if (d == 0) { dst[0] = Ms[hh]; dst[1] = lc[u]; }
        }
    }
}

constexpr int MB1 = 128;      // chunk partials requested at once (a 32k context: 128 chunks)
constexpr int MBAT = 32;      // further partials per register batch beyond those
constexpr int MFG = 16;       // merge factors read from LDS per group

// One workgroup of D threads per (row b, query head h); thread d folds o[d].  The chunk maxima
// and sums of the row go to LDS sized for the call's chunk count (5 floats per chunk), the
// running maximum is scanned by one thread exactly as the fold takes it, and every chunk's
// (alpha, beta) pair is evaluated in parallel.  Each thread requests its first MB1 partials
// o_c[d] in one go, before the scan (a 32k context needs no more), and further ones MBAT at a
// time, the next batch while the current one is folded.
__global__ __launch_bounds__(D) void attn_decode_merge_kernel(const int32_t* __restrict__ pos,
                                                              int Hq, int Tmax, int nchunks,
                                                              const float* __restrict__ ws,
                                                              float* __restrict__ O) {
    extern __shared__ __attribute__((aligned(16))) float mlds[];
    const int n4 = (nchunks + 3) & ~3;  // per-array stride, whole float4s
    float* Mc = mlds;                   // chunk maxima
    float* Mr = Mc + n4;                // running maximum after chunk c
    float* Lc = Mr + n4;
    float* Al = Lc + n4;
    float* Be = Al + n4;
    const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
    const int p = pos[b];
    if (p < 0 || p >= Tmax) {
        O[((int64_t)b * Hq + h) * D + d] = __builtin_nanf("");
        return;
    }
    const int nc = p / CHUNK + 1;
    const int D2 = D + 2;
    const float* src = ws + ((int64_t)b * Hq + h) * nchunks * D2;
    // partials o_c[d] of chunks 1 .. MB1 (indices past nc - 1 repeat nc - 1: valid addresses
    // whose values are never folded)
    float ov[MB1];
#pragma unroll
    for (int u = 0; u < MB1; ++u) ov[u] = src[(int64_t)min(1 + u, nc - 1) * D2 + 2 + d];
    for (int c = d; c < nc; c += D) { Mc[c] = src[(int64_t)c * D2]; Lc[c] = src[(int64_t)c * D2 + 1]; }
    for (int c = nc + d; c < ((nc + 3) & ~3); c += D) Mc[c] = 0.0f;   // padding of the last float4
    __syncthreads();
    // Running maximum Mr[c] = max(Mr[c - 1], Mc[c]) in the fold's comparison (the later value
    // only when strictly greater).  Without NaN among the maxima that comparison is associative
    // (ties can differ only in the sign of a zero, which no factor sees: exp_f(+-0) = 1), so
    // each thread scans a contiguous segment from the maximum of the segments before it; any
    // NaN sends the whole scan to one thread, in order.
    const int per = (nc + D - 1) / D;
    const int s0 = min(nc, d * per), s1 = min(nc, s0 + per);
    float seg = -__builtin_inff();
    int nan = 0;
    for (int c = s0; c < s1; ++c) {
        const float mc = Mc[c];
        nan |= mc != mc;
        seg = (mc > seg) ? mc : seg;
    }
    if (__syncthreads_or(nan)) {
        if (d == 0) {
            float m = Mc[0];
            Mr[0] = m;
            for (int c = 1; c < nc; ++c) { const float mc = Mc[c]; m = (mc > m) ? mc : m; Mr[c] = m; }
        }
    } else {
        // exclusive prefix maximum of the segment maxima over the D threads
        const int lane = d & 63, wv = d >> 6;
        float incl = seg;
        for (int off = 1; off < 64; off <<= 1) {
            const float t = __shfl_up(incl, off);
            if (lane >= off) incl = (incl > t) ? incl : t;
        }
        float excl = __shfl_up(incl, 1);
        if (lane == 0) excl = -__builtin_inff();
        // the first wavefront's total, through an Mr entry rewritten below (after the barrier)
        if (lane == 63 && wv == 0) Mr[n4 - 1] = incl;
        __syncthreads();
        if (wv == 1) {
            const float w0 = Mr[n4 - 1];
            excl = (excl > w0) ? excl : w0;
        }
        __syncthreads();
        float m = excl;
        for (int c = s0; c < s1; ++c) {
            const float mc = Mc[c];
            m = (c == 0) ? mc : ((mc > m) ? mc : m);
            Mr[c] = m;
        }
    }
    __syncthreads();
    for (int c = 1 + d; c < nc; c += D) {
        Al[c] = exp_f(Mr[c - 1] - Mr[c]);
        Be[c] = exp_f(Mc[c] - Mr[c]);
    }
    __syncthreads();
    float l = Lc[0], o = src[2 + d];
    // chunks 1 .. MB1 from the registers requested first; the factors of MFG chunks are read
    // from LDS ahead of their part of the serial fold
#pragma unroll
    for (int g0 = 0; g0 < MB1; g0 += MFG) {
        if (1 + g0 < nc) {
            float fa[MFG], fb[MFG], fl[MFG];
#pragma unroll
            for (int u = 0; u < MFG; ++u) {
                const int cc = min(1 + g0 + u, nc - 1);
                fa[u] = Al[cc]; fb[u] = Be[cc]; fl[u] = Lc[cc];
            }
#pragma unroll
            for (int u = 0; u < MFG; ++u) {
                if (1 + g0 + u < nc) {
                    l = (l * fa[u]) + (fl[u] * fb[u]);
                    o = (o * fa[u]) + (ov[g0 + u] * fb[u]);
                }
            }
        }
    }
    // longer contexts: the remaining chunks, MBAT partials at a time
    if (1 + MB1 < nc) {
        float cur[MBAT], nxt[MBAT];
#pragma unroll
        for (int u = 0; u < MBAT; ++u) cur[u] = src[(int64_t)min(1 + MB1 + u, nc - 1) * D2 + 2 + d];
        for (int c0 = 1 + MB1; c0 < nc; c0 += MBAT) {
            if (c0 + MBAT < nc) {
#pragma unroll
                for (int u = 0; u < MBAT; ++u) nxt[u] = src[(int64_t)min(c0 + MBAT + u, nc - 1) * D2 + 2 + d];
            }
#pragma unroll
            for (int u = 0; u < MBAT; ++u) {
                const int cc = c0 + u;
                if (cc < nc) {
                    l = (l * Al[cc]) + (Lc[cc] * Be[cc]);
                    o = (o * Al[cc]) + (cur[u] * Be[cc]);
                }
            }
#pragma unroll
            for (int u = 0; u < MBAT; ++u) cur[u] = nxt[u];
        }
    }
    O[((int64_t)b * Hq + h) * D + d] = o / l;
}

// The fold of the split prefill: rows see few chunks (a row at position p has p / 256 + 1), so
// each thread (row, head, d) runs the sequential merge itself -- running maximum in the same
// comparison, m' = (m_c > m) ? m_c : m, a = exp_f(m - m'), b = exp_f(m_c - m'), l = l a + l_c b,
// o = o a + o_c b, chunks ascending from (m_0, l_0, o_0) -- the arithmetic of the decode merge
// and of the single-task loop.  Partials row y is query row r0 + y % (Tq - r0) of sequence
// y / (Tq - r0).  One workgroup per (row, head).
__global__ __launch_bounds__(D) void attn_prefill_merge_kernel(int Hq, int Tq, int q_start, int r0, int nchunks,
                                                               const float* __restrict__ ws,
                                                               float* __restrict__ O) {
    const int h = blockIdx.x, y = blockIdx.y, d = threadIdx.x;
    const int nsr = Tq - r0, row = r0 + y % nsr;
    const int nc = (q_start + row) / CHUNK + 1;
    const int D2 = D + 2;
    const float* src = ws + ((int64_t)y * Hq + h) * nchunks * D2;
    float m = src[0], l = src[1], o = src[2 + d];
    for (int c = 1; c < nc; ++c) {
        const float* pc = src + (int64_t)c * D2;
        const float mc = pc[0], lc = pc[1], oc = pc[2 + d];
        const float mn = (mc > m) ? mc : m;
        const float al = exp_f(m - mn), be = exp_f(mc - mn);
        l = (l * al) + (lc * be);
        o = (o * al) + (oc * be);
        m = mn;
    }
    O[(((int64_t)(y / nsr) * Tq + row) * Hq + h) * D + d] = o / l;
}

}  // namespace

template <int NW, int SBK, bool SPLIT>
hipError_t launch_prefill_nw(const AttnArgs& a, const PrefillSplit& sp, int ntasks, hipStream_t st) {
    dim3 grid((SPLIT ? ntasks : (a.Tq + 16 * NW - 1) / (16 * NW)) * a.Hq * a.B);
    if (a.dtype == 1)
        hipLaunchKernelGGL((attn_prefill_kernel<1, NW, SBK, SPLIT>), grid, dim3(64 * NW), 0, st, a.Q, a.Kc, a.Vc,
                           a.B, a.Tq, a.q_start, a.Tmax, a.Hq, a.Hkv, a.scale, a.O, sp);
    else
        hipLaunchKernelGGL((attn_prefill_kernel<0, NW, SBK, SPLIT>), grid, dim3(64 * NW), 0, st, a.Q, a.Kc, a.Vc,
                           a.B, a.Tq, a.q_start, a.Tmax, a.Hq, a.Hkv, a.scale, a.O, sp);
    return hipGetLastError();
}

// 128-row workgroups (8 wavefronts, 64-key sub-blocks) when they give at least two per CU;
// else 64-row ones (4 wavefronts, 32-key sub-blocks) for twice the grid.  The rows' bits do
// not depend on the choice.
int attention_prefill_waves(int64_t B, int64_t Tq, int64_t Hq) {
    const int64_t wg128 = ((Tq + 127) / 128) * Hq * B;
    return wg128 >= 512 ? 8 : 4;
}

// The split of a small prefill grid: with 64-row blocks giving fewer than two workgroups per CU,
// blocks are cut into tasks of PREFILL_SPLIT_R chunks.  Returns the task count (0: no split).
constexpr int PREFILL_SPLIT_R = 1;
int64_t prefill_split_plan(int64_t B, int64_t Tq, int64_t q_start, int64_t Hq, int* R, int* r_split, int* nch) {
    if (attention_prefill_waves(B, Tq, Hq) != 4) return 0;
    const int64_t BQ = 64, nqb = (Tq + BQ - 1) / BQ;
    if (nqb * Hq * B >= 512) return 0;
    int64_t ntasks = 0, first = -1;
    for (int64_t qb = 0; qb < nqb; ++qb) {
        const int64_t n = (q_start + std::min(Tq, (qb + 1) * BQ) - 1) / CHUNK + 1;
        ntasks += (n + PREFILL_SPLIT_R - 1) / PREFILL_SPLIT_R;
        if (first < 0 && n > PREFILL_SPLIT_R) first = qb;
    }
    if (first < 0) return 0;                      // no block has more than R chunks
    *R = PREFILL_SPLIT_R;
    *r_split = (int)(first * BQ);
    *nch = (int)((q_start + Tq + CHUNK - 1) / CHUNK);
    return ntasks;
}

size_t prefill_split_ws_bytes(int64_t B, int64_t Tq, int64_t q_start, int64_t Hq) {
    int R, r_split, nch;
    if (!prefill_split_plan(B, Tq, q_start, Hq, &R, &r_split, &nch)) return 0;
    return sizeof(float) * (size_t)(B * (Tq - r_split) * Hq * (int64_t)nch * (D + 2));
}

hipError_t launch_attention_prefill(const AttnArgs& a, float* ws, size_t ws_bytes, hipStream_t st) {
    if (ws) {
        PrefillSplit sp{0, 0, 0, ws};
        const int64_t ntasks = prefill_split_plan(a.B, a.Tq, a.q_start, a.Hq, &sp.R, &sp.r_split, &sp.nch);
        if (ntasks > 0 && ws_bytes >= prefill_split_ws_bytes(a.B, a.Tq, a.q_start, a.Hq)) {
            hipError_t e = launch_prefill_nw<4, 32, true>(a, sp, (int)ntasks, st);
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL(attn_prefill_merge_kernel, dim3(a.Hq, a.B * (a.Tq - sp.r_split)), dim3(D), 0, st,
                               a.Hq, a.Tq, a.q_start, sp.r_split, sp.nch, ws, a.O);
            return hipGetLastError();
        }
    }
    const PrefillSplit none{0, 0, 0, nullptr};
    if (attention_prefill_waves(a.B, a.Tq, a.Hq) == 8) return launch_prefill_nw<8, 64, false>(a, none, 0, st);
    return launch_prefill_nw<4, 32, false>(a, none, 0, st);
}

namespace {

template <int DT, int GT>
hipError_t launch_partial(const AttnArgs& a, const int32_t* pos, float* ws, int nchunks, hipStream_t st) {
    dim3 grid(nchunks, a.Hkv, a.B);
    hipLaunchKernelGGL((attn_decode_partial_kernel<DT, GT>), grid, dim3(256), 0, st, a.Q, a.Kc, a.Vc,
                       pos, a.Tmax, a.Hq, a.Hkv, a.scale, nchunks, ws);
    return hipGetLastError();
}

template <int DT>
hipError_t launch_partial_dt(const AttnArgs& a, const int32_t* pos, float* ws, int nchunks, hipStream_t st) {
    const int G = a.Hq / a.Hkv;
    if (G <= 1) return launch_partial<DT, 1>(a, pos, ws, nchunks, st);
    if (G <= 2) return launch_partial<DT, 2>(a, pos, ws, nchunks, st);
    if (G <= 4) return launch_partial<DT, 4>(a, pos, ws, nchunks, st);
    if (G <= 8) return launch_partial<DT, 8>(a, pos, ws, nchunks, st);
    return launch_partial<DT, GMAX>(a, pos, ws, nchunks, st);
}

}  // namespace

// Scratch memory of the allocation-free decode entry point: the chunk partials of one call
// (B * Hq * ceil(Tmax / 256) * (D + 2) floats) for callers that cannot allocate.  Each GPU the
// library runs on holds its own copy until the process ends; every call on that GPU shares it,
// so calls that overlap on one GPU race.  Nothing needs clearing: the partial kernel writes
// every (row, head, chunk) entry the merge reads, in the same call.
static __device__ __align__(256) unsigned char scratch[DECODE_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex scratch_mutex;
void* scratch_ptr[MAX_DEVICES];   // device address of `scratch` on each GPU, looked up once
}  // namespace

// The device address of the current GPU's copy of `scratch`, looked up with that GPU current the
// first time it is needed (the array's name on the host is only a stand-in for the symbol).
hipError_t decode_scratch(float** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        scratch_ptr[dev] = p;
    }
    *out = reinterpret_cast<float*>(scratch_ptr[dev]);
    return hipSuccess;
}

hipError_t launch_attention_decode(const AttnArgs& a, const int32_t* pos, float* ws, hipStream_t st) {
    const int nchunks = (a.Tmax + CHUNK - 1) / CHUNK;
    hipError_t e = a.dtype == 1 ? launch_partial_dt<1>(a, pos, ws, nchunks, st)
                                : launch_partial_dt<0>(a, pos, ws, nchunks, st);
    if (e != hipSuccess) return e;
    // LDS: maxima, running maxima, sums and both factors of every chunk (the chunk count
    // rounded up to whole float4s for the scan's vector reads)
    const int nch4 = (nchunks + 3) & ~3;
    hipLaunchKernelGGL(attn_decode_merge_kernel, dim3(a.Hq, a.B), dim3(D), 5 * nch4 * sizeof(float), st, pos,
                       a.Hq, a.Tmax, nchunks, ws, a.O);
    return hipGetLastError();
}

}  // namespace invnum
