"""The kernel instantiations that the benchmark times, compared directly with the oracle at
shapes that route to them (each test asserts its route through inv_kernel_route).

The pinned order is per output, so a kernel's launch geometry must never change a bit; the
other GPU tests check that across sizes.  Here every instantiation the decoder runs at the
Llama-8B shapes (prefill blocks of 16384 tokens over a 32k context, decode at batch 1 and
16) is checked against the CPU oracle itself: element by element at sizes the oracle
finishes in seconds that still span many tiles and a ragged tail, and on sampled outputs
(rows spread over both row halves of the 128-row tiles, every wavefront column and the
last tile) at the benchmark's own sizes.  Bitwise batch-invariant operators with a bitwise
regression check are the Meituan page's key practice ("key practices" list).
"""
import numpy as np
import pytest

import synth
from gpu_util import assert_bitwise, bf16, f32, host, i32, requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]

D = 128
LM_KEYS = ("logprob", "margin", "top1", "top2", "recomputed")


def inv():
    import invariant_numerics_amd as m
    return m


def route(op, a, b):
    return inv().inv_kernel_route(op, a, b)


def sample_rows(M, seed, extra=()):
    """Rows from every part of a 128-row tile (both 64-row wavefront halves, first and last
    rows of 16-row groups), the first and last tiles, and a seeded spread."""
    rows = {0, 1, 15, 16, 63, 64, 65, 100, 127, 128, M - 1, M - 2, M - 64, M - 65}
    rows |= set(int(r) for r in synth.permutation(seed, M)[:16])
    rows |= set(extra)
    return np.array(sorted(r for r in rows if 0 <= r < M))


def sample_cols(N, seed, n=192):
    """Columns covering each 32-wide wavefront column of a 256-wide tile, the tile edges and
    the ragged last tile."""
    cols = {0, 31, 32, 63, 64, 127, 128, 255, 256, N - 1, N - 2, N - 33}
    cols |= set(int(c) for c in synth.permutation(seed, N)[:n])
    return np.array(sorted(c for c in cols if 0 <= c < N))


# ------------------------------------------------------------------ GEMM tiles --

@pytest.mark.parametrize("M,K,N2", [(1024, 520, 8192), (1000, 264, 8000)])
def test_gated_gemm_large_tile_matches_oracle(orc, M, K, N2):
    """Gated W1||W3 projection on the 128 x 256 tile with the SwiGLU epilogue (the
    benchmark's prefill W1||W3 instantiation), element by element: full K slices plus a
    partial slice (K = 520 = 2 x 256 + 8), ragged rows and columns."""
    assert route("gated_gemm", M, N2) == "gemm_mfma_kernel<128,256,2,4,2>"
    say("anchor gated", M, K, N2)
    X = synth.normal(12000 + K, (M, K))
    W13 = synth.bf16_normal(12001 + N2, (N2, K), 0.05)     # [gate rows | up rows]
    F = N2 // 2
    Wi = np.empty_like(W13)
    Wi[0::2], Wi[1::2] = W13[:F], W13[F:]
    got = host(inv().inv_gated_gemm(f32(X), bf16(Wi)))
    want = orc.swiglu(orc.gemm(X, W13[:F]), orc.gemm(X, W13[F:]))
    assert_bitwise(got, want, "gated %dx%dx%d" % (M, K, N2))


@pytest.mark.parametrize("M,K,N", [(1024, 264, 8192), (1030, 520, 7100)])
def test_residual_gemm_large_tile_matches_oracle(orc, M, K, N):
    """ROLE 0 projection with the residual epilogue on the 128 x 256 tile (the benchmark's
    prefill O and W2 instantiation), element by element."""
    assert route("gemm", M, N) == "gemm_mfma_kernel<128,256,2,4,0>"
    say("anchor residual", M, K, N)
    X = synth.normal(12100 + K, (M, K))
    W = synth.bf16_normal(12101 + N, (N, K), 0.05)
    R = synth.normal(12102 + N, (M, N))
    got = host(inv().inv_fixed_order_gemm(f32(X), bf16(W), R=f32(R)))
    want = (R + orc.gemm(X, W)).astype(np.float32)     # one FP32 add after the dot, as the oracle decoder
    assert_bitwise(got, want, "residual %dx%dx%d" % (M, K, N))
    got0 = host(inv().inv_fixed_order_gemm(f32(X), bf16(W)))
    assert_bitwise(got0, orc.gemm(X, W), "plain %dx%dx%d" % (M, K, N))


@pytest.mark.parametrize("name,N,K,kind", [
    ("qkv", 6144, 4096, "plain"), ("o", 4096, 4096, "residual"),
    ("w13", 28672, 4096, "gated"), ("w2", 4096, 14336, "residual")])
def test_c5_prefill_projections_sampled(orc, name, N, K, kind):
    """The four body projections of one 16384-token prefill block at the Llama-8B shapes, on
    the instantiation the benchmark times, against the oracle on sampled outputs."""
    M = 16384
    op = "gated_gemm" if kind == "gated" else "gemm"
    assert route(op, M, N) == "gemm_mfma_kernel<128,256,2,4,%d>" % (2 if kind == "gated" else 0)
    say("anchor c5 projection", name, M, N, K)
    X = synth.normal(12200 + K, (M, K))
    W = synth.bf16_normal(12201 + N, (N, K))
    rows = sample_rows(M, 12202)
    if kind == "gated":
        F = N // 2
        Wi = np.empty_like(W)
        Wi[0::2], Wi[1::2] = W[:F], W[F:]
        got = host(inv().inv_gated_gemm(f32(X), bf16(Wi)))
        cols = sample_cols(F, 12203)
        want = orc.swiglu(orc.gemm(X[rows], W[cols]), orc.gemm(X[rows], W[F + cols]))
    elif kind == "residual":
        R = synth.normal(12204 + N, (M, N))
        got = host(inv().inv_fixed_order_gemm(f32(X), bf16(W), R=f32(R)))
        cols = sample_cols(N, 12203)
        want = (R[rows][:, cols] + orc.gemm(X[rows], W[cols])).astype(np.float32)
    else:
        got = host(inv().inv_fixed_order_gemm(f32(X), bf16(W)))
        cols = sample_cols(N, 12203)
        want = orc.gemm(X[rows], W[cols])
    assert_bitwise(got[rows][:, cols], want, "%s sampled" % name)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 16, 32])
def test_c5_decode_projections_match_oracle(orc, M):
    """The decode-step projections at the Llama-8B shapes (batch 1 and 2 rows: the slice GEMV's
    VALU chains; 3 and 4: its 4x4x1 matrix chains; 16 and 32: the one- and two-tile matrix-core
    GEMVs), element by element: QKV, O and W2 with the residual, W1||W3 with the gated
    epilogue."""
    H, F, QKV = 4096, 14336, 6144
    X = synth.normal(12300 + M, (M, H))
    Xf = synth.normal(12301 + M, (M, F))
    R = synth.normal(12302 + M, (M, H))
    Wqkv = synth.bf16_normal(12303, (QKV, H))
    Wo = synth.bf16_normal(12304, (H, H))
    W13 = synth.bf16_normal(12305, (2 * F, H))
    W2 = synth.bf16_normal(12306, (H, F))
    say("anchor decode projections", M, route("gemm", M, QKV), route("gated_gemm", M, 2 * F))
    assert_bitwise(host(inv().inv_fixed_order_gemm(f32(X), bf16(Wqkv))), orc.gemm(X, Wqkv), "qkv M=%d" % M)
    assert_bitwise(host(inv().inv_fixed_order_gemm(f32(X), bf16(Wo), R=f32(R))),
                   (R + orc.gemm(X, Wo)).astype(np.float32), "o M=%d" % M)
    assert_bitwise(host(inv().inv_fixed_order_gemm(f32(Xf), bf16(W2), R=f32(R))),
                   (R + orc.gemm(Xf, W2)).astype(np.float32), "w2 M=%d" % M)
    Wi = np.empty_like(W13)
    Wi[0::2], Wi[1::2] = W13[:F], W13[F:]
    cols = sample_cols(F, 12307, 1024)
    got = host(inv().inv_gated_gemm(f32(X), bf16(Wi)))
    want = orc.swiglu(orc.gemm(X, W13[cols]), orc.gemm(X, W13[F + cols]))
    assert_bitwise(got[:, cols], want, "w13 M=%d" % M)


# ------------------------------------------------------------------ attention --

def rand_qkv(seed, B, Tq, Tmax, Hq, Hkv, bf):
    q = synth.normal(seed, (B, Tq, Hq, D))
    k = synth.normal(seed + 1, (B, Hkv, Tmax, D))
    v = synth.normal(seed + 2, (B, Hkv, Tmax, D))
    if bf:
        return synth.to_bf16_bits(q), synth.to_bf16_bits(k), synth.to_bf16_bits(v)
    return q, k, v


def dev(a):
    return bf16(a) if a.dtype == np.uint16 else f32(a)


@pytest.mark.parametrize("Tq,q_start,bf", [(512, 1536, False), (512, 1536, True), (500, 1541, False)])
def test_prefill_eight_wave_matches_oracle(orc, Tq, q_start, bf):
    """128-row, 8-wavefront prefill workgroups (the benchmark's attention instantiation):
    4 sequences x 32 query heads over 8 kv heads, a block of queries at an offset into a
    2048-slot cache, element by element.  Rows at 1536.. see six whole chunks (the
    straight-line path) and a diagonal chunk; the ragged case starts off a 64-key boundary
    and ends mid-tile."""
    B, Hq, Hkv, Tmax = 4, 32, 8, 2048
    assert route("attention_prefill", B * Hq, Tq) == "attn_prefill_kernel<DT,8,64>"
    say("anchor prefill 8-wave", Tq, q_start, bf)
    q, k, v = rand_qkv(12400 + Tq + int(bf), B, Tq, Tmax, Hq, Hkv, bf)
    got = host(inv().inv_attention_prefill(dev(q), dev(k), dev(v), q_start=q_start))
    assert_bitwise(got, orc.attention(q, k, v, q_start=q_start), "prefill 8-wave")


def test_prefill_bench_blocks_sampled(orc):
    """Both 16384-row prefill blocks of a 32k sequence (32 query heads, 8 kv heads, FP32
    cache of 32768 slots), as the benchmark launches them, against the oracle on sampled
    query rows (every head)."""
    Hq, Hkv, T, blk = 32, 8, 32768, 16384
    assert route("attention_prefill", Hq, blk) == "attn_prefill_kernel<DT,8,64>"
    say("anchor prefill bench blocks")
    q, k, v = rand_qkv(12500, 1, T, T, Hq, Hkv, False)
    kd, vd = f32(k), f32(v)
    for q0 in (0, blk):
        qb = q[:, q0:q0 + blk]
        got = host(inv().inv_attention_prefill(f32(qb), kd, vd, q_start=q0))
        for r in sample_rows(blk, 12501 + q0):
            want = orc.attention(qb[:, r:r + 1], k, v, q_start=q0 + r)
            assert_bitwise(got[:, r:r + 1], want, "block %d row %d" % (q0, r))


def test_decode_at_32k_matches_oracle(orc):
    """Decode rows at a 32k context (the benchmark's decode attention: chunk partials plus
    the ascending merge), batch 4 with ragged positions, against the oracle row."""
    B, Hq, Hkv, T = 4, 32, 8, 32768
    say("anchor decode 32k")
    k = synth.normal(12601, (B, Hkv, T, D))
    v = synth.normal(12602, (B, Hkv, T, D))
    qd = synth.normal(12603, (B, Hq, D))
    pos = np.array([32766, 32767, 256 * 77, 12345], np.int32)
    got = host(inv().inv_attention_decode(f32(qd), f32(k), f32(v), i32(pos)))
    for b in range(B):
        want = orc.attention(qd[b][None, None], k[b:b + 1], v[b:b + 1], q_start=int(pos[b]))
        assert_bitwise(got[b], want[0, 0], "decode b=%d pos=%d" % (b, pos[b]))


# ------------------------------------------------------------------- LM head --

@pytest.fixture(scope="module")
def c4():
    d = synth.c4_inputs()
    d["wd"] = bf16(d["w"])
    return d


def lm(h, wd, tgt, tau):
    r = inv().inv_lmhead_logprob_top2(f32(h), wd, i32(tgt), tau)
    return {k_: host(v_) for k_, v_ in r.items()}


@pytest.mark.parametrize("B,tau", [(1, 0.0), (1, 0.1), (1, np.inf), (2, 0.1), (4, 0.1), (8, 0.1)])
def test_lmhead_full_vocabulary_small_batch(orc, c4, B, tau):
    """The full 128256-entry vocabulary at decode batch sizes, element by element: one row
    alone (the slice GEMV's VALU chains over 1 or 2 operand rows), 2 rows (4 operand rows: its
    4x4x1 matrix chains), 4 and 8 rows (8 and 16 operand rows: the one-tile matrix-core
    GEMV)."""
    M = 2 * B if tau > 0 else B
    say("anchor lmhead", B, tau, route("gemm", M, 128256))
    got = lm(c4["h"][:B], c4["wd"], c4["target"][:B], tau)
    mode = 0 if np.isfinite(tau) else 2
    want = orc.lmhead(c4["h"][:B], c4["w"], c4["target"][:B], tau=np.float32(tau), mode=mode)
    for key in LM_KEYS:
        assert_bitwise(got[key], want[key], "B=%d tau=%s %s" % (B, tau, key))


def test_lmhead_bench_rows_sampled(orc, c4):
    """The LM head over one 16384-row prefill block (the 128 x 256 vocabulary tile for the
    primary pass and for the separate FP32 pass over the compacted rows) against the oracle
    on sampled rows, recomputed and not."""
    B = 16384
    assert route("lmhead_gemm", B, 128256) == "gemm_mfma_kernel<128,256,2,4,1>"
    say("anchor lmhead bench rows")
    h = synth.normal(12700, (B, 4096))
    tgt = synth.uniform_int(12701, (B,), 128256)
    got = lm(h, c4["wd"], tgt, 0.1)
    flagged = np.flatnonzero(got["recomputed"])
    plain = np.flatnonzero(got["recomputed"] == 0)
    assert 0 < flagged.size < B
    rows = sample_rows(B, 12702, extra=list(flagged[:6]) + list(flagged[-3:]) + list(plain[:3]))
    want = orc.lmhead(h[rows], c4["w"], tgt[rows])
    for key in LM_KEYS:
        assert_bitwise(got[key][rows], want[key], "bench rows %s" % key)
