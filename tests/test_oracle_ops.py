"""Pins of the oracle's compound steps: closed forms, exact special cases, textbook
sequential sums in exact rational arithmetic, float64 brute force within error bounds,
and the batch-composition invariant the pages state (a row's bits must not depend on the
other rows it is computed with)."""
from fractions import Fraction
import math

import numpy as np
import pytest

import exact
import synth
from oracle import ref64


def bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


def bf16_of(x):
    return synth.to_bf16_bits(np.asarray(x, np.float32))


# ------------------------------------------------------------------- dot_KS --

def test_dot_short_is_textbook_sequential_fma(orc):
    """K <= 256: one slice, i.e. c = fma(x_k, w_k, c) for k ascending from +0 (exact model)."""
    rng = np.random.default_rng(7)
    for K in (1, 3, 8, 37, 128, 256):
        x = rng.standard_normal(K).astype(np.float32)
        w = rng.standard_normal(K).astype(np.float32)
        got = float(orc.dot_ks(x, w))
        want = exact.seq_dot32([float(v) for v in x], [float(v) for v in w])
        assert exact.bits32(got) == exact.bits32(want), K


def test_dot_slices_then_left_fold(orc):
    """K > 256: slices of 256 summed separately, then folded left to right.  Closed-form
    cases whose result differs between this order and a single running sum."""
    K = 768
    x = np.zeros(K, np.float32)
    w = np.ones(K, np.float32)
    x[0] = 2.0 ** 25
    x[256:260] = 1.0            # slice 1 sums to 4 exactly
    # slices: c0 = 2^25, c1 = 4, c2 = 0 -> T = 2^25 + 4 (a single running sum stays at 2^25)
    assert float(orc.dot_ks(x, w)) == 2.0 ** 25 + 4
    # fold order: c0 = 1, c1 = 2^25, c2 = -2^25: ((1 + 2^25) - 2^25) = 0, not 1
    x = np.zeros(K, np.float32)
    x[0], x[256], x[512] = 1.0, 2.0 ** 25, -(2.0 ** 25)
    assert float(orc.dot_ks(x, w)) == 0.0
    # within a slice the order is ascending k: (2^25 + 1) + 1 + 1 + 1 stays 2^25 ...
    x = np.zeros(K, np.float32)
    x[0], x[1:4] = 2.0 ** 25, 1.0
    assert float(orc.dot_ks(x, w)) == 2.0 ** 25
    # ... whereas the ones first give 2^25 + 4 (reversed order inside the slice)
    x = np.zeros(K, np.float32)
    x[0:3], x[3] = 1.0, 2.0 ** 25
    x[4] = 1.0
    assert float(orc.dot_ks(x, w)) == 2.0 ** 25 + 4


def test_dot_partial_last_slice_and_fold_exact_model(orc):
    rng = np.random.default_rng(11)
    for K in (257, 520, 1000):
        x = rng.standard_normal(K).astype(np.float32)
        w = rng.standard_normal(K).astype(np.float32)
        parts = [exact.seq_dot32([float(v) for v in x[s:s + 256]], [float(v) for v in w[s:s + 256]])
                 for s in range(0, K, 256)]
        T = parts[0]
        for p in parts[1:]:
            T = exact.rn32(Fraction(T) + Fraction(p))
        assert exact.bits32(float(orc.dot_ks(x, w))) == exact.bits32(T)


def test_gemm_small_integers_exact(orc):
    """All partial sums are integers below 2^24, so every order gives the exact product."""
    rng = np.random.default_rng(3)
    M, N, K = 5, 7, 4096
    X = rng.integers(-2, 3, size=(M, K)).astype(np.float32)
    Wf = rng.integers(-2, 3, size=(N, K)).astype(np.float32)
    Y = orc.gemm(X, bf16_of(Wf))
    assert np.array_equal(Y, (X.astype(np.int64) @ Wf.astype(np.int64).T).astype(np.float32))


def test_gemm_identity_weight(orc):
    rng = np.random.default_rng(4)
    X = rng.standard_normal((9, 512)).astype(np.float32)
    W = np.zeros((512, 512), np.uint16)
    W[np.arange(512), np.arange(512)] = 0x3F80  # BF16 1.0
    assert np.array_equal(bits(orc.gemm(X, W)), bits(X))


def test_gemm_within_higham_bound(orc):
    """|Y - Y64| <= gamma_K * sum|x w|, gamma_K = K u / (1 - K u), u = 2^-24."""
    X = synth.normal(91, (16, 4096))
    W = synth.bf16_normal(92, (64, 4096))
    Y = orc.gemm(X, W).astype(np.float64)
    Wf = ref64.up(W)
    Y64 = X.astype(np.float64) @ Wf.T
    absum = np.abs(X.astype(np.float64)) @ np.abs(Wf).T
    u = 2.0 ** -24
    # slice chains have 256 terms plus a 16-term fold: depth 272
    g = 272 * u / (1 - 272 * u)
    assert np.all(np.abs(Y - Y64) <= g * absum)


def test_gemm_rows_independent_of_batch(orc):
    X = synth.normal(93, (12, 1024))
    W = synth.bf16_normal(94, (96, 1024))
    Y = orc.gemm(X, W)
    perm = synth.permutation(95, 12)
    assert np.array_equal(bits(orc.gemm(X[perm], W)), bits(Y[perm]))
    dup = np.concatenate([X[3:4], X[3:4], X[:2]])
    Yd = orc.gemm(dup, W)
    assert np.array_equal(bits(Yd[0]), bits(Y[3])) and np.array_equal(bits(Yd[1]), bits(Y[3]))
    for m in range(12):
        assert np.array_equal(bits(orc.gemm(X[m:m + 1], W)[0]), bits(Y[m]))


# ------------------------------------------------------------ GEMM backward --

def test_gemm_backward_small_integers_exact(orc):
    """Integer operands with all partial sums below 2^24: dX = dY W and dW = dY^T X exactly."""
    rng = np.random.default_rng(31)
    M, N, K = 300, 260, 40
    dY = rng.integers(-2, 3, size=(M, N)).astype(np.float32)
    X = rng.integers(-2, 3, size=(M, K)).astype(np.float32)
    Wf = rng.integers(-2, 3, size=(N, K)).astype(np.float32)
    dX, dW = orc.gemm_backward(dY, X, bf16_of(Wf))
    i64 = lambda a: a.astype(np.int64)  # noqa: E731
    assert np.array_equal(dX, (i64(dY) @ i64(Wf)).astype(np.float32))
    assert np.array_equal(dW, (i64(dY).T @ i64(X)).astype(np.float32))


def test_gemm_backward_one_hot_gradients(orc):
    """dY = e_(m, n): dX row m is up(W[n]) exactly and dW row n is X[m] exactly; every other
    output is +0."""
    X = synth.normal(301, (70, 96))
    W = synth.bf16_normal(302, (33, 96))
    for m, n in ((0, 0), (69, 32), (17, 5)):
        dY = np.zeros((70, 33), np.float32)
        dY[m, n] = 1.0
        dX, dW = orc.gemm_backward(dY, X, W)
        want_x = np.zeros_like(dX)
        want_x[m] = ref64.up(W[n]).astype(np.float32)
        want_w = np.zeros_like(dW)
        want_w[n] = X[m]
        assert np.array_equal(bits(dX), bits(want_x)) and np.array_equal(bits(dW), bits(want_w))


def test_gemm_backward_reduces_in_slices_along_the_reduced_index(orc):
    """The token sum of dW runs in 256-token slices folded left to right (closed forms that a
    single running sum would not give), and so does the output sum of dX."""
    M = 768
    dY = np.ones((M, 1), np.float32)
    X = np.zeros((M, 2), np.float32)
    X[0, 0] = 2.0 ** 25
    X[256:260, 0] = 1.0          # slices 2^25 | 4 | 0 -> 2^25 + 4
    X[0, 1], X[256, 1], X[512, 1] = 1.0, 2.0 ** 25, -(2.0 ** 25)   # fold ((1 + 2^25) - 2^25) = 0
    W = bf16_of(np.ones((1, 2), np.float32))
    _, dW = orc.gemm_backward(dY, X, W, dx=False)
    assert dW[0, 0] == 2.0 ** 25 + 4 and dW[0, 1] == 0.0
    N = 768
    dY = np.zeros((1, N), np.float32)
    dY[0, 0] = 2.0 ** 25
    dY[0, 256:260] = 1.0
    Wo = bf16_of(np.ones((N, 1), np.float32))
    dX, _ = orc.gemm_backward(dY, np.zeros((1, 1), np.float32), Wo, dw=False)
    assert dX[0, 0] == 2.0 ** 25 + 4


def test_gemm_backward_within_bound_and_sampled_outputs(orc):
    """Random operands: within the slice-then-fold error bound of the float64 products, and the
    single-output entry point gives the same bits as the full computation."""
    dY = synth.normal(303, (600, 520))
    X = synth.normal(304, (600, 72))
    W = synth.bf16_normal(305, (520, 72))
    dX, dW = orc.gemm_backward(dY, X, W)
    u = 2.0 ** -24
    Wf = ref64.up(W)
    d64 = dY.astype(np.float64)
    for got, want, absum, depth in (
            (dX, d64 @ Wf, np.abs(d64) @ np.abs(Wf), 256 + 3),
            (dW, d64.T @ X.astype(np.float64), np.abs(d64).T @ np.abs(X.astype(np.float64)), 256 + 3)):
        g = depth * u / (1 - depth * u)
        assert np.all(np.abs(got.astype(np.float64) - want) <= g * absum)
    rows = np.array([0, 599, 311]); cols = np.array([0, 71, 40])
    assert np.array_equal(bits(orc.gemm_backward_at("dx", dY, X, W, rows, cols)), bits(dX[rows, cols]))
    rows = np.array([0, 519, 260])
    assert np.array_equal(bits(orc.gemm_backward_at("dw", dY, X, W, rows, cols)), bits(dW[rows, cols]))


# ------------------------------------------------------------ logit gradient --

def test_logit_grad_zero_weights_closed_form(orc):
    """W = 0: z = 0, M = 0, S = V exactly, p = RN(1/V) for every v, and
    g_v = RN(coef * RN([v == t] - p))."""
    V, K = 3000, 64
    h = synth.normal(401, (3, K))
    W = np.zeros((V, K), np.uint16)
    tgt = np.array([0, 2999, 1234], np.int32)
    coef = np.array([1.0, -0.5, 3.0], np.float32)
    G, lp = orc.lmhead_logit_grad(h, W, tgt, coef)
    p = np.float32(1.0) / np.float32(V)
    for b in range(3):
        q = np.full(V, -p, np.float32)
        q[tgt[b]] = np.float32(1.0) - p
        want = (coef[b] * q).astype(np.float32)
        assert np.array_equal(bits(G[b]), bits(want))
    assert np.allclose(lp, -np.log(V), rtol=1e-6)


def test_logit_grad_vs_float64_and_forward(orc):
    """Against the float64 softmax gradient of the float64 logits (within 1e-5 of the largest
    entry); the rows sum to ~0; lp is the forward's FP32-pass logprob bit for bit."""
    B, K, V = 4, 256, 2500
    h = synth.normal(402, (B, K))
    W = synth.bf16_normal(403, (V, K), 0.1)
    tgt = synth.uniform_int(404, (B,), V)
    coef = np.array([1.0, -2.0, 0.25, 1.5], np.float32)
    G, lp = orc.lmhead_logit_grad(h, W, tgt, coef)
    z64 = h.astype(np.float64) @ ref64.up(W).T
    p64 = np.exp(z64 - z64.max(axis=1, keepdims=True))
    p64 /= p64.sum(axis=1, keepdims=True)
    onehot = np.zeros_like(p64)
    onehot[np.arange(B), tgt] = 1.0
    g64 = coef[:, None].astype(np.float64) * (onehot - p64)
    assert np.max(np.abs(G - g64)) <= 1e-5 * np.max(np.abs(g64))
    assert np.all(np.abs(G.astype(np.float64).sum(axis=1)) <= 1e-5 * np.abs(coef))
    fwd = orc.lmhead(h, W, tgt, mode=2)
    assert np.array_equal(bits(lp), bits(fwd["logprob"]))


# ------------------------------------------------------------------ RMSNorm --

def test_rmsnorm_constant_row_closed_form(orc):
    """x = c everywhere: y = c / sqrt(c^2 + eps) * gamma (closed form, within 2 ulp)."""
    for c in (0.5, 1.0, 3.0, -2.25, 1e-3):
        X = np.full((1, 4096), c, np.float32)
        g = np.full(4096, 0x3F80, np.uint16)
        y = orc.rmsnorm(X, g)[0]
        want = c / math.sqrt(c * c + float(np.float32(1e-5)))
        ulp = float(np.spacing(np.float32(abs(want))))
        assert np.all(np.abs(y.astype(np.float64) - want) <= 2 * ulp), c


def test_rmsnorm_vs_float64(orc):
    X = synth.normal(101, (32, 4096))
    g = synth.to_bf16_bits(np.float32(1.0) + synth.normal(102, (4096,), 0.02))
    y = orc.rmsnorm(X, g).astype(np.float64)
    y64 = ref64.rmsnorm(X, g)
    assert np.max(np.abs(y - y64) / np.maximum(np.abs(y64), 1e-3)) < 1e-6


# --------------------------------------------------------------------- RoPE --

def test_rope_position_zero_is_identity_and_matches_float64(orc):
    cos_t, sin_t = synth.rope_tables(64, 128)
    X = synth.normal(111, (10, 4, 128))
    pos = np.arange(10, dtype=np.int32) * 5
    Y = orc.rope(X, pos, cos_t, sin_t)
    assert np.array_equal(bits(Y[0]), bits(X[0]))  # cos 1, sin 0: exact
    Y64 = ref64.rope(X, pos, cos_t, sin_t)
    assert np.max(np.abs(Y - Y64)) < 4 * 2.0 ** -23 * np.max(np.abs(X))
    # the rotation preserves the norm of each (i, i+64) pair
    n0 = X[..., :64] ** 2 + X[..., 64:] ** 2
    n1 = Y64[..., :64] ** 2 + Y64[..., 64:] ** 2
    assert np.allclose(n0, n1, rtol=1e-6)


# ------------------------------------------------------------------- SwiGLU --

def test_swiglu_vs_float64(orc):
    G = synth.normal(121, (8, 2048)) * np.float32(4)
    U = synth.normal(122, (8, 2048))
    h = orc.swiglu(G, U).astype(np.float64)
    h64 = ref64.swiglu(G, U)
    tol = 4 * np.spacing(np.abs(h64).astype(np.float32)).astype(np.float64) + 1e-30
    assert np.all(np.abs(h - h64) <= tol)
    z = orc.swiglu(np.zeros((1, 4), np.float32), np.ones((1, 4), np.float32))
    assert np.all(z == 0)
    big = orc.swiglu(np.array([[100.0, -100.0, -1000.0]], np.float32), np.ones((1, 3), np.float32))
    assert big[0, 0] == 100.0 and big[0, 1] == 0.0 and big[0, 2] == 0.0


# ---------------------------------------------------------------- attention --

def _attn_inputs(seed, B, T, Hq, Hkv, D, bf=False):
    q = synth.normal(seed, (B, T, Hq, D))
    k = synth.normal(seed + 1, (B, Hkv, T, D))
    v = synth.normal(seed + 2, (B, Hkv, T, D))
    if bf:
        return bf16_of(q), bf16_of(k), bf16_of(v)
    return q, k, v


def test_attention_single_chunk_vs_float64(orc):
    q, k, v = _attn_inputs(131, 1, 200, 2, 2, 128)
    O = orc.attention(q, k, v)
    O64 = ref64.attention(q, k, v)
    assert np.max(np.abs(O - O64)) < 1e-5


def test_attention_multi_chunk_vs_float64_gqa(orc):
    """T = 600 crosses two chunk boundaries (256, 512); GQA 4 query heads per kv head."""
    q, k, v = _attn_inputs(141, 2, 600, 4, 1, 64)
    O = orc.attention(q, k, v)
    O64 = ref64.attention(q, k, v)
    assert np.max(np.abs(O - O64)) < 1e-5


def test_attention_bf16_inputs_vs_float64(orc):
    q, k, v = _attn_inputs(151, 1, 300, 2, 2, 128, bf=True)
    O = orc.attention(q, k, v)
    O64 = ref64.attention(q, k, v)
    assert np.max(np.abs(O - O64)) < 1e-5


def test_attention_unit_values_give_exactly_one(orc):
    """V = 1: o_c mirrors l_c step by step and the merge treats both alike, so out = l/l = 1."""
    q, k, _ = _attn_inputs(161, 1, 700, 2, 2, 128)
    v = np.ones_like(k)
    O = orc.attention(q, k, v)
    assert np.all(O == 1.0)


def test_attention_identical_keys_average_values(orc):
    q, _, v = _attn_inputs(171, 1, 520, 1, 1, 32)
    k = np.broadcast_to(synth.normal(172, (1, 1, 1, 32)), v.shape).copy()
    O = orc.attention(q, k, v)
    csum = np.cumsum(v[0, 0].astype(np.float64), axis=0) / np.arange(1, 521)[:, None]
    assert np.max(np.abs(O[0, :, 0, :] - csum)) < 1e-5


def test_attention_sharp_key_selects_value(orc):
    """One key far above the rest: the output is that key's value (other weights underflow)."""
    D = 16
    q = np.zeros((1, 300, 1, D), np.float32)
    q[..., 0] = 1.0
    k = np.zeros((1, 1, 300, D), np.float32)
    k[0, 0, 5, 0] = 5000.0
    v = synth.normal(181, (1, 1, 300, D))
    O = orc.attention(q, k, v, scale=np.float32(1.0))
    assert np.array_equal(O[0, 5:, 0, :], np.broadcast_to(v[0, 0, 5], (295, D)))


def test_attention_chunked_queries_and_batch_invariance(orc):
    """Rows computed in query blocks (q_start > 0), per sequence, or in a batch agree bitwise."""
    q, k, v = _attn_inputs(191, 3, 530, 2, 1, 32)
    O = orc.attention(q, k, v)
    O2 = orc.attention(q[:, 300:], k, v, q_start=300)
    assert np.array_equal(bits(O[:, 300:]), bits(O2))
    O1 = orc.attention(q[1:2], k[1:2], v[1:2])
    assert np.array_equal(bits(O[1]), bits(O1[0]))
    # a single decode row = the prefill row at that position
    Od = orc.attention(q[:, 511:512], k, v, q_start=511)
    assert np.array_equal(bits(O[:, 511:512]), bits(Od))


# ------------------------------------------------------------------ LM head --

def test_lmhead_zero_weights_closed_form(orc):
    """W = 0: every logit is 0, so S = V exactly and logprob = -log V; the top-2 tie gives
    margin 0, top1 0, top2 1, and the recompute fires (0 < tau)."""
    for V, K in ((4096, 256), (128256, 64)):
        h = synth.normal(201, (3, K))
        W = np.zeros((V, K), np.uint16)
        r = orc.lmhead(h, W, np.array([0, 5, V - 1], np.int32))
        want = -math.log(V)
        assert np.all(np.abs(r["logprob"].astype(np.float64) - want) <= np.spacing(np.float32(abs(want))))
        assert np.all(r["margin"] == 0) and np.all(r["top1"] == 0) and np.all(r["top2"] == 1)
        assert np.all(r["recomputed"] == 1)


def test_lmhead_duplicate_rows_tie_break(orc):
    h = synth.normal(211, (4, 256))
    W = synth.bf16_normal(212, (1000, 256))
    r0 = orc.lmhead(h, W, np.zeros(4, np.int32), mode=1)
    # copy each row's argmax row to a lower index and a higher index
    for i in range(4):
        W2 = W.copy()
        t = int(r0["top1"][i])
        lo, hi = (t // 2, min(999, t + 7)) if t > 0 else (0, 10)
        W2[lo] = W[t]
        W2[hi] = W[t]
        r = orc.lmhead(h[i:i + 1], W2, np.zeros(1, np.int32), mode=1)
        tied = sorted({lo, t, hi})
        assert r["top1"][0] == tied[0] and r["top2"][0] == tied[1] and r["margin"][0] == 0


def test_lmhead_threshold_limits_and_selection(orc):
    d = synth.c1_inputs(rows=32)
    P = orc.lmhead(d["h"], d["w"], d["target"], mode=1)
    F = orc.lmhead(d["h"], d["w"], d["target"], mode=2)
    r0 = orc.lmhead(d["h"], d["w"], d["target"], tau=np.float32(0.0))
    rinf = orc.lmhead(d["h"], d["w"], d["target"], tau=np.float32(np.inf))
    for key in ("logprob", "margin", "top1", "top2"):
        assert np.array_equal(r0[key], P[key]) and np.array_equal(rinf[key], F[key])
    assert np.all(r0["recomputed"] == 0) and np.all(rinf["recomputed"] == 1)
    r = orc.lmhead(d["h"], d["w"], d["target"])
    sel = P["margin"] < np.float32(0.1)
    assert np.array_equal(r["recomputed"].astype(bool), sel)
    for key in ("logprob", "margin", "top1", "top2"):
        assert np.array_equal(r[key], np.where(sel, F[key], P[key]))
    assert 0 < sel.sum() < 32


def test_lmhead_vs_float64(orc):
    """|lp - lp64| / max(|lp64|, 1) <= 1e-5 for both passes (P uses bf(h) in the reference too);
    top-2 indices agree wherever the float64 margin is clear of rounding."""
    d = synth.c1_inputs(rows=16)
    h = d["h"]
    for mode, A in ((1, ref64.up(bf16_of(h))), (2, h.astype(np.float64))):
        r = orc.lmhead(h, d["w"], d["target"], mode=mode)
        r64 = ref64.lmhead_pass(A, d["w"], d["target"])
        err = np.abs(r["logprob"] - r64["logprob"]) / np.maximum(np.abs(r64["logprob"]), 1.0)
        assert np.max(err) <= 1e-5
        clear = r64["margin"] > 1e-4
        assert np.array_equal(r["top1"][clear], r64["top1"][clear])
        assert np.max(np.abs(r["margin"] - r64["margin"])) < 1e-5


def test_lmhead_wide_vocab_tile_tail_vs_float64(orc):
    """V = 128256 = 125 full tiles + 256 entries of a partial tile."""
    h = synth.normal(221, (2, 64))
    W = synth.bf16_normal(222, (128256, 64), 0.2)
    tgt = np.array([128255, 7], np.int32)
    r = orc.lmhead(h, W, tgt, mode=2)
    r64 = ref64.lmhead_pass(h.astype(np.float64), W, tgt)
    err = np.abs(r["logprob"] - r64["logprob"]) / np.maximum(np.abs(r64["logprob"]), 1.0)
    assert np.max(err) <= 1e-5


def test_lmhead_rows_independent_of_batch(orc):
    d = synth.c1_inputs(rows=64)
    full = orc.lmhead(d["h"], d["w"], d["target"])
    for B in (1, 2, 4, 8):
        for s in range(0, 64, B):
            r = orc.lmhead(d["h"][s:s + B], d["w"], d["target"][s:s + B])
            for key in full:
                a = full[key][s:s + B]
                b = r[key]
                if a.dtype == np.float32:
                    a, b = bits(a), bits(b)
                assert np.array_equal(a, b), (B, s, key)


# ------------------------------------------------------------------ decoder --

@pytest.fixture(scope="module")
def tiny_model():
    return synth.decoder_model(synth.TINY, 640, seed_base=9000, gamma_std=0.02)


def test_decoder_tiny_vs_float64(orc, tiny_model):
    """Two layers, 4/2 heads, d 16, T = 600 (three KV chunks): all-F logprobs against the
    float64 forward within 1e-5 relative."""
    toks = synth.tokens(9100, 1, 600, synth.TINY["vocab"])[0]
    r = orc.decoder(toks, tiny_model, tau=np.float32(np.inf), return_hidden=True)
    hid64 = ref64.decoder(toks, tiny_model)
    assert np.max(np.abs(r["hidden"] - hid64) / np.maximum(np.abs(hid64), 1.0)) < 1e-5
    r64 = ref64.lmhead_pass(hid64[:-1], tiny_model["whead"], toks[1:])
    err = np.abs(r["logprob"] - r64["logprob"]) / np.maximum(np.abs(r64["logprob"]), 1.0)
    assert np.max(err) <= 1e-5
    assert np.all(r["recomputed"] == 1)


def test_decoder_prefix_and_batch_invariance(orc, tiny_model):
    """Scoring a prefix gives the same bits as the full sequence at those positions
    (prefill of T tokens vs. prefill of a shorter prompt: causal rows only)."""
    toks = synth.tokens(9200, 1, 300, synth.TINY["vocab"])[0]
    full = orc.decoder(toks, tiny_model)
    part = orc.decoder(toks[:270], tiny_model)
    for key in full:
        a, b = full[key][:269], part[key]
        if a.dtype == np.float32:
            a, b = bits(a), bits(b)
        assert np.array_equal(a, b), key


def test_decoder_storage_rounding_vs_float64(orc):
    """BF16 / FP16 activation storage: the oracle against the float64 forward that rounds at
    the same points (NumPy conversions), one layer, T = 64, four random models.  Between
    those two only rare rounding-boundary cases differ, so most final hidden values agree
    exactly; dropping any single rounding point from the oracle (checked when this pin was
    written: q, k, attention output, projection output, residual sum, norm output, gate/up,
    SwiGLU product, final norm) brings the FP16 mean to <= 0.94 and BF16 to <= 0.95."""
    cfg = dict(synth.TINY, layers=1)
    agree = {"fp16": [], "bf16": []}
    for sd in (9000, 9300, 9600, 9900):
        m = synth.decoder_model(cfg, 640, seed_base=sd, gamma_std=0.02)
        toks = synth.tokens(sd + 100, 1, 64, cfg["vocab"])[0]
        for act in agree:
            r = orc.decoder(toks, m, tau=np.float32(np.inf), return_hidden=True, act=act)["hidden"]
            h64 = ref64.decoder(toks, m, act=act)
            agree[act].append(np.mean(r.astype(np.float64) == h64))
            # every stored value is representable in the format
            if act == "fp16":
                assert np.array_equal(r, r.astype(np.float16).astype(np.float32))
            else:
                assert not np.any(r.view(np.uint32) & 0xFFFF)
            # and within a few units of the format's rounding of the float64 result
            rel = np.abs(r - h64) / np.maximum(np.abs(h64), 1.0)
            assert rel.max() < {"fp16": 2.0 ** -6, "bf16": 2.0 ** -4}[act]
    assert min(agree["bf16"]) >= 0.98, agree
    assert np.mean(agree["fp16"]) >= 0.96, agree


def test_decoder_policies_differ_and_fp32_is_layercast(orc, tiny_model):
    """The FP32 policy is the LayerCast decoder (same bits); BF16 and FP16 storage change the
    hidden states by about their unit roundoff (2^-9, 2^-12) relative to it."""
    toks = synth.tokens(9150, 1, 120, synth.TINY["vocab"])[0]
    base = orc.decoder(toks, tiny_model, return_hidden=True)
    same = orc.decoder(toks, tiny_model, return_hidden=True, act="fp32")
    for k in base:
        assert np.array_equal(bits(base[k]) if base[k].dtype == np.float32 else base[k],
                              bits(same[k]) if same[k].dtype == np.float32 else same[k]), k
    h = base["hidden"].astype(np.float64)
    for act, u in (("bf16", 2.0 ** -9), ("fp16", 2.0 ** -12)):
        r = orc.decoder(toks, tiny_model, return_hidden=True, act=act)["hidden"]
        err = np.median(np.abs(r - h) / np.maximum(np.abs(h), 1e-3))
        assert u / 4 < err < 16 * u, (act, err)


def test_oracle_greedy_consistent_with_scoring(orc, tiny_model):
    """Each greedy token is the top-1 of scoring the grown sequence, and scoring the final
    sequence gives the same top-1 at every generated position (prefix invariance)."""
    prompt = synth.tokens(9170, 1, 9, synth.TINY["vocab"])[0]
    g = orc.greedy(prompt, tiny_model, 8, act="fp16", tau=np.float32(0.1))
    seq = np.concatenate([prompt, g["tokens"]]).astype(np.int32)
    r = orc.decoder(seq, tiny_model, act="fp16", tau=np.float32(0.1), targets=np.zeros(len(seq), np.int32))
    assert np.array_equal(r["top1"][len(prompt) - 1:-1], g["tokens"])
    assert np.array_equal(bits(r["margin"][len(prompt) - 1:-1]), bits(g["margin"]))
    assert np.array_equal(g["top1"], g["tokens"])


def test_lmhead_nan_logits_never_win(orc):
    """NaN logits are unordered, so they take no part in the top-2: NaN at index 0 or 1 or in
    the middle leaves the finite logits' lowest-index maximum pair; a row with one finite
    logit pairs it with the lowest other index; an all-NaN row gives (0, 1)."""
    z = synth.normal(231, (3000,), 1.0)
    order = np.lexsort((np.arange(3000), -z))
    for nan_at in ([0], [1], [0, 1], [int(order[0])], [int(order[1]), 5]):
        y = z.copy()
        y[nan_at] = np.nan
        fin = [v for v in order if v not in nan_at]
        M, S, t1, t2 = orc.lmhead_stats(y)
        assert (t1, t2) == (fin[0], fin[1]), nan_at
        assert M == z[fin[0]] and np.isnan(S)
    y = np.full(16, np.nan, np.float32)
    assert orc.lmhead_stats(y)[2:] == (0, 1)
    y[9] = 2.0
    assert orc.lmhead_stats(y)[2:] == (9, 0)
    y[:] = np.nan
    y[0] = -1.0
    assert orc.lmhead_stats(y)[2:] == (0, 1)
