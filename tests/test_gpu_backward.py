"""Fixed-order backward of the LayerCast matmul on the GPU: dX (sum over the N outputs, the
forward GEMM on the transposed weights) and dW (sum over the M tokens, FP32 matrix cores)
bitwise equal to the oracle on ragged shapes, at a signed-zero edge, and on sampled outputs
of full-size projections; row-independence of dX across batch sizes."""
import numpy as np
import pytest

import synth
from gpu_util import assert_bitwise, bf16, f32, host, i32, requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]


def inv():
    import invariant_numerics_amd as m
    return m


@pytest.mark.parametrize("M,N,K", [(1, 8, 4), (33, 64, 68), (300, 264, 40), (600, 520, 72),
                                   (257, 1024, 260), (31, 136, 132)])
def test_backward_matches_oracle(orc, M, N, K):
    say("gemm backward", M, N, K)
    dY = synth.normal(8100 + M, (M, N))
    X = synth.normal(8200 + K, (M, K))
    W = synth.bf16_normal(8300 + N, (N, K))
    dX, dW = inv().inv_gemm_backward(f32(dY), f32(X), bf16(W))
    want_x, want_w = orc.gemm_backward(dY, X, W)
    assert_bitwise(host(dX), want_x, "dX %dx%dx%d" % (M, N, K))
    assert_bitwise(host(dW), want_w, "dW %dx%dx%d" % (M, N, K))


def test_backward_signed_zero_and_partial_stage(orc):
    """33 tokens (a partial 32-token stage and one token of a second): products that round to
    -0 keep a token sum at -0, which the padding of the partial stage must not turn into +0."""
    say("gemm backward signed zero")
    M, N, K = 33, 8, 4
    dY = np.zeros((M, N), np.float32)
    X = np.zeros((M, K), np.float32)
    dY[:, 0] = -(2.0 ** -100)
    X[:, 0] = 2.0 ** -100            # every product is -2^-200: each fma gives -0
    dY[:, 1] = 1.0
    X[:, 1] = -0.0
    W = synth.bf16_normal(8400, (N, K))
    dX, dW = inv().inv_gemm_backward(f32(dY), f32(X), bf16(W))
    want_x, want_w = orc.gemm_backward(dY, X, W)
    assert want_w[0, 0] == 0 and np.signbit(want_w[0, 0])
    assert_bitwise(host(dW), want_w, "dW")
    assert_bitwise(host(dX), want_x, "dX")


def test_backward_only_one_gradient(orc):
    say("gemm backward dx or dw only")
    dY = synth.normal(8501, (70, 96))
    X = synth.normal(8502, (70, 44))
    W = synth.bf16_normal(8503, (96, 44))
    want_x, want_w = orc.gemm_backward(dY, X, W)
    dX, none = inv().inv_gemm_backward(f32(dY), None, bf16(W), dw=False)
    assert none is None
    assert_bitwise(host(dX), want_x, "dX only")
    none, dW = inv().inv_gemm_backward(f32(dY), f32(X), bf16(W), dx=False)
    assert none is None
    assert_bitwise(host(dW), want_w, "dW only")


@pytest.mark.parametrize("M,N,K", [(16384, 4096, 4096), (4096, 28672, 4096), (4096, 4096, 14336)])
def test_backward_full_size_sampled(orc, M, N, K):
    """Projection shapes of the 4-layer hidden-4096 decoder (the O projection over a
    16384-token block; W1||W3 and W2 over 4096 tokens): 96 sampled outputs of each gradient
    equal the oracle's; dX rows of a 1-, 7- and 64-row batch equal the full batch's rows."""
    import torch
    say("gemm backward full", M, N, K)
    dY = synth.normal(8600, (M, N), 0.01)
    X = synth.normal(8601, (M, K))
    W = synth.bf16_normal(8602, (N, K))
    dYd, Xd, Wd = f32(dY), f32(X), bf16(W)
    dX, dW = inv().inv_gemm_backward(dYd, Xd, Wd)
    dXh, dWh = host(dX), host(dW)
    rng = np.random.default_rng(M + N + K)
    rx = rng.integers(0, M, 96); cx = rng.integers(0, K, 96)
    rw = rng.integers(0, N, 96); cw = rng.integers(0, K, 96)
    say("gemm backward oracle samples")
    assert_bitwise(dXh[rx, cx], orc.gemm_backward_at("dx", dY, X, W, rx, cx), "dX samples")
    assert_bitwise(dWh[rw, cw], orc.gemm_backward_at("dw", dY, X, W, rw, cw), "dW samples")
    for rows in (1, 7, 64):
        part, _ = inv().inv_gemm_backward(dYd[:rows].contiguous(), None, Wd, dw=False)
        assert_bitwise(host(part), dXh[:rows], "dX batch %d" % rows)
    del dX, dW
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B,K,V", [(1, 8, 2), (3, 264, 1025), (5, 256, 4096)])
def test_logit_grad_matches_oracle(orc, B, K, V):
    say("logit grad", B, K, V)
    h = synth.normal(8700 + V, (B, K))
    W = synth.bf16_normal(8701 + V, (V, K), 0.1)
    tgt = synth.uniform_int(8702 + V, (B,), V)
    if B > 1:
        tgt[1] = V + 3                     # outside the vocabulary: no +1 term, logprob NaN
    coef = synth.normal(8703 + V, (B,))
    G, lp = inv().inv_lmhead_logit_grad(f32(h), bf16(W), i32(tgt), f32(coef),
                                        logprob=True)
    want_g, want_lp = orc.lmhead_logit_grad(h, W, tgt, coef)
    assert_bitwise(host(G), want_g, "G")
    got_lp = host(lp)
    assert np.array_equal(np.isnan(got_lp), np.isnan(want_lp))
    fin = ~np.isnan(want_lp)
    assert_bitwise(got_lp[fin], want_lp[fin], "logprob")


def test_logit_grad_full_vocab_and_head_backward(orc):
    """Vocabulary 128256, hidden 4096: four rows of G bitwise equal to the oracle and equal
    between batch 4 and batch 1; the head backward on G (hidden-state gradient summed over the
    128256 logits, weight gradient over the 4 tokens) equals the oracle on sampled outputs."""
    d = synth.c4_inputs(rows=4)
    h, W, tgt = d["h"], d["w"], d["target"]
    coef = np.array([1.0, -0.75, 0.5, 2.0], np.float32)
    say("logit grad full vocab")
    Wd = bf16(W)
    G = inv().inv_lmhead_logit_grad(f32(h), Wd, i32(tgt), f32(coef))
    want_g, _ = orc.lmhead_logit_grad(h, W, tgt, coef)
    Gh = host(G)
    assert_bitwise(Gh, want_g, "G full vocab")
    one = inv().inv_lmhead_logit_grad(f32(h[2:3]), Wd, i32(tgt[2:3]), f32(coef[2:3]))
    assert_bitwise(host(one)[0], Gh[2], "G batch 1 vs 4")
    say("head backward on G")
    dH, dW = inv().inv_gemm_backward(G, f32(h), Wd)
    rng = np.random.default_rng(9)
    rx = rng.integers(0, 4, 32); cx = rng.integers(0, 4096, 32)
    rw = rng.integers(0, 128256, 32); cw = rng.integers(0, 4096, 32)
    assert_bitwise(host(dH)[rx, cx], orc.gemm_backward_at("dx", want_g, h, W, rx, cx), "dH samples")
    assert_bitwise(host(dW)[rw, cw], orc.gemm_backward_at("dw", want_g, h, W, rw, cw), "dW samples")
