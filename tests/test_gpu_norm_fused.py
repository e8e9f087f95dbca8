"""The RMSNorm-fused projections (inv_rmsnorm_gemm, inv_rmsnorm_qkv_rope_kv_append: the norm
computed in the GEMV's prologue by every workgroup) against the oracle's rmsnorm followed by
its gemm, swiglu and rope, element by element, for one to four rows: the VALU chains (one and
two rows; 4- and 16-row workgroups) and the 4x4x1 matrix chains (three and four rows), rows of
one and of several 16-slice groups (K = 4096, 8200, 14336), a ragged last slice (K = 264, 72),
the residual epilogue and the gated (SwiGLU) epilogue."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import assert_bitwise, bf16, f32, host, i32, requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]


def inv():
    import invariant_numerics_amd as m
    return m


def _rows(seed, M, K):
    # rows of different scales, so every row has its own r
    X = synth.normal(seed, (M, K))
    return (X * np.float32([0.25, 3.0, 1.0, 40.0])[:M, None]).astype(np.float32)


def _gamma(seed, K):
    return synth.to_bf16_bits(np.float32(1.0) + synth.normal(seed, (K,), 0.1))


@pytest.mark.parametrize("M,K,N", [(1, 4096, 4096), (1, 4096, 28672), (2, 4096, 6144), (2, 4096, 16400),
                                   (3, 4096, 4096), (4, 4096, 1040), (1, 8200, 520), (4, 8200, 16400),
                                   (2, 14336, 256), (3, 264, 40), (1, 72, 24), (4, 72, 16), (1, 8, 5),
                                   (2, 16, 33), (4, 16384, 20)])
def test_rmsnorm_gemm_matches_oracle(orc, M, K, N):
    """Routes: N below 16384 with one or two rows runs 4-row workgroups, else 16-row ones;
    three and four rows run the 4x4x1 matrix chains."""
    say("rmsnorm gemm", M, K, N)
    X = _rows(16100 + M, M, K)
    g = _gamma(16102 + K, K)
    W = synth.bf16_normal(16104 + N, (N, K))
    R = synth.normal(16106 + N, (M, N))
    eps = np.float32(1e-5)
    n = orc.rmsnorm(X, g, eps)
    want = orc.gemm(n, W)
    Y = inv().inv_rmsnorm_gemm(f32(X), bf16(g), bf16(W), eps=float(eps))
    assert_bitwise(host(Y), want, "rmsnorm gemm")
    # residual epilogue: R + dot, one rounding (R aliases the output, as in the decoder)
    Rd = f32(R)
    inv().inv_rmsnorm_gemm(f32(X), bf16(g), bf16(W), eps=float(eps), R=Rd, out=Rd)
    assert_bitwise(host(Rd), (R + want).astype(np.float32), "rmsnorm gemm + residual")


@pytest.mark.parametrize("M,K,F", [(1, 4096, 14336), (2, 4096, 14336), (3, 4096, 2048), (4, 4096, 14336),
                                   (2, 264, 20), (1, 8200, 300)])
def test_rmsnorm_gated_gemm_matches_oracle(orc, M, K, F):
    say("rmsnorm gated", M, K, F)
    X = _rows(16110 + M, M, K)
    g = _gamma(16112 + K, K)
    W = synth.bf16_normal(16114 + F, (2 * F, K))       # rows interleaved gate i, up i
    eps = np.float32(1e-5)
    z = orc.gemm(orc.rmsnorm(X, g, eps), W)
    want = orc.swiglu(z[:, 0::2], z[:, 1::2])
    H = inv().inv_rmsnorm_gemm(f32(X), bf16(g), bf16(W), eps=float(eps), gated=True)
    assert_bitwise(host(H), want, "rmsnorm gated gemm")


@pytest.mark.parametrize("M,K,Hq,Hkv", [(1, 4096, 32, 8), (2, 4096, 32, 8), (3, 4096, 32, 8), (4, 4096, 32, 8),
                                        (1, 264, 2, 1), (4, 8200, 4, 2)])
def test_rmsnorm_qkv_rope_kv_append_matches_oracle(orc, M, K, Hq, Hkv):
    D, Tmax, Bc = 128, 300, 5
    say("rmsnorm qkv rope", M, K, Hq, Hkv)
    N = (Hq + 2 * Hkv) * D
    X = _rows(16120 + M, M, K)
    g = _gamma(16122 + K, K)
    W = synth.bf16_normal(16124 + K, (N, K))
    cos_t, sin_t = synth.rope_tables(Tmax, D)
    seq = np.array([2, 0, 1, 4][:M], np.int32)
    pos = np.array([299, 7, 150, 0][:M], np.int32)
    eps = np.float32(1e-5)
    Q = torch.full((M, Hq, D), -7.0, device="cuda")
    Kc = torch.full((Bc, Hkv, Tmax, D), -7.0, device="cuda")
    Vc = torch.full((Bc, Hkv, Tmax, D), -7.0, device="cuda")
    inv().inv_rmsnorm_qkv_rope_kv_append(f32(X), bf16(g), bf16(W), Hq, Hkv, D, i32(seq), i32(pos), f32(cos_t),
                                         f32(sin_t), Q, Kc, Vc, eps=float(eps))
    qkv = orc.gemm(orc.rmsnorm(X, g, eps), W)
    wq = orc.rope(qkv[:, :Hq * D].reshape(M, Hq, D), pos, cos_t, sin_t)
    wk = orc.rope(qkv[:, Hq * D:(Hq + Hkv) * D].reshape(M, Hkv, D), pos, cos_t, sin_t)
    wv = qkv[:, (Hq + Hkv) * D:].reshape(M, Hkv, D)
    assert_bitwise(host(Q), wq, "q")
    Kh, Vh = host(Kc), host(Vc)
    for m in range(M):
        assert_bitwise(Kh[seq[m], :, pos[m]], wk[m], "k row %d" % m)
        assert_bitwise(Vh[seq[m], :, pos[m]], wv[m], "v row %d" % m)


def test_rmsnorm_fused_rejects_more_than_four_rows():
    X = torch.zeros((5, 256), device="cuda")
    g = torch.zeros(256, dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((16, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(inv().InvError):
        inv().inv_rmsnorm_gemm(X, g, W)
