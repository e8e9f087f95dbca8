"""The fused QKV entry point (inv_qkv_rope_kv_append: the QKV projection with RoPE and the KV
append) against the oracle's gemm and rope in sequence: one launch for one to four rows, the
projection and the rotation kernel otherwise; bitwise equal either way, and a row whose
position lies outside the cache writes nothing."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import assert_bitwise, bf16, f32, host, i32, requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]


def inv():
    import invariant_numerics_amd as m
    return m


@pytest.mark.parametrize("M,K,Hq,Hkv", [(1, 4096, 32, 8), (2, 4096, 32, 8), (3, 4096, 32, 8), (4, 512, 4, 2),
                                        (1, 264, 2, 1), (5, 4096, 32, 8), (2, 8200, 4, 4),
                                        (4, 8200, 4, 2), (3, 72, 2, 2)])
def test_qkv_rope_kv_append_matches_oracle(orc, M, K, Hq, Hkv):
    D, Tmax, Bc = 128, 300, 5
    say("qkv rope", M, K, Hq, Hkv)
    N = (Hq + 2 * Hkv) * D
    X = synth.normal(15320 + M, (M, K))
    W = synth.bf16_normal(15322 + K, (N, K))
    cos_t, sin_t = synth.rope_tables(Tmax, D)
    seq = np.array([2, 0, 1, 4, 3][:M], np.int32)
    pos = np.array([299, 7, 150, 0, 255][:M], np.int32)
    Q = torch.full((M, Hq, D), -7.0, device="cuda")
    Kc = torch.full((Bc, Hkv, Tmax, D), -7.0, device="cuda")
    Vc = torch.full((Bc, Hkv, Tmax, D), -7.0, device="cuda")
    inv().inv_qkv_rope_kv_append(f32(X), bf16(W), Hq, Hkv, D, i32(seq), i32(pos), f32(cos_t), f32(sin_t), Q, Kc, Vc)
    qkv = orc.gemm(X, W)
    wq = orc.rope(qkv[:, :Hq * D].reshape(M, Hq, D), pos, cos_t, sin_t)
    wk = orc.rope(qkv[:, Hq * D:(Hq + Hkv) * D].reshape(M, Hkv, D), pos, cos_t, sin_t)
    wv = qkv[:, (Hq + Hkv) * D:].reshape(M, Hkv, D)
    assert_bitwise(host(Q), wq, "q")
    Kh, Vh = host(Kc), host(Vc)
    for m in range(M):
        assert_bitwise(Kh[seq[m], :, pos[m]], wk[m], "k row %d" % m)
        assert_bitwise(Vh[seq[m], :, pos[m]], wv[m], "v row %d" % m)
    written = np.zeros((Bc, Tmax), bool)
    written[seq, pos] = True
    assert np.all(Kh.transpose(0, 2, 1, 3)[~written] == -7.0) and np.all(Vh.transpose(0, 2, 1, 3)[~written] == -7.0)
    # a row outside the cache (position -1 or past Tmax) is skipped
    bad = pos.copy()
    bad[0] = -1 if M % 2 else Tmax
    Kc2 = torch.full_like(Kc, -7.0)
    Vc2 = torch.full_like(Vc, -7.0)
    inv().inv_qkv_rope_kv_append(f32(X), bf16(W), Hq, Hkv, D, i32(seq), i32(bad), f32(cos_t), f32(sin_t), Q, Kc2, Vc2)
    assert np.all(host(Kc2)[seq[0]] == -7.0) and np.all(host(Vc2)[seq[0]] == -7.0)
