"""fixed_order_gemm on the GPU: bitwise equal to the oracle, and rows bitwise identical
whatever M (batch size), row position and kernel variant (slice-parallel for M <= 16,
register-tiled above)."""
import numpy as np
import pytest

import synth
from gpu_util import assert_bitwise, bf16, f32, host, requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]


def inv():
    import invariant_numerics_amd as m
    return m


@pytest.mark.parametrize("M,K,N", [
    (1, 8, 5), (1, 264, 70), (2, 4096, 130), (3, 520, 257), (4, 8200, 33), (4, 72, 17), (2, 16, 1),
    (3, 8, 5), (4, 16, 300), (3, 4104, 66),
    (5, 1000, 64), (16, 4096, 33),
    (8, 8, 5), (8, 1000, 12300), (11, 520, 257), (16, 264, 12289), (13, 4104, 70), (9, 8200, 70),
    (17, 264, 129), (20, 8200, 2049), (32, 520, 12300), (33, 520, 2050), (64, 1032, 4096),
    (40, 4096, 200), (64, 768, 64), (65, 256, 300), (130, 1032, 257), (200, 4096, 129),
    (190, 264, 8300), (260, 520, 9000), (129, 264, 300), (193, 520, 8300),
    (24, 520, 6150), (17, 4104, 4100), (32, 264, 12287), (47, 264, 3072), (33, 8200, 1024),
    (40, 264, 6144), (64, 264, 8192), (49, 520, 3072),
])
def test_gemm_matches_oracle_small(orc, M, K, N):
    say("gemm", M, K, N)
    X = synth.normal(7000 + M, (M, K))
    W = synth.bf16_normal(7100 + N, (N, K))
    Y = host(inv().inv_fixed_order_gemm(f32(X), bf16(W)))
    assert_bitwise(Y, orc.gemm(X, W), "gemm %dx%dx%d" % (M, K, N))


def test_gemm_residual_epilogue(orc):
    say("gemm residual")
    X = synth.normal(7201, (37, 512))
    W = synth.bf16_normal(7202, (96, 512))
    R = synth.normal(7203, (37, 96))
    want = (R + orc.gemm(X, W)).astype(np.float32)   # float32 add, as in the oracle decoder
    got = host(inv().inv_fixed_order_gemm(f32(X), bf16(W), R=f32(R)))
    assert_bitwise(got, want, "residual")
    for rows in (4, 10, 131):                   # 131 = 128 + a 3-row tail on the skinny GEMV
        Xs = synth.normal(7204 + rows, (rows, 512))
        Rs = synth.normal(7205 + rows, (rows, 96))
        got = host(inv().inv_fixed_order_gemm(f32(Xs), bf16(W), R=f32(Rs)))
        assert_bitwise(got, (Rs + orc.gemm(Xs, W)).astype(np.float32), "residual %d rows" % rows)


@pytest.mark.parametrize("M,K,N", [(50, 264, 4096), (64, 520, 3072), (40, 1032, 2048), (29, 264, 6144),
                                   (64, 264, 6144)])
def test_gemm_row_groups_with_residual(orc, M, K, N):
    """Routes that cut the activation rows into grid rows of 32 or 16 (33-64 rows at N =
    1024-4096, 17-32 rows at N = 4097-12287), with the residual epilogue: every group's rows,
    residual rows and output rows are its own."""
    say("gemm row groups", M, K, N, inv().inv_kernel_route("gemm", M, N))
    assert "row groups" in inv().inv_kernel_route("gemm", M, N)
    X = synth.normal(7210 + M, (M, K))
    W = synth.bf16_normal(7211 + N, (N, K))
    R = synth.normal(7212 + M, (M, N))
    want = (R + orc.gemm(X, W)).astype(np.float32)
    Rd = f32(R)
    inv().inv_fixed_order_gemm(f32(X), bf16(W), R=Rd, out=Rd)
    assert_bitwise(host(Rd), want, "row groups + residual")


def test_gemm_worked_example_k3_padded():
    """0.1 + 0.2 + (-0.1) as a K = 3 dot, padded with exact zeros to K = 8: the left fold."""
    say("gemm worked example")
    x = np.zeros((1, 8), np.float32)
    x[0, :3] = np.array([0.1, 0.2, -0.1], np.float32)
    W = np.zeros((1, 8), np.uint16)
    W[0, :3] = 0x3F80
    y = host(inv().inv_fixed_order_gemm(f32(x), bf16(W)))[0, 0]
    a, b, c = np.float32(0.1), np.float32(0.2), np.float32(-0.1)
    assert y.view(np.uint32) == ((a + b) + c).view(np.uint32)
    assert y != a + (b + c)


def test_gemm_special_values(orc):
    """Identity weights reproduce X exactly; small integers give exact products."""
    say("gemm special")
    X = synth.normal(7301, (20, 512))
    Wi = np.zeros((512, 512), np.uint16)
    Wi[np.arange(512), np.arange(512)] = 0x3F80
    assert_bitwise(host(inv().inv_fixed_order_gemm(f32(X), bf16(Wi))), X, "identity")
    rng = np.random.default_rng(5)
    Xi = rng.integers(-2, 3, size=(9, 4096)).astype(np.float32)
    Wf = rng.integers(-2, 3, size=(77, 4096)).astype(np.float32)
    want = (Xi.astype(np.int64) @ Wf.astype(np.int64).T).astype(np.float32)
    assert_bitwise(host(inv().inv_fixed_order_gemm(f32(Xi), bf16(synth.to_bf16_bits(Wf)))), want, "ints")


@pytest.mark.parametrize("n,k", [(4096, 4096), (14336, 4096), (4096, 14336)])
def test_gemm_full_size_batch_invariance(orc, n, k):
    """Full sizes (4096x4096, 4096x14336 and the down projection 14336->4096): rows of
    every M in {1,3,16,64,257,512} and of a shuffled batch are bitwise the same rows;
    sampled outputs equal the oracle's."""
    say("gemm full", n, k)
    if k == 4096:
        d = synth.c3_inputs(n=n, k=k)
    else:
        d = dict(x=synth.normal(synth.SEEDS["c3_xdown"], (512, k)),
                 w=synth.bf16_normal(synth.SEEDS["c3_wdown"], (n, k)))
    X, W = d["x"], d["w"]
    Xd, Wd = f32(X), bf16(W)
    full = host(inv().inv_fixed_order_gemm(Xd, Wd))
    for M in (1, 3, 8, 12, 16, 64, 257):
        say("gemm full M", M)
        part = host(inv().inv_fixed_order_gemm(Xd[:M].contiguous(), Wd))
        assert_bitwise(part, full[:M], "M=%d" % M)
    perm = synth.permutation(7400, 512)
    shuf = host(inv().inv_fixed_order_gemm(f32(X[perm]), Wd))
    assert_bitwise(shuf, full[perm], "shuffled")
    # oracle on sampled rows and columns (each output is one row's dot product)
    rows = [0, 1, 2, 63, 64, 256, 511]
    cols = np.sort(synth.permutation(7401, n)[:192])
    want = orc.gemm(X[rows], W[cols])
    assert_bitwise(full[rows][:, cols], want, "oracle sample")


@pytest.mark.parametrize("M,K,F", [(1, 4096, 14336), (2, 264, 37), (3, 520, 70), (4, 8200, 37), (5, 1000, 64), (16, 4096, 130),
                                   (12, 520, 4200), (9, 264, 6500), (8, 4096, 14336), (6, 8456, 50), (17, 264, 129), (24, 520, 1030),
                                   (48, 264, 1100), (64, 768, 64), (65, 4096, 300), (20, 520, 3000),
                                   (64, 264, 2048),
                                   (300, 1032, 257), (190, 264, 4200), (130, 264, 300)])
def test_gated_gemm_equals_gemm_then_swiglu(orc, M, K, F):
    """inv_gated_gemm on gate/up rows interleaved equals inv_fixed_order_gemm followed by
    inv_swiglu on its even and odd columns, bit for bit, on the one-wavefront GEMV path
    (M <= 2), the 16-row GEMV path, the 32 x 32 matrix-core tiles (M <= 16 with many weight
    rows, M <= 64) and the large tiles; small shapes also match the oracle's gemm + swiglu on
    the two halves."""
    say("gated gemm", M, K, F)
    X = synth.normal(9960 + K, (M, K)) * np.float32(2)
    W13 = synth.bf16_normal(9961 + F, (2 * F, K), 0.05)
    Wi = np.empty_like(W13)
    Wi[0::2] = W13[:F]
    Wi[1::2] = W13[F:]
    Xd, Wid = f32(X), bf16(Wi)
    Y = inv().inv_fixed_order_gemm(Xd, Wid)
    ref = inv().inv_swiglu(Y[:, 0::2].contiguous(), Y[:, 1::2].contiguous())
    got = inv().inv_gated_gemm(Xd, Wid)
    assert tuple(got.shape) == (M, F)
    assert_bitwise(host(got), host(ref), "gated vs gemm + swiglu")
    if M * K * F <= 300 * 1032 * 257:
        want = orc.swiglu(orc.gemm(X, W13[:F]), orc.gemm(X, W13[F:]))
        assert_bitwise(host(got), want, "oracle")
