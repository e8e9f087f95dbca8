"""The FP32 matrix instructions the attention and GEMM kernels use: one
v_mfma_f32_16x16x4_f32 must equal four sequential fused multiply-adds in k order
(c = fma(a_k, b_k, c), k = 0..3, each rounded once), and one v_mfma_f32_32x32x2_f32 two
(k = 0, then 1), which is the slice chain of dot_KS.  Checked against the oracle's own fma
chain on random, wide-exponent, cancelling and signed-zero/subnormal inputs."""
import numpy as np
import pytest

from gpu_util import assert_bitwise, f32, host, requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]


def wide(rng, shape, lo, hi):
    m = rng.uniform(1, 2, shape) * rng.choice([-1, 1], shape)
    return (m * 2.0 ** rng.integers(lo, hi, shape)).astype(np.float32)


def oracle_chain(orc, A, B, C):
    """D[t, i, j] = fma chain over k ascending starting from C[t, i, j] (oracle fmaf).  The
    oracle's dot starts from +0, so C enters as the first product C * 1 (exact)."""
    n, R, _ = A.shape
    D = np.empty_like(C)
    for t in range(n):
        for i in range(R):
            for j in range(R):
                x = np.concatenate([[C[t, i, j]], A[t, i, :]]).astype(np.float32)
                w = np.concatenate([[1.0], B[t, :, j]]).astype(np.float32)
                D[t, i, j] = orc.dot_ks(x, w)
    return D


def operands(kind, R, Kk, n):
    rng = np.random.default_rng({"normal": 1, "wide": 2, "cancel": 3, "tiny": 4}[kind] + 10 * Kk)
    sa, sb, sc = (n, R, Kk), (n, Kk, R), (n, R, R)
    if kind == "normal":
        A, B, C = (rng.standard_normal(s).astype(np.float32) for s in (sa, sb, sc))
    elif kind == "wide":
        A, B, C = wide(rng, sa, -12, 12), wide(rng, sb, -12, 12), wide(rng, sc, -20, 20)
    elif kind == "cancel":
        A, B, C = wide(rng, sa, 0, 3), wide(rng, sb, 0, 3), wide(rng, sc, 2, 8)
    else:  # products and sums in the subnormal range
        A, B = wide(rng, sa, -70, -60), wide(rng, sb, -70, -60)
        C = wide(rng, sc, -140, -126)
    C[C == 0] = 1.0  # the reference chain starts from C via an exact C * 1 product
    return A, B, C


@pytest.mark.parametrize("kind", ["normal", "wide", "cancel", "tiny"])
def test_mfma_f32_is_sequential_fma(orc, kind):
    import invariant_numerics_amd as inv
    say("mfma 16x16x4 check", kind)
    A, B, C = operands(kind, 16, 4, 48)
    D = host(inv.inv_mfma_f32_check(f32(A), f32(B), f32(C)))
    assert_bitwise(D, oracle_chain(orc, A, B, C), kind)


@pytest.mark.parametrize("kind", ["normal", "wide", "cancel", "tiny"])
def test_mfma32_f32_is_sequential_fma(orc, kind):
    import invariant_numerics_amd as inv
    say("mfma 32x32x2 check", kind)
    A, B, C = operands(kind, 32, 2, 12)
    D = host(inv.inv_mfma32_f32_check(f32(A), f32(B), f32(C)))
    assert_bitwise(D, oracle_chain(orc, A, B, C), kind)

