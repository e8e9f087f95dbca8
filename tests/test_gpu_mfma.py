"""The FP32 matrix instruction the GEMM and attention kernels use: one
v_mfma_f32_16x16x4_f32 must equal four sequential fused multiply-adds in k order
(c = fma(a_k, b_k, c), k = 0..3, each rounded once), which is the slice chain of dot_KS.
Checked against the oracle's own fma chain on random, wide-exponent, cancelling and
signed-zero/subnormal inputs."""
import numpy as np
import pytest

from gpu_util import assert_bitwise, f32, host, requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]


def wide(rng, shape, lo, hi):
    m = rng.uniform(1, 2, shape) * rng.choice([-1, 1], shape)
    return (m * 2.0 ** rng.integers(lo, hi, shape)).astype(np.float32)


def oracle_chain(orc, A, B, C):
    """D[t, i, j] = fma chain over k = 0..3 starting from C[t, i, j] (oracle fmaf).  The
    oracle's dot starts from +0, so C enters as the first product C * 1 (exact)."""
    n = A.shape[0]
    D = np.empty_like(C)
    for t in range(n):
        for i in range(16):
            for j in range(16):
                x = np.concatenate([[C[t, i, j]], A[t, i, :]]).astype(np.float32)
                w = np.concatenate([[1.0], B[t, :, j]]).astype(np.float32)
                D[t, i, j] = orc.dot_ks(x, w)
    return D


@pytest.mark.parametrize("kind", ["normal", "wide", "cancel", "tiny"])
def test_mfma_f32_is_sequential_fma(orc, kind):
    import invariant_numerics_amd as inv
    say("mfma check", kind)
    rng = np.random.default_rng({"normal": 1, "wide": 2, "cancel": 3, "tiny": 4}[kind])
    n = 48
    if kind == "normal":
        A, B, C = (rng.standard_normal(s).astype(np.float32) for s in ((n, 16, 4), (n, 4, 16), (n, 16, 16)))
    elif kind == "wide":
        A, B, C = wide(rng, (n, 16, 4), -12, 12), wide(rng, (n, 4, 16), -12, 12), wide(rng, (n, 16, 16), -20, 20)
    elif kind == "cancel":
        A, B, C = wide(rng, (n, 16, 4), 0, 3), wide(rng, (n, 4, 16), 0, 3), wide(rng, (n, 16, 16), 2, 8)
    else:  # products and sums in the subnormal range
        A, B = wide(rng, (n, 16, 4), -70, -60), wide(rng, (n, 4, 16), -70, -60)
        C = wide(rng, (n, 16, 16), -140, -126)
    C[C == 0] = 1.0  # the reference chain starts from C via an exact C * 1 product
    D = host(inv.inv_mfma_f32_check(f32(A), f32(B), f32(C)))
    assert_bitwise(D, oracle_chain(orc, A, B, C), kind)
