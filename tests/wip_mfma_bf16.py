"""BF16 matrix instruction (v_mfma_f32_16x16x32_bf16) through the lane-form diagnostic:
its lane layout pinned with small integers, and the search of the accumulation model family
of tests/mfma_models.py.  Not collected by pytest until it has run on the GPU."""
import numpy as np
import pytest

from gpu_util import f32, host, requires_gpu, say
from test_gpu_mfma import wide

pytestmark = [pytest.mark.gpu, requires_gpu]


# ------------------------------------------------------------- BF16 matrix core --

def bf16_operands(kind, n):
    import mfma_models as mm  # noqa: F401
    import synth
    rng = np.random.default_rng({"normal": 21, "wide": 22, "cancel": 23}[kind])
    if kind == "normal":
        A = rng.standard_normal((n, 16, 32))
        B = rng.standard_normal((n, 32, 16))
        C = rng.standard_normal((n, 16, 16))
    elif kind == "wide":
        A, B, C = wide(rng, (n, 16, 32), -10, 10), wide(rng, (n, 32, 16), -10, 10), wide(rng, (n, 16, 16), -16, 16)
    else:
        A, B, C = wide(rng, (n, 16, 32), 0, 3), wide(rng, (n, 32, 16), 0, 3), wide(rng, (n, 16, 16), 3, 9)
    return synth.to_bf16_bits(A.astype(np.float32)), synth.to_bf16_bits(B.astype(np.float32)), C.astype(np.float32)


def run_bf16(A, B, C):
    import torch
    import invariant_numerics_amd as inv
    import mfma_models as mm
    la, lb, lc = mm.to_lanes(A, B, C)
    dv = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    ld = host(inv.inv_mfma_bf16_check(dv(la), dv(lb), f32(lc)))
    return mm.from_lanes(ld)


def test_mfma_bf16_lane_layout_exact_integers():
    """Small-integer operands: every summation order gives the exact sum, so the instruction
    must return C + A B exactly under the documented lane layout (lane l holds A[l % 16][8 (l /
    16) + i], B[8 (l / 16) + i][l % 16], results D[4 (l / 16) + v][l % 16])."""
    import synth
    say("mfma bf16 layout")
    rng = np.random.default_rng(31)
    A = rng.integers(-8, 9, (16, 16, 32)).astype(np.float32)
    B = rng.integers(-8, 9, (16, 32, 16)).astype(np.float32)
    C = rng.integers(-1000, 1000, (16, 16, 16)).astype(np.float32)
    D = run_bf16(synth.to_bf16_bits(A), synth.to_bf16_bits(B), C)
    want = C.astype(np.int64) + np.einsum("tik,tkj->tij", A.astype(np.int64), B.astype(np.int64))
    assert np.array_equal(D, want.astype(np.float32))


def test_mfma_bf16_accumulation_model_search():
    """Which model of the family in tests/mfma_models.py reproduces every output bit of the
    instruction on normal, wide-exponent and cancelling operands.  The result decides whether
    the BF16 LM-head pass may use the instruction: only under a model that fits every output
    could the CPU check reproduce it."""
    import mfma_models as mm
    names = mm.family()
    alive = set(names)
    hits = {n: 0 for n in names}
    total = 0
    for kind in ("normal", "wide", "cancel"):
        say("mfma bf16 search", kind)
        A, B, C = bf16_operands(kind, 8)
        D = run_bf16(A, B, C)
        for t in range(A.shape[0]):
            for i in range(16):
                for j in range(16):
                    p = mm.products(A[t, i, :], B[t, :, j])
                    got = D[t, i, j].view(np.uint32)
                    total += 1
                    for n in list(alive) if total > 512 else names:
                        v = np.float32(mm.model_value(n, float(C[t, i, j]), p)).view(np.uint32)
                        if v == got:
                            hits[n] += 1
                        elif total > 512:
                            alive.discard(n)
            if total == 512:
                alive = {n for n in names if hits[n] == 512}
    best = sorted(hits.items(), key=lambda kv: -kv[1])[:8]
    print("[mfma bf16] outputs %d; fitting every output: %s; best: %s" % (
        total, sorted(n for n in alive if hits[n] == total), best), flush=True)
    assert total == 3 * 8 * 256
