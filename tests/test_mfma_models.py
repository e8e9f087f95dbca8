"""Pins of the BF16 matrix-instruction model family (tests/mfma_models.py) against the exact
rational definitions in tests/exact.py: the rounding helper, the sequential and one-rounding
models, and the aligned-truncation models in their limiting cases."""
from fractions import Fraction

import numpy as np

import exact
import mfma_models as mm
import synth


def rand_bf16(seed, n, lo=-8, hi=8):
    rng = np.random.default_rng(seed)
    m = rng.uniform(1, 2, n) * rng.choice([-1, 1], n) * 2.0 ** rng.integers(lo, hi, n)
    return synth.to_bf16_bits(m.astype(np.float32))


def frac(mp):
    m, e = mp
    return Fraction(m) * Fraction(2) ** e


def test_rounding_helper_matches_exact_model():
    rng = np.random.default_rng(1)
    for _ in range(3000):
        m = int(rng.integers(-2 ** 40, 2 ** 40))
        e = int(rng.integers(-190, 80))
        want = exact.rn32(Fraction(m) * Fraction(2) ** e)
        assert exact.bits32(mm.to_f32(m, e)) == exact.bits32(want) or (m == 0 and want == 0.0)


def test_products_exact_and_sequential_model_is_fma_chain():
    for seed in range(20):
        a, b = rand_bf16(seed, 32), rand_bf16(100 + seed, 32)
        c = float(synth.normal(200 + seed, (1,))[0])
        p = mm.products(a, b)
        for (x, y), q in zip(zip(a, b), p):
            assert frac(q) == Fraction(mm.bf16_value(x)) * Fraction(mm.bf16_value(y))
        r = c
        for x, y in zip(a, b):
            r = exact.fma32(mm.bf16_value(x), mm.bf16_value(y), r)
        assert exact.bits32(mm.model_value("seq+", c, p)) == exact.bits32(r)
        tot = Fraction(c) + sum(frac(q) for q in p)
        assert exact.bits32(mm.model_value("exact", c, p)) == exact.bits32(exact.rn32(tot))


def test_align_limits():
    """With the accumulator in the group and enough guard bits, alignment loses nothing:
    'align 32/g/c/rne' equals the exact one-rounding model whenever the terms span fewer than
    g + 24 bits; with 0 guard bits it drops every term below the largest term's precision."""
    for seed in range(20):
        a, b = rand_bf16(300 + seed, 32, -2, 2), rand_bf16(400 + seed, 32, -2, 2)
        c = 1.5
        p = mm.products(a, b)
        assert mm.model_value("align 32/24/c/rne", c, p) == mm.model_value("exact", c, p)
    big = mm.f32_parts(2.0 ** 20)
    tiny = (1, -30)                           # 2^-30: below 2^(20-23) = 2^-3
    assert mm.model_value("align 32/0/c/rne", 0.0, [big, tiny] + [(0, 0)] * 30) == 2.0 ** 20
    assert mm.model_value("exact", 2.0 ** 20, [tiny] * 32) == 2.0 ** 20


def test_lane_layout_round_trip():
    A = np.arange(2 * 16 * 32).reshape(2, 16, 32)
    B = np.arange(2 * 32 * 16).reshape(2, 32, 16)
    C = np.arange(2 * 256).reshape(2, 16, 16)
    la, lb, lc = mm.to_lanes(A, B, C)
    assert la[0, 17, 3] == A[0, 1, 11] and lb[1, 40, 7] == B[1, 23, 8]
    assert np.array_equal(mm.from_lanes(lc), C)
