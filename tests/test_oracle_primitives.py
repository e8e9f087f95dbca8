"""Pins of the oracle's scalar primitives against things other than the oracle itself:
the pages' worked example, format definitions, exact rational rounding, libm in double
precision over whole input domains, and closed-form special values."""
import ctypes
from fractions import Fraction
import json
import math
import os

import numpy as np
import pytest

import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_worked_example_bf16_orders_differ(orc):
    """FP32 write-up, section 1: (0.1+0.2)+(-0.1) and 0.1+(0.2+(-0.1)) differ in low precision."""
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    a, b, c = (float(s) for s in g["operands"])
    # operands stored as BF16 (nearest), exactly as a rational rounding defines them
    ab, bb, cb = (exact.bits_bf16(exact.rnbf16(Fraction(s))) for s in g["operands"])
    assert [ab, bb, cb] == [int(x) for x in orc.bf16_rne(np.array([a, b, c], np.float32))]
    left = orc.add_bf16(orc.add_bf16(ab, bb), cb)
    right = orc.add_bf16(ab, orc.add_bf16(bb, cb))
    assert left != right  # the page's claim
    up = lambda x: float(orc.bf16_up(np.uint16(x)))  # noqa: E731
    # each BF16 step equals the exact sum rounded once to BF16
    exp_left = exact.rnbf16(Fraction(exact.rnbf16(Fraction(up(ab)) + Fraction(up(bb)))) + Fraction(up(cb)))
    exp_right = exact.rnbf16(Fraction(up(ab)) + Fraction(exact.rnbf16(Fraction(up(bb)) + Fraction(up(cb)))))
    assert up(left) == exp_left and up(right) == exp_right


def test_worked_example_fp32_and_other_formats(orc):
    a, b, c = np.float32(0.1), np.float32(0.2), np.float32(-0.1)
    left = orc.add_f32(orc.add_f32(a, b), c)
    right = orc.add_f32(a, orc.add_f32(b, c))
    # NumPy's own binary32 arithmetic and exact rational rounding agree with the oracle
    assert left == (a + b) + c and right == a + (b + c)
    assert float(left) == exact.rn32(Fraction(exact.rn32(Fraction(float(a)) + Fraction(float(b)))) + Fraction(float(c)))
    assert left != right
    # FP16 (10 fraction bits) differs too, FP64 as well (both via library arithmetic)
    h = [np.float16(x) for x in (0.1, 0.2, -0.1)]
    assert (h[0] + h[1]) + h[2] != h[0] + (h[1] + h[2])
    assert (0.1 + 0.2) + (-0.1) != 0.1 + (0.2 + (-0.1))
    # dot_KS with unit weights is the left fold of the same three terms
    d = orc.dot_ks(np.array([a, b, c], np.float32), np.ones(3, np.float32))
    assert exact.bits32(float(d)) == exact.bits32(float(left))


def test_format_bit_layouts(orc):
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))["format_bits"]
    assert g["fp32"]["fraction"] == np.finfo(np.float32).nmant
    assert g["fp16"]["fraction"] == np.finfo(np.float16).nmant
    # BF16 = the top 16 bits of FP32: 7 fraction bits, same 8-bit exponent.
    one_plus_ulp = orc.bf16_up(np.uint16(0x3F81))
    assert float(one_plus_ulp) - 1.0 == 2.0 ** -g["bf16"]["fraction"]
    # largest finite BF16: all 7 fraction bits set, exponent 127
    assert float(orc.bf16_up(np.uint16(0x7F7F))) == (2 - 2.0 ** -g["bf16"]["fraction"]) * 2.0 ** 127


def test_bf16_rne_exhaustive(numcheck):
    """All 2^32 binary32 patterns: oracle rounding == nearest-neighbour rounding in double."""
    assert numcheck.check_bf16_range(0, 1 << 32) == 0


def test_bf16_rne_special_cases(orc):
    cases = {0x3F808000: 0x3F80,  # tie, even stays
             0x3F818000: 0x3F82,  # tie, odd rounds up
             0x3F808001: 0x3F81,  # above tie
             0x7F7FFFFF: 0x7F80,  # overflow to inf
             0x80000000: 0x8000,  # -0
             0x00000001: 0x0000}  # smallest subnormal rounds to +0
    for fb, want in cases.items():
        x = np.array([fb], np.uint32).view(np.float32)
        assert int(orc.bf16_rne(x)[0]) == want, hex(fb)


def test_f16_rne_exhaustive(numcheck):
    """All 2^32 binary32 patterns: oracle FP16 rounding == nearer FP16 grid point in double."""
    assert numcheck.check_f16_range(0, 1 << 32) == 0
    assert numcheck.check_f16_up() == 0


def test_f16_rne_special_cases(orc):
    lib = orc.lib()
    cases = {65504.0: 0x7BFF,                  # largest finite
             65519.99609375: 0x7BFF,           # just below the midpoint to 2^16
             65520.0: 0x7C00,                  # midpoint ties to the even neighbour, 2^16 = inf
             2.0 ** -24: 0x0001,               # smallest subnormal
             2.0 ** -25: 0x0000,               # half of it: tie to even (zero)
             3 * 2.0 ** -25: 0x0002,           # 1.5 quanta: tie to even (2)
             2.0 ** -14 - 2.0 ** -25: 0x0400,  # rounds up into the smallest normal
             1.0 + 2.0 ** -11: 0x3C00,         # tie, even stays
             1.0 + 3 * 2.0 ** -11: 0x3C02,     # tie, odd rounds up
             -0.0: 0x8000}
    for v, want in cases.items():
        assert int(lib.orc_f16_rne(float(np.float32(v)))) == want, v
    assert float(lib.orc_f16_up(0x7BFF)) == 65504.0 and float(lib.orc_f16_up(0x0001)) == 2.0 ** -24


def test_round_act_matches_library_conversions(orc):
    """The decoder's storage rounding: FP16 against NumPy's float16 conversion and BF16
    against the nearest-BF16 definition in exact rationals, on wide random patterns and the
    FP16 edge region; FP32 is the identity."""
    rng = np.random.default_rng(77)
    u = rng.integers(0, 1 << 32, 1 << 20, dtype=np.uint64).astype(np.uint32)
    edge = (np.arange(0x33000000, 0x33000000 + (1 << 20), 7, dtype=np.uint32),      # ~2^-25
            np.arange(0x387fc000, 0x38804000, dtype=np.uint32),                      # ~2^-14
            np.arange(0x477fe000, 0x47800010, dtype=np.uint32))                      # ~65504..2^16
    x = np.concatenate([u] + list(edge)).view(np.float32)
    x = x[np.isfinite(x)]
    with np.errstate(over="ignore"):
        want16 = x.astype(np.float16).astype(np.float32)
    assert np.array_equal(orc.round_act(x, "fp16").view(np.uint32), want16.view(np.uint32))
    assert np.array_equal(orc.round_act(x, "fp32").view(np.uint32), x.view(np.uint32))
    few = x[:2000]
    want_bf = [exact.rnbf16(Fraction(float(v))) for v in few]
    got_bf = orc.round_act(few, "bf16")
    assert all(float(g) == w for g, w in zip(got_bf, want_bf) if np.isfinite(g))


def test_exp_f_within_one_ulp_everywhere(numcheck):
    """Whole finite domain of exp_f against libm exp in double (error bound: 2 ulp)."""
    w = ctypes.c_uint32()
    pos = numcheck.max_ulp_err(0, 0, 0x42B17217, ctypes.byref(w))   # [0, ln 2^128)
    neg = numcheck.max_ulp_err(0, 0x80000000, 0xC2AEAC50, ctypes.byref(w))  # [ln 2^-126, -0]
    assert pos < 1.0 and neg < 1.0, (pos, neg)


def test_log_f_within_one_ulp_everywhere(numcheck):
    w = ctypes.c_uint32()
    err = numcheck.max_ulp_err(1, 1, 0x7F7FFFFF, ctypes.byref(w))  # every positive finite float
    assert err < 1.0, (err, hex(w.value))


def test_exp_log_special_values(orc):
    cut = np.float32(-87.3365478515625)            # binary32 nearest to ln(2^-126)
    x = np.array([0.0, -0.0, cut, np.nextafter(cut, np.float32(-np.inf)), -1000.0,
                  88.72283935546875, 89.0, 1000.0], np.float32)
    y = orc.exp_f(x)
    assert y[0] == 1.0 and y[1] == 1.0
    assert 0 < y[2] < 2.0 ** -125      # at the pinned cutoff: still evaluated
    assert y[3] == 0.0 and y[4] == 0.0 and not np.signbit(y[3])  # below it: +0
    assert np.isinf(y[5]) and np.isinf(y[6]) and np.isinf(y[7])
    L = orc.log_f(np.array([1.0, 2.0, 0.5, 0.0, np.inf], np.float32))
    assert L[0] == 0.0 and not np.signbit(L[0])
    assert L[1] == np.float32(math.log(2.0)) and L[2] == np.float32(-math.log(2.0))
    assert L[3] == -np.inf and L[4] == np.inf
    # integer powers of two: log_f(2^e) = e ln2 correctly rounded (within 1 ulp)
    e = np.arange(-149, 128)
    xs = np.ldexp(np.float32(1.0), e).astype(np.float32)
    got = orc.log_f(xs).astype(np.float64)
    ref = e * math.log(2.0)
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(got - ref) <= ulp)


def test_constants_are_exact_roundings(orc):
    """Each constant equals the exact binary32 rounding of its mathematical definition."""
    fc, ic = orc.constants()
    ln2 = Fraction("0.69314718055994530941723212145817656807550013436026")
    hi = exact.rn32(ln2)
    # ln2 with 16 significant bits
    q = ln2 * 2 ** 16
    fl = q.numerator // q.denominator
    hi16 = Fraction(fl + (1 if q - fl > Fraction(1, 2) else 0), 2 ** 16)
    want = [exact.rn32(1 / ln2), hi, exact.rn32(ln2 - Fraction(hi)), exact.rn32(-126 * ln2),
            exact.rn32(128 * ln2)] + [exact.rn32(Fraction(1, math.factorial(k))) for k in range(8)] + \
           [float(hi16), exact.rn32(ln2 - hi16)] + [exact.rn32(Fraction(2, 2 * k + 1)) for k in range(1, 6)]
    assert [exact.bits32(float(v)) for v in fc] == [exact.bits32(v) for v in want]
    assert list(ic) == [256, 256, 1024, 64]


def test_attention_scale_is_exact_rounding():
    """The attention scale is RN(1/sqrt(128)) = 0x3DB504F3 (exact rational rounding of
    sqrt(2)/16), the value the binding passes by default and the oracle computes as
    1/sqrt(128) in binary32."""
    import decimal
    from fractions import Fraction
    decimal.getcontext().prec = 60
    want = exact.rn32(Fraction(decimal.Decimal(2).sqrt() / 16))
    assert exact.bits32(want) == 0x3DB504F3
    assert (np.float32(1.0) / np.sqrt(np.float32(128))).view(np.uint32) == 0x3DB504F3
    from invariant_numerics_amd import binding
    assert exact.bits32(binding.SCALE_D128) == 0x3DB504F3
