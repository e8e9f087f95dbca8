"""Exact rational model of IEEE-754 binary32 / bfloat16 rounding (round to nearest, ties to
even, subnormals kept), written from the format definition with Python's Fraction.
Used by the tests to pin the oracle; shares nothing with the oracle or the HIP library."""
from fractions import Fraction
import math
import struct


def f32_to_frac(x):
    return Fraction(float(x))


def round_to_format(q, mant_bits, emin, emax):
    """Round rational q to the binary format with `mant_bits` stored fraction bits,
    minimum normal exponent `emin`, maximum exponent `emax`.  Returns float or +-inf."""
    if q == 0:
        return 0.0
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    # fix off-by-one from float log2
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - mant_bits)
    m = a / quantum
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = fl * quantum
    if v >= Fraction(2) ** (emax + 1):
        return sign * math.inf
    return sign * float(v)


def rn32(q):
    return round_to_format(Fraction(q), 23, -126, 127)


def rnbf16(q):
    return round_to_format(Fraction(q), 7, -126, 127)


def f32(x):
    """Python float -> nearest binary32 value (as a Python float)."""
    return rn32(Fraction(x))


def bits32(x):
    return struct.unpack("<I", struct.pack("<f", x))[0]


def bits_bf16(x):
    return bits32(x) >> 16


def fma32(a, b, c):
    return rn32(Fraction(a) * Fraction(b) + Fraction(c))


def seq_dot32(x, w):
    """Textbook sequential dot in binary32 with one rounding per fused step, from +0."""
    c = 0.0
    for a, b in zip(x, w):
        c = fma32(a, b, c)
    return c
