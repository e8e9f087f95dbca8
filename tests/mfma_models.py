"""Candidate models of one BF16 matrix instruction's accumulation (v_mfma_f32_16x16x32_bf16:
D = C + sum over 32 k of A[i][k] B[k][j]), in exact integer arithmetic written from the
binary32 / bfloat16 definitions.  The test suite runs the instruction through the library's
lane-form diagnostic and asks which model, if any, reproduces every output bit; a BF16 LM
head ("Greedy Decoding Is Not Precision-Invariant", abstract) could use the instruction only
under a model that does.

A value is carried as (m, e) = m * 2**e with m a Python int.  Every BF16 x BF16 product is
exact in binary32 (8 x 8 significant bits), so the models differ only in how the 32
products and the accumulator are added and rounded.

The family:
  * "seq+"/"seq-": one rounding per product in k order (ascending / descending);
  * "exact": the exact sum of the accumulator and all products, rounded once;
  * "prod-then-c": the products' exact sum rounded, then added to the accumulator;
  * "groups G": products in consecutive groups of G summed exactly, each group sum added to
    the running accumulator with one rounding;
  * "align G/g/c/r": per group of G products (and the accumulator when c is set), every
    term is truncated toward zero to g bits below binary32 precision relative to the
    largest term's leading bit, the truncated terms are summed exactly, and the result is
    rounded to binary32 by r (nearest-even or toward zero); without c, that group value is
    then added to the accumulator with one rounding to nearest even.
"""
import struct

import numpy as np


def f32_parts(x):
    """binary32 value -> (m, e) exactly (m signed int).  x is a Python float holding a binary32
    value."""
    if x == 0.0 or x != x:
        return (0, 0)
    b = struct.unpack("<I", struct.pack("<f", x))[0]
    s = -1 if b >> 31 else 1
    ex = (b >> 23) & 0xFF
    fr = b & 0x7FFFFF
    if ex == 0:
        return (s * fr, -149)
    return (s * (fr | 0x800000), ex - 150)


def to_f32(m, e, mode="rne"):
    """Round m * 2**e to binary32 (nearest-even or toward zero), subnormals kept, overflow to
    inf.  Returns a Python float."""
    if m == 0:
        return 0.0
    s = -1.0 if m < 0 else 1.0
    a = -m if m < 0 else m
    top = a.bit_length() - 1 + e           # exponent of the leading bit
    q = max(top - 23, -149)                # quantum exponent of the result
    shift = q - e
    if shift > 0:
        fl = a >> shift
        rem = a - (fl << shift)
        half = 1 << (shift - 1)
        if mode == "rne" and (rem > half or (rem == half and fl & 1)):
            fl += 1
        a, e = fl, q
    elif shift < 0:
        a, e = a << (-shift), q
    if a == 0:
        return s * 0.0
    if a.bit_length() - 1 + e > 127:
        return s * float("inf")
    return s * float(a) * 2.0 ** e


def add_exact(terms):
    """Exact sum of (m, e) terms as (m, e)."""
    nz = [(m, e) for m, e in terms if m]
    if not nz:
        return (0, 0)
    e0 = min(e for _, e in nz)
    return (sum(m << (e - e0) for m, e in nz), e0)


def trunc_rel(m, e, emax, g):
    """m * 2**e truncated toward zero to a multiple of 2**(emax - 23 - g)."""
    q = emax - 23 - g
    if e >= q:
        return (m, e)
    a = -m if m < 0 else m
    a >>= (q - e)
    return (-a if m < 0 else a, q)


def lead(m, e):
    a = -m if m < 0 else m
    return a.bit_length() - 1 + e


def model_value(name, c, prods):
    """Evaluate model `name` on accumulator c (Python float, binary32) and the 32 exact products
    (list of (m, e)).  Returns a Python float."""
    cm = f32_parts(c)
    if name in ("seq+", "seq-"):
        r = c
        for p in (prods if name == "seq+" else prods[::-1]):
            r = to_f32(*add_exact([f32_parts(r), p]))
        return r
    if name == "exact":
        return to_f32(*add_exact([cm] + prods))
    if name == "prod-then-c":
        return to_f32(*add_exact([cm, f32_parts(to_f32(*add_exact(prods)))]))
    kind, rest = name.split(" ", 1)
    if kind == "groups":
        G = int(rest)
        r = c
        for i in range(0, len(prods), G):
            r = to_f32(*add_exact([f32_parts(r)] + prods[i:i + G]))
        return r
    if kind == "align":
        G, g, inc, rm = rest.split("/")
        G, g, inc = int(G), int(g), inc == "c"
        r = c
        for i in range(0, len(prods), G):
            grp = [p for p in prods[i:i + G] if p[0]]
            rp = f32_parts(r)
            terms = grp + ([rp] if inc and rp[0] else [])
            if not terms:
                continue
            emax = max(lead(m, e) for m, e in terms)
            s = add_exact([trunc_rel(m, e, emax, g) for m, e in terms])
            if inc:
                r = to_f32(*s, mode=rm)
            else:
                r = to_f32(*add_exact([rp, f32_parts(to_f32(*s, mode=rm))]))
        return r
    raise ValueError(name)


def family():
    names = ["seq+", "seq-", "exact", "prod-then-c"] + ["groups %d" % G for G in (2, 4, 8, 16)]
    for G in (4, 8, 16, 32):
        for g in (0, 1, 2, 3, 4, 8, 24):
            for inc in ("c", "n"):
                for rm in ("rne", "rz"):
                    names.append("align %d/%d/%s/%s" % (G, g, inc, rm))
    return names


def bf16_value(bits):
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def products(a_bits, b_bits):
    """Exact products of BF16 pairs as (m, e)."""
    out = []
    for x, y in zip(a_bits, b_bits):
        ma, ea = f32_parts(bf16_value(x))
        mb, eb = f32_parts(bf16_value(y))
        out.append((ma * mb, ea + eb))
    return out


# lane form of the instruction: lane l holds A[l % 16][8 (l / 16) + i] and B[8 (l / 16) + i][l % 16]
# for i = 0..7, and results D[4 (l / 16) + v][l % 16] for v = 0..3
def to_lanes(A, B, C):
    """Matrices [n, 16, 32] (A), [n, 32, 16] (B), [n, 16, 16] (C) -> lane arrays [n, 64, 8],
    [n, 64, 8], [n, 64, 4] under the layout above."""
    n = A.shape[0]
    la = np.empty((n, 64, 8), A.dtype)
    lb = np.empty((n, 64, 8), B.dtype)
    lc = np.empty((n, 64, 4), C.dtype)
    for l in range(64):
        g, r = l // 16, l % 16
        la[:, l] = A[:, r, 8 * g:8 * g + 8]
        lb[:, l] = B[:, 8 * g:8 * g + 8, r]
        lc[:, l] = C[:, 4 * g:4 * g + 4, r]
    return la, lb, lc


def from_lanes(ld):
    """Lane results [n, 64, 4] -> D [n, 16, 16]."""
    n = ld.shape[0]
    D = np.empty((n, 16, 16), ld.dtype)
    for l in range(64):
        g, r = l // 16, l % 16
        D[:, 4 * g:4 * g + 4, r] = ld[:, l]
    return D
