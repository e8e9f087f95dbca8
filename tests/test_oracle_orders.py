"""Exact pins of the two reduction orders whose other checks are order-blind: the LM head's
softmax denominator S (vocabulary tiles of 1024, 64 lanes striding the tile, a pairwise lane
tree, tiles folded in ascending order) and the attention chunk merge (absolute chunks of 256
keys, per-chunk max / sum / weighted values, a left fold that rounds each product before the
add).  The pages name these sums as the ones whose order changes the bits (Meituan page,
principles list: attention score summation, softmax denominator reduction, logprob
accumulation) and fix no tree, so the order is a pinned choice.

Each pin is a model of that order in exact rational arithmetic (tests/exact.py: round to
nearest even from the format definition) that shares nothing with the oracle; exp_f and
log_f enter as the oracle's own scalar functions, which are pinned on their own over every
binary32 input of their domains.  Beside each model, plausible wrong orders (another lane
stride, tile or chunk size, a reversed tree, a fused merge) are evaluated on the same
inputs and shown to differ from the oracle, so a mistake of that kind fails the pin.
"""
from fractions import Fraction

import numpy as np
import pytest

import exact
import synth

TV, LW, CHUNK = 1024, 64, 256


def add32(a, b):
    return exact.rn32(Fraction(a) + Fraction(b))


def mul32(a, b):
    return exact.rn32(Fraction(a) * Fraction(b))


def sub32(a, b):
    return exact.rn32(Fraction(a) - Fraction(b))


def div32(a, b):
    return exact.rn32(Fraction(a) / Fraction(b))


def b32(x):
    return exact.bits32(float(x))


# ------------------------------------------------------------ LM-head S tree --

def exp_terms(orc, z, M):
    """e_v = exp_f(z_v - M), the subtraction rounded once (exact model), exp_f the oracle's."""
    d = np.array([sub32(float(v), float(M)) for v in z], np.float32)
    return [float(e) for e in orc.exp_f(d)]


def s_tree(e, tv=TV, lw=LW, lane_major=False, tree="pairwise", fold="left"):
    """The denominator over terms e in a given order.  Defaults are the pinned order; the
    keyword arguments describe the wrong orders the pin must reject."""
    V = len(e)
    per = tv // lw
    tiles = []
    for u in range((V + tv - 1) // tv):
        lanes = []
        for l in range(lw):
            acc = 0.0
            for j in range(per):
                v = u * tv + (l * per + j if lane_major else j * lw + l)
                if v < V:
                    acc = add32(acc, e[v])
            lanes.append(acc)
        if tree == "pairwise":            # a_l += a_{l+w} for l = 0 mod 2w, w = 1, 2, ..., 32
            w = 1
            while w < lw:
                for l in range(0, lw, 2 * w):
                    lanes[l] = add32(lanes[l], lanes[l + w])
                w *= 2
            tiles.append(lanes[0])
        elif tree == "halving":           # a_l += a_{l+w} for l < w, w = 32, 16, ..., 1
            w = lw // 2
            while w >= 1:
                for l in range(w):
                    lanes[l] = add32(lanes[l], lanes[l + w])
                w //= 2
            tiles.append(lanes[0])
        else:                             # lanes folded left to right
            acc = lanes[0]
            for a in lanes[1:]:
                acc = add32(acc, a)
            tiles.append(acc)
    if fold == "left":
        S = tiles[0]
        for t in tiles[1:]:
            S = add32(S, t)
        return S
    while len(tiles) > 1:                 # pairwise over tiles
        tiles = [add32(tiles[i], tiles[i + 1]) if i + 1 < len(tiles) else tiles[i]
                 for i in range(0, len(tiles), 2)]
    return tiles[0]


def logit_rows(seed, n, V, std):
    return [synth.normal(seed + i, (V,), std) for i in range(n)]


@pytest.mark.parametrize("V", [4096 + 300, 3 * 1024])
def test_softmax_denominator_is_the_pinned_tree(orc, V):
    """S over a spread of logits (N(0, 4): terms over ~20 binades, so the order matters) is
    the pinned tree bit for bit, with a partial last tile; the top-2 and M are the row's
    lowest-index maximum pair."""
    for z in logit_rows(13000 + V, 3, V, 4.0):
        M, S, t1, t2 = orc.lmhead_stats(z)
        order = sorted(range(V), key=lambda v: (-float(z[v]), v))
        assert (t1, t2) == (order[0], order[1]) and b32(M) == b32(z[order[0]])
        assert b32(S) == b32(s_tree(exp_terms(orc, z, M)))


def test_softmax_denominator_rejects_other_orders(orc):
    """Each plausible wrong order differs from the oracle's S on these rows: lanes owning 16
    contiguous entries instead of a stride of 64, tiles of 512 or 2048, the lane tree halving
    from the top, lanes folded in sequence, tiles folded pairwise."""
    V = 4096 + 300
    rows = logit_rows(13100, 6, V, 4.0)
    stats = [orc.lmhead_stats(z) for z in rows]
    terms = [exp_terms(orc, z, st[0]) for z, st in zip(rows, stats)]
    for e, st in zip(terms, stats):
        assert b32(st[1]) == b32(s_tree(e))
    wrong = {
        "contiguous lanes": dict(lane_major=True),
        "tile 512": dict(tv=512),
        "tile 2048": dict(tv=2048),
        "halving tree": dict(tree="halving"),
        "sequential lanes": dict(tree="left"),
        "pairwise tiles": dict(fold="pairwise"),
    }
    for name, kw in wrong.items():
        differs = sum(b32(st[1]) != b32(s_tree(e, **kw)) for e, st in zip(terms, stats))
        assert differs >= 1, name


def short_term(orc, below):
    """An input d whose exp_f(d) = eps has at most 20 significant bits (so sums of up to 16
    equal terms, and doublings of them, are exact) with 1024 eps just below `below`: found by
    scanning binary32 inputs around ln(below / 1024) with the oracle's exp_f."""
    c = np.float32(np.log(below / 1024.0))
    u = int(c.view(np.uint32))
    d = np.arange(u - 4000, u + 4000, dtype=np.uint32).view(np.float32)
    e = orc.exp_f(d)
    ok = ((e.view(np.uint32) & 7) == 0) & (e.astype(np.float64) * 1024 < below) & \
         (e.astype(np.float64) * 1024 > 0.99 * below)
    i = int(np.flatnonzero(ok)[0])
    return d[i], float(e[i])


def test_softmax_denominator_tile_crossing_closed_form(orc):
    """Closed form that only an ascending tile fold gives.  Four tiles: the row's maximum
    (term 1) at index 0 and every other logit d below it, whose term eps has 1024 eps just
    under 2^-24 (half a unit in the last place of 1).  Tile 0 sums to exactly 1 (each lane's
    eps terms are absorbed by 1); tiles 1-3 sum to exactly 1024 eps each; folded in ascending
    order 1 + 1024 eps rounds back to 1 three times, so S = 1 exactly.  A pairwise fold over
    tiles gives 1 + 2^-23, a descending fold 1 + 2^-23 or more, and tiles of 2048 give
    1 + 2^-23 as well."""
    d, eps = short_term(orc, 2.0 ** -24)
    V = 4 * TV
    z = np.full(V, d, np.float32)
    z[0] = 0.0
    M, S, t1, t2 = orc.lmhead_stats(z)
    assert (b32(M), t1, t2) == (b32(0.0), 0, 1)
    assert b32(S) == b32(1.0)
    e = exp_terms(orc, z, M)
    assert all(b32(x) == b32(eps) for x in e[1:])
    assert b32(s_tree(e)) == b32(1.0)
    assert b32(s_tree(e[TV:2 * TV])) == b32(1024 * eps)
    assert b32(s_tree(e, fold="pairwise")) == b32(1.0 + 2.0 ** -23)
    assert b32(s_tree(e[::-1])) != b32(1.0)
    assert b32(s_tree(e, tv=2048)) == b32(1.0 + 2.0 ** -23)
    # log-softmax of the maximum is then exactly (0 - 0) - log_f(1) = +0
    assert b32(orc.log_f(np.array([S], np.float32))[0]) == b32(0.0)


# ------------------------------------------------------------ attention merge --

def attention_row_model(orc, q, K, V, i, scale, chunk=CHUNK, fused_merge=False, relative=False):
    """One causal attention row (keys 0..i) in the pinned order, exact rational arithmetic:
    s_j = RN(dot_seq(q, k_j)) * scale; chunks of `chunk` keys at absolute positions (or, with
    relative=True, counted back from the row: a wrong reading); per chunk m_c, then for j
    ascending p = exp_f(s_j - m_c), l_c += p, o_c = fma(p, v_j, o_c); merge from chunk 0
    ascending with m' = max, a = exp_f(m - m'), b = exp_f(m_c - m'), l = l*a + l_c*b,
    o = o*a + o_c*b (each product rounded, or one fused step with fused_merge=True)."""
    D = len(q)
    s = [mul32(exact.seq_dot32(q, K[j]), scale) for j in range(i + 1)]
    if relative:
        bounds = []
        hi = i
        while hi >= 0:
            bounds.append((max(0, hi - chunk + 1), hi))
            hi -= chunk
        bounds.reverse()
    else:
        bounds = [(c * chunk, min(c * chunk + chunk - 1, i)) for c in range(i // chunk + 1)]
    m = l = None
    o = None
    for (j0, j1) in bounds:
        mc = s[j0]
        for j in range(j0 + 1, j1 + 1):
            if s[j] > mc:
                mc = s[j]
        diffs = np.array([sub32(s[j], mc) for j in range(j0, j1 + 1)], np.float32)
        ps = [float(p) for p in orc.exp_f(diffs)]
        lc = 0.0
        oc = [0.0] * D
        for t, j in enumerate(range(j0, j1 + 1)):
            lc = add32(lc, ps[t])
            oc = [exact.fma32(ps[t], V[j][d], oc[d]) for d in range(D)]
        if m is None:
            m, l, o = mc, lc, oc
            continue
        mn = mc if mc > m else m
        a, b = (float(x) for x in orc.exp_f(np.array([sub32(m, mn), sub32(mc, mn)], np.float32)))
        if fused_merge:
            l = exact.fma32(l, a, mul32(lc, b))
            o = [exact.fma32(o[d], a, mul32(oc[d], b)) for d in range(D)]
        else:
            l = add32(mul32(l, a), mul32(lc, b))
            o = [add32(mul32(o[d], a), mul32(oc[d], b)) for d in range(D)]
        m = mn
    return [div32(o[d], l) for d in range(D)]


def attn_inputs(seed, T, D, spread):
    q = synth.normal(seed, (1, T, 1, D), spread)
    k = synth.normal(seed + 1, (1, 1, T, D))
    v = synth.normal(seed + 2, (1, 1, T, D))
    return q, k, v


ROWS = (0, 1, 200, 255, 256, 257, 300, 511, 512, 513, 599)


def test_attention_row_is_the_pinned_chunk_merge(orc):
    """Rows across two chunk boundaries (T = 600, head dim 4, scale 1/2) equal the exact
    model bit for bit, including the rows just before and after 256 and 512."""
    D, T = 4, 600
    q, k, v = attn_inputs(13200, T, D, 1.5)
    scale = 0.5
    O = orc.attention(q, k, v, scale=np.float32(scale))
    K = [[float(x) for x in k[0, 0, j]] for j in range(T)]
    Vv = [[float(x) for x in v[0, 0, j]] for j in range(T)]
    for i in ROWS:
        want = attention_row_model(orc, [float(x) for x in q[0, i, 0]], K, Vv, i, scale)
        assert [b32(x) for x in O[0, i, 0]] == [b32(x) for x in want], i


def test_attention_merge_rejects_other_orders(orc):
    """Chunks of 128 or 512, a fused multiply-add merge, and chunk bounds counted back from
    the row (not absolute) each change some output bits of the rows that cross a boundary."""
    D, T = 4, 600
    q, k, v = attn_inputs(13300, T, D, 1.5)
    scale = 0.5
    O = orc.attention(q, k, v, scale=np.float32(scale))
    K = [[float(x) for x in k[0, 0, j]] for j in range(T)]
    Vv = [[float(x) for x in v[0, 0, j]] for j in range(T)]
    rows = [i for i in ROWS if i >= 256]
    got = {i: [b32(x) for x in O[0, i, 0]] for i in rows}
    for i in rows:
        assert got[i] == [b32(x) for x in attention_row_model(orc, [float(x) for x in q[0, i, 0]], K, Vv, i, scale)]
    wrong = {"chunk 128": dict(chunk=128), "chunk 512": dict(chunk=512),
             "fused merge": dict(fused_merge=True), "relative bounds": dict(relative=True)}
    for name, kw in wrong.items():
        differs = sum(got[i] != [b32(x) for x in attention_row_model(
            orc, [float(x) for x in q[0, i, 0]], K, Vv, i, scale, **kw)] for i in rows)
        assert differs >= 1, name


def test_attention_merge_rounds_each_product(orc):
    """Closed form across a chunk boundary that only the two-rounding merge gives.  Row 256
    sees key 0 (score 0, value [3, 1]) in chunk 0, key 256 (score x = 0.75, value [-RN(3a), 1]
    with a = exp_f(-x)) in chunk 1, and keys 1..255 far below (weights exactly +0).  Chunk 0:
    m = 0, l = 1, o = [3, 1]; chunk 1: m = x, l = 1, o = [-RN(3a), 1]; the merge takes
    alpha = exp_f(0 - x) = a and beta = exp_f(0) = 1, so o_0 = RN(RN(3 a) + -RN(3 a)) = +0 and
    the output is exactly +0, while a fused merge RN(3 a - RN(3 a)) leaves the product's
    rounding error.  The second value column gives l / l = 1 exactly; row 255 gives [3, 1]."""
    D, T = 2, 257
    x = np.float32(0.75)
    a = float(orc.exp_f(np.array([-x], np.float32))[0])
    p3 = mul32(3.0, a)
    assert Fraction(p3) != 3 * Fraction(a)           # the product is inexact: the two merges differ
    q = np.zeros((1, T, 1, D), np.float32)
    q[..., 0] = 1.0
    k = np.zeros((1, 1, T, D), np.float32)
    k[0, 0, :, 0] = -1000.0
    k[0, 0, 0, 0] = 0.0
    k[0, 0, 256, 0] = x
    v = synth.normal(13400, (1, 1, T, D))
    v[0, 0, 0] = (3.0, 1.0)
    v[0, 0, 256] = (-p3, 1.0)
    O = orc.attention(q, k, v, scale=np.float32(1.0))
    assert [b32(t) for t in O[0, 256, 0]] == [b32(0.0), b32(1.0)]
    assert [b32(t) for t in O[0, 255, 0]] == [b32(3.0), b32(1.0)]
    fused = exact.fma32(3.0, a, -p3)
    assert fused != 0.0
    K = [[float(t) for t in k[0, 0, j]] for j in range(T)]
    Vv = [[float(t) for t in v[0, 0, j]] for j in range(T)]
    qi = [float(t) for t in q[0, 256, 0]]
    assert [b32(t) for t in attention_row_model(orc, qi, K, Vv, 256, 1.0)] == [b32(0.0), b32(1.0)]
    assert b32(attention_row_model(orc, qi, K, Vv, 256, 1.0, fused_merge=True)[0]) != b32(0.0)


def test_attention_chunk_crossing_cancellation(orc):
    """Closed form across a chunk boundary: keys 0..255 all score 0 with values +1, and keys
    256..511 all score 0 with values -1 (scale 1, q = 0, so every score is exactly 0 and every
    weight exp_f(0) = 1).  Chunk sums are l_c = 256, o_c = +-256 exactly; the merge factors
    are exp_f(0) = 1, so row 511 gives o = 256 + -256 = +0 and out = +0 / 512 = +0 exactly.
    A row in chunk 1 before its end (row 300) gives (256 - 45) / 301 rounded once."""
    D = 2
    T = 512
    q = np.zeros((1, T, 1, D), np.float32)
    k = synth.normal(13400, (1, 1, T, D))
    v = np.ones((1, 1, T, D), np.float32)
    v[0, 0, 256:] = -1.0
    O = orc.attention(q, k, v, scale=np.float32(1.0))
    assert b32(O[0, 511, 0, 0]) == b32(0.0) and b32(O[0, 511, 0, 1]) == b32(0.0)
    assert b32(O[0, 300, 0, 0]) == b32(div32(211.0, 301.0))
    assert b32(O[0, 255, 0, 0]) == b32(1.0)
