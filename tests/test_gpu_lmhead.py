"""lmhead_logprob_top2 on the GPU: bitwise equal to the oracle (logprob, margin, top-2,
recompute flag), per-row bits independent of the batch size, tau limits, ties."""
import numpy as np
import pytest

import synth
from gpu_util import assert_bitwise, bf16, f32, host, i32, requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]

KEYS = ("logprob", "margin", "top1", "top2", "recomputed")


def inv():
    import invariant_numerics_amd as m
    return m


def run(h, W, tgt, tau=0.1, Wd=None):
    r = inv().inv_lmhead_logprob_top2(f32(h), Wd if Wd is not None else bf16(W), i32(tgt), tau)
    return {k: host(v) for k, v in r.items()}


def check(got, want, what):
    for k in KEYS:
        assert_bitwise(got[k], want[k], "%s %s" % (what, k))


def test_c1_all_batch_sizes(orc):
    """hidden 256, vocab 4096, 64 tokens, batch 1/2/4/8: per-row bits equal across batch
    sizes and equal to the oracle."""
    say("lmhead C1")
    d = synth.c1_inputs()
    want = orc.lmhead(d["h"], d["w"], d["target"])
    Wd = bf16(d["w"])
    assert 0 < want["recomputed"].sum() < 64
    for B in (1, 2, 4, 8):
        parts = [run(d["h"][s:s + B], None, d["target"][s:s + B], Wd=Wd) for s in range(0, 64, B)]
        got = {k: np.concatenate([p[k] for p in parts]) for k in KEYS}
        check(got, want, "B=%d" % B)


@pytest.mark.parametrize("B,K,V", [(1, 8, 2), (3, 264, 1025), (17, 256, 3000), (40, 512, 4096)])
def test_shapes_match_oracle(orc, B, K, V):
    say("lmhead shape", B, K, V)
    h = synth.normal(9000 + V, (B, K))
    W = synth.bf16_normal(9100 + V, (V, K), 0.1)
    tgt = synth.uniform_int(9200 + V, (B,), V)
    check(run(h, W, tgt), orc.lmhead(h, W, tgt), "shape")


def test_fused_and_separate_recompute_paths_agree(orc):
    """Up to 32 rows the FP32 logits share the primary sweep over W; above, flagged rows get
    their own pass.  Both give the oracle's bits, for tau 0.1, +inf and 0."""
    d = synth.c1_inputs(rows=40)
    Wd = bf16(d["w"])
    for tau, mode in ((0.1, 0), (np.inf, 2), (0.0, 1)):
        say("lmhead paths tau", tau)
        want = orc.lmhead(d["h"], d["w"], d["target"], tau=np.float32(tau), mode=mode)
        sep = run(d["h"], None, d["target"], tau=tau, Wd=Wd)
        check(sep, want, "B=40 tau=%s" % tau)
        for B in (20, 16, 5, 1):
            parts = [run(d["h"][s:s + B], None, d["target"][s:s + B], tau=tau, Wd=Wd) for s in range(0, 40, B)]
            check({k: np.concatenate([p[k] for p in parts]) for k in KEYS}, want, "B=%d tau=%s" % (B, tau))


@pytest.mark.parametrize("B", [33, 100])
def test_fp32_pass_head_and_rest(orc, B):
    """Above 32 rows the FP32 pass runs its first 32 compacted rows on their own GEMV and the
    rest on 64 x 64 tiles (live rows on the device): with every row flagged at a finite tau
    (1e30) both parts carry rows, with tau = 0.1 usually only the first; tau = +inf runs the
    pass as one GEMM."""
    d = synth.c1_inputs(rows=B)
    Wd = bf16(d["w"])
    for tau, mode in ((1e30, 0), (np.inf, 2), (0.1, 0)):
        say("lmhead fp32 head/rest", B, tau)
        want = orc.lmhead(d["h"], d["w"], d["target"], tau=np.float32(tau), mode=mode)
        check(run(d["h"], None, d["target"], tau=tau, Wd=Wd), want, "B=%d tau=%s" % (B, tau))


def test_tau_limits_and_ties(orc):
    say("lmhead tau/ties")
    d = synth.c1_inputs(rows=16)
    for tau, mode in ((0.0, 1), (np.inf, 2)):
        check(run(d["h"], d["w"], d["target"], tau=tau), orc.lmhead(d["h"], d["w"], d["target"], mode=mode),
              "tau=%s" % tau)
    W0 = np.zeros((4096, 256), np.uint16)
    got = run(d["h"], W0, d["target"])
    assert np.all(got["top1"] == 0) and np.all(got["top2"] == 1) and np.all(got["margin"] == 0)
    assert np.all(got["recomputed"] == 1)
    check(got, orc.lmhead(d["h"], W0, d["target"]), "W=0")
    W = d["w"].copy()
    W[10] = W[3000] = W[20]
    check(run(d["h"], W, d["target"]), orc.lmhead(d["h"], W, d["target"]), "duplicate rows")


@pytest.fixture(scope="module")
def c4():
    return synth.c4_inputs()


def test_c4_batch_invariance_and_oracle_sample(orc, c4):
    """hidden 4096, vocab 128256: batches 1..256 give the same per-row bits; sampled rows
    equal the oracle (selective recompute, margin < 0.1)."""
    h, W, tgt = c4["h"], c4["w"], c4["target"]
    Wd = bf16(W)
    say("lmhead C4 B=256")
    full = run(h, None, tgt, Wd=Wd)
    for B in (1, 2, 3, 4, 8, 16, 32, 64, 128):
        say("lmhead C4 B", B)
        got = run(h[:B], None, tgt[:B], Wd=Wd)
        check(got, {k: v[:B] for k, v in full.items()}, "B=%d" % B)
    frac = full["recomputed"].mean()
    assert 0.1 < frac < 0.6, frac
    rows = [0, 1, 5, 100, 255]
    say("lmhead C4 oracle rows", rows)
    want = orc.lmhead(h[rows], W, tgt[rows])
    check({k: v[rows] for k, v in full.items()}, want, "oracle rows")


def test_c4_margin_stress(orc):
    """Near-tied weight rows (w_b = w_a + N(0, 1e-3)) make small margins common."""
    d = synth.c4_inputs(rows=16, stress=True)
    say("lmhead C4 stress")
    got = run(d["h"], d["w"], d["target"])
    rows = [0, 7, 15]
    want = orc.lmhead(d["h"][rows], d["w"], d["target"][rows])
    check({k: v[rows] for k, v in got.items()}, want, "stress")
    assert got["recomputed"].mean() > 0.5


def test_nan_rows_stay_in_bounds(orc):
    """Rows whose logits are all NaN (NaN hidden state): no logit is orderable, so the top-2
    takes the scan's starting choice (0, 1) and logprob is NaN; finite rows beside them are
    unaffected.  (Regression: the reduction once indexed past the row in this case.)"""
    say("lmhead NaN rows")
    d = synth.c1_inputs(rows=4)
    h = d["h"].copy()
    h[1, :] = np.nan
    got = run(h, d["w"], d["target"])
    assert np.isnan(got["logprob"][1]) and got["top1"][1] == 0 and got["top2"][1] == 1
    assert got["recomputed"][1] == 0
    rows = [0, 2, 3]
    want = orc.lmhead(d["h"][rows], d["w"], d["target"][rows])
    check({k: v[rows] for k, v in got.items()}, want, "finite rows")


def test_partly_nan_rows_match_oracle(orc):
    """Rows with NaN logits among finite ones (an infinite product sum meeting its negative in
    the slice fold): NaN never takes part in the top-2, so top-1, top-2, margin and the
    recompute flag come from the finite logits, and the logprob is NaN (the NaN terms reach
    the denominator).  NaN at vocabulary index 0, at index 1, at both, and in the middle."""
    say("lmhead partly-NaN rows")
    K, V = 512, 3000
    W = synth.bf16_normal(9300, (V, K), 0.1)
    W[:, [0, 1, 2, 256, 257, 258]] = 0
    for v, c in ((0, 0), (1, 1), (2000, 2)):          # vocabulary row v: +2 at column c, -2 at c + 256
        W[v, c], W[v, c + 256] = 0x4000, 0xC000
    h = synth.normal(9301, (5, K))
    big = np.float32(3e38)
    for r, cols in ((0, [0]), (1, [1]), (2, [0, 1]), (3, [2])):
        for c in cols:
            h[r, c] = h[r, c + 256] = big                 # row 4 stays finite
    tgt = np.array([0, 5, 1, 2000, 7], np.int32)
    for tau in (0.1, np.inf):
        got = run(h, W, tgt, tau=tau)
        want = orc.lmhead(h, W, tgt, tau=np.float32(tau))
        for k in ("margin", "top1", "top2", "recomputed"):
            assert_bitwise(got[k], want[k], "tau=%s %s" % (tau, k))
        assert np.array_equal(np.isnan(got["logprob"]), np.isnan(want["logprob"]))
        assert np.isnan(want["logprob"][:4]).all() and np.isfinite(want["margin"]).all()
        assert_bitwise(got["logprob"][4:], want["logprob"][4:], "finite row")
        assert want["top1"][0] != 0 and want["top1"][1] != 1 and 0 not in want["top1"][2:3]
