"""Host bookkeeping of the cross-precision agreement harness on hand-built runs: divergence
index, exact agreement, the comparable-step window and the flip-versus-margin rule."""
import numpy as np

from invariant_numerics_amd import agreement


def run(tokens, margin, top2):
    tokens = np.asarray(tokens, np.int32)
    return {"tokens": tokens, "top1": tokens.copy(), "top2": np.asarray(top2, np.int32),
            "margin": np.asarray(margin, np.float32), "recomputed": np.zeros(tokens.shape, np.uint8)}


def test_divergence_index_edges():
    a = np.array([[1, 2, 3], [1, 2, 3], [1, 2, 3]])
    b = np.array([[1, 2, 3], [9, 2, 3], [1, 2, 9]])
    assert agreement.divergence_index(a, b).tolist() == [3, 0, 2]


def test_compare_counts_flips_at_the_divergence_only():
    # prompt 0 agrees everywhere; prompt 1 flips at step 1 (B ranks A's pair the other way),
    # after which the prefixes differ and nothing more is compared
    A = run([[5, 6, 7], [5, 6, 7]], [[0.5, 0.4, 0.3], [0.5, 0.02, 0.3]], [[1, 1, 1], [1, 8, 1]])
    B = run([[5, 6, 7], [5, 8, 0]], [[0.49, 0.41, 0.3], [0.51, 0.01, 9.0]], [[1, 1, 1], [1, 6, 4]])
    r = agreement.compare(A, B)
    assert r["exact_agreement"] == 0.5
    assert r["divergence_index"] == [3, 1]
    assert r["comparable_steps"] == 3 + 2
    assert r["flips"] == 1 and r["flips_other_pair"] == 0
    # at the flip: m_A = 0.02, g_B = -0.01, d = 0.03 > m_A
    assert abs(r["median_abs_perturbation_at_flip"] - 0.03) < 1e-6
    assert abs(r["median_margin_at_flip"] - 0.02) < 1e-6
    assert r["flip_iff_perturbation_exceeds_margin"]


def test_compare_other_pair_and_identical_runs():
    A = run([[3, 4]], [[0.2, 0.2]], [[7, 1]])
    B = run([[9, 4]], [[0.1, 0.2]], [[3, 1]])      # B's top two are (9, 3): not A's pair
    r = agreement.compare(A, B)
    assert r["flips"] == 1 and r["flips_other_pair"] == 1 and r["median_margin_at_flip"] is None
    same = agreement.compare(A, A)
    assert same["exact_agreement"] == 1.0 and same["flips"] == 0
    assert same["median_abs_perturbation_no_flip"] == 0.0
