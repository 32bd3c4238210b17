"""Pins of the oracle's causal top-k (page "Sparse latent attention": up to
2,048 positions per query, selection over top_2048 of the masked score;
page "Rotate first features": topk(min(index_topk, end_pos))).

Reading under test: k_eff = min(K, n_valid); order (score desc, position
asc); -0 == +0; output ascending, padded with -1.
"""
import numpy as np
import pytest

import oracle
import synth


def lexsort_topk(row, n, K):
    """Independent formulation: numpy's lexsort on (position, -score)."""
    v = row[:n].astype(np.float64)
    v = np.where(v == 0.0, 0.0, v)               # -0 -> +0
    order = np.lexsort((np.arange(n), -v))
    keep = np.sort(order[:min(K, n)])
    out = np.full(K, -1, np.int32)
    out[:keep.size] = keep
    return out


@pytest.mark.parametrize("kind", ["normal", "ties", "zeros", "constant", "wide"])
def test_matches_lexsort(kind):
    L, K = 700, 64
    sc = synth.topk_scores(31, 12, L, kind)
    nv = np.array([700, 1, 2, 63, 64, 65, 100, 699, 500, 0, 350, 128], np.int32)
    got = oracle.topk(sc, nv, K)
    for r in range(12):
        assert np.array_equal(got[r], lexsort_topk(sc[r], nv[r], K)), (kind, r)


def test_all_equal_scores_take_lowest_positions():
    sc = np.zeros((1, 5000))
    got = oracle.topk(sc, [5000], 2048)[0]
    assert np.array_equal(got, np.arange(2048))


def test_budget_larger_than_prefix_returns_prefix():
    sc = synth.topk_scores(32, 3, 3000, "normal")
    got = oracle.topk(sc, [1000, 2048, 1], 2048)
    assert np.array_equal(got[0, :1000], np.arange(1000)) and np.all(got[0, 1000:] == -1)
    assert np.array_equal(got[1], np.arange(2048))
    assert got[2, 0] == 0 and np.all(got[2, 1:] == -1)


def test_negative_zero_ties_with_positive_zero():
    sc = np.array([[-0.0, 0.0, -1.0, -0.0, 0.0]])
    assert oracle.topk(sc, [5], 2).tolist() == [[0, 1]]
    sc = np.array([[-1.0, 0.0, -0.0]])
    assert oracle.topk(sc, [3], 2).tolist() == [[1, 2]]


def test_permuting_distinct_values_permutes_selection():
    g = np.random.Generator(np.random.PCG64(33))
    v = g.permutation(4096).astype(np.float64)        # distinct
    perm = g.permutation(4096)
    a = oracle.topk(v[None], [4096], 100)[0]
    b = oracle.topk(v[perm][None], [4096], 100)[0]
    assert np.array_equal(np.sort(perm[b]), a)
    assert set(v[a]) == set(range(3996, 4096))


def test_causal_bound_excludes_later_positions():
    sc = np.zeros((1, 10))
    sc[0, 7:] = 100.0                                    # beyond n_valid=7
    assert oracle.topk(sc, [7], 3).tolist() == [[0, 1, 2]]
