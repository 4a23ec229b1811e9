"""Pins for the oracle's top-K selection: brute force and special cases (no GPU)."""
import math

import numpy as np
import pytest

from oracle import ref_select, ref_select_varlen


def _better(gi, i, gj, j):
    """True when token i outranks token j: a number beats NaN, a larger value
    beats a smaller one, and equal values go to the lower index."""
    ni, nj = math.isnan(gi), math.isnan(gj)
    if ni != nj:
        return nj
    if not ni and gi != gj:
        return gi > gj
    return i < j


def brute_force_select(g, k, q):
    """O(N^2) definition: a document token is kept iff fewer than Kd document
    tokens outrank it; the question tail is always kept."""
    g = [float(x) for x in np.asarray(g, dtype=np.float32)]
    n = len(g)
    doc = n - q
    kd = min(k, n) - q
    kept = []
    for j in range(doc):
        rank = sum(1 for i in range(doc) if i != j and _better(g[i], i, g[j], j))
        if rank < kd:
            kept.append(j)
    return np.array(kept + list(range(doc, n)), dtype=np.int64)


@pytest.mark.parametrize("seed", range(12))
def test_select_matches_brute_force_rank_definition(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 160))
    q = int(rng.integers(0, min(n, 20) + 1))
    k = int(rng.integers(q, n + 10))
    kind = seed % 4
    if kind == 0:
        g = rng.random(n).astype(np.float32)
    elif kind == 1:      # heavy ties
        g = (rng.integers(0, 4, n) / 4.0).astype(np.float32)
    elif kind == 2:      # signed zeros, NaNs and infinities mixed in
        g = rng.standard_normal(n).astype(np.float32)
        g[rng.random(n) < 0.1] = np.nan
        g[rng.random(n) < 0.1] = -0.0
        g[rng.random(n) < 0.1] = 0.0
        g[rng.random(n) < 0.05] = -np.inf
    else:                # saturated gate values: many exact 1.0f
        g = np.where(rng.random(n) < 0.4, 1.0, rng.random(n)).astype(np.float32)
    np.testing.assert_array_equal(ref_select(g, k, q), brute_force_select(g, k, q))


def test_select_budget_at_or_above_n_is_identity():
    g = np.random.default_rng(3).random(50).astype(np.float32)
    for k in (50, 51, 1000):
        np.testing.assert_array_equal(ref_select(g, k, 7), np.arange(50))


def test_select_budget_equal_to_question_keeps_only_the_tail():
    g = np.random.default_rng(4).random(40).astype(np.float32)
    np.testing.assert_array_equal(ref_select(g, 8, 8), np.arange(32, 40))


def test_select_all_equal_scores_keep_lowest_indices_then_tail():
    g = np.full(100, 0.25, dtype=np.float32)
    np.testing.assert_array_equal(ref_select(g, 30, 10), np.concatenate([np.arange(20), np.arange(90, 100)]))


def test_select_tie_storm_threshold_goes_to_lower_indices():
    # Two levels: 5 tokens at 0.9 are all kept; the remaining 3 slots go to the
    # three lowest-index tokens at 0.5.
    g = np.full(20, 0.5, dtype=np.float32)
    g[[4, 9, 11, 15, 17]] = 0.9
    got = ref_select(g, 8 + 2, 2)
    np.testing.assert_array_equal(got, [0, 1, 2, 4, 9, 11, 15, 17, 18, 19])


def test_select_order_is_ascending_and_kept_scores_dominate():
    rng = np.random.default_rng(5)
    g = rng.random(300).astype(np.float32)
    idx = ref_select(g, 64, 16)
    assert len(idx) == 64 and np.all(np.diff(idx) > 0)
    np.testing.assert_array_equal(idx[-16:], np.arange(284, 300))
    doc_kept = idx[:-16]
    dropped = np.setdiff1d(np.arange(284), doc_kept)
    assert g[doc_kept].min() >= g[dropped].max()


def test_select_question_tail_kept_even_with_lowest_scores():
    g = np.ones(30, dtype=np.float32)
    g[-5:] = 0.0
    np.testing.assert_array_equal(ref_select(g, 10, 5)[-5:], np.arange(25, 30))


def test_select_rejects_question_longer_than_budget():
    with pytest.raises(ValueError):
        ref_select(np.zeros(10, np.float32), 3, 4)
    with pytest.raises(ValueError):
        ref_select(np.zeros(3, np.float32), 10, 4)


def test_select_nan_ranks_last_and_signed_zeros_tie():
    g = np.array([np.nan, -0.0, 0.0, -1.0, np.nan], dtype=np.float32)
    # Kd = 3 of 5 document tokens (no tail): -0.0 and +0.0 tie (index 1 first),
    # then -1.0; both NaNs drop.
    np.testing.assert_array_equal(ref_select(g, 3, 0), [1, 2, 3])


def test_select_varlen_is_per_prompt():
    rng = np.random.default_rng(6)
    ns, qs = [40, 7, 90], [5, 7, 12]
    cu = np.concatenate([[0], np.cumsum(ns)])
    g = rng.random(cu[-1]).astype(np.float32)
    idx, cu_kept = ref_select_varlen(g, cu, qs, 20)
    np.testing.assert_array_equal(cu_kept, [0, 20, 27, 47])
    for b in range(3):
        np.testing.assert_array_equal(idx[cu_kept[b]:cu_kept[b + 1]],
                                      brute_force_select(g[cu[b]:cu[b + 1]], 20, qs[b]))
