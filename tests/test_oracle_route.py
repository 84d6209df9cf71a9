"""Pins for the oracle's router, top-k and grouping (CPU only).

Definitions pinned: "Hand-writing a DeepSeek inference engine in pure C"
(hnwysp.cn/news/134870) §3.4 (softmax with the maximum subtracted), §3.5
(router = linear layer + softmax, top-k by a greater-first partial sort of
(score, index) pairs, tokens grouped per expert, weighted sum); the
renormalised top-k weights summing to one and exactly k distinct experts are
the workload's definition.
"""
import math

import numpy as np
import pytest

import oracle


def brute_topk(l, k):
    # a full sort with the same comparator: larger logit, then larger index
    return sorted(range(len(l)), key=lambda e: (-l[e], -e))[:k]


@pytest.mark.parametrize("E,k", [(256, 6), (8, 2), (4, 4), (1, 1), (64, 1)])
def test_topk_matches_full_sort(E, k):
    rng = np.random.default_rng(20)
    T = 50
    L = rng.standard_normal((T, E))
    # plant exact ties
    L[:, E // 2] = L[:, 0]
    idx, w, gap = oracle.route(L, k)
    for t in range(T):
        assert list(idx[t]) == brute_topk(list(L[t]), k)
        assert len(set(idx[t])) == k
        assert abs(w[t].sum() - 1.0) <= 8 * 2.0 ** -53 * k
        # renormalised weights == softmax over the selected logits only
        sel = L[t, idx[t]]
        ref = np.exp(sel - sel.max()) / np.exp(sel - sel.max()).sum()
        np.testing.assert_allclose(w[t], ref, rtol=1e-14)
        srt = sorted(L[t], reverse=True)
        assert gap[t] == (math.inf if k == E else srt[k - 1] - srt[k])


def test_tie_breaks_to_higher_index():
    L = np.zeros((1, 256))
    L[0, 3] = 5.0
    L[0, 200] = 5.0
    L[0, 100] = 4.0
    idx, w, _ = oracle.route(L, 3)
    assert list(idx[0]) == [200, 3, 100]
    assert w[0, 0] == w[0, 1]


def test_closed_form_weights():
    # logits ln(1..6): selected weights are proportional to 6,5,4
    L = np.log(np.arange(1, 7, dtype=np.float64))[None, :]
    idx, w, _ = oracle.route(L, 3)
    assert list(idx[0]) == [5, 4, 3]
    np.testing.assert_allclose(w[0], np.array([6, 5, 4]) / 15.0, rtol=1e-15)


def test_large_logits_do_not_overflow():
    # without the max subtraction exp(1000) overflows to inf and gives NaN
    L = np.array([[1000.0, 1000.0 - math.log(2.0), -1000.0]])
    idx, w, _ = oracle.route(L, 2)
    assert list(idx[0]) == [0, 1]
    assert np.isfinite(w).all()
    # 1000 - ln 2 is itself rounded to the fp64 grid near 1000 (ulp 1.1e-13)
    np.testing.assert_allclose(w[0], [2.0 / 3.0, 1.0 / 3.0], rtol=2e-13)


def test_rejects_non_finite_and_bad_k():
    with pytest.raises(ValueError):
        oracle.route(np.array([[0.0, np.nan]]), 1)
    with pytest.raises(ValueError):
        oracle.route(np.zeros((1, 4)), 5)


def test_router_linear_layer_matches_library():
    rng = np.random.default_rng(21)
    X = rng.standard_normal((3, 96))
    Wr = rng.standard_normal((10, 96)) * 0.02
    b = rng.standard_normal(10)
    L, S = oracle.router_f64(X, Wr, b)
    np.testing.assert_allclose(L, X @ Wr.T + b, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(S, np.abs(X) @ np.abs(Wr).T, rtol=1e-13)


@pytest.mark.parametrize("T,k,E", [(1, 6, 256), (32, 6, 256), (7, 2, 4), (300, 6, 256)])
def test_group_is_stable_counting_sort(T, k, E):
    rng = np.random.default_rng(22)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, perm = oracle.group(idx, E)
    flat = idx.reshape(-1)
    # library sort of (expert, entry) pairs gives the same order
    ref = sorted(range(T * k), key=lambda j: (flat[j], j))
    assert list(perm) == ref
    np.testing.assert_array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and offsets[-1] == T * k
    np.testing.assert_array_equal(np.diff(offsets), counts)
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert (flat[seg] == e).all()
