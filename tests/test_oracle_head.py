"""Pins for the oracle's output-head selection (CPU only).

Definition pinned: the next token is chosen from the output projection's
logits ("Hand-writing a DeepSeek inference engine in pure C",
hnwysp.cn/news/134870, §2.1; "ds4 code walkthrough", the session API's
argmax / sample step), and the end-to-end check compares the argmax at
every position ("Running a 284B-parameter LLM from 3.2 GB of RAM in plain
C").  Reading: the k largest logits in rank order, larger value first, equal
values to the smaller index (the first maximum a plain greater-than scan
keeps), NaN below every number.
"""
import math

import numpy as np
import pytest

import oracle


def scan_argmax(y):
    # the plain loop: keep the first strictly greater value; NaN never wins
    # against a number
    best = None
    for i, v in enumerate(y):
        if math.isnan(v):
            continue
        if best is None or v > y[best]:
            best = i
    if best is None:  # all NaN: the first one
        best = 0
    return best


def brute_rank(y):
    # a full sort with an explicit key: numbers before NaNs, larger value
    # first (with -0 == +0), smaller index first
    def key(i):
        v = float(y[i])
        if math.isnan(v):
            return (1, 0.0, i)
        return (0, -v, i)
    return sorted(range(len(y)), key=key)


@pytest.mark.parametrize("N,k", [(1, 1), (7, 3), (50, 50), (1000, 1), (1000, 64), (4097, 17)])
def test_topk_matches_full_sort(N, k):
    rng = np.random.default_rng(70 + N)
    y = rng.standard_normal(N).astype(np.float32)
    idx, val = oracle.topk(y, k)
    ref = brute_rank(y)[:k]
    assert list(idx) == ref
    np.testing.assert_array_equal(val, y[ref])


def test_topk_ties_go_to_the_smaller_index():
    # integer-valued logits: many exact ties
    rng = np.random.default_rng(71)
    y = rng.integers(-3, 4, size=300).astype(np.float32)
    idx, val = oracle.topk(y, 40)
    assert list(idx) == brute_rank(y)[:40]
    for r in range(39):
        assert val[r] > val[r + 1] or (val[r] == val[r + 1] and idx[r] < idx[r + 1])


def test_topk_signed_zero_and_infinities():
    y = np.array([0.0, -0.0, -np.inf, np.inf, -0.0, 1.0, np.inf, 0.0], np.float32)
    idx, val = oracle.topk(y, 8)
    # +inf (3, 6), 1.0 (5), zeros of either sign in index order (0, 1, 4, 7), -inf
    assert list(idx) == [3, 6, 5, 0, 1, 4, 7, 2]


def test_topk_nan_ranks_last():
    y = np.array([np.nan, -5.0, np.nan, -np.inf, 2.0], np.float32)
    idx, _ = oracle.topk(y, 5)
    assert list(idx) == [4, 1, 3, 0, 2]


@pytest.mark.parametrize("seed", range(5))
def test_argmax_is_the_plain_scan(seed):
    rng = np.random.default_rng(80 + seed)
    y = rng.integers(-20, 21, size=5000).astype(np.float32)
    y[rng.integers(0, 5000, size=50)] = np.nan
    idx, val = oracle.topk(y, 1)
    assert idx[0] == scan_argmax(list(y))
    # a NaN-free vector: numpy's argmax (first maximum)
    z = rng.standard_normal(5000).astype(np.float32)
    z[3000] = z[100] = z.max() + 1.0
    assert oracle.topk(z, 1)[0][0] == np.argmax(z) == 100


def test_topk_full_length_is_a_sorted_permutation():
    rng = np.random.default_rng(72)
    y = rng.standard_normal(513).astype(np.float32)
    idx, val = oracle.topk(y, 513)
    assert sorted(idx) == list(range(513))
    assert np.all(np.diff(val) <= 0)


def test_topk_rejects_bad_k():
    y = np.zeros(4, np.float32)
    for k in (0, 5):
        with pytest.raises(ValueError):
            oracle.topk(y, k)
