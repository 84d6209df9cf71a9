"""Pins for the oracle's RMSNorm (CPU only).

Definition pinned: each block normalises its input with RMSNorm before the
feed-forward / MoE step and adds the residual after it ("Hand-writing a
DeepSeek inference engine in pure C", hnwysp.cn/news/134870, §2.1); the
epsilon is 1e-6 ("ds4 code walkthrough", the model constants).  The pages
name RMSNorm without printing it; the standard form is read:
x / sqrt(mean(x^2) + eps) * g, per row.

Each pin fails for a plausible slip: the sum instead of the mean, a missing
square root, eps outside the root, a dropped weight, the wrong axis.
"""
import math

import numpy as np
import pytest

import oracle

EPS = 1e-6


def test_worked_example_three_four():
    # x = (3, 4): mean square 12.5, so x / sqrt(12.5) = (0.6, 0.8) * sqrt(2);
    # the weight (2, 0.5) scales each column
    x = np.array([[3.0, 4.0]], np.float32)
    out = oracle.rmsnorm_f64(x, np.array([2.0, 0.5], np.float32), 0.0)
    np.testing.assert_allclose(out[0], [1.2 * math.sqrt(2.0), 0.4 * math.sqrt(2.0)],
                               rtol=1e-15)
    # with eps the root is taken of mean + eps
    out = oracle.rmsnorm_f64(x, np.ones(2, np.float32), EPS)
    np.testing.assert_allclose(out[0], [3 / math.sqrt(12.5 + EPS), 4 / math.sqrt(12.5 + EPS)],
                               rtol=1e-15)


@pytest.mark.parametrize("c", [1.0, -0.5, 1e-3, 7.25])
def test_constant_row(c):
    # every element c: the row becomes g * c / sqrt(c^2 + eps)
    H = 96
    g = np.linspace(0.5, 2.0, H).astype(np.float32)
    out = oracle.rmsnorm_f64(np.full((1, H), c, np.float32), g, EPS)
    c32 = float(np.float32(c))
    np.testing.assert_allclose(out[0], g.astype(np.float64) * c32 / math.sqrt(c32 * c32 + EPS),
                               rtol=1e-14)


def test_mean_square_of_the_result():
    # with g = 1 the result's mean square is ms / (ms + eps)
    rng = np.random.default_rng(3)
    for H in (1, 7, 4096):
        x = rng.standard_normal((3, H)).astype(np.float32) * np.float32(0.01)
        out = oracle.rmsnorm_f64(x, np.ones(H, np.float32), EPS)
        ms = (x.astype(np.float64) ** 2).mean(axis=1)
        np.testing.assert_allclose((out ** 2).mean(axis=1), ms / (ms + EPS), rtol=1e-12)


def test_power_of_two_scaling_is_exact_without_eps():
    # x * 2^j scales the root by exactly 2^j, so the result is bitwise equal
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2, 333)).astype(np.float32)
    g = rng.standard_normal(333).astype(np.float32)
    base = oracle.rmsnorm_f64(x, g, 0.0)
    for j in (-6, 3, 20):
        scaled = (x * np.float32(2.0 ** j)).astype(np.float32)
        np.testing.assert_array_equal(oracle.rmsnorm_f64(scaled, g, 0.0), base)


def test_sign_symmetry_and_zero_row():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 64)).astype(np.float32)
    g = np.ones(64, np.float32)
    np.testing.assert_array_equal(oracle.rmsnorm_f64(-x, g, EPS), -oracle.rmsnorm_f64(x, g, EPS))
    assert not oracle.rmsnorm_f64(np.zeros((1, 64), np.float32), g, EPS).any()


def test_rows_are_independent():
    # a batch normalises each row over its own elements only
    rng = np.random.default_rng(6)
    x = rng.standard_normal((5, 40)).astype(np.float32)
    x[2] *= np.float32(100.0)
    g = rng.standard_normal(40).astype(np.float32)
    batch = oracle.rmsnorm_f64(x, g, EPS)
    for t in range(5):
        np.testing.assert_array_equal(batch[t], oracle.rmsnorm_f64(x[t:t + 1], g, EPS)[0])


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.rmsnorm_f64(np.ones((1, 4), np.float32), np.ones(3, np.float32), EPS)
    with pytest.raises(ValueError):
        oracle.rmsnorm_f64(np.ones((1, 4), np.float32), np.ones(4, np.float32), -1.0)
