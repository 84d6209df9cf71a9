"""Pins for the oracle's fused-dequant matmul (CPU only).

Definitions pinned: "Hand-writing a DeepSeek inference engine in pure C"
(hnwysp.cn/news/134870) §3.2 (dequantize inside the matmul's inner loop) and
§3.3 (C = A * B, reduction over K, OpenMP over independent outputs);
"Running a 284B-parameter LLM from 3.2 GB of RAM in plain C"
(feinterview.poetries.top): scalar and OpenMP paths bitwise identical.
"""
import numpy as np
import pytest

import oracle
from test_oracle_quant import grid_groups


@pytest.mark.parametrize("bits,group", [(8, 64), (4, 64), (8, 128), (4, 128)])
def test_exact_arithmetic_special_case(bits, group):
    """Weights on a power-of-two grid with scales 2^-6..2^-8, X small
    integers: every product and partial sum is a multiple of 2^-8 below 2^14,
    hence exact in fp32 in any order.  The fp32 fused path must then equal
    the exact result bit for bit, and so must the fp64 reference."""
    rng = np.random.default_rng(10)
    N, K, M = 7, group * 4, 3
    v, _, _, _, _ = grid_groups(rng, N, K, bits, group)
    # rescale groups to 2^-6..2^-8 steps: regenerate with a narrow exponent
    qmax = (1 << bits) - 1
    ng = K // group
    e = rng.integers(6, 9, size=(N, ng))
    z = rng.integers(0, qmax + 1, size=(N, ng))
    j = rng.integers(0, qmax + 1, size=(N, ng, group))
    j[:, :, 0] = 0
    j[:, :, 1] = qmax
    w = ((j - z[:, :, None]) * np.ldexp(1.0, -e)[:, :, None]).reshape(N, K).astype(np.float32)
    m = oracle.quantize(w, bits, group)
    X = rng.integers(-4, 5, size=(M, K)).astype(np.float32)
    exact = X.astype(np.float64) @ w.astype(np.float64).T   # exact in fp64 too
    Y32 = oracle.qmatmul_f32(X, m)
    Y64, S = oracle.qmatmul_ref(X, m)
    np.testing.assert_array_equal(Y64, exact)
    np.testing.assert_array_equal(Y32.astype(np.float64), exact)
    # a dropped zero-point would not survive this case
    assert (m.zp != 0).any()


@pytest.mark.parametrize("bits", [8, 4])
def test_reference_matches_library_matmul(bits):
    rng = np.random.default_rng(11)
    M, N, K = 5, 9, 192                      # K != N: a transposed operand fails
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    m = oracle.quantize(w, bits, 64)
    X = rng.standard_normal((M, K))
    Y, S = oracle.qmatmul_ref(X, m)
    wd = m.dequant_f64()
    np.testing.assert_allclose(Y, X @ wd.T, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(S, np.abs(X) @ np.abs(wd).T, rtol=1e-13)


def test_one_hot_returns_dequantized_column():
    rng = np.random.default_rng(12)
    N, K = 33, 256
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    for bits in (8, 4):
        m = oracle.quantize(w, bits, 64)
        X = np.eye(K, dtype=np.float32)[[0, 5, 63, 64, 200, 255]]
        Y = oracle.qmatmul_f32(X, m)
        cols = m.dequant_f64()[:, [0, 5, 63, 64, 200, 255]].T
        np.testing.assert_array_equal(Y, cols.astype(np.float32))


def test_scalar_and_openmp_bitwise_identical():
    rng = np.random.default_rng(13)
    w = (rng.standard_normal((300, 1024)) * 0.02).astype(np.float32)
    X = rng.standard_normal((4, 1024)).astype(np.float32)
    m = oracle.quantize(w, 4, 64)
    oracle.set_threads(1)
    a = oracle.qmatmul_f32(X, m)
    oracle.set_threads(8)
    b = oracle.qmatmul_f32(X, m)
    np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("bits,group", [(8, 64), (4, 64), (8, 128)])
def test_fp32_method_within_tolerance_of_reference(bits, group):
    """The fp32 fused path meets the fp32 gate |err| <= 1e-5 * sum|x*w| at a
    decode-sized K, so the gate is attainable by honest fp32 arithmetic."""
    rng = np.random.default_rng(14)
    N, K = 64, 4096
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    X = rng.standard_normal((2, K)).astype(np.float32)
    m = oracle.quantize(w, bits, group)
    Y32 = oracle.qmatmul_f32(X, m)
    Y64, S = oracle.qmatmul_ref(X, m)
    assert (np.abs(Y32 - Y64) <= 1e-5 * S).all()
