"""Pins for the oracle's expert SwiGLU and MoE combine (CPU only).

Definitions pinned: "Hand-writing a DeepSeek inference engine in pure C"
(hnwysp.cn/news/134870) §3.5 (experts run on the tokens routed to them, the
outputs are summed with the routing weights; grouping by expert must not
change the result).  The expert form down(silu(gate) * up) is the workload's
definition (the pages only call experts feed-forward networks).
"""
import numpy as np
import pytest

import oracle


def make_experts(rng, E, H, I, bits, group):
    ex = {}
    for e in range(E):
        wg = (rng.standard_normal((I, H)) * 0.02).astype(np.float32)
        wu = (rng.standard_normal((I, H)) * 0.02).astype(np.float32)
        wd = (rng.standard_normal((H, I)) * 0.02).astype(np.float32)
        ex[e] = oracle.quantize_expert(wg, wu, wd, bits, group)
    return ex


def silu(z):
    return z / (1.0 + np.exp(-z))


@pytest.mark.parametrize("bits", [4, 8])
def test_expert_matches_library_matmuls(bits):
    rng = np.random.default_rng(30)
    H, I = 256, 128                        # H != I catches a swapped operand
    ex = make_experts(rng, 1, H, I, bits, 64)[0]
    x = rng.standard_normal(H)
    y, Sd, Pd, g, u, h = oracle.expert_f64(x, ex, want_gu=True)
    Wg, Wu, Wd = ex.gate.dequant_f64(), ex.up.dequant_f64(), ex.down.dequant_f64()
    np.testing.assert_allclose(g, Wg @ x, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(u, Wu @ x, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(h, silu(Wg @ x) * (Wu @ x), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(y, Wd @ h, rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(Sd, np.abs(Wd) @ np.abs(h), rtol=1e-12)
    assert (Pd >= 0).all()


def test_single_expert_reduces_to_dense_swiglu():
    """E = 1, k = 1: the router always picks expert 0 with weight 1 and the
    MoE layer is one dense SwiGLU FFN."""
    rng = np.random.default_rng(31)
    H, I, T = 128, 64, 5
    ex = make_experts(rng, 1, H, I, 8, 64)
    X = rng.standard_normal((T, H))
    idx, w, _ = oracle.route(rng.standard_normal((T, 1)), 1)
    assert (idx == 0).all() and (w == 1.0).all()
    Y, SY, PY = oracle.moe_combine_f64(X, range(T), idx, w, ex)
    Wg, Wu, Wd = (m.dequant_f64() for m in (ex[0].gate, ex[0].up, ex[0].down))
    ref = (silu(X @ Wg.T) * (X @ Wu.T)) @ Wd.T
    np.testing.assert_allclose(Y, ref, rtol=1e-11, atol=1e-13)


def test_combine_is_weighted_sum_in_slot_order():
    rng = np.random.default_rng(32)
    H, I, E, T, k = 64, 64, 6, 4, 3
    ex = make_experts(rng, E, H, I, 4, 64)
    X = rng.standard_normal((T, H))
    idx, w, _ = oracle.route(rng.standard_normal((T, E)), k)
    Y, _, _ = oracle.moe_combine_f64(X, range(T), idx, w, ex)
    for t in range(T):
        ref = sum(w[t, i] * oracle.expert_f64(X[t], ex[int(idx[t, i])])[0] for i in range(k))
        np.testing.assert_array_equal(Y[t], ref)


@pytest.mark.parametrize("bits", [4, 8])
def test_grouped_equals_token_loop_bitwise(bits):
    rng = np.random.default_rng(33)
    H, I, E, T, k = 128, 64, 8, 9, 2
    ex = make_experts(rng, E, H, I, bits, 64)
    X = rng.standard_normal((T, H)).astype(np.float32)
    idx, w, _ = oracle.route(rng.standard_normal((T, E)), k)
    a = oracle.moe_f32(X, idx, w, ex, E, grouped=True)
    b = oracle.moe_f32(X, idx, w, ex, E, grouped=False)
    np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))


def test_fp32_moe_within_first_order_bound():
    rng = np.random.default_rng(34)
    H, I, E, T, k = 512, 256, 8, 6, 3
    ex = make_experts(rng, E, H, I, 4, 64)
    X = rng.standard_normal((T, H)).astype(np.float32)
    idx, w, _ = oracle.route(rng.standard_normal((T, E)), k)
    Y32 = oracle.moe_f32(X, idx, w.astype(np.float32), ex, E)
    Y, SY, PY = oracle.moe_combine_f64(X.astype(np.float64), range(T), idx, w, ex)
    assert (np.abs(Y32 - Y) <= 1e-5 * (SY + PY)).all()
