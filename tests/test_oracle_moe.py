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
    """The oracle's own silu (pinned below by closed forms), elementwise."""
    return np.vectorize(oracle.silu, otypes=[np.float64])(np.asarray(z, np.float64))


def dsilu(z):
    return np.vectorize(oracle.dsilu, otypes=[np.float64])(np.asarray(z, np.float64))


def test_silu_closed_forms():
    """silu(z) = z / (1 + e^-z): values fixed by the definition alone."""
    ln3 = np.log(3.0)
    assert oracle.silu(0.0) == 0.0
    # e^-ln3 = 1/3, so silu(ln 3) = ln3 / (4/3); e^ln3 = 3, silu(-ln 3) = -ln3 / 4
    assert abs(oracle.silu(ln3) - 0.75 * ln3) <= 4e-16
    assert abs(oracle.silu(-ln3) + 0.25 * ln3) <= 4e-16
    # silu(z) - silu(-z) = z for every z (the logistic is symmetric about 1/2)
    for z in (0.1, 1.0, 2.5, 7.0, 30.0):
        assert abs(oracle.silu(z) - oracle.silu(-z) - z) <= 4e-16 * max(1.0, z)
    # limits: silu(z) -> z for large z, -> 0 from below for large -z
    assert oracle.silu(40.0) == 40.0
    assert -1e-15 < oracle.silu(-40.0) < 0.0
    assert oracle.silu(-800.0) == 0.0 or abs(oracle.silu(-800.0)) < 1e-300
    # an odd sign pattern: silu < 0 exactly on z < 0
    assert oracle.silu(-1e-3) < 0.0 < oracle.silu(1e-3)


def test_dsilu_closed_forms_and_derivative():
    """silu'(z) = s (1 + z (1 - s)), s the logistic: silu'(0) = 1/2,
    silu'(ln 3) = 3/4 (1 + ln3 / 4), the limits 1 and 0, and central
    differences of the oracle's own silu."""
    ln3 = np.log(3.0)
    assert oracle.dsilu(0.0) == 0.5
    assert abs(oracle.dsilu(ln3) - 0.75 * (1.0 + ln3 / 4.0)) <= 4e-16
    assert abs(oracle.dsilu(-ln3) - 0.25 * (1.0 - 3.0 * ln3 / 4.0)) <= 4e-16
    assert abs(oracle.dsilu(40.0) - 1.0) <= 1e-15
    assert abs(oracle.dsilu(-40.0)) <= 1e-15
    # silu'(z) + silu'(-z) = 1 (derivative of silu(z) - silu(-z) = z)
    for z in (0.3, 1.7, 5.0):
        assert abs(oracle.dsilu(z) + oracle.dsilu(-z) - 1.0) <= 1e-15
    h = 1e-5
    for z in (-6.0, -2.0, -0.5, 0.0, 0.4, 1.3, 3.0, 8.0):
        fd = (oracle.silu(z + h) - oracle.silu(z - h)) / (2 * h)
        assert abs(fd - oracle.dsilu(z)) <= 1e-9, z


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


@pytest.mark.parametrize("bits", [4, 8])
def test_expert_sensitivity_helper_is_the_worst_first_order_change(bits):
    """Pd[n] (the oracle's tolerance helper) is the largest first-order change
    of y[n] when every gate sum g_j and up sum u_j moves by at most
    delta * (its own magnitude sum Sg_j, Su_j), divided by delta.  The largest
    change is reached by moving each sum in the direction that raises y[n]:
    g_j by delta Sg_j sign(silu'(g_j) u_j Wd[n][j]), u_j by delta Su_j
    sign(silu(g_j) Wd[n][j]).  A finite difference of the expert's output
    under exactly that perturbation must reproduce Pd[n]; a dropped term, a
    wrong derivative or a missing absolute value fails it."""
    rng = np.random.default_rng(35)
    H, I = 192, 128
    ex = make_experts(rng, 1, H, I, bits, 64)[0]
    x = rng.standard_normal(H)
    y, Sd, Pd, g, u, h = oracle.expert_f64(x, ex, want_gu=True)
    Wg, Wu, Wd = ex.gate.dequant_f64(), ex.up.dequant_f64(), ex.down.dequant_f64()
    _, Sg = oracle.matmul_f64(x[None, :], Wg)
    _, Su = oracle.matmul_f64(x[None, :], Wu)
    Sg, Su = Sg[0], Su[0]
    delta = 1e-7
    for n in (0, 5, 77, H - 1):
        dg = delta * Sg * np.sign(dsilu(g) * u * Wd[n])
        du = delta * Su * np.sign(silu(g) * Wd[n])
        y1 = float(Wd[n] @ (silu(g + dg) * (u + du)))
        fd = (y1 - y[n]) / delta
        assert abs(fd - Pd[n]) <= 1e-4 * Pd[n], (n, fd, Pd[n])
        # and no other sign pattern does better (a random one does worse)
        sg, su = rng.choice([-1.0, 1.0], I), rng.choice([-1.0, 1.0], I)
        y2 = float(Wd[n] @ (silu(g + delta * Sg * sg) * (u + delta * Su * su)))
        assert abs(y2 - y[n]) / delta <= Pd[n] * (1 + 1e-4)


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
    """The pages' fp32 CPU MoE against the fp64 oracle: inside 1e-5 * S_Y,
    the magnitude sum of the down projection weighted by the routing
    weights (the routing weights are given, so no weight error enters)."""
    rng = np.random.default_rng(34)
    H, I, E, T, k = 512, 256, 8, 6, 3
    ex = make_experts(rng, E, H, I, 4, 64)
    X = rng.standard_normal((T, H)).astype(np.float32)
    idx, w, _ = oracle.route(rng.standard_normal((T, E)), k)
    w32 = w.astype(np.float32)
    Y32 = oracle.moe_f32(X, idx, w32, ex, E)
    Y, SY, PY = oracle.moe_combine_f64(X.astype(np.float64), range(T), idx,
                                       w32.astype(np.float64), ex)
    assert (np.abs(Y32 - Y) <= 1e-5 * SY).all()
