"""Pins for the oracle's quantizer and dequantizer (CPU only).

Definitions pinned: "Hand-writing a DeepSeek inference engine in pure C"
(hnwysp.cn/news/134870) §2.3 (dequant (q - zp) * scale, groups of 64/128)
and §3.2 (scale = (max - min) / (2^bits - 1), zp = round(-min / scale),
q = clamp(round(v / scale) + zp), INT4 two values per byte, range 0..15),
§5.1 (zero scale is an error).
"""
import numpy as np
import pytest

import oracle

CASES = [(8, 64), (8, 128), (4, 64), (4, 128)]


def grid_groups(rng, rows, K, bits, group, half_points=False):
    """Weights on an exact power-of-two grid: within each group
    v = (j - z) * 2^-e with j in 0..qmax, both end points present.  The
    closed form of the pages' rule is then scale = 2^-e, zp = z, q = j."""
    qmax = (1 << bits) - 1
    ng = K // group
    e = rng.integers(3, 12, size=(rows, ng))
    z = rng.integers(0, qmax + 1, size=(rows, ng))
    j = rng.integers(0, qmax + 1, size=(rows, ng, group))
    for r in range(rows):
        for g in range(ng):
            pos = rng.permutation(group)[:2]
            j[r, g, pos[0]] = 0
            j[r, g, pos[1]] = qmax
    frac = np.zeros_like(j, dtype=np.float64)
    if half_points:
        # every non-end-point value sits exactly half-way between two levels
        frac = np.where((j != 0) & (j != qmax), 0.5, 0.0)
        j = np.where((j != 0) & (j != qmax), np.minimum(j, qmax - 1), j)
    step = np.ldexp(1.0, -e)[:, :, None]
    v = ((j - z[:, :, None]) + frac) * step
    return v.reshape(rows, K).astype(np.float32), e, z, j, frac


@pytest.mark.parametrize("bits,group", CASES)
def test_closed_form_power_of_two_grid(bits, group):
    rng = np.random.default_rng(1)
    rows, K = 5, group * 3
    v, e, z, j, _ = grid_groups(rng, rows, K, bits, group)
    m = oracle.quantize(v, bits, group)
    assert (m.flags == 0).all()
    np.testing.assert_array_equal(m.scale, np.ldexp(1.0, -e).astype(np.float32))
    np.testing.assert_array_equal(m.zp, z.astype(np.float32))
    np.testing.assert_array_equal(oracle.unpack_q(m), j.reshape(rows, K))
    # the grid is reproduced exactly by the dequantizer
    np.testing.assert_array_equal(m.dequant_f64(), v.astype(np.float64))
    np.testing.assert_array_equal(m.dequant_f32(), v)


@pytest.mark.parametrize("bits,group", CASES)
def test_half_way_values_round_away_from_zero(bits, group):
    """roundf (the printed routine) rounds x.5 away from zero; rintf would
    round to even and fail here."""
    rng = np.random.default_rng(2)
    rows, K = 4, group * 2
    v, e, z, j, frac = grid_groups(rng, rows, K, bits, group, half_points=True)
    m = oracle.quantize(v, bits, group)
    t = (j - z[:, :, None]) + frac            # exact v / scale
    expect = np.where(frac > 0, np.where(t > 0, np.floor(t) + 1, np.ceil(t) - 1), t)
    expect = np.clip(expect + z[:, :, None], 0, (1 << bits) - 1).reshape(rows, K)
    np.testing.assert_array_equal(oracle.unpack_q(m), expect.astype(np.int32))
    # and at least some of them are ties that rint would have sent elsewhere
    rint = np.clip(np.rint(t) + z[:, :, None], 0, (1 << bits) - 1).reshape(rows, K)
    assert (rint != expect).any()


def test_int4_nibble_order():
    """Canonical INT4 byte j holds k = 2j in the low nibble, k = 2j+1 high."""
    rng = np.random.default_rng(3)
    v, e, z, j, _ = grid_groups(rng, 3, 128, 4, 64)
    m = oracle.quantize(v, 4, 64)
    jj = j.reshape(3, 128)
    np.testing.assert_array_equal(m.q, (jj[:, 0::2] | (jj[:, 1::2] << 4)).astype(np.uint8))


@pytest.mark.parametrize("bits,group", CASES)
def test_invariants_random_normal(bits, group):
    rng = np.random.default_rng(4)
    rows, K = 64, group * 8
    w = (rng.standard_normal((rows, K)) * 0.02).astype(np.float32)
    m = oracle.quantize(w, bits, group)
    qmax = (1 << bits) - 1
    q = oracle.unpack_q(m)
    assert (m.flags == 0).all()
    assert q.min() >= 0 and q.max() <= qmax
    wg = w.reshape(rows, K // group, group)
    qg = q.reshape(rows, K // group, group)
    amin = wg.argmin(axis=2)
    amax = wg.argmax(axis=2)
    qa = np.take_along_axis(qg, amin[..., None], 2)[..., 0]
    qb = np.take_along_axis(qg, amax[..., None], 2)[..., 0]
    assert (qa == 0).all()                       # roundf is odd-symmetric
    assert np.isin(qb, [qmax - 1, qmax]).all()
    # round trip within half a step: |(q - zp) * s - v| <= s/2 (+ fp32 slack of
    # the v/s division and of the scale itself, both below 2^-12 s here)
    dq = m.dequant_f64().reshape(rows, K // group, group)
    s = m.scale.astype(np.float64)[..., None]
    err = np.abs(dq - wg.astype(np.float64))
    assert (err <= s * (0.5 + 2.0 ** -12)).all()
    # zp is an exact integer and lies in range since every group spans 0
    assert (m.zp == np.round(m.zp)).all()
    assert (m.zp >= 0).all() and (m.zp <= qmax).all()


@pytest.mark.parametrize("bits,group", CASES)
def test_brute_force_nearest_level(bits, group):
    """Each code is the nearest of all 2^bits levels (up to near-ties)."""
    rng = np.random.default_rng(5)
    rows, K = 6, group * 2
    w = (rng.standard_normal((rows, K)) * rng.uniform(0.01, 3, size=(rows, 1))).astype(np.float32)
    m = oracle.quantize(w, bits, group)
    qmax = (1 << bits) - 1
    q = oracle.unpack_q(m)
    gi = np.arange(K) // group
    for r in range(rows):
        s = m.scale[r, gi].astype(np.float64)
        zp = m.zp[r, gi].astype(np.float64)
        levels = (np.arange(qmax + 1)[None, :] - zp[:, None]) * s[:, None]
        errs = np.abs(levels - w[r].astype(np.float64)[:, None])
        best = errs.min(axis=1)
        mine = errs[np.arange(K), q[r]]
        assert (mine <= best + s * 2.0 ** -12).all()


def test_flags_degenerate_and_nonfinite():
    w = (np.random.default_rng(6).standard_normal((3, 256)) * 0.02).astype(np.float32)
    w[0, 64:128] = 0.37                       # constant group: scale 0
    w[1, 0] = np.nan
    w[1, 200] = np.inf
    w[2, 128:192] = 1000.0                    # tiny span far from 0: |zp| > 2^24
    w[2, 130] = np.nextafter(np.float32(1000.0), np.float32(2000.0))
    m = oracle.quantize(w, 8, 64)
    expect = np.zeros((3, 4), np.uint8)
    expect[0, 1] = oracle.FLAG_DEGENERATE
    expect[1, 0] = oracle.FLAG_NONFINITE
    expect[1, 3] = oracle.FLAG_NONFINITE
    expect[2, 2] = oracle.FLAG_DEGENERATE
    np.testing.assert_array_equal(m.flags, expect)
    bad = m.flags != 0
    assert (m.scale[bad] == 0).all() and (m.zp[bad] == 0).all()
    q = oracle.unpack_q(m).reshape(3, 4, 64)
    assert (q[bad] == 0).all()
    # unflagged groups of the same rows are quantized normally
    m2 = oracle.quantize(w[:, 192:256].copy(), 8, 64)
    np.testing.assert_array_equal(m2.q, m.q[:, 192:256])


def test_rejects_bad_shapes():
    w = np.zeros((2, 100), np.float32)
    with pytest.raises(ValueError):
        oracle.quantize(w, 8, 64)
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros((2, 128), np.float32), 5, 64)


def test_threads_do_not_change_codes():
    w = (np.random.default_rng(7).standard_normal((257, 512)) * 0.02).astype(np.float32)
    oracle.set_threads(1)
    a = oracle.quantize(w, 4, 64)
    oracle.set_threads(8)
    b = oracle.quantize(w, 4, 64)
    np.testing.assert_array_equal(a.q, b.q)
    np.testing.assert_array_equal(a.scale, b.scale)
    np.testing.assert_array_equal(a.zp, b.zp)
