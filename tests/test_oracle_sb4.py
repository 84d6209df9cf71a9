"""Pins for the oracle's two-level super-block 4-bit format (CPU only).

The block is the one "ds4 code walkthrough" prints in trace 4 (quant block
struct sizes): fp16 d, fp16 dmin, 12 bytes of scales, 128 bytes of nibbles
for 256 weights, 144 bytes.  The pages fix the fields and the sizes only; the
reading pinned here (oracle.c states it in full): 8 sub-blocks of 32 weights,
each with a 6-bit scale sc_j and 6-bit min m_j (sc_0..7 then m_0..7 as a
little-endian stream of 6-bit fields), a weight dequantizes to
d*sc_j*q - dmin*m_j, and the quantizer follows the group rule level by level.

The field parser below is written from that description alone (it shares
nothing with oracle.c), so a slip in the C packing, the nibble order or the
dequant formula fails here.
"""
import numpy as np
import pytest

import oracle


def parse(blocks):
    """(d, dmin, sc[.., 8], m[.., 8], q[.., 256]) of blocks[..., 144]."""
    b = np.asarray(blocks, np.uint8)
    d = b[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    dmin = b[..., 2:4].copy().view(np.float16)[..., 0].astype(np.float64)
    s12 = b[..., 4:16].astype(np.uint64)
    stream = np.zeros(b.shape[:-1], np.uint64)
    word_hi = np.zeros(b.shape[:-1], np.uint64)
    for i in range(8):                       # bytes 0..7 -> bits 0..63
        stream |= s12[..., i] << np.uint64(8 * i)
    for i in range(8, 12):                   # bytes 8..11 -> bits 64..95
        word_hi |= s12[..., i] << np.uint64(8 * (i - 8))
    fields = np.zeros(b.shape[:-1] + (16,), np.int64)
    for f in range(16):
        v = 0
        for bit in range(6):
            pos = 6 * f + bit
            src = stream if pos < 64 else word_hi
            p = pos if pos < 64 else pos - 64
            v = v | (((src >> np.uint64(p)) & np.uint64(1)).astype(np.int64) << bit)
        fields[..., f] = v
    nib = b[..., 16:144]
    q = np.empty(b.shape[:-1] + (256,), np.int64)
    q[..., 0::2] = nib & 0x0F
    q[..., 1::2] = nib >> 4
    return d, dmin, fields[..., :8], fields[..., 8:], q


def dequant_from_fields(blocks):
    d, dmin, sc, m, q = parse(blocks)
    j = np.arange(256) // 32
    return d[..., None] * sc[..., j] * q - dmin[..., None] * m[..., j]


def test_fp16_conversion_is_numpy_round_to_nearest_even():
    rng = np.random.default_rng(1)
    vals = [rng.standard_normal(2000) * s for s in (1e-8, 1e-6, 1e-3, 1.0, 300.0, 2e4)]
    special = [0.0, -0.0, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 2.0 ** -24, 2.0 ** -25,
               3 * 2.0 ** -26, 1.5 * 2.0 ** -24, 2.0 ** -14 * (1 - 2.0 ** -11), 65504.0,
               65519.0, 65520.0, 1e6, -65520.0, 6.1e-5, np.inf, -np.inf]
    x = np.concatenate(vals + [np.array(special)]).astype(np.float32)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(oracle.f16_bits(x), ref)
    nan = oracle.f16_bits(np.array([np.nan], np.float32))[0]
    assert (nan & 0x7C00) == 0x7C00 and (nan & 0x03FF) != 0
    bits = rng.integers(0, 0x7C00, 3000).astype(np.uint16)
    np.testing.assert_array_equal(oracle.f16_value(bits),
                                  bits.view(np.float16).astype(np.float64))


def test_block_is_144_bytes_per_256_weights():
    m = oracle.sb4_quantize(np.zeros((3, 768), np.float32))
    assert m.blocks.shape == (3, 3, 144)
    with pytest.raises(ValueError):
        oracle.sb4_quantize(np.zeros((1, 300), np.float32))


@pytest.mark.parametrize("seed", range(4))
def test_exact_grid_recovers_every_field(seed):
    """Weights built as d*sc_j*q - dmin*m_j from fp16-exact d, dmin with
    every sub-block holding the codes 0 and 15, one scale and one min at 63:
    the quantizer must return exactly those fields and codes."""
    rng = np.random.default_rng(10 + seed)
    rows, nb = 3, 2
    d = 2.0 ** -7 * rng.integers(1, 4, (rows, nb))       # exact in fp16
    dmin = 2.0 ** -8 * rng.integers(1, 4, (rows, nb))
    sc = rng.integers(1, 64, (rows, nb, 8))
    m = rng.integers(0, 64, (rows, nb, 8))
    sc[..., 0] = 63
    m[..., 1] = 63
    q = rng.integers(0, 16, (rows, nb, 256))
    q[..., 0::32] = 0
    q[..., 1::32] = 15
    j = np.arange(256) // 32
    w = d[..., None] * sc[..., j] * q - dmin[..., None] * m[..., j]
    w32 = w.astype(np.float32)
    assert np.array_equal(w32.astype(np.float64), w)     # the grid is exact in fp32
    mat = oracle.sb4_quantize(w32.reshape(rows, nb * 256))
    pd, pdm, psc, pm, pq = parse(mat.blocks)
    np.testing.assert_array_equal(pd, d)
    np.testing.assert_array_equal(pdm, dmin)
    np.testing.assert_array_equal(psc, sc)
    np.testing.assert_array_equal(pm, m)
    np.testing.assert_array_equal(pq, q)
    np.testing.assert_array_equal(mat.dequant_f64(), w.reshape(rows, nb * 256))
    assert not mat.flags.any()


@pytest.mark.parametrize("std", [0.02, 1.0])
def test_codes_are_the_nearest_level(std):
    """Brute force over the 16 levels d*sc_j*q' - dmin*m_j of each weight's
    sub-block: the stored code is the nearest one (half a level of slack for
    the fp32 division and the half-way rounding)."""
    rng = np.random.default_rng(20)
    w = (rng.standard_normal((6, 1024)) * std).astype(np.float32)
    w[1, :256] += np.float32(3 * std)                  # an all-positive block
    w[2, 256:512] -= np.float32(3 * std)               # an all-negative block
    mat = oracle.sb4_quantize(w)
    d, dmin, sc, m, q = parse(mat.blocks)
    j = np.arange(256) // 32
    S = (d[..., None] * sc[..., j]).reshape(6, 1024)
    M = (dmin[..., None] * m[..., j]).reshape(6, 1024)
    q = q.reshape(6, 1024)
    levels = S[..., None] * np.arange(16) - M[..., None]
    dist = np.abs(w.astype(np.float64)[..., None] - levels)
    chosen = np.take_along_axis(dist, q[..., None], -1)[..., 0]
    assert (chosen <= dist.min(axis=-1) + 1e-6 * S).all()


def test_block_scale_invariants():
    rng = np.random.default_rng(30)
    w = (rng.standard_normal((8, 2048)) * 0.02).astype(np.float32)
    mat = oracle.sb4_quantize(w)
    d, dmin, sc, m, q = parse(mat.blocks)
    assert ((sc >= 0) & (sc <= 63)).all() and ((m >= 0) & (m <= 63)).all()
    assert ((q >= 0) & (q <= 15)).all()
    # d is the largest sub-block step / 63 rounded to fp16 (relative error
    # <= 2^-11), so that step maps back to exactly 63; the same for dmin
    assert (sc.max(axis=-1) == 63).all() and (m.max(axis=-1) == 63).all()
    # the levels of every sub-block reach its extremes to within half a step
    # plus the rounding of the 6-bit scales
    ws = w.astype(np.float64).reshape(8, 8, 8, 32)
    S = d[..., None] * sc
    M = dmin[..., None] * m
    lo_err = -M - ws.min(axis=-1)
    hi_err = ws.max(axis=-1) - (15 * S - M)
    tol = S / 2 + 15 * d[..., None] / 2 + dmin[..., None] / 2
    assert (lo_err <= tol).all() and (hi_err <= tol).all()


def test_dequant_is_the_field_formula():
    rng = np.random.default_rng(40)
    w = (rng.standard_normal((5, 512)) * 0.05).astype(np.float32)
    mat = oracle.sb4_quantize(w)
    np.testing.assert_array_equal(mat.dequant_f64(),
                                  dequant_from_fields(mat.blocks).reshape(5, 512))


def test_nonfinite_and_overflowing_blocks_are_zero_and_flagged():
    rng = np.random.default_rng(50)
    w = (rng.standard_normal((2, 768)) * 0.02).astype(np.float32)
    w[0, 300] = np.nan
    w[1, 10] = 1e8             # step / 63 = 1.06e5 overflows fp16
    mat = oracle.sb4_quantize(w)
    assert mat.flags[0, 1] == oracle.FLAG_NONFINITE and mat.flags[1, 0] == oracle.FLAG_DEGENERATE
    assert not mat.blocks[0, 1].any() and not mat.blocks[1, 0].any()
    assert mat.flags[0, 0] == 0 and mat.flags[0, 2] == 0 and mat.flags[1, 1] == 0
    deq = mat.dequant_f64()
    assert not deq[0, 256:512].any() and not deq[1, :256].any()
    ok = oracle.sb4_quantize(w[:, 512:])
    np.testing.assert_array_equal(mat.blocks[:, 2], ok.blocks[:, 0])


def test_zero_and_constant_blocks():
    z = oracle.sb4_quantize(np.zeros((1, 256), np.float32))
    assert not z.blocks.any() and not z.flags.any()
    for c in (0.75, -0.3):
        mat = oracle.sb4_quantize(np.full((1, 256), c, np.float32))
        deq = mat.dequant_f64()
        # a constant block is reproduced to within fp16's relative precision
        assert np.allclose(deq, c, rtol=2.0 ** -10, atol=0)
