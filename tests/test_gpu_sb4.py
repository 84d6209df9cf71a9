"""GPU parity: the two-level super-block 4-bit format (group = 256) -- the
packer bit for bit against the oracle's quantizer, the GEMV against the fp64
reference on the oracle's dequantized weights.

The block is the one "ds4 code walkthrough" prints in trace 4 (quant block
struct sizes): fp16 d, fp16 dmin, 12 bytes of 6-bit scales and mins, 128
bytes of nibbles per 256 weights; the fields' arithmetic is the reading the
oracle states (weight = d*sc_j*q - dmin*m_j).  Bounds:
  packed blocks: bit-exact after the independent layout reader turns the
                 device bytes back into canonical 144-byte blocks;
  GEMV         : |y - y_ref| <= 1e-5 * sum_k |x_k w_k| per output, with w the
                 oracle's exactly dequantized weights.
"""
import numpy as np
import pytest
import torch

import layout_v1
import oracle
from gpu_util import assert_bounded, say
from group_quantized_moe_dsq_amd import dsq, synth

pytestmark = pytest.mark.gpu


def pack_sb(w: torch.Tensor, flags=None) -> dsq.QWeight:
    if w.dim() == 2:
        w = w[None]
    B, N, K = w.shape
    qw = dsq.QWeight(4, 256, K, N, B)
    dsq.pack_weights(w.contiguous(), qw, flags=flags)
    return qw


def device_blocks(qw: dsq.QWeight, b: int = 0) -> np.ndarray:
    return layout_v1.decode_sb_entry(qw.buf.cpu().numpy(), b, qw.K, qw.N)


def weights(N, K, seed):
    w = synth.normal((N, K), 0.02, 0, synth.W, seed, device="cuda")
    # rows of very different magnitude: d and dmin span many binades,
    # down to fp16 subnormals
    w *= torch.exp(synth.normal((N, 1), 2.5, 0, synth.W, seed + 1, device="cuda"))
    return w.contiguous()


@pytest.mark.parametrize("N,K", [(1, 256), (5, 512), (33, 1024), (64, 4096), (7, 12288)])
def test_sb4_pack_bit_exact(N, K):
    say(f"sb4 pack N={N} K={K}")
    w = weights(N, K, 300 + N)
    qw = pack_sb(w)
    ref = oracle.sb4_quantize(w.cpu().numpy())
    assert not ref.flags.any()
    np.testing.assert_array_equal(device_blocks(qw), ref.blocks)


def test_sb4_pack_special_blocks_and_flags():
    """Zero, constant, tiny (fp16-subnormal d), all-positive, all-negative,
    NaN and fp16-overflowing blocks, and a batch packed in two calls."""
    say("sb4 pack special blocks")
    rng = np.random.default_rng(60)
    w = (rng.standard_normal((3, 6, 2048)) * 0.02).astype(np.float32)
    w[0, 0, 0:256] = 0.0
    w[0, 1, 256:512] = 0.4375
    w[0, 2, 512:768] *= np.float32(1e-3)          # d in fp16's subnormal range
    w[0, 3, 768:1024] = np.abs(w[0, 3, 768:1024]) + np.float32(0.01)
    w[0, 4, 1024:1280] = -np.abs(w[0, 4, 1024:1280]) - np.float32(0.01)
    w[1, 0, 300] = np.nan
    w[1, 1, 600] = np.inf
    w[2, 5, 10] = 1e8                              # step / 63 overflows fp16
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    qw = dsq.QWeight(4, 256, 2048, 6, 3)
    dsq.pack_weights(torch.from_numpy(w[1:]).cuda(), qw, first=1, flags=flags)
    dsq.pack_weights(torch.from_numpy(w[0]).cuda(), qw, first=0, flags=flags)
    want = 0
    for b in range(3):
        ref = oracle.sb4_quantize(w[b])
        want |= int(np.bitwise_or.reduce(ref.flags.reshape(-1)))
        np.testing.assert_array_equal(device_blocks(qw, b), ref.blocks)
    assert want == oracle.FLAG_NONFINITE | oracle.FLAG_DEGENERATE
    assert int(flags.item()) == want


def gemv_check(N, K, seed, rows=None):
    w = weights(N, K, seed)
    x = synth.normal((K,), 1.0, 0, synth.X, seed, device="cuda")
    qw = pack_sb(w)
    y = dsq.gemv(qw, x).cpu().numpy()
    rows = np.arange(N) if rows is None else rows
    m = oracle.sb4_quantize(w[torch.from_numpy(rows).cuda()].cpu().numpy())
    ref, S = oracle.qmatmul_sb4_ref(x.cpu().numpy()[None, :], m)
    assert_bounded(y[rows], ref[0], 1e-5 * S[0], f"sb4 gemv N={N} K={K}")
    return qw, x, y


# K = 256 .. 8192 keep the lane's x slice in registers (1..4 chunks per lane),
# 12288 takes the long-row kernel; N covers ragged row blocks
@pytest.mark.parametrize("N,K", [(1, 256), (5, 512), (37, 4096), (300, 8192), (3, 12288),
                                 (1000, 2048)])
def test_sb4_gemv(N, K):
    say(f"sb4 gemv N={N} K={K}")
    gemv_check(N, K, 500 + N)


def test_sb4_gemv_vocab_full_size_and_head():
    """The vocab projection in the super-block format, K = 4096, N = 129280:
    1024 sampled rows plus the first and last against fp64, then the top-1 of
    the logits equals the oracle's selection on the same values."""
    say("sb4 gemv vocab full size")
    N, K = 129280, 4096
    rows = np.unique(np.concatenate([[0, 1, N - 2, N - 1],
                                     np.random.default_rng(61).choice(N, 1024, replace=False)]))
    qw, x, y = gemv_check(N, K, 900, rows)
    y2, idx, val = dsq.gemv_topk(qw, x, 1)
    np.testing.assert_array_equal(y2.cpu().numpy(), y)
    ref_idx, ref_val = oracle.topk(y, 1)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    del qw
    torch.cuda.empty_cache()
