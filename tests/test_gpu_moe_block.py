"""GPU parity: the MoE step of a block with its RMSNorm and residual,
Y = X + moe(rmsnorm(X) * g), through dsq_moe_block.

Method: each block normalises with RMSNorm before the feed-forward / MoE
step and adds the residual after it ("Hand-writing a DeepSeek inference
engine in pure C", hnwysp.cn/news/134870, §2.1; epsilon 1e-6 from the model
constants of "ds4 code walkthrough"); the MoE layer itself as §3.4-§3.5.

Checks, each against the oracle:
  xn : the normalised rows (returned through xn_out) against the fp64
       RMSNorm, |xn - xn_ref| <= (H/256 + 16) * 2^-24 * |xn_ref|.  Derived
       from the kernels' arithmetic: each thread adds H/256 squares in order
       (fused multiply-add), six butterfly levels and three cross-wave adds
       follow (relative error of a sum of positive terms <= depth * 2^-24),
       the square root halves that, and the reciprocal and two products add
       one rounding each.
  MoE: logits, routing and weights checked on the GPU's own xn (the rows the
       router and the experts saw), with the bounds of the MoE layer test.
  Y  : the oracle's X + moe(xn) within the MoE output bound plus one fp32
       rounding of the residual addition, 2^-24 * |X + moe|.
Also: repeated calls are bitwise identical, and the in-place form (Y = X)
equals the out-of-place one bitwise.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import MoeFixture, assert_bounded, assert_normwise, check_moe_result, say
from group_quantized_moe_dsq_amd import dsq, synth

pytestmark = pytest.mark.gpu

EPS = 1e-6


def norm_weight(H, seed):
    return (synth.normal((H,), 0.25, seed, synth.X, 900, device="cuda") + 1.0).contiguous()


def check_block(fx: MoeFixture, X, g, k, math, rel, tokens=None):
    T, H = X.shape
    lay = fx.layer(k)
    xn = torch.empty((T, H), dtype=torch.float32, device="cuda")
    logits = torch.empty((T, fx.E), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    counts = torch.empty((fx.E,), dtype=torch.int32, device="cuda")
    Y = dsq.moe_block(lay, X, g, EPS, math=math, xn_out=xn, logits_out=logits, idx_out=idx,
                      w_out=w, counts_out=counts)
    Y2 = dsq.moe_block(lay, X, g, EPS, math=math)
    Xin = X.clone()
    dsq.moe_block(lay, Xin, g, EPS, math=math, Y=Xin)  # in place
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2), "moe_block is not deterministic"
    assert torch.equal(Y, Xin), "in-place moe_block differs from out-of-place"

    Xh = X.cpu().numpy()
    xn_h = xn.cpu().numpy()
    xref = oracle.rmsnorm_f64(Xh, g.cpu().numpy(), EPS)
    assert_bounded(xn_h, xref, (H / 256 + 16) * 2.0 ** -24 * np.abs(xref), "rmsnorm")

    tok, mref, bound = check_moe_result(fx, xn_h, logits.cpu().numpy(), idx.cpu().numpy(),
                                        w.cpu().numpy(), counts.cpu().numpy(), k, rel, tokens)
    Yref = Xh[tok].astype(np.float64) + mref
    Yh = Y.cpu().numpy()[tok]
    assert_bounded(Yh, Yref, bound + 2.0 ** -24 * np.abs(Yref), "block output")
    if rel > 1e-5:
        assert_normwise(Yh - Xh[tok], mref, rel, "block moe part")
    return idx.cpu().numpy()


# T <= 4: decode kernels with the norm fused into the router; 5..32: grouped
# kernels, norm fused into the router; > 32: separate norm kernel
CASES = [(8, 256, 128, 4, 64, 2, 1, dsq.MATH_FP32), (16, 512, 256, 8, 128, 6, 4, dsq.MATH_FP32),
         (8, 256, 128, 4, 64, 2, 5, dsq.MATH_FP32), (16, 128, 192, 8, 64, 4, 33, dsq.MATH_FP32),
         (8, 256, 128, 8, 128, 2, 64, dsq.MATH_BF16_MFMA), (4, 8192, 128, 8, 64, 2, 2, dsq.MATH_FP32),
         # norm kernel, then the matrix-core router with K in 8 slices
         (24, 2048, 128, 4, 64, 2, 40, dsq.MATH_FP32)]


@pytest.mark.parametrize("E,H,I,bits,group,k,T,math", CASES)
def test_moe_block_small(E, H, I, bits, group, k, T, math):
    say(f"moe block E={E} H={H} I={I} bits={bits} group={group} k={k} T={T} math={math}")
    fx = MoeFixture(E, H, I, bits, group, seed=7, bias_std=0.5 if T > 5 else None)
    X = synth.normal((T, H), 1.0, 7, synth.X, T, device="cuda")
    X[T // 2] *= 50.0   # rows of very different scale: the norm must be per row
    g = norm_weight(H, 7)
    check_block(fx, X, g, k, math, 1e-2 if math == dsq.MATH_BF16_MFMA else 1e-5)


def test_moe_block_decode_one_token_full_size():
    """One token through the full layer shape: hidden 4096, 256 INT4 group-64
    experts (I = 2048), top-6, fp32 router."""
    say("moe block decode T=1 full size")
    fx = MoeFixture(256, 4096, 2048, 4, 64, seed=0)
    X = synth.normal((1, 4096), 3.0, 0, synth.X, 11, device="cuda")
    check_block(fx, X, norm_weight(4096, 0), 6, dsq.MATH_FP32, 1e-5)
