"""GPU parity: the whole routed MoE layer (router, top-k, grouping, expert
SwiGLU GEMMs, weighted combine) against the oracle.

Method: "Hand-writing a DeepSeek inference engine in pure C"
(hnwysp.cn/news/134870) §3.4-§3.5.  Bounds:
  logits : |l - l_ref| <= 1e-5 * sum_h |x_h wr_h|  (+ one fp32 rounding of the
           bias addition);
  idx    : the same expert set as the oracle's for every token whose oracle
           margin between the k-th and (k+1)-th logit exceeds twice the logit
           bound; for the others (near-ties, where both choices are right) the
           GPU's set must be one of the sets the oracle admits within that
           bound; slots ordered by the kernel's own fp32 scores;
  w      : first-order softmax propagation of the logit bound, + 1e-6;
  Y      : rel * S_Y + sum_i dw_i |y_i|, S_Y = sum_i w_i S_i with S_i the
           magnitude sum of expert i's down projection (fp64, from the
           oracle), dw_i the weight bound; rel = 1e-5 (fp32) or 1e-2 (bf16
           MFMA, plus a normwise relative error of at most 1e-2).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import MoeFixture, assert_bounded, assert_normwise, check_moe_result, say
from group_quantized_moe_dsq_amd import dsq, synth

pytestmark = pytest.mark.gpu


def run_moe(fx: MoeFixture, X, k, math):
    T = X.shape[0]
    lay = fx.layer(k)
    logits = torch.empty((T, fx.E), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    counts = torch.empty((fx.E,), dtype=torch.int32, device="cuda")
    Y = dsq.moe_ffn(lay, X, math=math, logits_out=logits, idx_out=idx, w_out=w,
                    counts_out=counts)
    Y2 = dsq.moe_ffn(lay, X, math=math)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2), "moe_ffn is not deterministic"
    return (Y.cpu().numpy(), logits.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy(),
            counts.cpu().numpy())


def check_moe(fx: MoeFixture, X, k, math, rel, tokens=None):
    Y, L, idx, w, counts = run_moe(fx, X, k, math)
    tok, Yref, bound = check_moe_result(fx, X.cpu().numpy(), L, idx, w, counts, k, rel, tokens)
    assert_bounded(Y[tok], Yref, bound, "moe output")
    if rel > 1e-5:
        assert_normwise(Y[tok], Yref, rel, "moe output")
    return idx


# T <= 4 runs the per-slot decode kernels, larger T the expert-grouped ones
SMALL = [(8, 256, 128, 4, 64, 2, 1), (8, 256, 128, 4, 64, 2, 5), (16, 128, 192, 8, 64, 4, 33),
         (8, 256, 128, 4, 64, 2, 3), (16, 512, 256, 8, 128, 6, 4), (4, 8192, 128, 8, 64, 2, 2),
         (4, 384, 128, 8, 128, 1, 17), (32, 512, 256, 4, 128, 6, 40),
         # ~20 tokens per expert: three token tiles of one expert in flight
         (4, 256, 128, 8, 64, 2, 40),
         # H a multiple of 1024: the matrix-core router with K split in 4 / 8
         # slices added by the top-k kernel (ragged token and expert tiles)
         (16, 1024, 128, 4, 64, 2, 9), (24, 2048, 128, 8, 128, 3, 40),
         # the largest top_k (32 of 64): decode kernels and the grouped path, and
         # top_k = 16 through the split router
         (64, 256, 128, 8, 64, 32, 3), (64, 256, 128, 4, 64, 32, 40), (64, 1024, 128, 8, 128, 16, 9),
         # INT4 decode: an odd top_k streams one slot per down step, an even one
         # two (g64 above, g128 here)
         (8, 256, 128, 4, 64, 3, 2), (16, 512, 256, 4, 128, 5, 1), (16, 512, 256, 4, 128, 4, 3),
         # 256 tokens per expert: 32 token tiles of 8 in every expert
         (16, 256, 128, 4, 64, 4, 1024)]


@pytest.mark.parametrize("E,H,I,bits,group,k,T", SMALL)
def test_moe_fp32_small(E, H, I, bits, group, k, T):
    say(f"moe fp32 E={E} H={H} I={I} bits={bits} group={group} k={k} T={T}")
    fx = MoeFixture(E, H, I, bits, group, seed=4, bias_std=0.5 if T > 5 else None)
    X = synth.normal((T, H), 1.0, 4, synth.X, T, device="cuda")
    check_moe(fx, X, k, dsq.MATH_FP32, 1e-5)


@pytest.mark.parametrize("E,H,I,bits,group,k,T", [(8, 256, 128, 8, 128, 2, 64),
                                                  (16, 512, 256, 4, 64, 4, 100),
                                                  (8, 128, 192, 8, 64, 3, 7),
                                                  (16, 1024, 256, 4, 64, 4, 100),
                                                  # ~770 tokens per expert: 49 token tiles
                                                  (16, 512, 256, 8, 128, 6, 2048)])
def test_moe_bf16_small(E, H, I, bits, group, k, T):
    say(f"moe bf16 E={E} H={H} I={I} bits={bits} group={group} k={k} T={T}")
    fx = MoeFixture(E, H, I, bits, group, seed=5)
    X = synth.normal((T, H), 1.0, 5, synth.X, T, device="cuda")
    check_moe(fx, X, k, dsq.MATH_BF16_MFMA, 1e-2)


def test_moe_single_expert_is_dense_swiglu():
    """E = 1, k = 1: the layer reduces to one dense SwiGLU FFN with weight 1."""
    say("moe E=1 k=1")
    fx = MoeFixture(1, 256, 128, 8, 64, seed=6)
    X = synth.normal((9, 256), 1.0, 6, synth.X, 9, device="cuda")
    idx = check_moe(fx, X, 1, dsq.MATH_FP32, 1e-5)
    assert (idx == 0).all()


def test_moe_decode_one_token_full_size():
    """One token, hidden 4096, 256 INT4 group-64 experts (I = 2048), top-6,
    fp32 router 4096x256."""
    say("moe decode T=1 full size")
    fx = MoeFixture(256, 4096, 2048, 4, 64, seed=0)
    X = synth.normal((1, 4096), 1.0, 0, synth.X, 3, device="cuda")
    check_moe(fx, X, 6, dsq.MATH_FP32, 1e-5)


def test_moe_batched_decode_32_tokens_skewed_full_size():
    """32 tokens through the same layer shape with a per-expert router bias
    ~N(0,1) that makes expert load uneven; experts grouped before the GEMMs."""
    say("moe batched decode T=32 full size, skewed")
    fx = MoeFixture(256, 4096, 2048, 4, 64, seed=0, bias_std=1.0)
    X = synth.normal((32, 4096), 1.0, 0, synth.X, 4, device="cuda")
    idx = check_moe(fx, X, 6, dsq.MATH_FP32, 1e-5)
    say(f"  distinct experts touched: {len(np.unique(idx))}, "
        f"max tokens per expert: {np.bincount(idx.reshape(-1)).max()}")


def test_moe_prefill_256_tokens_full_size():
    """256 tokens, 256 INT8 group-128 SwiGLU experts, bf16 MFMA path; the
    routing and the output of every token are checked (so every (expert,
    token tile) item of the grouped GEMMs is compared)."""
    say("moe prefill T=256 full size INT8 g128 bf16")
    fx = MoeFixture(256, 4096, 2048, 8, 128, seed=0)
    X = synth.normal((256, 4096), 1.0, 0, synth.X, 5, device="cuda")
    check_moe(fx, X, 6, dsq.MATH_BF16_MFMA, 1e-2)
