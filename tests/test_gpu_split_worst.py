"""GPU: the fp32-accuracy matrix-core path driven to its worst case.

Batched tokens (dsq_gemm FP32 with M >= 2, and the MoE expert GEMMs) run on
the matrix cores with the weights as exact integer codes and each activation
split into two bf16 parts, x = hi + lo.  Two round-to-nearest bf16 steps
leave |x - hi - lo| <= 2^-17 |x|; the bound is reached at the significand
1.0019607543945312 (bits 0x4040 above the exponent: the residual is
0.998 * 2^-17 x, with x > hi + lo).  Here every activation has that
significand (exponents vary) and every weight is positive, so every group's
minimum is above zero, every (q - zp) is positive and every product has the
same sign: the split's errors all add up in one direction, the worst case
for the per-output gate |err| <= 1e-5 * sum_k |x_k w_k| (the fp32-FMA gate of
the workload).  The accumulation error of the fp32 sums comes on top.

Method: "Hand-writing a DeepSeek inference engine in pure C"
(hnwysp.cn/news/134870) §3.2-§3.3 (dequantized (q - zero_point) * scale
inside the matmul).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import MoeFixture, assert_bounded, check_moe_result, say
from group_quantized_moe_dsq_amd import dsq

pytestmark = pytest.mark.gpu

WORST = 1.0019607543945312


def split_residual(x):
    """x - hi - lo in fp64 for the two-part bf16 split (round to nearest even)."""
    def bf16(v):
        b = v.view(np.uint32).astype(np.uint64)
        return ((b + ((b >> 16) & 1) + 0x7FFF) & 0xFFFF0000).astype(np.uint32).view(np.float32)
    hi = bf16(x)
    lo = bf16((x - hi).astype(np.float32))
    return x.astype(np.float64) - hi.astype(np.float64) - lo.astype(np.float64)


def adversarial_x(shape, seed):
    rng = np.random.default_rng(seed)
    return (WORST * np.exp2(rng.integers(-3, 3, size=shape))).astype(np.float32)


def positive_w(shape, seed):
    rng = np.random.default_rng(seed)
    return (0.02 * (1.0 + rng.random(shape))).astype(np.float32)


def test_worst_significand_reaches_the_bound():
    x = adversarial_x((4096,), 0)
    r = split_residual(x) / x
    assert (r > 0.998 * 2.0 ** -17).all() and (r <= 2.0 ** -17).all()


@pytest.mark.parametrize("bits,group", [(8, 64), (4, 64), (8, 128), (4, 128)])
@pytest.mark.parametrize("M", [2, 8, 33])
def test_gemm_fp32_worst_case_split(bits, group, M):
    N, K = 96, 4096
    say(f"gemm fp32 worst-case split M={M} N={N} K={K} bits={bits} g{group}")
    w = positive_w((N, K), 1)
    X = adversarial_x((M, K), 2 + M)
    m = oracle.quantize(w, bits, group)
    assert (m.zp < 0).all(), "every group's minimum is above zero"
    qw = dsq.QWeight(bits, group, K, N)
    dsq.pack_weights(torch.from_numpy(w).cuda(), qw)
    Y = dsq.gemm(qw, torch.from_numpy(X).cuda(), math=dsq.MATH_FP32).cpu().numpy()
    ref, S = oracle.qmatmul_ref(X, m)
    assert np.allclose(np.abs(ref), S, rtol=1e-12), "every product is positive"
    assert_bounded(Y, ref, 1e-5 * S, "worst-case split, fp32 gate")


def positive_experts(e, H, I, seed):
    g = positive_w((I, H), 100 + 3 * e)
    u = positive_w((I, H), 101 + 3 * e)
    d = positive_w((H, I), 102 + 3 * e)
    return tuple(torch.from_numpy(a).cuda() for a in (g, u, d))


@pytest.mark.parametrize("T", [1, 3, 9])
def test_moe_fp32_worst_case_split(T):
    """The expert GEMMs (decode kernels for T <= 4, grouped kernels above) on
    worst-case activations.  The output is bounded by the first-order worst
    case of contractions each within 1e-5 of their magnitude sums:
    1e-5 * (S_Y + P_Y), P_Y carrying the gate/up errors through SwiGLU and
    the down projection."""
    E, H, I, k = 8, 1024, 256, 2
    say(f"moe fp32 worst-case split T={T} E={E} H={H} I={I}")
    fx = MoeFixture(E, H, I, 4, 64, seed=21, weights=positive_experts)
    X = torch.from_numpy(adversarial_x((T, H), 30 + T)).cuda()
    lay = fx.layer(k)
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    counts = torch.empty((E,), dtype=torch.int32, device="cuda")
    Y = dsq.moe_ffn(lay, X, math=dsq.MATH_FP32, logits_out=logits, idx_out=idx, w_out=w,
                    counts_out=counts)
    torch.cuda.synchronize()
    tok, Yref, bound = check_moe_result(fx, X.cpu().numpy(), logits.cpu().numpy(),
                                        idx.cpu().numpy(), w.cpu().numpy(),
                                        counts.cpu().numpy(), k, 1e-5, propagated=True)
    assert_bounded(Y.cpu().numpy()[tok], Yref, bound, "moe output, worst-case split")
