"""GPU parity: the batched fused-dequant GEMM (fp32 and bf16-MFMA paths) and
the router top-k.  Method: "Hand-writing a DeepSeek inference engine in pure
C" (hnwysp.cn/news/134870) §3.2-§3.5."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_bounded, assert_normwise, gpu_weights, pack_gpu, say
from group_quantized_moe_dsq_amd import dsq, synth

pytestmark = pytest.mark.gpu

FP32_CASES = [(8, 64, 2, 300, 512), (4, 64, 7, 129, 4096), (8, 128, 9, 64, 2048),
              (4, 128, 31, 100, 384), (8, 64, 33, 257, 1024), (4, 64, 8, 4096, 4096),
              (8, 64, 100, 300, 1024)]


@pytest.mark.parametrize("bits,group,M,N,K", FP32_CASES)
def test_gemm_fp32_within_bound(bits, group, M, N, K):
    say(f"gemm fp32 bits={bits} group={group} M={M} N={N} K={K}")
    w = gpu_weights((N, K), 1, synth.W, M + N + K)
    X = synth.normal((M, K), 1.0, 1, synth.X, M, device="cuda")
    qw = pack_gpu(w, bits, group)
    Y = dsq.gemm(qw, X, math=dsq.MATH_FP32).cpu().numpy()
    m = oracle.quantize(w.cpu().numpy(), bits, group)
    ref, S = oracle.qmatmul_ref(X.cpu().numpy(), m)
    assert_bounded(Y, ref, 1e-5 * S, "gemm fp32 vs fp64")


BF16_CASES = [(8, 128, 1, 64, 256), (8, 128, 16, 128, 1024), (4, 64, 33, 100, 320),
              (8, 64, 64, 257, 512), (4, 128, 100, 64, 4096), (8, 128, 256, 512, 4096),
              # three and five 128-row tiles of M, the last ragged (and a ragged N tile)
              (4, 64, 300, 640, 2048), (8, 64, 513, 200, 768)]


@pytest.mark.parametrize("bits,group,M,N,K", BF16_CASES)
def test_gemm_bf16_within_bound(bits, group, M, N, K):
    say(f"gemm bf16 bits={bits} group={group} M={M} N={N} K={K}")
    w = gpu_weights((N, K), 2, synth.W, M + N + K)
    X = synth.normal((M, K), 1.0, 2, synth.X, M, device="cuda")
    qw = pack_gpu(w, bits, group)
    Y = dsq.gemm(qw, X, math=dsq.MATH_BF16_MFMA).cpu().numpy()
    m = oracle.quantize(w.cpu().numpy(), bits, group)
    ref, S = oracle.qmatmul_ref(X.cpu().numpy(), m)
    assert_bounded(Y, ref, 1e-2 * S, "gemm bf16 vs fp64")
    assert_normwise(Y, ref, 1e-2, "gemm bf16 vs fp64")


@pytest.mark.parametrize("bits,group", [(8, 128), (4, 64), (8, 64)])
def test_gemm_bf16_exact_special_case_bitwise(bits, group):
    """Grid weights (q - zp) * 2^-e with |q - zp| <= 255 and small-integer X
    are exactly representable in bf16, their products and partial sums are
    exact in fp32: the MFMA path must reproduce the exact product bit for
    bit.  This pins the operand and output lane layouts of the MFMA tiles."""
    say(f"gemm bf16 exact bits={bits} group={group}")
    rng = np.random.default_rng(60)
    M, N, K = 48, 80, group * 4
    qmax = (1 << bits) - 1
    ng = K // group
    e = rng.integers(6, 9, size=(N, ng))
    z = rng.integers(0, qmax + 1, size=(N, ng))
    j = rng.integers(0, qmax + 1, size=(N, ng, group))
    j[:, :, 0] = 0
    j[:, :, 1] = qmax
    w = ((j - z[:, :, None]) * np.ldexp(1.0, -e)[:, :, None]).reshape(N, K).astype(np.float32)
    X = rng.integers(-4, 5, size=(M, K)).astype(np.float32)
    qw = pack_gpu(torch.from_numpy(w).cuda(), bits, group)
    Y = dsq.gemm(qw, torch.from_numpy(X).cuda(), math=dsq.MATH_BF16_MFMA).cpu().numpy()
    exact = X.astype(np.float64) @ w.astype(np.float64).T
    np.testing.assert_array_equal(Y.astype(np.float64), exact)
    Yf = dsq.gemm(qw, torch.from_numpy(X).cuda(), math=dsq.MATH_FP32).cpu().numpy()
    np.testing.assert_array_equal(Yf.astype(np.float64), exact)


def test_gemm_prefill_dense_full_size_sampled():
    """The dense INT8 group-128 4096x4096 projection applied to 256 tokens on
    the bf16 MFMA path; 512 sampled output columns of all 256 rows are
    checked."""
    say("gemm prefill dense M=256 K=N=4096 INT8 g128 bf16")
    N = K = 4096
    M = 256
    w = synth.normal((N, K), 0.02, 0, synth.W, 5, device="cuda")
    X = synth.normal((M, K), 1.0, 0, synth.X, 5, device="cuda")
    qw = pack_gpu(w, 8, 128)
    Y = dsq.gemm(qw, X, math=dsq.MATH_BF16_MFMA).cpu().numpy()
    cols = np.sort(np.random.default_rng(61).choice(N, 512, replace=False))
    m = oracle.quantize(w[torch.from_numpy(cols).cuda()].cpu().numpy(), 8, 128)
    ref, S = oracle.qmatmul_ref(X.cpu().numpy(), m)
    assert_bounded(Y[:, cols], ref, 1e-2 * S, "prefill gemm sampled columns")
    assert_normwise(Y[:, cols], ref, 1e-2, "prefill gemm sampled columns")


ROUTE_CASES = [(100, 256, 6, False), (37, 256, 6, True), (50, 8, 2, False), (20, 64, 1, True),
               (9, 1000, 32, False), (5, 4096, 8, True), (3, 1, 1, False), (4, 16, 16, False)]


@pytest.mark.parametrize("T,E,k,with_bias", ROUTE_CASES)
def test_route_topk_bit_exact(T, E, k, with_bias):
    say(f"route T={T} E={E} k={k} bias={with_bias}")
    L = synth.normal((T, E), 1.0, 3, synth.LOGITS, E, device="cuda")
    # plant exact ties between experts
    if E >= 4:
        L[:, E - 1] = L[:, 0]
        L[: T // 2, 1] = L[: T // 2, 2]
    bias = synth.normal((E,), 0.5, 3, synth.BIAS, E, device="cuda") if with_bias else None
    idx, w = dsq.moe_route_topk(L, k, bias=bias)
    # the scores the kernel ranks: one IEEE fp32 addition, redone on the host
    scores = L.cpu().numpy()
    if with_bias:
        scores = (scores + bias.cpu().numpy()[None, :]).astype(np.float32)
    ref_idx, ref_w, _ = oracle.route(scores.astype(np.float64), k)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    np.testing.assert_allclose(w.cpu().numpy(), ref_w, rtol=0, atol=1e-6)
    assert np.allclose(w.cpu().numpy().sum(1), 1.0, atol=1e-6)


def test_route_all_equal_scores_pick_highest_indices():
    say("route all-equal")
    L = torch.zeros((3, 256), device="cuda")
    idx, w = dsq.moe_route_topk(L, 6)
    assert (idx.cpu().numpy() == np.arange(255, 249, -1)).all()
    np.testing.assert_allclose(w.cpu().numpy(), 1.0 / 6, rtol=0, atol=1e-7)
