"""A seeded sweep over supported shapes, beyond the hand-picked ragged cases of
the other GPU tests.  Every case draws its sizes from a fixed generator (the
case number is its seed; the sizes are printed before it runs) and checks the
library against the oracle with the bounds those tests use: the fp32 paths
within 1e-5 * sum|x w| per output, the bf16 matrix-core paths within
1e-2 * sum|x w| plus a normwise relative error of at most 1e-2, the MoE
layer through the same routing, weight and output checks as test_gpu_moe,
the super-block GEMV as test_gpu_sb4 does, and the top-k selection bitwise
(indices and value bits) as test_gpu_head does."""
import numpy as np
import pytest

import oracle
from gpu_util import MoeFixture, assert_bounded, assert_normwise, gpu_weights, pack_gpu, say
from group_quantized_moe_dsq_amd import dsq, synth
from test_gpu_moe import check_moe

pytestmark = pytest.mark.gpu


def rng(kind, case):
    return np.random.default_rng([7919, kind, case])


def qformat(r):
    return int(r.choice([4, 8])), int(r.choice([64, 128]))


@pytest.mark.parametrize("case", range(16))
def test_sweep_gemv(case):
    r = rng(1, case)
    bits, group = qformat(r)
    N = int(r.integers(1, 3000))
    # up to 12288 columns: INT8 rows beyond 4096 take the long-row kernel
    K = group * int(r.integers(1, 12288 // group + 1))
    say(f"sweep gemv case={case} bits={bits} group={group} N={N} K={K}")
    w = gpu_weights((N, K), 11, synth.W, case)
    x = synth.normal((K,), 1.0, 11, synth.X, case, device="cuda")
    qw = pack_gpu(w, bits, group)
    y = dsq.gemv(qw, x).cpu().numpy()
    m = oracle.quantize(w.cpu().numpy(), bits, group)
    ref, S = oracle.qmatmul_ref(x.cpu().numpy()[None, :], m)
    assert_bounded(y, ref[0], 1e-5 * S[0], "gemv vs fp64")


@pytest.mark.parametrize("case", range(10))
def test_sweep_gemm_bf16(case):
    r = rng(2, case)
    bits, group = qformat(r)
    M = int(r.integers(2, 600))
    N = int(r.integers(1, 700))
    K = 128 * int(r.integers(1, 33))  # a multiple of the 64-wide K step and of the group
    say(f"sweep gemm bf16 case={case} bits={bits} group={group} M={M} N={N} K={K}")
    w = gpu_weights((N, K), 12, synth.W, case)
    X = synth.normal((M, K), 1.0, 12, synth.X, case, device="cuda")
    qw = pack_gpu(w, bits, group)
    Y = dsq.gemm(qw, X, math=dsq.MATH_BF16_MFMA).cpu().numpy()
    m = oracle.quantize(w.cpu().numpy(), bits, group)
    ref, S = oracle.qmatmul_ref(X.cpu().numpy(), m)
    assert_bounded(Y, ref, 1e-2 * S, "gemm bf16 vs fp64")
    assert_normwise(Y, ref, 1e-2, "gemm bf16 vs fp64")


@pytest.mark.parametrize("case", range(8))
def test_sweep_gemm_fp32(case):
    r = rng(3, case)
    bits, group = qformat(r)
    M = int(r.integers(2, 130))
    N = int(r.integers(1, 700))
    K = group * int(r.integers(1, 4096 // group + 1))
    say(f"sweep gemm fp32 case={case} bits={bits} group={group} M={M} N={N} K={K}")
    w = gpu_weights((N, K), 13, synth.W, case)
    X = synth.normal((M, K), 1.0, 13, synth.X, case, device="cuda")
    qw = pack_gpu(w, bits, group)
    Y = dsq.gemm(qw, X, math=dsq.MATH_FP32).cpu().numpy()
    m = oracle.quantize(w.cpu().numpy(), bits, group)
    ref, S = oracle.qmatmul_ref(X.cpu().numpy(), m)
    assert_bounded(Y, ref, 1e-5 * S, "gemm fp32 vs fp64")


@pytest.mark.parametrize("case", range(10))
def test_sweep_moe(case):
    r = rng(4, case)
    bits, group = qformat(r)
    E = int(r.integers(1, 65))
    k = int(r.integers(1, min(E, 8) + 1))
    H = group * int(r.integers(1, 13))
    I = group * int(r.integers(1, 9))
    T = int(r.integers(1, 71))
    math = int(r.choice([dsq.MATH_FP32, dsq.MATH_BF16_MFMA]))
    bias = float(r.choice([0.0, 0.5]))
    say(f"sweep moe case={case} E={E} k={k} H={H} I={I} T={T} bits={bits} group={group} "
        f"math={math} bias={bias}")
    fx = MoeFixture(E, H, I, bits, group, seed=14 + case, bias_std=bias or None)
    X = synth.normal((T, H), 1.0, 14, synth.X, case, device="cuda")
    check_moe(fx, X, k, math, 1e-5 if math == dsq.MATH_FP32 else 1e-2)


@pytest.mark.parametrize("case", range(8))
def test_sweep_superblock_gemv(case):
    from test_gpu_sb4 import gemv_check
    r = rng(5, case)
    N = int(r.integers(1, 2500))
    K = 256 * int(r.integers(1, 49))  # up to 12288: the long-row kernel too
    say(f"sweep sb4 gemv case={case} N={N} K={K}")
    gemv_check(N, K, 900 + case)


@pytest.mark.parametrize("case", range(12))
def test_sweep_topk(case):
    import torch

    from test_gpu_head import bits, values
    r = rng(6, case)
    N = int(r.integers(1, 200000))
    k = int(r.integers(1, min(N, 256) + 1))
    pattern = str(r.choice(["normal", "ties", "special"]))
    say(f"sweep topk case={case} N={N} k={k} pattern={pattern}")
    y = values(N, pattern, 1000 + case)
    idx, val = dsq.topk(torch.from_numpy(y).cuda(), k)
    ref_idx, ref_val = oracle.topk(y, k)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    np.testing.assert_array_equal(bits(val.cpu().numpy()), bits(ref_val))
