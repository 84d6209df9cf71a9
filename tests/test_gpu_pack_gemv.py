"""GPU parity: the packer (bit-exact against the oracle's quantizer) and the
fused-dequant GEMV (fp32 gate |err| <= 1e-5 * sum|x*w|, exact cases
bitwise).  Method: "Hand-writing a DeepSeek inference engine in pure C"
(hnwysp.cn/news/134870) §2.3, §3.2, §3.3."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (as_qmat, assert_bounded, device_entry, gpu_weights, pack_gpu, say)
from group_quantized_moe_dsq_amd import dsq, synth
from test_oracle_quant import grid_groups

pytestmark = pytest.mark.gpu

PACK_CASES = [(8, 64, 33, 192), (4, 64, 33, 192), (8, 128, 7, 384), (4, 128, 65, 256),
              (8, 64, 256, 4096), (4, 64, 300, 4096), (4, 128, 3, 2048)]


@pytest.mark.parametrize("bits,group,N,K", PACK_CASES)
def test_pack_bit_exact(bits, group, N, K):
    say(f"pack bits={bits} group={group} N={N} K={K}")
    w = gpu_weights((N, K), 0, synth.W, N * 1000 + K)
    # vary magnitudes across rows so scales span many binades
    w *= torch.exp(synth.normal((N, 1), 2.0, 0, synth.W, 7, device="cuda"))
    qw = pack_gpu(w, bits, group)
    q, s, z = device_entry(qw)
    ref = oracle.quantize(w.cpu().numpy(), bits, group)
    assert (ref.flags == 0).all()
    np.testing.assert_array_equal(q, ref.q)
    np.testing.assert_array_equal(s.view(np.uint32), ref.scale.view(np.uint32))
    np.testing.assert_array_equal(z.view(np.uint32), ref.zp.view(np.uint32))


@pytest.mark.parametrize("bits,group", [(8, 64), (4, 64), (8, 128), (4, 128)])
def test_pack_half_way_ties(bits, group):
    """Exact half-way values: the GPU must round them away from zero too."""
    say(f"pack ties bits={bits} group={group}")
    rng = np.random.default_rng(50)
    v, *_ = grid_groups(rng, 9, group * 4, bits, group, half_points=True)
    qw = pack_gpu(torch.from_numpy(v).cuda(), bits, group)
    q, s, z = device_entry(qw)
    ref = oracle.quantize(v, bits, group)
    np.testing.assert_array_equal(q, ref.q)
    np.testing.assert_array_equal(s, ref.scale)
    np.testing.assert_array_equal(z, ref.zp)


def test_pack_batch_entries_and_offsets():
    say("pack batch entries")
    B, N, K = 3, 40, 256
    w = gpu_weights((B, N, K), 0, synth.W, 99)
    qw = dsq.QWeight(4, 64, K, N, B)
    dsq.pack_weights(w[1:].contiguous(), qw, first=1)
    dsq.pack_weights(w[0].contiguous(), qw, first=0)
    for b in range(B):
        q, s, z = device_entry(qw, b)
        ref = oracle.quantize(w[b].cpu().numpy(), 4, 64)
        np.testing.assert_array_equal(q, ref.q)
        np.testing.assert_array_equal(s, ref.scale)
        np.testing.assert_array_equal(z, ref.zp)


def test_pack_flags_degenerate_and_nonfinite():
    say("pack flags")
    w = (np.random.default_rng(51).standard_normal((3, 256)) * 0.02).astype(np.float32)
    w[0, 64:128] = 0.37
    w[1, 0] = np.nan
    w[1, 200] = np.inf
    w[2, 128:192] = 1000.0
    w[2, 130] = np.nextafter(np.float32(1000.0), np.float32(2000.0))
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    qw = dsq.QWeight(8, 64, 256, 3, 1)
    dsq.pack_weights(torch.from_numpy(w).cuda(), qw, flags=flags)
    q, s, z = device_entry(qw)
    ref = oracle.quantize(w, 8, 64)
    assert int(flags.item()) == (dsq.FLAG_DEGENERATE | dsq.FLAG_NONFINITE)
    np.testing.assert_array_equal(q, ref.q)
    np.testing.assert_array_equal(s, ref.scale)
    np.testing.assert_array_equal(z, ref.zp)
    # a clean matrix leaves the word untouched
    flags.zero_()
    dsq.pack_weights(torch.from_numpy(w[:, 192:256].copy()[[0]]).cuda(),
                     dsq.QWeight(8, 64, 64, 1, 1), flags=flags)
    assert int(flags.item()) == 0


GEMV_CASES = [(8, 64, 4096, 4096), (4, 64, 4096, 4096), (8, 128, 1000, 2048),
              (4, 128, 33, 384), (8, 64, 17, 64), (4, 64, 5, 8192), (8, 64, 3, 16384),
              (4, 64, 2048, 4096), (8, 128, 4096, 2048), (4, 64, 129, 1088),
              # very long rows (the kernel that re-reads x per chunk)
              (8, 64, 5, 65536), (4, 128, 3, 131072)]


@pytest.mark.parametrize("bits,group,N,K", GEMV_CASES)
def test_gemv_within_fp32_bound(bits, group, N, K):
    say(f"gemv bits={bits} group={group} N={N} K={K}")
    w = gpu_weights((N, K), 0, synth.W, 5 + N + K)
    x = synth.normal((K,), 1.0, 0, synth.X, K, device="cuda")
    qw = pack_gpu(w, bits, group)
    y = dsq.gemv(qw, x)
    y2 = dsq.gemv(qw, x)
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "GEMV is not deterministic"
    m = oracle.quantize(w.cpu().numpy(), bits, group)
    ref, S = oracle.qmatmul_ref(x.cpu().numpy()[None, :], m)
    assert_bounded(y.cpu().numpy(), ref[0], 1e-5 * S[0], "gemv vs fp64")


@pytest.mark.parametrize("bits,group", [(8, 64), (4, 64), (8, 128), (4, 128)])
def test_gemv_exact_special_case_bitwise(bits, group):
    """Power-of-two grid weights and small-integer x: every partial sum is
    exact in fp32, so any summation order must give the exact result."""
    say(f"gemv exact bits={bits} group={group}")
    rng = np.random.default_rng(52)
    N, K = 70, group * 6
    qmax = (1 << bits) - 1
    ng = K // group
    e = rng.integers(6, 9, size=(N, ng))
    z = rng.integers(0, qmax + 1, size=(N, ng))
    j = rng.integers(0, qmax + 1, size=(N, ng, group))
    j[:, :, 0] = 0
    j[:, :, 1] = qmax
    w = ((j - z[:, :, None]) * np.ldexp(1.0, -e)[:, :, None]).reshape(N, K).astype(np.float32)
    x = rng.integers(-4, 5, size=K).astype(np.float32)
    qw = pack_gpu(torch.from_numpy(w).cuda(), bits, group)
    y = dsq.gemv(qw, torch.from_numpy(x).cuda()).cpu().numpy()
    exact = w.astype(np.float64) @ x.astype(np.float64)
    np.testing.assert_array_equal(y.astype(np.float64), exact)


def test_gemv_one_hot_returns_dequantized_columns():
    say("gemv one-hot")
    N, K = 257, 512
    w = gpu_weights((N, K), 0, synth.W, 3)
    for bits in (8, 4):
        qw = pack_gpu(w, bits, 64)
        m = oracle.quantize(w.cpu().numpy(), bits, 64)
        cols = m.dequant_f32()
        for k in (0, 15, 16, 63, 64, 255, 511):
            x = torch.zeros(K, device="cuda")
            x[k] = 1.0
            y = dsq.gemv(qw, x).cpu().numpy()
            np.testing.assert_array_equal(y, cols[:, k])


@pytest.mark.parametrize("bits,group", [(8, 64), (4, 64), (4, 128)])
def test_gemv_vocab_projection_full_size_sampled(bits, group):
    """Vocab projection K=4096, N=129280 (the whole matrix is packed and
    multiplied on the GPU, in the large-matrix launch shape: every wave runs
    many row blocks); 1024 sampled rows are checked against the oracle, whose
    codes for those rows are recomputed from the same fp32 weights (rows
    quantize independently)."""
    say(f"gemv vocab 129280 x 4096 bits={bits} g{group}")
    N, K = 129280, 4096
    w = synth.normal((N, K), 0.02, 0, synth.W, 2, device="cuda")
    x = synth.normal((K,), 1.0, 0, synth.X, 2, device="cuda")
    qw = pack_gpu(w, bits, group)
    y = dsq.gemv(qw, x).cpu().numpy()
    rows = np.sort(np.random.default_rng(53).choice(N, 1024, replace=False))
    rows[-1] = N - 1
    wr = w[torch.from_numpy(rows).cuda()].cpu().numpy()
    m = oracle.quantize(wr, bits, group)
    ref, S = oracle.qmatmul_ref(x.cpu().numpy()[None, :], m)
    assert_bounded(y[rows], ref[0], 1e-5 * S[0], "vocab gemv sampled rows")
    # the packed codes of those rows are the oracle's
    q, s, z = device_entry(qw)
    np.testing.assert_array_equal(q[rows], m.q)
    np.testing.assert_array_equal(s[rows].view(np.uint32), m.scale.view(np.uint32))
    np.testing.assert_array_equal(z[rows].view(np.uint32), m.zp.view(np.uint32))
    del w, qw
    torch.cuda.empty_cache()
