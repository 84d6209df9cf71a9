"""HIP graph capture of the compute entry points.

Every compute call only enqueues kernels on the caller's stream (no
allocation, copy, memset or synchronisation), so a graph captured from one
call replays it.  Each case captures one call on fixed buffers, then, per
replay: rewrites the inputs in place, replays, keeps the outputs, poisons
them, runs the same call eagerly and checks the replay's outputs bitwise
against the eager ones (the library's reductions are deterministic), with a
synchronisation before the next replay.  Correctness of the eager call itself
against the oracle is the other GPU tests' subject.
"""
import pytest
import torch

from gpu_util import MoeFixture, pack_gpu, say
from group_quantized_moe_dsq_amd import dsq, synth

pytestmark = pytest.mark.gpu

REPLAYS = 3


def poison(t):
    if t.dtype.is_floating_point:
        t.fill_(float("nan"))
    else:
        t.fill_(-7)


def replay_check(name, call, outputs, refill):
    """call(): the library call on the current stream, reading the inputs
    refill(r) writes and writing `outputs`."""
    say(f"graph: {name}")
    refill(0)
    call()  # first call outside the capture (one-time set-up, if any)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        refill(r + 1)
        for o in outputs:
            poison(o)
        g.replay()
        got = [o.clone() for o in outputs]
        for o in outputs:
            poison(o)
        call()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(got, outputs)):
            assert torch.equal(a, b), f"{name}: replay {r} output {i} differs from the eager call"
            if a.dtype.is_floating_point:
                assert torch.isfinite(a).all(), f"{name}: replay {r} output {i} not written"
    del g


def normal_into(t, seed, std=1.0):
    t.copy_(synth.normal(tuple(t.shape), std, 7, synth.X, seed, device="cuda"))


@pytest.mark.parametrize("bits", [8, 4])
def test_graph_gemv_and_head(bits):
    N, K = 1000, 1024
    W = pack_gpu(synth.normal((N, K), 0.02, 7, synth.W, bits, device="cuda"), bits, 64)
    x = torch.empty(K, device="cuda")
    y = torch.empty(N, device="cuda")
    replay_check(f"gemv INT{bits}", lambda: dsq.gemv(W, x, y), [y], lambda r: normal_into(x, r))
    for k in (1, 8):
        idx = torch.empty(k, dtype=torch.int32, device="cuda")
        val = torch.empty(k, device="cuda")
        ws = torch.empty(dsq.topk_workspace_bytes(N, k) + 256, dtype=torch.uint8, device="cuda")
        replay_check(f"gemv_topk INT{bits} k={k}",
                     lambda: dsq.gemv_topk(W, x, k, y=y, idx=idx, values=val, workspace=ws),
                     [y, idx, val], lambda r: normal_into(x, 100 + r))


@pytest.mark.parametrize("M,math", [(64, dsq.MATH_BF16_MFMA), (256, dsq.MATH_BF16_MFMA),
                                    (8, dsq.MATH_FP32), (40, dsq.MATH_FP32)])
def test_graph_gemm(M, math):
    N, K = 512, 2048
    W = pack_gpu(synth.normal((N, K), 0.02, 7, synth.W, 20 + M, device="cuda"), 8, 128)
    X = torch.empty((M, K), device="cuda")
    Y = torch.empty((M, N), device="cuda")
    ws = torch.empty(dsq.gemm_workspace_bytes(M, N, K, math) + 256, dtype=torch.uint8,
                     device="cuda")
    replay_check(f"gemm M={M} math={math}", lambda: dsq.gemm(W, X, Y, math=math, workspace=ws),
                 [Y], lambda r: normal_into(X, 200 + r))


@pytest.fixture(scope="module")
def fx():
    return MoeFixture(16, 512, 256, 4, 64, seed=8, bias_std=0.5)


@pytest.mark.parametrize("T,k,math", [(1, 6, dsq.MATH_FP32), (3, 3, dsq.MATH_FP32),
                                      (40, 4, dsq.MATH_FP32), (64, 6, dsq.MATH_BF16_MFMA)])
def test_graph_moe(fx, T, k, math):
    lay = fx.layer(k)
    H, E = fx.H, fx.E
    X = torch.empty((T, H), device="cuda")
    Y = torch.empty((T, H), device="cuda")
    logits = torch.empty((T, E), device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), device="cuda")
    counts = torch.empty((E,), dtype=torch.int32, device="cuda")
    ws = torch.empty(dsq.moe_workspace_bytes(T, E, k, H, fx.I, math) + 256, dtype=torch.uint8,
                     device="cuda")
    replay_check(f"moe_ffn T={T} k={k} math={math}",
                 lambda: dsq.moe_ffn(lay, X, math=math, Y=Y, workspace=ws, logits_out=logits,
                                     idx_out=idx, w_out=w, counts_out=counts),
                 [Y, logits, idx, w, counts], lambda r: normal_into(X, 300 + T + r))
    # the entry point without a workspace argument, on the library's scratch
    replay_check(f"moe_ffn_noalloc T={T} k={k} math={math}",
                 lambda: dsq.moe_ffn_noalloc(lay, X, math=math, Y=Y, idx_out=idx, w_out=w),
                 [Y, idx, w], lambda r: normal_into(X, 400 + T + r))


@pytest.mark.parametrize("T", [1, 40])
def test_graph_moe_block(fx, T):
    k = 4
    lay = fx.layer(k)
    H = fx.H
    X = torch.empty((T, H), device="cuda")
    Y = torch.empty((T, H), device="cuda")
    xn = torch.empty((T, H), device="cuda")
    gamma = synth.normal((H,), 0.25, 7, synth.X, 900, device="cuda") + 1.0
    ws = torch.empty(dsq.moe_block_workspace_bytes(T, fx.E, k, H, fx.I, dsq.MATH_FP32) + 256,
                     dtype=torch.uint8, device="cuda")
    replay_check(f"moe_block T={T}",
                 lambda: dsq.moe_block(lay, X, gamma, math=dsq.MATH_FP32, Y=Y, workspace=ws,
                                       xn_out=xn),
                 [Y, xn], lambda r: normal_into(X, 500 + T + r))
