"""GPU: dsq_moe_ffn_noalloc (the MoE layer on the library's fixed scratch,
for callers that cannot allocate) gives bitwise the results of dsq_moe_ffn
with a caller workspace, call after call on the shared scratch, the second
call smaller than the first; sizes beyond the scratch are refused on the
host."""
import ctypes

import pytest
import torch

from gpu_util import MoeFixture, say
from group_quantized_moe_dsq_amd import dsq, synth

pytestmark = pytest.mark.gpu


def both(fx, k, X, math):
    T, E = X.shape[0], fx.E
    outs = []
    for fn in (dsq.moe_ffn_noalloc, dsq.moe_ffn):
        L = torch.empty((T, E), dtype=torch.float32, device="cuda")
        idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, k), dtype=torch.float32, device="cuda")
        c = torch.empty((E,), dtype=torch.int32, device="cuda")
        Y = fn(fx.layer(k), X, math=math, logits_out=L, idx_out=idx, w_out=w, counts_out=c)
        outs.append((Y, L, idx, w, c))
    torch.cuda.synchronize()
    for a, b, name in zip(outs[0], outs[1], ("Y", "logits", "idx", "w", "counts")):
        assert torch.equal(a, b), f"{name} differs from dsq_moe_ffn"


@pytest.mark.parametrize("calls", [[(8, dsq.MATH_FP32), (1, dsq.MATH_FP32)],
                                   [(64, dsq.MATH_BF16_MFMA), (3, dsq.MATH_FP32)]])
def test_noalloc_matches_workspace_entry_full_size(calls):
    fx = MoeFixture(256, 4096, 2048, 4, 64, seed=0, bias_std=1.0)
    for i, (T, math) in enumerate(calls):
        say(f"moe noalloc full size call {i}: T={T} math={math}")
        X = synth.normal((T, 4096), 1.0, 0, synth.X, 700 + 10 * i + T, device="cuda")
        both(fx, 6, X, math)


def test_noalloc_small_layer_twice():
    fx = MoeFixture(8, 256, 128, 8, 128, seed=3)
    for i, T in enumerate((40, 5)):
        say(f"moe noalloc small call {i}: T={T}")
        X = synth.normal((T, 256), 1.0, 3, synth.X, 800 + T, device="cuda")
        both(fx, 2, X, dsq.MATH_FP32)


def test_noalloc_refuses_sizes_beyond_the_scratch():
    fx = MoeFixture(256, 4096, 2048, 4, 64, seed=0)
    T = 256
    assert dsq.moe_workspace_bytes(T, 256, 6, 4096, 2048, dsq.MATH_FP32) > \
        dsq.NOALLOC_SCRATCH_BYTES
    X = torch.zeros((T, 4096), device="cuda")
    Y = torch.full((T, 4096), 7.0, device="cuda")
    with pytest.raises(dsq.DsqError) as ei:
        dsq.moe_ffn_noalloc(fx.layer(6), X, math=dsq.MATH_FP32, Y=Y)
    assert ei.value.status == -4
    torch.cuda.synchronize()
    assert bool((Y == 7.0).all()), "a refused call wrote its output"
