"""GPU parity: the routed MoE layer with its experts behind the expert cache
(dsq_moe_ffn_cached): host-resident experts streamed into HBM slots, least
recently used out ("Running a 284B-parameter LLM from 3.2 GB of RAM in plain
C": per token the router decides which experts are needed and only those are
read into an LRU cache).

Each call of a token stream is checked as the MoE layer test checks
dsq_moe_ffn (logits, routing, weights and output against the oracle, the
bounds of that test), and:
  - the same expert sets as dsq_moe_ffn on the same tokens;
  - the slots used are the ones the cache tables hold for those experts, and
    the hit/miss counts follow the LRU rule on the routing the GPU produced;
  - the bytes copied are the misses times one expert's three packed matrices.
"""
import numpy as np
import pytest
import torch

from gpu_util import MoeFixture, assert_bounded, check_moe_result, say
from group_quantized_moe_dsq_amd import dsq, synth
from test_expert_cache_cpu import LruModel

pytestmark = pytest.mark.gpu


def cache_for(fx: MoeFixture, slots: int) -> dsq.ExpertCache:
    c = dsq.ExpertCache(fx.bits, fx.group, fx.H, fx.I, fx.E, slots)
    # the fixture's packed layer holds all E entries back to back: the host
    # stores are its bytes
    for m, q in enumerate((fx.gate, fx.up, fx.down)):
        c.host[m].copy_(q.buf)
    torch.cuda.synchronize()
    return c


def run_stream(fx, k, slots, sizes, seed, rel=1e-5, math=dsq.MATH_FP32):
    c = cache_for(fx, slots)
    model = LruModel(fx.E, slots)
    bias = fx.bias
    for n, T in enumerate(sizes):
        say(f"  call {n}: T={T}")
        X = synth.normal((T, fx.H), 1.0, seed, synth.X, 1000 + n, device="cuda")
        logits = torch.empty((T, fx.E), device="cuda")
        idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, k), device="cuda")
        Y = dsq.moe_ffn_cached(fx.router, bias, c, X, k, math=math, logits_out=logits,
                               idx_out=idx, w_out=w)
        # the direct layer on the same tokens picks the same experts
        idx_d = torch.empty((T, k), dtype=torch.int32, device="cuda")
        dsq.moe_ffn(fx.layer(k), X, math=math, idx_out=idx_d)
        torch.cuda.synchronize()
        idx_h = idx.cpu().numpy()
        for t in range(T):
            assert set(idx_h[t]) == set(idx_d.cpu().numpy()[t]), f"call {n} token {t}"
        counts = np.bincount(idx_h.reshape(-1), minlength=fx.E)
        tok, Yref, bound = check_moe_result(fx, X.cpu().numpy(), logits.cpu().numpy(), idx_h,
                                            w.cpu().numpy(), counts, k, rel)
        assert_bounded(Y.cpu().numpy()[tok], Yref, bound, "cached moe output")
        # slots and counters follow the LRU rule on the GPU's routing
        slots_used, _ = model.call(idx_h.reshape(-1).tolist())
        assert c.last_slots.reshape(-1).tolist() == slots_used
        assert (c.hits, c.misses) == (model.hits, model.misses)
        for e, s in zip(idx_h.reshape(-1), c.last_slots.reshape(-1)):
            assert c.expert_of[s] == e and c.slot_of[e] == s
    assert c.bytes_copied == c.misses * sum(c.strides)
    return c


@pytest.mark.parametrize("bits,group", [(4, 64), (8, 128)])
def test_cached_moe_small_stream(bits, group):
    """16 experts in 8 slots, top-2: decode calls (given-routing decode
    kernels) and grouped calls mixed, with hits, misses and evictions (a call
    of T tokens needs up to 2T distinct experts, at most the 8 slots)."""
    say(f"cached moe small bits={bits} group={group}")
    fx = MoeFixture(16, 256, 128, bits, group, seed=8)
    c = run_stream(fx, 2, 8, [1, 2, 1, 1, 3, 2, 1, 1, 4, 1, 2, 1], seed=8)
    assert c.hits > 0 and c.misses > 0


def test_cached_moe_grouped_and_bf16():
    """Larger calls through the grouped kernels, fp32 and bf16 MFMA."""
    say("cached moe grouped")
    fx = MoeFixture(32, 256, 128, 8, 128, seed=9, bias_std=0.5)
    run_stream(fx, 2, 16, [5, 7, 6], seed=9)
    run_stream(fx, 2, 24, [8, 8], seed=10, rel=1e-2, math=dsq.MATH_BF16_MFMA)


def test_cached_moe_decode_full_size():
    """Decode tokens through the full layer shape (256 INT4 group-64 experts,
    H = 4096, I = 2048, top-6) with 16 slots."""
    say("cached moe decode full size")
    fx = MoeFixture(256, 4096, 2048, 4, 64, seed=0)
    run_stream(fx, 6, 16, [1, 1, 1, 1], seed=11)


def test_cached_moe_many_tokens_matrix_core_router():
    """Calls of 40 and 36 tokens: the routing runs on the matrix-core router
    (H a multiple of 1024), all 16 experts fit the 16 slots."""
    say("cached moe many tokens")
    fx = MoeFixture(16, 1024, 128, 4, 64, seed=12, bias_std=0.5)
    run_stream(fx, 2, 16, [40, 36], seed=12)
