"""Expert cache, host logic only (no GPU): the slot mapping, fills and
counters of dsq_expert_cache_plan against a plain LRU model written from the
rule the header states, and the pages' observation that a cache smaller than
the set of experts a pass cycles through never hits ("Running a
284B-parameter LLM from 3.2 GB of RAM in plain C", the --budget section: a
budget below one forward pass's experts evicts every entry before its layer
comes back, 0 hits).
"""
import numpy as np
import pytest

from group_quantized_moe_dsq_amd import dsq


class LruModel:
    """Per call: a requested expert already in a slot is a hit; a miss takes
    an empty slot (lowest index) or the least recently used slot not used in
    this call.  Every request stamps its slot in request order."""

    def __init__(self, E, slots):
        self.slot_of = [-1] * E
        self.expert_of = [-1] * slots
        self.last = [0] * slots
        self.clock = 0
        self.hits = self.misses = 0

    def call(self, experts):
        first = self.clock + 1
        out, fills = [], []
        for e in experts:
            self.clock += 1
            now = self.clock
            s = self.slot_of[e]
            if s >= 0:
                self.hits += 1
            else:
                cands = [(0 if self.expert_of[j] < 0 else self.last[j], j)
                         for j in range(len(self.expert_of))]
                cands = [c for c in cands if c[0] < first]
                if not cands:
                    raise RuntimeError("working set larger than the cache")
                _, s = min(cands)
                if self.expert_of[s] >= 0:
                    self.slot_of[self.expert_of[s]] = -1
                self.expert_of[s] = e
                self.slot_of[e] = s
                self.misses += 1
                fills.append((e, s))
            self.last[s] = now
            out.append(s)
        return out, fills


def make_cache(E, slots):
    # host-side descriptors only: the "device" slot buffers are CPU tensors,
    # which plan() never touches
    return dsq.ExpertCache(4, 64, 256, 128, E, slots, device="cpu", pinned=False)


@pytest.mark.parametrize("E,slots,seed", [(32, 4, 0), (32, 8, 1), (32, 31, 2), (32, 32, 3),
                                          (256, 16, 4)])
def test_plan_matches_the_lru_rule(E, slots, seed):
    rng = np.random.default_rng(seed)
    c = make_cache(E, slots)
    model = LruModel(E, slots)
    for _ in range(200):
        n = int(rng.integers(1, min(slots, 6) + 1))
        # skewed requests with repeats inside a call
        req = rng.zipf(1.3, size=n) % E
        distinct = len(set(req.tolist()))
        if distinct > slots:
            continue
        got, fe, fs = c.plan(req)
        want, fills = model.call(req.tolist())
        assert got.tolist() == want
        assert list(zip(fe.tolist(), fs.tolist())) == fills
        # the tables are each other's inverse
        for e in range(E):
            if c.slot_of[e] >= 0:
                assert c.expert_of[c.slot_of[e]] == e
        for s in range(slots):
            if c.expert_of[s] >= 0:
                assert c.slot_of[c.expert_of[s]] == s
    assert (c.hits, c.misses) == (model.hits, model.misses)
    assert c.hits + c.misses > 0


def test_a_cache_below_the_cycle_never_hits():
    """Experts requested in a repeating cycle of 10 (one per call): 9 slots
    evict every expert before it comes back, 10 slots hit on every request
    after the first cycle."""
    for slots, want_hits in ((9, 0), (10, 90)):
        c = make_cache(16, slots)
        for rep in range(10):
            for e in range(10):
                c.plan(np.array([e]))
        assert c.hits == want_hits and c.misses == 100 - want_hits


def test_working_set_larger_than_the_cache_is_rejected():
    c = make_cache(32, 4)
    c.plan(np.array([1, 2]))
    with pytest.raises(dsq.DsqError) as ei:
        c.plan(np.array([3, 4, 5, 6, 7]))       # five distinct experts, four slots
    assert ei.value.status == -5
    # the tables stay consistent
    for s in range(4):
        if c.expert_of[s] >= 0:
            assert c.slot_of[c.expert_of[s]] == s
    with pytest.raises(dsq.DsqError) as ei:
        c.plan(np.array([40]))                  # expert out of range
    assert ei.value.status == -1


def test_cached_step_validation():
    c = make_cache(32, 8)
    L = dsq.lib()
    import ctypes
    fake = ctypes.c_void_p(0x40000)
    need = dsq.moe_cached_workspace_bytes(2, 32, 8, 2, 256, 128, dsq.MATH_FP32)
    assert need == (dsq.moe_workspace_bytes(2, 8, 2, 256, 128, dsq.MATH_FP32)
                    + 256 + 3 * 256)                  # logits [2][32], ids, weights, slots
    h = (ctypes.c_int32 * 4)()
    args = lambda ws, k=2: (fake, fake, None, ctypes.byref(c.desc), 2, k, 0, fake, fake, ws, h, h,
                            None, None, None, None)
    assert L.dsq_moe_ffn_cached(*args(need - 1)) == -4      # workspace too small
    assert L.dsq_moe_ffn_cached(*args(need, k=9)) == -2     # top_k > slots
    assert L.dsq_moe_ffn_cached(fake, fake, None, ctypes.byref(c.desc), 2, 2, 0, fake, fake,
                                need, None, h, None, None, None, None) == -1  # no host buffer
