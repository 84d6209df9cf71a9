"""Helpers for the GPU parity tests: build packed weights through the C ABI,
read them back through the independent layout reader, and compare results
with the oracle under the bounds the tests state."""
import sys

import numpy as np
import torch

import layout_v1
import oracle
from group_quantized_moe_dsq_amd import dsq, synth


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def pack_gpu(w: torch.Tensor, bits: int, group: int) -> dsq.QWeight:
    """w: fp32 [N][K] or [B][N][K] on the GPU."""
    if w.dim() == 2:
        w = w[None]
    B, N, K = w.shape
    qw = dsq.QWeight(bits, group, K, N, B)
    dsq.pack_weights(w.contiguous(), qw)
    return qw


def device_entry(qw: dsq.QWeight, b: int = 0):
    raw = qw.buf.cpu().numpy()
    return layout_v1.decode_entry(raw, b, qw.bits, qw.group, qw.K, qw.N)


def as_qmat(q, s, z, bits, group, K, N) -> oracle.QMat:
    return oracle.QMat(np.ascontiguousarray(q), np.ascontiguousarray(s),
                       np.ascontiguousarray(z), None, N, K, bits, group)


def assert_bounded(y, ref, bound, what, min_ratio_report=True):
    """|y - ref| <= bound elementwise; reports the worst ratio."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(y - ref)
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    ratio = err / np.maximum(bound, 1e-300)
    worst = float(ratio.max()) if ratio.size else 0.0
    say(f"  {what}: max |err|/bound = {worst:.3g} (n={ratio.size})")
    assert (err <= bound).all(), f"{what}: {(err > bound).sum()} outputs exceed the bound, " \
                                 f"worst ratio {worst:.3g}"


def assert_normwise(y, ref, rel, what):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    r = np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-300)
    say(f"  {what}: normwise rel err = {r:.3g}")
    assert r <= rel, f"{what}: normwise relative error {r:.3g} > {rel}"


def gpu_weights(shape, seed, tid, index=0, std=0.02):
    return synth.normal(shape, std, seed, tid, index, device="cuda")


class MoeFixture:
    """A routed MoE layer built on the GPU from seeded weights.  Expert
    weights are generated per expert (counter-keyed), packed through the C
    ABI, and regenerated on demand for the oracle."""

    def __init__(self, E, H, I, bits, group, seed=0, bias_std=None):
        self.E, self.H, self.I, self.bits, self.group, self.seed = E, H, I, bits, group, seed
        self.router = synth.normal((E, H), 0.02, seed, synth.ROUTER, 0, device="cuda")
        self.bias = (None if bias_std is None else
                     synth.normal((E,), bias_std, seed, synth.BIAS, 0, device="cuda"))
        self.gate = dsq.QWeight(bits, group, H, I, E)
        self.up = dsq.QWeight(bits, group, H, I, E)
        self.down = dsq.QWeight(bits, group, I, H, E)
        for e in range(E):
            g, u, d = synth.expert_weights(e, H, I, seed, device="cuda")
            dsq.pack_weights(g, self.gate, first=e)
            dsq.pack_weights(u, self.up, first=e)
            dsq.pack_weights(d, self.down, first=e)
        torch.cuda.synchronize()
        self._cache = {}

    def layer(self, top_k):
        return dsq.MoeLayer(self.router, self.gate, self.up, self.down, self.bias, top_k)

    def oracle_expert(self, e):
        """Oracle-quantized expert e from the regenerated fp32 weights."""
        if e not in self._cache:
            g, u, d = synth.expert_weights(e, self.H, self.I, self.seed, device="cuda")
            self._cache[e] = oracle.quantize_expert(g.cpu().numpy(), u.cpu().numpy(),
                                                    d.cpu().numpy(), self.bits, self.group)
        return self._cache[e]
