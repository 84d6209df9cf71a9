"""Helpers for the GPU parity tests: build packed weights through the C ABI,
read them back through the independent layout reader, and compare results
with the oracle under the bounds the tests state."""
import itertools
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

    def __init__(self, E, H, I, bits, group, seed=0, bias_std=None, weights=None):
        """weights: optional f(e, H, I, seed) -> (gate, up, down) fp32 CUDA
        tensors in place of synth.expert_weights."""
        self.E, self.H, self.I, self.bits, self.group, self.seed = E, H, I, bits, group, seed
        self.weights = weights or (lambda e, H, I, seed: synth.expert_weights(e, H, I, seed,
                                                                              device="cuda"))
        self.router = synth.normal((E, H), 0.02, seed, synth.ROUTER, 0, device="cuda")
        self.bias = (None if bias_std is None else
                     synth.normal((E,), bias_std, seed, synth.BIAS, 0, device="cuda"))
        self.gate = dsq.QWeight(bits, group, H, I, E)
        self.up = dsq.QWeight(bits, group, H, I, E)
        self.down = dsq.QWeight(bits, group, I, H, E)
        for e in range(E):
            g, u, d = self.weights(e, H, I, seed)
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
            g, u, d = self.weights(e, self.H, self.I, self.seed)
            self._cache[e] = oracle.quantize_expert(g.cpu().numpy(), u.cpu().numpy(),
                                                    d.cpu().numpy(), self.bits, self.group)
        return self._cache[e]


def check_moe_result(fx, Xin, L, idx, w, counts, k, rel, tokens=None, propagated=False):
    """Checks a MoE layer's logits, routing and weights on the rows Xin (the
    rows the layer's router and experts saw) against the oracle, and returns
    (tokens, reference output, bound) for the output check:
      logits : |l - l_ref| <= 1e-5 * sum_h |x_h wr_h|  (+ one fp32 rounding of
               the bias addition);
      idx    : the same expert set as the oracle's for every token whose
               oracle margin between the k-th and (k+1)-th logit exceeds twice
               the logit bound; for the others (near-ties, where both choices
               are right) the GPU's set must be one of the sets the oracle
               admits within that bound; slots ordered by the kernel's own
               fp32 scores;
      w      : first-order softmax propagation of the logit bound, + 1e-6;
      Y      : rel * S_Y + sum_i dw_i |y_i|, with S_Y = sum_i w_i S_i and S_i
               the magnitude sum of expert i's down projection
               (sum_j |h_j Wd[n][j]|, fp64, from the oracle), dw_i the weight
               bound: the workload's gate (1e-5 * sum|a w| for the fp32 paths,
               1e-2 for bf16) on the last contraction, with the routing
               weights' own error added.  The first-order propagation of
               errors in the gate/up sums (P_i, about 100 S_i at the full
               layer shape) is printed as a diagnostic only: the gate does
               not widen by it -- unless `propagated`, for inputs built to
               drive every contraction to its worst case, where the bound is
               the first-order worst case of contractions each within
               rel * (its magnitude sum): rel * (S_Y + P_Y) + sum_i dw_i |y_i|."""
    T = Xin.shape[0]
    Xc = np.asarray(Xin, np.float64)
    bias = None if fx.bias is None else fx.bias.cpu().numpy().astype(np.float64)
    Lref, SL = oracle.router_f64(Xc, fx.router.cpu().numpy(), bias)
    lb = 1e-5 * SL + 2.0 ** -23 * np.abs(Lref)
    assert_bounded(L, Lref, lb, "router logits")

    ref_idx, ref_w, gap = oracle.route(Lref, k)
    delta = lb.max(axis=1)
    clear = gap > 2 * delta
    say(f"  routing: {int(clear.sum())}/{T} tokens with a clear top-{k} margin")
    for t in range(T):
        if clear[t]:
            assert set(idx[t]) == set(ref_idx[t]), f"token {t}: top-{k} set differs"
        else:
            kth = np.sort(Lref[t])[::-1][k - 1]
            certain = np.nonzero(Lref[t] > kth + 2 * delta[t])[0]
            cand = np.nonzero(np.abs(Lref[t] - kth) <= 2 * delta[t])[0]
            valid = [set(certain) | set(c) for c in
                     itertools.combinations(cand, k - len(certain))]
            assert set(idx[t]) in valid, f"token {t}: {sorted(idx[t])} is not a valid top-{k}"
        # slot order: descending in the kernel's own fp32 scores, ties to the
        # higher expert index
        s = L[t, idx[t]]
        for i in range(k - 1):
            assert s[i] > s[i + 1] or (s[i] == s[i + 1] and idx[t, i] > idx[t, i + 1])
    # the grouping counts are the routing histogram
    np.testing.assert_array_equal(counts, np.bincount(idx.reshape(-1), minlength=fx.E))
    sel_idx = idx.copy()        # validated above against the oracle's sets
    # routing weights of the selected sets, from the oracle's logits
    sel_l = np.take_along_axis(Lref, sel_idx.astype(np.int64), 1)
    ex = np.exp(sel_l - sel_l.max(axis=1, keepdims=True))
    wref = ex / ex.sum(axis=1, keepdims=True)
    d_l = np.take_along_axis(lb, sel_idx.astype(np.int64), 1)
    dw = wref * (d_l + (wref * d_l).sum(axis=1, keepdims=True)) + 1e-6
    assert_bounded(w, wref, dw, "routing weights")

    tokens = range(T) if tokens is None else tokens
    H = fx.H
    Yref = np.zeros((len(tokens), H))
    bound = np.zeros((len(tokens), H))
    SY = np.zeros((len(tokens), H))
    PY = np.zeros((len(tokens), H))
    for r, t in enumerate(tokens):
        for i in range(k):
            e = int(sel_idx[t, i])
            y, Sd, Pd = oracle.expert_f64(Xc[t], fx.oracle_expert(e))
            Yref[r] += wref[t, i] * y
            SY[r] += wref[t, i] * Sd
            PY[r] += wref[t, i] * Pd
            bound[r] += dw[t, i] * np.abs(y)
    bound += rel * (SY + PY) if propagated else rel * SY
    say(f"  output gate rel * S_Y (rel = {rel:g}); P_Y / S_Y median "
        f"{float(np.median(PY / np.maximum(SY, 1e-300))):.3g} (not in the gate)")
    return np.asarray(list(tokens)), Yref, bound
