"""GPU parity: grouping the routed entries by expert, bit-exact against the
oracle's stable counting sort.

Method: "Hand-writing a DeepSeek inference engine in pure C"
(hnwysp.cn/news/134870) §3.5: the tokens routed to one expert are gathered
so that its weights are read once.  The grouping is integer work, so counts,
offsets, perm and pos must equal the oracle's exactly, for the one-workgroup
kernel (up to 256 tokens) and the three-kernel path beyond it.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import MoeFixture, assert_bounded, check_moe_result, say
from group_quantized_moe_dsq_amd import dsq, synth

pytestmark = pytest.mark.gpu


def distinct_rows(rng, T, E, k, skew=None):
    """idx [T][k]: k distinct experts per token; with skew, experts drawn
    with probabilities proportional to exp(skew * N(0,1)) (uneven load)."""
    if skew is None:
        return np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32) \
            if T else np.zeros((0, k), np.int32)
    p = np.exp(skew * rng.standard_normal(E))
    p /= p.sum()
    return np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(T)]).astype(np.int32)


def check_group(idx, E, what):
    T, k = idx.shape
    counts, offsets, perm, pos = dsq.moe_group(torch.from_numpy(idx).cuda(), E)
    torch.cuda.synchronize()
    rc, ro, rp = oracle.group(idx, E)
    np.testing.assert_array_equal(counts.cpu().numpy(), rc, err_msg=f"{what}: counts")
    np.testing.assert_array_equal(offsets.cpu().numpy(), ro, err_msg=f"{what}: offsets")
    np.testing.assert_array_equal(perm.cpu().numpy(), rp, err_msg=f"{what}: perm")
    rpos = np.empty(T * k, np.int32)
    rpos[rp] = np.arange(T * k, dtype=np.int32)
    np.testing.assert_array_equal(pos.cpu().numpy(), rpos, err_msg=f"{what}: pos")
    say(f"  {what}: bit-exact ({T * k} entries, {int((rc > 0).sum())} experts touched, "
        f"largest {int(rc.max()) if rc.size else 0})")


# (T, E, k): both paths (T <= 256 one workgroup, beyond it three kernels),
# ragged word boundaries (T % 32), one expert, the largest E and k
CASES = [(0, 8, 2), (1, 256, 6), (5, 8, 8), (31, 64, 6), (32, 256, 6), (33, 256, 6),
         (255, 256, 6), (256, 256, 6), (257, 256, 6), (300, 1, 1), (1000, 64, 32),
         (4096, 256, 6), (4099, 4096, 6), (65536, 256, 6)]


@pytest.mark.parametrize("T,E,k", CASES)
def test_group_bit_exact(T, E, k):
    say(f"group T={T} E={E} k={k}")
    rng = np.random.default_rng(T * 7 + E + k)
    check_group(distinct_rows(rng, T, E, k), E, "uniform")


@pytest.mark.parametrize("T", [200, 4096])
def test_group_skewed_load(T):
    """A few experts take most tokens (router bias ~N(0,1)-like skew)."""
    say(f"group skewed T={T}")
    rng = np.random.default_rng(11 + T)
    check_group(distinct_rows(rng, T, 256, 6, skew=2.0), 256, "skewed")


@pytest.mark.parametrize("T", [40, 600])
def test_group_entries_outside_the_experts(T):
    """Entries with an expert outside [0, E) are grouped nowhere (pos = -1);
    the rest are grouped as the oracle groups them with those entries
    removed."""
    say(f"group with invalid entries T={T}")
    E, k = 32, 4
    rng = np.random.default_rng(12 + T)
    idx = distinct_rows(rng, T, E, k)
    bad = rng.random(idx.shape) < 0.1
    idx[bad] = np.where(rng.random(idx.shape) < 0.5, -1, E + 3)[bad]
    counts, offsets, perm, pos = dsq.moe_group(torch.from_numpy(idx).cuda(), E)
    # the oracle on the same entries with the invalid ones sent to an extra
    # expert E, which sorts after every real one
    idx2 = np.where(bad, E, idx).astype(np.int32)
    rc, ro, rp = oracle.group(idx2, E + 1)
    nvalid = int(ro[E])
    np.testing.assert_array_equal(counts.cpu().numpy(), rc[:E])
    np.testing.assert_array_equal(offsets.cpu().numpy(), ro[:E + 1])
    np.testing.assert_array_equal(perm.cpu().numpy()[:nvalid], rp[:nvalid])
    rpos = np.full(idx.size, -1, np.int32)
    rpos[rp[:nvalid]] = np.arange(nvalid, dtype=np.int32)
    np.testing.assert_array_equal(pos.cpu().numpy(), rpos)


def test_group_matches_moe_layer_counts():
    """The MoE layer's expert counts are the grouping's counts."""
    fx = MoeFixture(16, 256, 128, 4, 64, seed=13, bias_std=1.0)
    X = synth.normal((300, 256), 1.0, 13, synth.X, 300, device="cuda")
    idx = torch.empty((300, 4), dtype=torch.int32, device="cuda")
    cnt = torch.empty(16, dtype=torch.int32, device="cuda")
    dsq.moe_ffn(fx.layer(4), X, math=dsq.MATH_FP32, idx_out=idx, counts_out=cnt)
    c2, _, _, _ = dsq.moe_group(idx, 16)
    assert torch.equal(cnt, c2)


@pytest.mark.parametrize("math,rel", [(dsq.MATH_FP32, 1e-5), (dsq.MATH_BF16_MFMA, 1e-2)])
def test_moe_layer_4096_tokens(math, rel):
    """A whole MoE layer at 4096 tokens (the three-kernel grouping feeds the
    grouped GEMMs): routing and every token's output against the oracle."""
    say(f"moe T=4096 E=64 H=256 I=128 INT4 g64 math={math}")
    fx = MoeFixture(64, 256, 128, 4, 64, seed=14, bias_std=0.5)
    T, k = 4096, 6
    X = synth.normal((T, 256), 1.0, 14, synth.X, T, device="cuda")
    lay = fx.layer(k)
    logits = torch.empty((T, 64), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    counts = torch.empty(64, dtype=torch.int32, device="cuda")
    Y = dsq.moe_ffn(lay, X, math=math, logits_out=logits, idx_out=idx, w_out=w,
                    counts_out=counts)
    torch.cuda.synchronize()
    tok, Yref, bound = check_moe_result(fx, X.cpu().numpy(), logits.cpu().numpy(),
                                        idx.cpu().numpy(), w.cpu().numpy(),
                                        counts.cpu().numpy(), k, rel)
    assert_bounded(Y.cpu().numpy()[tok], Yref, bound, "moe output")
