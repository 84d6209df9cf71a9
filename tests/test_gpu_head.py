"""GPU parity: output-head selection (the k largest logits) and the whole
output head (vocab GEMV + selection).  Method: the output projection's
logits choose the next token ("Hand-writing a DeepSeek inference engine in
pure C", hnwysp.cn/news/134870, §2.1; "ds4 code walkthrough", the session
API's argmax / sample step); the end-to-end check compares the argmax
("Running a 284B-parameter LLM from 3.2 GB of RAM in plain C").

The selection is a decision taken on fp32 values, so the GPU and the oracle
take it on the same fp32 logits (the GPU's own) and must agree exactly;
the logits themselves are checked against the fp64 reference under the
GEMV's bound."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_bounded, pack_gpu, say
from group_quantized_moe_dsq_amd import dsq, synth

pytestmark = pytest.mark.gpu


def bits(v):
    return np.ascontiguousarray(v, np.float32).view(np.uint32)


def values(N, pattern, seed):
    rng = np.random.default_rng(seed)
    if pattern == "normal":
        return rng.standard_normal(N).astype(np.float32)
    if pattern == "ties":  # integer values: many exact ties
        return rng.integers(-4, 5, size=N).astype(np.float32)
    y = rng.standard_normal(N).astype(np.float32)  # specials mixed in
    sel = rng.integers(0, N, size=max(1, N // 20))
    y[sel] = rng.choice(np.array([np.nan, np.inf, -np.inf, 0.0, -0.0, 3.0], np.float32),
                        size=sel.size)
    return y


CASES = [(1, 1, "normal"), (5, 5, "ties"), (1023, 64, "normal"), (1024, 1, "special"),
         (1025, 256, "ties"), (2049, 17, "special"), (70000, 50, "normal"),
         (70000, 256, "ties"), (129280, 1, "special"), (300001, 100, "special"),
         # either side of the pick / sort switch (k <= 6 picks)
         (129280, 6, "special"), (129280, 7, "ties"), (5000, 8, "special")]


@pytest.mark.parametrize("N,k,pattern", CASES)
def test_topk_matches_oracle(N, k, pattern):
    say(f"topk N={N} k={k} {pattern}")
    y = values(N, pattern, 90 + N + k)
    idx, val = dsq.topk(torch.from_numpy(y).cuda(), k)
    ref_idx, ref_val = oracle.topk(y, k)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    np.testing.assert_array_equal(bits(val.cpu().numpy()), bits(ref_val))


def test_topk_all_equal_takes_the_first_indices():
    say("topk all equal")
    y = np.full(5000, 0.25, np.float32)
    idx, _ = dsq.topk(torch.from_numpy(y).cuda(), 40)
    np.testing.assert_array_equal(idx.cpu().numpy(), np.arange(40))


def test_topk_repeated_calls_reuse_the_workspace():
    say("topk workspace reuse")
    ws = torch.empty(dsq.topk_workspace_bytes(129280, 64) + 256, dtype=torch.uint8, device="cuda")
    for s, k in [(1, 64), (2, 3), (3, 64)]:
        y = values(129280, "normal", 200 + s)
        idx, _ = dsq.topk(torch.from_numpy(y).cuda(), k, workspace=ws)
        np.testing.assert_array_equal(idx.cpu().numpy(), oracle.topk(y, k)[0])


@pytest.mark.parametrize("k", [1, 50])
def test_gemv_topk_vocab_full_size(k):
    """The output head at full size: INT8 group-64 vocab projection K=4096,
    N=129280, then the top k.  The selection equals the oracle's on the
    GPU's logits; the logits of the selected rows and of 1024 sampled rows
    are within the GEMV bound of the fp64 reference, and no sampled row's
    fp64 logit beats a selected one by more than the two rows' bounds."""
    say(f"gemv topk vocab k={k}")
    N, K = 129280, 4096
    w = synth.normal((N, K), 0.02, 0, synth.W, 2, device="cuda")
    x = synth.normal((K,), 1.0, 0, synth.X, 3 + k, device="cuda")
    qw = pack_gpu(w, 8, 64)
    y, idx, val = dsq.gemv_topk(qw, x, k)
    y, idx, val = y.cpu().numpy(), idx.cpu().numpy(), val.cpu().numpy()
    ref_idx, ref_val = oracle.topk(y, k)
    np.testing.assert_array_equal(idx, ref_idx)
    np.testing.assert_array_equal(bits(val), bits(ref_val))
    # logits of the selected rows and of sampled rows against fp64
    sample = np.random.default_rng(54).choice(N, 1024, replace=False)
    rows = np.unique(np.concatenate([idx.astype(np.int64), sample]))
    m = oracle.quantize(w[torch.from_numpy(rows).cuda()].cpu().numpy(), 8, 64)
    ref, S = oracle.qmatmul_ref(x.cpu().numpy()[None, :], m)
    bound = 1e-5 * S[0]
    assert_bounded(y[rows], ref[0], bound, "head logits")
    # y[s] >= y[u] for a selected s and any other u, and |y - ref| <= bound,
    # so ref[u] - bound[u] <= ref[s] + bound[s] must hold for every pair
    pos = {int(r): i for i, r in enumerate(rows)}
    lim = min(ref[0][pos[int(s)]] + bound[pos[int(s)]] for s in idx)
    chosen = set(int(s) for s in idx)
    for i, r in enumerate(rows):
        if int(r) not in chosen:
            assert ref[0][i] - bound[i] <= lim, f"row {r} outranks the selection"
    del w, qw
    torch.cuda.empty_cache()


# top-1 through the GEMV that ranks its own outputs: small and ragged N (waves
# without rows write the padding key), both code widths, rows of 1..4 chunks
# per lane, and a row length past that (the separate selection pass)
@pytest.mark.parametrize("nbits,group,N,K", [(8, 64, 1, 256), (4, 64, 37, 512), (8, 128, 1000, 4096),
                                            (4, 128, 5003, 8192), (8, 64, 4097, 2048),
                                            (8, 64, 300, 12288), (4, 64, 129280, 4096)])
def test_gemv_top1_matches_selection_on_its_logits(nbits, group, N, K):
    say(f"gemv top-1 bits={nbits} group={group} N={N} K={K}")
    w = synth.normal((N, K), 0.02, 0, synth.W, 60 + N, device="cuda")
    # duplicated rows: equal logits, the smaller index must win
    if N > 8:
        w[N - 1] = w[N // 2]
        w[3] = w[N // 2]
    x = synth.normal((K,), 1.0, 0, synth.X, 61 + N, device="cuda")
    qw = pack_gpu(w.contiguous(), nbits, group)
    y, idx, val = dsq.gemv_topk(qw, x, 1)
    y_plain = dsq.gemv(qw, x)
    y_h = y.cpu().numpy()
    np.testing.assert_array_equal(y_h, y_plain.cpu().numpy())
    ref_idx, ref_val = oracle.topk(y_h, 1)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    np.testing.assert_array_equal(bits(val.cpu().numpy()), bits(ref_val))


def test_gemv_top1_ties_take_the_smallest_index():
    """Every row equal: all logits tie, so row 0 is the answer."""
    say("gemv top-1 all rows equal")
    N, K = 3000, 1024
    row = synth.normal((1, K), 0.02, 0, synth.W, 70, device="cuda")
    qw = pack_gpu(row.repeat(N, 1).contiguous(), 8, 64)
    x = synth.normal((K,), 1.0, 0, synth.X, 71, device="cuda")
    _, idx, _ = dsq.gemv_topk(qw, x, 1)
    assert int(idx.item()) == 0
