"""Pins against the values the pages print (tests/golden/printed_values.txt,
each with its page and section): the super-block layout, the workload's
model constants, and the expert cache's behaviour below one forward pass.
CPU only."""
import os

import numpy as np

import oracle
from group_quantized_moe_dsq_amd import dsq

HERE = os.path.dirname(os.path.abspath(__file__))


def printed():
    vals = {}
    with open(os.path.join(HERE, "golden", "printed_values.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, value = (t.strip() for t in line.split("="))
            vals[name] = float(value) if any(c in value for c in ".e") else int(value)
    return vals


def test_super_block_layout_matches_the_printed_struct():
    v = printed()
    fields = (v["q4_block_d_bytes"] + v["q4_block_dmin_bytes"] + v["q4_block_scales_bytes"] +
              v["q4_block_codes_bytes"])
    assert fields == v["q4_block_bytes"] == oracle.SB_BYTES
    # 4-bit codes: two per byte
    assert v["q4_block_codes_bytes"] * 2 == v["q4_block_weights"]
    w = np.random.default_rng(0).standard_normal((2, 2 * v["q4_block_weights"])).astype(np.float32)
    assert oracle.sb4_quantize(w).blocks.shape == (2, 2, v["q4_block_bytes"])
    # the device layout carries the same bytes per block: codes plus a 16-byte header
    assert dsq.packed_bytes(4, 256, v["q4_block_weights"], 1) >= v["q4_block_bytes"]


def test_workload_uses_the_printed_model_constants():
    import bench
    v = printed()
    assert bench.N_EMBD == v["n_embd"]
    assert bench.N_VOCAB == v["n_vocab"]
    assert bench.N_EXPERT == v["n_expert"]
    assert bench.N_EXPERT_USED == v["n_expert_used"]
    assert bench.RMS_EPS == v["rms_eps"]
    # the pages' per-pass expert count is the layers times the experts per token
    assert v["n_layer"] * v["n_expert_used"] == v["experts_per_pass"]


def test_expert_cache_below_one_pass_never_hits():
    """The printed run: every layer's experts requested in turn (43 calls of 6
    per pass, 258 distinct experts per pass) for 10,320 requests.  A cache one
    slot short of a pass evicts each expert before its layer comes back: 0
    hits.  One slot more keeps the pass and hits on every later request."""
    v = printed()
    per_pass = v["experts_per_pass"]
    calls = per_pass // v["n_expert_used"]
    passes = v["budget_below_pass_requests"] // per_pass
    assert passes * per_pass == v["budget_below_pass_requests"]
    for slots, want_hits in ((per_pass - 1, v["budget_below_pass_hits"]),
                             (per_pass, v["budget_below_pass_requests"] - per_pass)):
        c = dsq.ExpertCache(4, 64, 256, 128, per_pass, slots, device="cpu", pinned=False)
        for _ in range(passes):
            for layer in range(calls):
                c.plan(np.arange(layer * v["n_expert_used"], (layer + 1) * v["n_expert_used"]))
        assert c.hits + c.misses == v["budget_below_pass_requests"]
        assert c.hits == want_hits
