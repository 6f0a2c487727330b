"""cg_sample_advance_fill against the separate calls: along a trajectory,
the ids, log-probabilities, states, steps and statuses equal those of
cg_sample_advance, and the mask it leaves behind equals cg_fill_bitmask of
the updated states, bit for bit ("Evaluator aware decoding", "Why isn't this
in production APIs yet?": the mask depends on the automaton's state alone)."""
import numpy as np
import pytest

import logit_masking_amd as cg
from logit_masking_amd import workloads as W
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg,V,B,n_steps,split", [(2, None, 32, 40, False), (3, 20000, 64, 60, False),
                                                   (3, None, 256, 12, True), (5, 8000, 48, 40, False),
                                                   (6, 20000, 48, 60, True), (1, None, 4, 30, False)])
def test_fused_fill_matches_separate_calls(cfg, V, B, n_steps, split):
    import torch
    say("fused fill", cfg, V, B, split)
    blob, off = W.make_vocab(cfg, V)
    V = len(off) - 1
    g = cg.Grammar(W.spec_json(cfg), blob, off)
    c = W.CONFIGS[cfg]
    temp = torch.full((B,), float(c["T"]), dtype=torch.float32, device="cuda")
    seeds = np.array(W.row_seeds(cfg, B), dtype=np.uint64)
    seed = torch.from_numpy(seeds.view(np.int64)).cuda()
    ws = cg.new_workspace(B, V)
    fws_a, fws_b = g.new_fill_workspace(B), g.new_fill_workspace(B)
    rows = []
    for _ in range(2):
        st = g.new_states(B)
        g.init_state(st)
        rows.append(dict(st=st, steps=torch.zeros(B, dtype=torch.int32, device="cuda"),
                         status=torch.zeros(B, dtype=torch.int32, device="cuda"),
                         mask=torch.full((B, g.W + 3), 0x5A5A5A5A5A5A5A5A, dtype=torch.int64, device="cuda"),
                         ids=torch.empty(B, dtype=torch.int32, device="cuda"),
                         lp=torch.empty(B, dtype=torch.float32, device="cuda")))
    a, b = rows
    g.fill_bitmask(b["st"], b["mask"], fws_b)
    for s in range(n_steps):
        logits = W.make_logits(cfg, s, B, V, "cuda")
        g.fill_bitmask(a["st"], a["mask"], fws_a)
        assert torch.equal(a["mask"], b["mask"]), (cfg, s)
        g.sample_advance(logits, a["mask"], temp, seed, a["steps"], ws, a["ids"], a["lp"], a["st"], a["status"])
        g.sample_advance_fill(logits, b["mask"], temp, seed, b["steps"], ws, b["ids"], b["lp"], b["st"],
                              b["status"], fws_b, split=split)
        if split:  # the second launch as a call of its own (cg_fill_walk)
            g.fill_walk(b["st"], b["mask"], fws_b)
        for key in ("ids", "lp", "st", "steps", "status"):
            assert torch.equal(a[key], b[key]), (cfg, s, key)
    g.fill_bitmask(a["st"], a["mask"], fws_a)
    assert torch.equal(a["mask"], b["mask"])
    assert int((a["status"] == cg.ROW_DONE).sum()) + int((a["steps"] > 0).sum()) > 0


def test_large_table_against_separate_calls():
    """A tool-call grammar of 24 tools (the eight tools under three names
    each), whose transition table is larger than the part the sampler fetches
    into registers (4096 entries; the rest is staged after the stream) and
    within the 60 KiB staged in LDS:
    cg_sample_advance_fill against cg_fill_bitmask + cg_apply_mask_sample +
    cg_advance along a trajectory, and the masks of rows at random prefixes
    against the oracle."""
    import json
    import torch
    from oracle import oracle as O
    from tests.gpu_util import device_rows, gpu_masks, oracle_masks, random_walk
    say("large table")
    spec = json.dumps({"kind": "tool_call", "ws_max": 4, "open_string_cap": 256, "depth_cap": 16,
                       "tools": [W._tool(f"{n}_v{k}", a) for k in range(3) for n, a in W.TOOLS]},
                      separators=(",", ":")).encode()
    blob, off = W.make_vocab(3, 20000)
    V = len(off) - 1
    toks = [blob[off[i]:off[i + 1]] for i in range(V)]
    g = cg.Grammar(spec, blob, off)
    assert g.info()["table_entries"] > 4096, g.info()
    og = O.load_spec(spec)
    rng = W.SplitMix(0x7AB1E)
    seqs, orows = [], []
    for _ in range(24):
        sq, row = random_walk(og, toks, rng.below(30), rng)
        seqs.append(sq)
        orows.append(row)
    st_o, _, _ = device_rows(g, seqs)
    want, _ = oracle_masks(og, orows, blob, off)
    got = gpu_masks(g, st_o)
    assert np.array_equal(got[:, :want.shape[1]], want)
    B, n_steps = 64, 40
    temp = torch.tensor([0.0 if r % 4 == 0 else 0.7 for r in range(B)], dtype=torch.float32, device="cuda")
    seed = torch.from_numpy(np.array(W.row_seeds(3, B), dtype=np.uint64).view(np.int64)).cuda()
    ws = cg.new_workspace(B, V)
    fws_a, fws_b = g.new_fill_workspace(B), g.new_fill_workspace(B)
    rows = []
    for _ in range(2):
        st = g.new_states(B)
        g.init_state(st)
        rows.append(dict(st=st, steps=torch.zeros(B, dtype=torch.int32, device="cuda"),
                         status=torch.zeros(B, dtype=torch.int32, device="cuda"),
                         mask=torch.empty((B, g.W), dtype=torch.int64, device="cuda"),
                         ids=torch.empty(B, dtype=torch.int32, device="cuda"),
                         lp=torch.empty(B, dtype=torch.float32, device="cuda")))
    a, b = rows
    g.fill_bitmask(b["st"], b["mask"], fws_b)
    for s in range(n_steps):
        logits = W.make_logits(3, s, B, V, "cuda")
        g.fill_bitmask(a["st"], a["mask"], fws_a)
        assert torch.equal(a["mask"], b["mask"]), s
        cg.apply_mask_sample(logits, a["mask"], temp, seed, a["steps"], ws, a["ids"], a["lp"])
        g.advance(a["st"], a["ids"], a["steps"], a["status"])
        g.sample_advance_fill(logits, b["mask"], temp, seed, b["steps"], ws, b["ids"], b["lp"], b["st"],
                              b["status"], fws_b)
        for key in ("ids", "st", "steps", "status"):
            assert torch.equal(a[key], b[key]), (s, key)
        assert torch.equal(a["lp"].view(torch.int32), b["lp"].view(torch.int32)), s
    g.fill_bitmask(a["st"], a["mask"], fws_a)
    assert torch.equal(a["mask"], b["mask"])
    assert int(a["steps"].sum()) > B
