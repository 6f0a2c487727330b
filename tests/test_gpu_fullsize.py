"""The step at the headline workloads' full sizes, in the launch the bench
times (cg_sample_advance_fill over the whole batch and vocabulary), against
the oracle on sampled rows: the tool-call grammar (vocab 128,256, batch 256,
bf16, T = 0.7), the integer answer (vocab 151,936, batch 1024, greedy) and
recursive JSON (vocab 256,000, batch 512, Student-t logits, T = 1.0).  The
batch is made of 32 rows at random legal prefixes repeated in a seeded
order; for 24 rows the mask, the pick, its log-probability and the next
step's mask are compared with the oracle's.  Two more cases of the tool-call
workload cover both cache policies of the sampler's stream (logits of a
launch above 32 MB are read with the non-temporal hint): its logits in
float32 (131 MB, the float32 kernel with the hint) and a batch of 64 rows
(16 MB, the bf16 kernel without it)."""
import numpy as np
import pytest

import logit_masking_amd as cg
from logit_masking_amd import workloads as W
from oracle import oracle as O
from tests.gpu_util import device_rows, oracle_masks, random_walk, say

pytestmark = pytest.mark.gpu

NEAR_TIE = 1e-6


@pytest.mark.parametrize("cfg,fp32,batch", [(3, False, None), (4, False, None), (5, False, None),
                                            (3, True, None), (3, False, 64)],
                         ids=["3", "4", "5", "3-fp32", "3-b64"])
def test_full_size_step_against_oracle(cfg, fp32, batch):
    import torch
    say("full size", cfg, "fp32" if fp32 else "", batch or "")
    c = W.CONFIGS[cfg]
    B, T = batch or c["B"], float(c["T"] or 0.0)
    blob, off = W.make_vocab(cfg)
    V = len(off) - 1
    toks = [blob[off[i]:off[i + 1]] for i in range(V)]
    g = cg.Grammar(W.spec_json(cfg), blob, off)
    og = O.load_spec(W.spec_json(cfg))
    rng = W.SplitMix(0xF011 + cfg)
    seqs = [random_walk(og, toks, rng.below(24), rng)[0] for _ in range(32)]
    st_p, steps_p, _ = device_rows(g, seqs)
    proto = np.random.default_rng(cfg).integers(0, 32, size=B)
    pick_t = torch.from_numpy(proto).cuda()
    st = st_p.index_select(0, pick_t).contiguous()
    steps = steps_p.index_select(0, pick_t).contiguous()
    status = torch.zeros(B, dtype=torch.int32, device="cuda")
    temp = torch.full((B,), T, dtype=torch.float32, device="cuda")
    seeds = np.array(W.row_seeds(cfg, B), dtype=np.uint64)
    seed = torch.from_numpy(seeds.view(np.int64)).cuda()
    ws = cg.new_workspace(B, V)
    fws = g.new_fill_workspace(B)
    mask = torch.full((B, g.W), 0x5A5A5A5A5A5A5A5A, dtype=torch.int64, device="cuda")
    ids = torch.empty(B, dtype=torch.int32, device="cuda")
    lp = torch.empty(B, dtype=torch.float32, device="cuda")
    logits = W.make_logits(cfg, 3, B, V, "cuda")
    if fp32:
        logits = logits.float()
    g.fill_bitmask(st, mask, fws)
    torch.cuda.synchronize()
    check = np.sort(np.random.default_rng(100 + cfg).choice(B, 24, replace=False))
    mask0 = mask.cpu().numpy().view(np.uint64)[check]
    steps0 = steps.cpu().numpy()[check]
    g.sample_advance_fill(logits, mask, temp, seed, steps, ws, ids, lp, st, status, fws)
    torch.cuda.synchronize()
    x = logits[torch.from_numpy(check).cuda()].float().cpu().numpy().astype(np.float64)
    ids_h, lp_h = ids.cpu().numpy()[check], lp.cpu().numpy()[check]
    mask1 = mask.cpu().numpy().view(np.uint64)[check]
    rows0, rows1 = [], []
    for k, r in enumerate(check):
        row = O.Row(og, W.GEN_CAP)
        for t in seqs[proto[r]]:
            row.advance(toks[t])
        rows0.append(row)
    want0, _ = oracle_masks(og, rows0, blob, off)
    assert np.array_equal(mask0[:, :want0.shape[1]], want0)
    ties = 0
    for k, r in enumerate(check):
        bits = O.unpack_mask(want0[k], V)
        i, l, info = O.sample_row(x[k], bits, T, int(seeds[r]), int(steps0[k]))
        if T > 0 and min(info["margin_chunk"], info["margin_token"]) < NEAR_TIE:
            ties += 1
            assert i < 0 or bits[ids_h[k]]
            i = int(ids_h[k])  # both sides continue with the device's pick
        else:
            assert ids_h[k] == i, (cfg, r, ids_h[k], i, info)
            if i >= 0:
                assert abs(lp_h[k] - l) < 1e-5, (cfg, r, lp_h[k], l)
        row = O.Row(og, W.GEN_CAP)
        for t in seqs[proto[r]]:
            row.advance(toks[t])
        if i >= 0:
            row.advance(toks[i])
        rows1.append(row)
    want1, _ = oracle_masks(og, rows1, blob, off)
    assert np.array_equal(mask1[:, :want1.shape[1]], want1)
    say("near-ties", ties)
    assert ties <= 2


def test_full_size_trajectory_tool_call():
    """The bench's own trajectory (tool-call grammar, vocab 128,256, batch
    256, T = 0.7, every row from the start state) for 30 steps of
    cg_sample_advance_fill, 16 rows followed in lock-step by the oracle:
    every step's mask, pick and log-probability equal the oracle's (a
    sampled near-tie adopts the device's pick on both sides)."""
    import torch
    say("full size trajectory")
    cfg = 3
    c = W.CONFIGS[cfg]
    B, T = c["B"], float(c["T"])
    blob, off = W.make_vocab(cfg)
    V = len(off) - 1
    toks = [blob[off[i]:off[i + 1]] for i in range(V)]
    g = cg.Grammar(W.spec_json(cfg), blob, off)
    og = O.load_spec(W.spec_json(cfg))
    st = g.new_states(B)
    g.init_state(st)
    steps = torch.zeros(B, dtype=torch.int32, device="cuda")
    status = torch.zeros(B, dtype=torch.int32, device="cuda")
    temp = torch.full((B,), T, dtype=torch.float32, device="cuda")
    seeds = np.array(W.row_seeds(cfg, B), dtype=np.uint64)
    seed = torch.from_numpy(seeds.view(np.int64)).cuda()
    ws = cg.new_workspace(B, V)
    fws = g.new_fill_workspace(B)
    mask = torch.empty((B, g.W), dtype=torch.int64, device="cuda")
    ids = torch.empty(B, dtype=torch.int32, device="cuda")
    lp = torch.empty(B, dtype=torch.float32, device="cuda")
    check = np.sort(np.random.default_rng(7).choice(B, 16, replace=False))
    check_t = torch.from_numpy(check).cuda()
    orows = [O.Row(og, W.GEN_CAP) for _ in check]
    g.fill_bitmask(st, mask, fws)
    ties = taken = 0
    for s in range(30):
        logits = W.make_logits(cfg, s, B, V, "cuda")
        torch.cuda.synchronize()
        got = mask.cpu().numpy().view(np.uint64)[check]
        want, _ = oracle_masks(og, orows, blob, off)
        assert np.array_equal(got[:, :want.shape[1]], want), s
        g.sample_advance_fill(logits, mask, temp, seed, steps, ws, ids, lp, st, status, fws)
        torch.cuda.synchronize()
        x = logits.index_select(0, check_t).float().cpu().numpy().astype(np.float64)
        ids_h, lp_h = ids.cpu().numpy()[check], lp.cpu().numpy()[check]
        for k, r in enumerate(check):
            bits = O.unpack_mask(want[k], V)
            i, l, info = O.sample_row(x[k], bits, T, int(seeds[r]), orows[k].step)
            if i >= 0 and min(info["margin_chunk"], info["margin_token"]) < NEAR_TIE:
                ties += 1
                assert bits[ids_h[k]]
                i = int(ids_h[k])
            else:
                assert ids_h[k] == i, (s, r, ids_h[k], i, info)
                if i >= 0:
                    assert abs(lp_h[k] - l) < 1e-5, (s, r, lp_h[k], l)
            if i >= 0:
                orows[k].advance(toks[i])
                taken += 1
    say("near-ties", ties, "of", taken, "sampled picks")
    assert ties <= 2 and taken > 100
