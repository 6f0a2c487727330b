"""GPU trajectories in lockstep with the oracle: every step runs
fill_bitmask -> apply_mask_sample -> advance on the device, and the oracle
recomputes each checked row's mask, pick and log-probability from the same
logits.  Near-ties (oracle margin < 1e-6) adopt the device's pick so both
trajectories stay in step; they are counted, not failed."""
import numpy as np
import pytest

import logit_masking_amd as cg
from logit_masking_amd import workloads as W
from oracle import oracle as O
from tests.gpu_util import NTHREADS, say

pytestmark = pytest.mark.gpu


def _run(cfg, B, steps, V=None, T=None, check_rows=None, gen_cap=W.GEN_CAP, fused=False):
    import torch
    c = W.CONFIGS[cfg]
    blob, off = W.make_vocab(cfg, V)
    V = len(off) - 1
    toks = [blob[off[i]:off[i + 1]] for i in range(V)]
    g = cg.Grammar(W.spec_json(cfg), blob, off, gen_cap=gen_cap)
    og = O.load_spec(W.spec_json(cfg))
    T = c["T"] if T is None else T
    st = g.new_states(B)
    g.init_state(st)
    stepc = torch.zeros(B, dtype=torch.int32, device="cuda")
    status = torch.zeros(B, dtype=torch.int32, device="cuda")
    mask = torch.empty((B, g.W), dtype=torch.int64, device="cuda")
    temp = torch.full((B,), float(T), dtype=torch.float32, device="cuda")
    seeds = np.array(W.row_seeds(cfg, B), dtype=np.uint64)
    seed_t = torch.from_numpy(seeds.view(np.int64)).cuda()
    ws = cg.new_workspace(B, V)
    ids = torch.empty(B, dtype=torch.int32, device="cuda")
    lp = torch.empty(B, dtype=torch.float32, device="cuda")
    rows_chk = list(range(B)) if check_rows is None else check_rows
    orows = {r: O.Row(og, gen_cap) for r in rows_chk}
    ties = done_steps = 0
    for s in range(steps):
        logits = W.make_logits(cfg, s, B, V, "cuda")
        g.fill_bitmask(st, mask)
        if fused:
            g.sample_advance(logits, mask, temp, seed_t, stepc, ws, ids, lp, st, status)
        else:
            cg.apply_mask_sample(logits, mask, temp, seed_t, stepc, ws, ids, lp)
        m_dev = mask.cpu().numpy().view(np.uint64)
        ids_dev = ids.cpu().numpy()
        lp_dev = lp.cpu().numpy()
        x = logits.float().cpu().numpy().astype(np.float64)
        words, _ = og.mask_rows([orows[r].conf for r in rows_chk], [orows[r].done for r in rows_chk], blob, off,
                                NTHREADS)
        forced = ids_dev.copy()
        for k, r in enumerate(rows_chk):
            if not np.array_equal(m_dev[r], words[k]):
                bad = np.nonzero(m_dev[r] != words[k])[0][0]
                raise AssertionError(f"cfg {cfg} step {s} row {r}: mask word {bad} differs")
            bits = O.unpack_mask(words[k], V)
            i, l, info = O.sample_row(x[r], bits, T, int(seeds[r]), orows[r].step)  # step before this token
            if i < 0:
                assert ids_dev[r] == -1, (s, r)
                continue
            if T > 0 and min(info["margin_chunk"], info["margin_token"]) < 1e-6:
                # sampled near-tie: both sides adopt the device's pick
                ties += 1
                assert bits[ids_dev[r]]
            else:
                assert ids_dev[r] == i, (cfg, s, r, ids_dev[r], i, info)
                assert abs(lp_dev[r] - l) < 1e-5, (cfg, s, r, lp_dev[r], l)
        if not fused:
            g.advance(st, ids, stepc, status)
        stat = status.cpu().numpy()
        for r in rows_chk:
            tok = None if ids_dev[r] < 0 else toks[ids_dev[r]]
            want = orows[r].advance(tok)
            assert stat[r] == want, (s, r, stat[r], want)
        if all(orows[r].done for r in rows_chk):
            done_steps = s + 1
            break
    # the device's step counters match
    sc = stepc.cpu().numpy()
    for r in rows_chk:
        assert sc[r] == orows[r].step
    return ties, {r: bytes(orows[r].text) for r in rows_chk}


@pytest.mark.parametrize("cfg,B,steps,V,T", [
    (1, 4, 30, None, 0.0),
    (2, 8, 60, None, None),
    (3, 6, 40, None, None),
    (4, 6, 40, None, None),
    (4, 4, 25, None, 0.7),
    (5, 4, 30, None, 1.0),
    (5, 4, 30, None, 0.0),
])
def test_trajectory(cfg, B, steps, V, T):
    say("trajectory", cfg, B, steps, T)
    ties, texts = _run(cfg, B, steps, V=V, T=T)
    assert ties <= 2


def test_trajectory_small_cap_finishes():
    """A tiny engine cap ends every row; afterwards masks are empty and picks -1."""
    say("trajectory cap")
    ties, texts = _run(5, 5, 12, V=3000, T=1.0, gen_cap=7)
    assert all(len(t) > 0 for t in texts.values())


@pytest.mark.parametrize("cfg,B,steps,T", [
    (1, 4, 30, 0.0),
    (3, 6, 40, None),
    (4, 6, 30, None),
    (5, 4, 30, 1.0),
])
def test_trajectory_fused_sample_advance(cfg, B, steps, T):
    """cg_sample_advance (pick + walk in one launch) against the oracle."""
    say("trajectory fused", cfg, B, steps, T)
    ties, texts = _run(cfg, B, steps, T=T, fused=True)
    assert ties <= 2


@pytest.mark.parametrize("cfg", [2, 3, 5])
def test_fused_equals_separate(cfg):
    """Same inputs through sample+advance and through the two separate calls:
    identical ids, log-probabilities (bitwise), states, steps and statuses,
    including finished rows, forced prefixes and a row at the cap."""
    import torch
    say("fused vs separate", cfg)
    c = W.CONFIGS[cfg]
    blob, off = W.make_vocab(cfg, 20000 if cfg != 2 else None)
    V = len(off) - 1
    toks = [blob[off[i]:off[i + 1]] for i in range(V)]
    g = cg.Grammar(W.spec_json(cfg), blob, off, gen_cap=25)
    og = O.load_spec(W.spec_json(cfg))
    B = 48
    rng = W.SplitMix(0x5EED + cfg)
    from tests.gpu_util import device_rows, random_walk
    seqs = [random_walk(og, toks, rng.below(30), rng, gen_cap=25)[0] for _ in range(B)]
    st0, steps0, _ = device_rows(g, seqs)
    mask = torch.empty((B, g.W), dtype=torch.int64, device="cuda")
    g.fill_bitmask(st0, mask)
    temp = torch.tensor([0.0 if r % 3 == 0 else float(c["T"] or 0.7) for r in range(B)], dtype=torch.float32,
                        device="cuda")
    seed = torch.from_numpy(np.array(W.row_seeds(cfg, B), dtype=np.uint64).view(np.int64)).cuda()
    ws = cg.new_workspace(B, V)
    for s in range(3):
        logits = W.make_logits(cfg, 100 + s, B, V, "cuda")
        st_a, st_b = st0.clone(), st0.clone()
        sa, sb = steps0.clone(), steps0.clone()
        ids_a = torch.empty(B, dtype=torch.int32, device="cuda")
        ids_b = torch.empty_like(ids_a)
        lp_a = torch.empty(B, dtype=torch.float32, device="cuda")
        lp_b = torch.empty_like(lp_a)
        stat_a = torch.full((B,), -9, dtype=torch.int32, device="cuda")
        stat_b = torch.full((B,), -9, dtype=torch.int32, device="cuda")
        cg.apply_mask_sample(logits, mask, temp, seed, sa, ws, ids_a, lp_a)
        g.advance(st_a, ids_a, sa, stat_a)
        g.sample_advance(logits, mask, temp, seed, sb, ws, ids_b, lp_b, st_b, stat_b)
        torch.cuda.synchronize()
        assert torch.equal(ids_a, ids_b)
        assert torch.equal(lp_a.view(torch.int32), lp_b.view(torch.int32))
        assert torch.equal(st_a, st_b)
        assert torch.equal(sa, sb)
        assert torch.equal(stat_a, stat_b)
        st0, steps0 = st_b, sb
        g.fill_bitmask(st0, mask)
