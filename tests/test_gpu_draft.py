"""Masks along a draft (speculative decoding) on the device, against the
oracle: for every row and every position j of its k-token draft, the mask
of the configuration after the first j draft tokens ("Constrained
decoding", "The guarantee": each position is masked by the automaton's
state there), how many draft tokens are legal in a row, and the states
along the path (equal, byte for byte, to walking the kept tokens with
cg_advance)."""
import numpy as np
import pytest

import logit_masking_amd as cg
from logit_masking_amd import workloads as W
from oracle import oracle as O
from tests.gpu_util import NTHREADS, device_rows, random_walk, say

pytestmark = pytest.mark.gpu


def _setup(cfg, V, gen_cap=W.GEN_CAP):
    blob, off = W.make_vocab(cfg, V)
    toks = [blob[off[i]:off[i + 1]] for i in range(len(off) - 1)]
    g = cg.Grammar(W.spec_json(cfg), blob, off, gen_cap=gen_cap)
    og = O.load_spec(W.spec_json(cfg))
    return g, og, blob, off, toks


def _drafts(og, toks, rows, k, rng):
    """Per row a draft of k ids: a legal continuation (a random walk from the
    row), sometimes broken by an illegal token or cut short with -1."""
    out = np.full((len(rows), k), -1, dtype=np.int32)
    V = len(toks)
    for r, row in enumerate(rows):
        cont = O.Row(og, row.gen_cap)
        cont.conf, cont.step, cont.complete, cont.capped = og.clone(row.conf), row.step, row.complete, row.capped
        seq = []
        while len(seq) < k and not cont.done:
            nb = sorted(og.next_bytes(cont.conf))
            pick = None
            for _ in range(32):
                t = 256 + rng.below(V - 256)
                c = og.clone(cont.conf)
                if og.feed(c, toks[t], model=True) == len(toks[t]):
                    pick = t
                    break
            if pick is None:
                if not nb:
                    break
                pick = nb[rng.below(len(nb))]
            cont.advance(toks[pick])
            seq.append(pick)
        u = rng.uniform()
        if seq and u < 0.25:
            seq[rng.below(len(seq))] = rng.below(V)      # most likely illegal
        elif seq and u < 0.4:
            seq = seq[:rng.below(len(seq) + 1)]          # padded with -1
        out[r, :len(seq)] = seq
    return out


def _oracle_path(og, row, draft, toks):
    """(configurations and done flags at positions 0..k, accepted count)."""
    cur = O.Row(og, row.gen_cap)
    cur.conf, cur.step, cur.complete, cur.capped = og.clone(row.conf), row.step, row.complete, row.capped
    confs, done = [og.clone(cur.conf)], [cur.done]
    acc, alive = 0, True
    for t in draft:
        if alive:
            st = cur.advance(None if t < 0 else toks[t])
            if st in (O.ROW_REJECTED, O.ROW_NOOP):
                alive = False
            else:
                acc += 1
        confs.append(og.clone(cur.conf))
        done.append(cur.done or not alive)
    return confs, done, acc


@pytest.mark.parametrize("cfg,V,k,B", [(2, None, 4, 24), (3, 20000, 4, 24), (3, 5000, 8, 16), (6, 8000, 6, 24),
                                       (5, 3000, 3, 16), (3, 20000, 0, 8), (1, None, 5, 16)])
def test_draft_masks(cfg, V, k, B):
    import torch
    say("draft", cfg, V, k, B)
    g, og, blob, off, toks = _setup(cfg, V)
    rng = W.SplitMix(0xD4A + cfg * 7 + k)
    seqs, rows = [], []
    for r in range(B):
        s, row = random_walk(og, toks, rng.below(40), rng)
        seqs.append(s)
        rows.append(row)
    st, steps, _ = device_rows(g, seqs)
    draft = _drafts(og, toks, rows, k, rng)
    d_draft = torch.from_numpy(draft).cuda().reshape(B, k)
    path = torch.full((B, k + 1, cg.STATE_BYTES), 0xA5, dtype=torch.uint8, device="cuda")
    masks = torch.full((B, k + 1, g.W), 0x5A5A5A5A5A5A5A5A, dtype=torch.int64, device="cuda")
    acc = torch.full((B,), -9, dtype=torch.int32, device="cuda")
    before = st.clone()
    g.fill_draft(st, steps, d_draft, path, masks, acc)
    torch.cuda.synchronize()
    assert torch.equal(before, st)  # the rows themselves are untouched
    got = masks.cpu().numpy().view(np.uint64)
    acc_h = acc.cpu().numpy()
    confs, dones = [], []
    for r in range(B):
        c, d, a = _oracle_path(og, rows[r], draft[r], toks)
        assert acc_h[r] == a, (r, acc_h[r], a, draft[r])
        confs += c
        dones += d
    want, _ = og.mask_rows(confs, dones, blob, off, NTHREADS)
    want = want.reshape(B, k + 1, -1)
    for r in range(B):
        for j in range(k + 1):
            assert np.array_equal(got[r, j], want[r, j]), (cfg, r, j, acc_h[r])
    # the path state at the accepted length equals cg_advance over the kept tokens
    kept = [list(seqs[r]) + [int(t) for t in draft[r][:acc_h[r]]] for r in range(B)]
    st2, steps2, _ = device_rows(g, kept)
    p = path.cpu().numpy()
    s2 = st2.cpu().numpy()
    for r in range(B):
        assert np.array_equal(p[r, acc_h[r]], s2[r]), r
    assert (acc_h > 0).sum() >= B // 4 or k == 0


def test_draft_k0_equals_fill():
    import torch
    say("draft k0")
    g, og, blob, off, toks = _setup(3, 20000)
    rng = W.SplitMix(77)
    seqs = [random_walk(og, toks, rng.below(30), rng)[0] for _ in range(32)]
    st, steps, _ = device_rows(g, seqs)
    m1 = torch.empty((32, g.W), dtype=torch.int64, device="cuda")
    g.fill_bitmask(st, m1)
    m2 = torch.empty((32, 1, g.W), dtype=torch.int64, device="cuda")
    path = torch.empty((32, 1, cg.STATE_BYTES), dtype=torch.uint8, device="cuda")
    acc = torch.empty(32, dtype=torch.int32, device="cuda")
    g.fill_draft(st, steps, torch.empty((32, 0), dtype=torch.int32, device="cuda"), path, m2, acc)
    assert torch.equal(m1, m2[:, 0]) and torch.equal(path[:, 0], st)
    assert not acc.any()


def test_draft_hits_the_cap():
    """A draft that crosses the engine cap: the token that reaches it is kept
    (CAPPED), the ones after it are not, and the masks after it are empty."""
    import torch
    say("draft cap")
    g, og, blob, off, toks = _setup(5, 3000, gen_cap=6)
    rng = W.SplitMix(5)
    seqs, rows = [], []
    for r in range(8):
        s, row = random_walk(og, toks, 3, rng, gen_cap=6)
        seqs.append(s)
        rows.append(row)
    st, steps, _ = device_rows(g, seqs)
    draft = _drafts(og, toks, rows, 6, W.SplitMix(6))
    k = draft.shape[1]
    path = torch.empty((8, k + 1, cg.STATE_BYTES), dtype=torch.uint8, device="cuda")
    masks = torch.empty((8, k + 1, g.W), dtype=torch.int64, device="cuda")
    acc = torch.empty(8, dtype=torch.int32, device="cuda")
    g.fill_draft(st, steps, torch.from_numpy(draft).cuda(), path, masks, acc)
    acc_h = acc.cpu().numpy()
    got = masks.cpu().numpy().view(np.uint64)
    for r in range(8):
        c, d, a = _oracle_path(og, rows[r], draft[r], toks)
        assert acc_h[r] == a and a <= 6 - rows[r].step
        w, _ = og.mask_rows(c, d, blob, off, NTHREADS)
        assert np.array_equal(got[r], w)
