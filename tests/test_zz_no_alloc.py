"""GPU test of cg_fill_bitmask_noalloc (the fill for callers that cannot
allocate: its tile lists live in the library's per-device scratch array)
against cg_fill_bitmask with a caller workspace, through the C ABI.

Two calls in a row share the scratch array, the second over fewer rows;
each must give the masks of cg_fill_bitmask word for word (integer work:
bit-exact), and words past the vocabulary are left untouched.  The size
limit is refused before anything is launched.
"""
import numpy as np
import pytest

import logit_masking_amd as cg
from logit_masking_amd import workloads as W
from oracle import oracle as O
from tests.gpu_util import device_rows, random_walk, say

pytestmark = pytest.mark.gpu


def _rows(cfg, B, V, seed, max_len):
    blob, off = W.make_vocab(cfg, V)
    toks = [blob[off[i]:off[i + 1]] for i in range(len(off) - 1)]
    g = cg.Grammar(W.spec_json(cfg), blob, off, gen_cap=W.GEN_CAP)
    og = O.load_spec(W.spec_json(cfg))
    rng = W.SplitMix(seed)
    seqs = [random_walk(og, toks, rng.below(max_len + 1), rng)[0] for _ in range(B)]
    st, _, _ = device_rows(g, seqs)
    return g, st


def _fill_both(g, st, extra_words):
    import torch
    B = st.shape[0]
    fill = 0x5A5A5A5A5A5A5A5A
    a = torch.full((B, g.W + extra_words), fill, dtype=torch.int64, device="cuda")
    b = torch.full((B, g.W + extra_words), fill, dtype=torch.int64, device="cuda")
    g.fill_bitmask(st, a, g.new_fill_workspace(B))
    g.fill_bitmask_noalloc(st, b)
    torch.cuda.synchronize()
    a = a.cpu().numpy().view(np.uint64)
    b = b.cpu().numpy().view(np.uint64)
    assert np.array_equal(a, b), f"{int((a != b).sum())} words differ"
    assert np.all(b[:, g.W:] == np.uint64(fill))
    return b


@pytest.mark.parametrize("cfg,B1,B2,V,max_len", [
    (3, 256, 37, None, 60),      # tool call at full vocabulary and batch, then a smaller ragged batch
    (5, 512, 100, None, 80),     # recursive JSON at full vocabulary and batch
    (2, 64, 5, None, 120),       # decision schema
    (6, 200, 3, 20000, 80),      # text with calc spans, engine-written regions
])
def test_fill_noalloc_matches_workspace(cfg, B1, B2, V, max_len):
    import torch
    say("fill_noalloc", cfg, B1, B2, V)
    g, st = _rows(cfg, B1, V, 1000 + cfg, max_len)
    first = _fill_both(g, st, 3)
    # the second call over fewer rows (other states) reuses the scratch array
    # holding the first call's lists
    g2, st2 = _rows(cfg, B2, V, 2000 + cfg, max_len)
    _fill_both(g2, st2, 1)
    # and the first rows again, after the smaller call
    again = torch.full((B1, g.W + 3), 0x5A5A5A5A5A5A5A5A, dtype=torch.int64, device="cuda")
    g.fill_bitmask_noalloc(st, again)
    torch.cuda.synchronize()
    assert np.array_equal(again.cpu().numpy().view(np.uint64), first)


def test_fill_noalloc_limits():
    import torch
    blob, off = W.make_vocab(4)
    g = cg.Grammar(W.spec_json(4), blob, off, gen_cap=W.GEN_CAP)
    per_row = g.fill_workspace_bytes(1)
    B = (cg.FILL_NOALLOC_SCRATCH_BYTES // per_row) + 1
    st = g.new_states(B)
    g.init_state(st)
    mask = torch.zeros((B, g.W), dtype=torch.int64, device="cuda")
    with pytest.raises(cg.CgError) as e:
        g.fill_bitmask_noalloc(st, mask)
    assert e.value.code == cg.CG_E_LIMIT
    # an empty batch is a no-op
    g.fill_bitmask_noalloc(st[:0], mask[:0])
    torch.cuda.synchronize()
