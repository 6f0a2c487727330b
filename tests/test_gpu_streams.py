"""The path on more than one stream, and under graph capture.

* The fill on a second stream, concurrent with other work on the main
  stream (the mask depends on the rows' states alone, so it may run while
  the model's forward pass does -- "Evaluator aware decoding", "Why isn't
  this in production APIs yet?"): the same trajectory as on one stream.
* A step captured as a graph (no allocation or memset inside any call) and
  replayed several times with eager work in between: every replay equals
  the eager step from the same inputs.
"""
import numpy as np
import pytest

import logit_masking_amd as cg
from logit_masking_amd import workloads as W
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def _setup(B=32, V=20000):
    import torch
    blob, off = W.make_vocab(3, V)
    g = cg.Grammar(W.spec_json(3), blob, off)
    V = len(off) - 1
    bufs = dict(
        mask=torch.empty((B, g.W), dtype=torch.int64, device="cuda"),
        temp=torch.full((B,), 0.7, dtype=torch.float32, device="cuda"),
        seed=torch.from_numpy(np.array(W.row_seeds(3, B), dtype=np.uint64).view(np.int64)).cuda(),
        ws=cg.new_workspace(B, V),
        fws=g.new_fill_workspace(B),
        ids=torch.empty(B, dtype=torch.int32, device="cuda"),
        lp=torch.empty(B, dtype=torch.float32, device="cuda"),
    )
    return g, B, V, bufs


def _fresh(g, B):
    import torch
    st = g.new_states(B)
    g.init_state(st)
    return st, torch.zeros(B, dtype=torch.int32, device="cuda"), torch.zeros(B, dtype=torch.int32, device="cuda")


def test_fill_on_second_stream():
    import torch
    say("streams")
    g, B, V, b = _setup()
    logits = [W.make_logits(3, s, B, V, "cuda") for s in range(40)]
    junk_a = torch.randn((2048, 2048), device="cuda")
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()

    def run(two):
        st, steps, status = _fresh(g, B)
        hist = []
        for s in range(40):
            if two:
                side.wait_stream(main)
                g.fill_bitmask(st, b["mask"], b["fws"], side)
                ev = torch.cuda.Event()
                ev.record(side)
                junk = junk_a @ junk_a  # unrelated work on the main stream meanwhile
                main.wait_event(ev)
            else:
                g.fill_bitmask(st, b["mask"], b["fws"], main)
            g.sample_advance(logits[s], b["mask"], b["temp"], b["seed"], steps, b["ws"], b["ids"], b["lp"], st,
                             status, main)
            hist.append(b["ids"].clone())
        torch.cuda.synchronize()
        return st, steps, torch.stack(hist)

    a = run(False)
    c = run(True)
    for x, y in zip(a, c):
        assert torch.equal(x, y)


def test_step_as_graph():
    import torch
    say("graph")
    g, B, V, b = _setup()
    st, steps, status = _fresh(g, B)
    logits = W.make_logits(3, 0, B, V, "cuda")
    # advance a few eager steps so the rows sit in varied states
    for s in range(5):
        g.fill_bitmask(st, b["mask"], b["fws"])
        g.sample_advance(W.make_logits(3, 100 + s, B, V, "cuda"), b["mask"], b["temp"], b["seed"], steps, b["ws"],
                         b["ids"], b["lp"], st, status)
    torch.cuda.synchronize()
    st0, steps0 = st.clone(), steps.clone()
    # eager reference of one step from (st0, steps0)
    g.fill_bitmask(st, b["mask"], b["fws"])
    g.sample_advance(logits, b["mask"], b["temp"], b["seed"], steps, b["ws"], b["ids"], b["lp"], st, status)
    torch.cuda.synchronize()
    ref = (st.clone(), steps.clone(), b["ids"].clone(), b["lp"].clone(), status.clone(), b["mask"].clone())
    # capture the same step
    graph = torch.cuda.CUDAGraph()
    st.copy_(st0)
    steps.copy_(steps0)
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            g.fill_bitmask(st, b["mask"], b["fws"], cap)
            g.sample_advance(logits, b["mask"], b["temp"], b["seed"], steps, b["ws"], b["ids"], b["lp"], st, status,
                             cap)
    for rep in range(4):
        st.copy_(st0)
        steps.copy_(steps0)
        b["mask"].fill_(0x5A)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (st, steps, b["ids"], b["lp"], status, b["mask"])
        for x, y in zip(got, ref):
            assert torch.equal(x, y), rep
        # eager work between replays
        _ = torch.randn(1024, device="cuda").sum().item()
