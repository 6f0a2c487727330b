"""Helpers of the GPU parity tests: drive rows on the device through the C ABI
and the same rows through the oracle, with identical token choices."""
from __future__ import annotations

import os

import numpy as np

import logit_masking_amd as cg
from logit_masking_amd import workloads as W
from oracle import oracle as O

NTHREADS = min(16, os.cpu_count() or 1)


def say(*a):
    print("[gpu-case]", *a, flush=True)


def random_walk(og: O.Grammar, toks, n_tokens, rng: W.SplitMix, multi=0.6, gen_cap=2048):
    """A legal token sequence of up to n_tokens tokens chosen with the
    oracle: random multi-byte tokens that continue legally, else a random
    allowed single byte (ids 0-255 are the bytes)."""
    row = O.Row(og, gen_cap)
    seq = []
    V = len(toks)
    while len(seq) < n_tokens and not row.done:
        pick = None
        if rng.uniform() < multi:
            for _ in range(64):
                t = 256 + rng.below(V - 256)
                c = og.clone(row.conf)
                if og.feed(c, toks[t], model=True) == len(toks[t]):
                    pick = t
                    break
        if pick is None:
            nb = sorted(og.next_bytes(row.conf))
            if not nb:
                break
            pick = nb[rng.below(len(nb))]
        row.advance(toks[pick])
        seq.append(pick)
    return seq, row


def device_rows(g: cg.Grammar, seqs, device="cuda"):
    """Rows at start, then advanced through cg_advance one token per call;
    returns (states, steps, last status)."""
    import torch
    B = len(seqs)
    st = g.new_states(B, device)
    g.init_state(st)
    steps = torch.zeros(B, dtype=torch.int32, device=device)
    status = torch.full((B,), -7, dtype=torch.int32, device=device)
    L = max((len(s) for s in seqs), default=0)
    ids_all = np.full((L, B), -1, dtype=np.int32)
    for r, s in enumerate(seqs):
        ids_all[:len(s), r] = s
    ids_dev = torch.from_numpy(ids_all).to(device)
    for k in range(L):
        g.advance(st, ids_dev[k].contiguous(), steps, status)
    return st, steps, status


def oracle_masks(og, rows, blob, off):
    confs = [r.conf for r in rows]
    done = [r.done for r in rows]
    words, walked = og.mask_rows(confs, done, blob, off, NTHREADS)
    return words, walked


def gpu_masks(g, states, W_words=None):
    import torch
    B = states.shape[0]
    Wn = g.W if W_words is None else W_words
    mask = torch.full((B, Wn), 0x5A5A5A5A5A5A5A5A, dtype=torch.int64, device=states.device)
    g.fill_bitmask(states, mask)
    torch.cuda.synchronize()
    return mask.cpu().numpy().view(np.uint64)
