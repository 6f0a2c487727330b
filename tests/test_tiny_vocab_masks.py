"""The oracle's token masks over a tiny vocabulary, against brute force (CPU only).

A mask bit is set exactly when the row is not done and the row's bytes
followed by the token's bytes are a prefix of some member of the language
("Constrained decoding", "The guarantee": every token the mask lets through
keeps the output inside the grammar, and no token that would is left out).
For tiny languages enumerated generatively (tests/langref.py, the same
specs as the byte-level brute force), the vocabulary here is every string of
one to three bytes over the language's test alphabet, and for sampled viable
prefixes p the oracle's mask (oracle.mask, the C routine that walks each
token) must equal, token by token, membership of p + token in the
enumerated prefix set.  Tokens that cross from a structural byte into a
string, a number or a key, and tokens that leave a string, are all in the
vocabulary, so the token walk is checked beyond single bytes.
"""
import itertools
import random

import numpy as np
import pytest

from oracle import oracle as O
from tests import langref
from tests.test_oracle_pins import TINY


def _vocab(sigma, max_len=3):
    toks = [bytes(t) for n in range(1, max_len + 1) for t in itertools.product(sorted(set(sigma)), repeat=n)]
    blob = b"".join(toks)
    off = np.zeros(len(toks) + 1, dtype=np.int64)
    off[1:] = np.cumsum([len(t) for t in toks])
    return toks, blob, off


def _check(spec, sigma, budget, min_room=0, n_prefixes=120, seed=7):
    g = O.load_spec(spec)
    M = langref.Enumerator(spec, sigma, budget).members()
    P = langref.prefixes(M)
    toks, blob, off = _vocab(sigma)
    V = len(toks)
    # prefixes whose every 3-byte extension is decided by the enumeration
    cand = sorted(p for p in P if len(p) + 3 + min_room <= budget)
    rng = random.Random(seed)
    short = [p for p in cand if len(p) <= 2]
    picked = short + rng.sample([p for p in cand if len(p) > 2], min(n_prefixes, max(0, len(cand) - len(short))))
    checked = allowed = 0
    for p in picked:
        c = g.start()
        assert g.feed(c, p) == len(p), p
        words = g.mask(c, blob, off)
        got = np.unpackbits(words.view(np.uint8), bitorder="little")[:V].astype(bool)
        want = np.array([(p + t) in P for t in toks])
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (p, [toks[i] for i in bad[:8]], got[bad[:8]].tolist())
        checked += 1
        allowed += int(want.sum())
    return checked, allowed


@pytest.mark.parametrize("name,spec,sigma,budget", TINY, ids=[t[0] for t in TINY])
def test_tiny_vocab_masks(name, spec, sigma, budget):
    checked, allowed = _check(spec, sigma, budget)
    assert checked > 5 and allowed > 0


def test_tiny_vocab_masks_calc():
    # the shortest completion of any non-empty viable prefix is at most 13
    # bytes ("<" + "calc>0</calc>"); tokens add up to 3 more
    spec = {"kind": "calc", "int_min": 0, "int_max": 12, "ws_max": 0, "depth_cap": 2}
    checked, allowed = _check(spec, b"<calc>/01+()", 26, min_room=13)
    assert checked > 50 and allowed > 0


def test_tiny_vocab_mask_of_finished_row():
    """A complete output takes no further token (the grammars are prefix-free),
    and a row at the generation cap has an empty mask whatever its bytes."""
    spec = TINY[1][1]  # ws-one-key: {"a":"x"} with up to two whitespace bytes
    g = O.load_spec(spec)
    toks, blob, off = _vocab(TINY[1][2])
    c = g.start()
    assert g.feed(c, b'{"a":"x"}') == 9 and g.complete(c)
    assert not g.mask(c, blob, off).any()
    row = O.Row(g, 2)
    assert row.advance(b'{"') == O.ROW_OK and row.advance(b'a') == O.ROW_CAPPED
    assert not g.mask_rows([row.conf], [row.done], blob, off)[0].any()
