"""Evaluator-aware spans with engine-written results (CPU only).

Page "Evaluator aware decoding": the model writes a <calc> span, the engine
evaluates it with a small local parser and injects <result>VALUE</result>
("The core idea"), or <result_error>...</result_error> on a failure; the
grammar must not let the model write the result block itself, and the
injection is a grammar transition the model did not choose ("A concrete
prototype on llama.cpp").

Pins of the oracle against things other than itself: the page's worked
example, a full-string regular-expression validator (tests/langref.py),
Python's own expression parser for precedence and associativity, and
exact integer arithmetic.  Then the library's host parts (the table walker
behind cg_try_input and the cg_eval_calc evaluator) against the oracle.
"""
import itertools
import re

import numpy as np
import pytest

from logit_masking_amd import workloads as W
from oracle import oracle as O
from tests import langref

SPEC = W.SPECS[6]
INT64 = O.INT64_RANGE


@pytest.fixture(scope="module")
def og():
    return O.load_spec(W.spec_json(6))


@pytest.fixture(scope="module")
def vocab():
    blob, off = W.make_vocab(6, 4096)
    return blob, off, [blob[off[i]:off[i + 1]] for i in range(len(off) - 1)]


# ---------------------------------------------------------------------------
# The page's worked example, as a row of the decode loop.
# ---------------------------------------------------------------------------
def test_page_example_injection(og, vocab):
    blob, off, toks = vocab
    row = O.Row(og, gen_cap=W.GEN_CAP)
    span = b"<calc>17 * 23 + 91</calc>"
    # the model writes the span (one byte per token), the last byte closes it
    sts = [row.advance(bytes([b])) for b in span]
    assert sts[:-1] == [O.ROW_OK] * (len(span) - 1)
    assert sts[-1] == O.ROW_INJECT
    # nothing the model could write is legal now
    assert not O.unpack_mask(og.mask(row.conf, blob, off), len(toks)).any()
    assert og.next_bytes(row.conf) == set()
    assert row.advance(b"<") == O.ROW_REJECTED
    # "The core idea": the span evaluates to 482
    assert O.eval_calc(span) == 482
    steps = row.step
    assert row.force(b"<result>482</result>") == O.ROW_OK
    assert row.step == steps  # an injection is not a generation step
    assert row.advance(b" so<end>") == O.ROW_DONE
    parts = langref.calc_text_parts(SPEC, bytes(row.text))
    assert parts == [("model", span), ("engine", b"<result>482</result>"), ("model", b" so"),
                     ("model", b"<end>")]


def test_model_cannot_write_result(og):
    c = og.start()
    # a result block the model opens in text is refused at its second byte
    assert og.feed(c, b"x <result>482</result>", model=True) == 3
    # a token may end where the engine's region starts, not run into it
    c = og.start()
    assert og.feed(c, b"<calc>1+2", model=True) == 9
    c2 = og.clone(c)
    assert og.feed(c2, b"</calc>", model=True) == 7 and og.in_engine(c2)
    c3 = og.clone(c)
    assert og.feed(c3, b"</calc><result>3</result>", model=True) == 7
    # the engine's own walk takes the same bytes
    c4 = og.clone(c)
    assert og.feed(c4, b"</calc><result>3</result>") == 25 and not og.in_engine(c4)
    # error blocks: any printable message but '<'
    c5 = og.clone(c2)
    assert og.feed(c5, b"<result_error>division by zero</result_error>") == 45
    c6 = og.clone(c2)
    assert og.feed(c6, b"<result_error>a<b</result_error>") == 16


def test_force_semantics(og):
    row = O.Row(og, gen_cap=4)
    assert row.force(b"") == O.ROW_NOOP
    assert row.force(b"abc") == O.ROW_OK and row.step == 0  # legal text, forced
    assert row.force(b"<result>") == O.ROW_REJECTED and bytes(row.text) == b"abc"
    assert row.advance(b"<calc>1") == O.ROW_OK
    assert row.advance(b"</calc>") == O.ROW_INJECT
    assert row.force(b"<result>1") == O.ROW_INJECT  # still inside the block
    assert row.force(b"</result>") == O.ROW_OK
    assert row.advance(b"x") == O.ROW_OK and row.step == 3
    assert row.advance(b"<end>") == O.ROW_DONE
    assert row.force(b"x") == O.ROW_REJECTED
    # the cap counts model tokens only; a capped row takes no more bytes
    row = O.Row(og, gen_cap=2)
    assert row.advance(b"<calc>5") == O.ROW_OK
    assert row.advance(b"</calc>") == O.ROW_CAPPED
    assert row.force(b"<result>5</result>") == O.ROW_REJECTED


# ---------------------------------------------------------------------------
# Random members: the oracle, the regular-expression validator and the
# model / engine split agree.
# ---------------------------------------------------------------------------
def _random_member(rng, n_spans):
    segs = W.calc_text_script(rng, SPEC, n_spans)
    out, parts = b"", []
    for s in segs[:-1]:
        r = rng.uniform()
        if r < 0.2:
            res = b"<result_error>" + bytes(0x20 + rng.below(28) for _ in range(rng.below(12))) + b"</result_error>"
        else:
            v = rng.below(10 ** (1 + rng.below(19)))
            res = b"<result>" + (b"-" if r < 0.4 else b"") + str(v).encode() + b"</result>"
        parts += [("model", s), ("engine", res)]
        out += s + res
    parts.append(("model", segs[-1]))
    return out + segs[-1], parts


def test_random_members_agree(og):
    rng = W.SplitMix(61)
    for i in range(300):
        data, parts = _random_member(rng, rng.below(4))
        assert langref.member(SPEC, data), data
        assert og.try_input(data) == (len(data), True), data
        # walk the pieces: the model's as model bytes, the engine's as forced
        c = og.start()
        for who, piece in parts:
            if who == "engine":
                assert og.in_engine(c)
                assert og.feed(og.clone(c), piece, model=True) == 0
                assert og.feed(c, piece) == len(piece)
            else:
                assert not og.in_engine(c)
                assert og.feed(c, piece, model=True) == len(piece)
        assert og.complete(c)


def test_mutations_agree_with_validator(og):
    """Membership of mutated members: the oracle and the validator agree."""
    rng = W.SplitMix(62)
    alphabet = b"<>/calcresultnd_error0123456789+-*() \nxy"
    n_in = n_out = 0
    for i in range(1500):
        data, _ = _random_member(rng, 1 + rng.below(2))
        d = bytearray(data)
        for _ in range(1 + rng.below(2)):
            k = rng.below(3)
            p = rng.below(len(d) + 1)
            if k == 0 and p < len(d):
                d[p] = alphabet[rng.below(len(alphabet))]
            elif k == 1:
                d.insert(p, alphabet[rng.below(len(alphabet))])
            elif p < len(d):
                del d[p]
        d = bytes(d)
        want = langref.member(SPEC, d)
        k, complete = og.try_input(d)
        assert complete == want, d
        n_in += want
        n_out += not want
    assert n_in > 50 and n_out > 500


def test_tiny_calc_text_bruteforce():
    """Viability by brute force over a tiny alphabet: with the bytes
    {a, e, n, d, <} no span can open, so every member ends in "<end>" and a
    string is a viable prefix iff it is completed by a suffix of "<end>"
    (the validator decides membership of each completion)."""
    spec = {"kind": "calc_text", "int_min": 0, "int_max": 9, "ws_max": 0, "depth_cap": 1}
    g = O.load_spec(spec)
    completions = [b"<end>"[j:] for j in range(6)]
    n_viable = 0
    for n in range(0, 7):
        for t in map(bytes, itertools.product(b"aend<", repeat=n)):
            k, complete = g.try_input(t)
            assert complete == langref.member(spec, t), t
            viable = any(langref.member(spec, t + s) for s in completions)
            assert (k == len(t)) == viable, t
            n_viable += viable
    assert n_viable > 1000
    # members built from text and closed spans with their results
    atoms = [b"a", b"<calc>7</calc><result>7</result>", b"<calc>(7)/0</calc><result_error>x</result_error>"]
    for parts in itertools.product(atoms, repeat=3):
        m = b"".join(parts) + b"<end>"
        assert g.try_input(m) == (len(m), True) and langref.member(spec, m)


# ---------------------------------------------------------------------------
# The evaluator: Python's parser fixes precedence and associativity.
# ---------------------------------------------------------------------------
class _TruncInt:
    """Integers whose / truncates toward zero; range-checked."""

    def __init__(self, v, bound):
        if bound is not None and not bound[0] <= v <= bound[1]:
            raise OverflowError
        self.v, self.bound = v, bound

    def _mk(self, v):
        return _TruncInt(v, self.bound)

    def __add__(self, o):
        return self._mk(self.v + o.v)

    def __sub__(self, o):
        return self._mk(self.v - o.v)

    def __mul__(self, o):
        return self._mk(self.v * o.v)

    def __truediv__(self, o):
        if o.v == 0:
            raise ZeroDivisionError
        q = abs(self.v) // abs(o.v)
        return self._mk(q if (self.v >= 0) == (o.v >= 0) else -q)


def _python_eval(body: bytes, bound=None):
    src = re.sub(rb"[0-9]+", lambda m: b"_T(" + m.group(0).lstrip(b"0").rjust(1, b"0") + b")", body)
    try:
        return eval(src.decode(), {"__builtins__": {}, "_T": lambda v: _TruncInt(v, bound)}).v
    except ZeroDivisionError:
        return "division by zero"
    except OverflowError:
        return "out of range"


def _oracle_eval(span, bound=None):
    try:
        return O.eval_calc(span, bound)
    except O.CalcError as e:
        return str(e)


def test_evaluator_examples():
    assert O.eval_calc(b"<calc>17 * 23 + 91</calc>") == 482   # the page's example
    assert O.eval_calc(b"<calc>8/2/2</calc>") == 2             # left to right
    assert O.eval_calc(b"<calc>10-3-2</calc>") == 5
    assert O.eval_calc(b"<calc>2+3*4</calc>") == 14            # * before +
    assert O.eval_calc(b"<calc>(2+3)*4</calc>") == 20
    assert O.eval_calc(b"<calc>0-7/2</calc>") == -3            # toward zero
    assert O.eval_calc(b"<calc>(0-7)/2</calc>") == -3
    assert _oracle_eval(b"<calc>5/(3-3)</calc>") == "division by zero"
    big = b"<calc>" + b"*".join([b"999"] * 7) + b"</calc>"
    assert O.eval_calc(big) == 999 ** 7
    assert _oracle_eval(big, INT64) == "out of range"
    assert _oracle_eval(b"<calc>" + b"*".join([b"999"] * 6) + b"</calc>", INT64) == 999 ** 6


def test_evaluator_against_python_parser():
    rng = W.SplitMix(63)
    spec = dict(SPEC, int_max=999999999)
    for i in range(3000):
        body = W.calc_expr(rng, spec if i % 3 == 0 else SPEC, budget=3 + rng.below(8))
        span = b"<calc>" + body + b"</calc>"
        bound = INT64 if i % 2 else None
        assert _oracle_eval(span, bound) == _python_eval(body, bound), span


# ---------------------------------------------------------------------------
# The library's host parts against the oracle.
# ---------------------------------------------------------------------------
def _cg():
    import logit_masking_amd as cg
    try:
        cg.lib()
    except (ImportError, OSError) as e:
        pytest.skip(f"libcg.so not built: {e}")
    return cg


def test_library_evaluator_matches_oracle():
    cg = _cg()
    rng = W.SplitMix(64)
    spec = dict(SPEC, int_max=999999999)
    cases = [b"<calc>17 * 23 + 91</calc>", b"<calc>5/(3-3)</calc>",
             b"<calc>" + b"*".join([b"999999999"] * 3) + b"</calc>",
             b"<calc>" + b"*".join([b"999"] * 6) + b"</calc>", b"<calc>0-9223372036854775807-1</calc>",
             b"<calc>0-9223372036854775807-2</calc>", b"<calc>9223372036854775807</calc>",
             b"<calc>9223372036854775808</calc>"]
    for i in range(4000):
        cases.append(b"<calc>" + W.calc_expr(rng, spec if i % 2 else SPEC, budget=3 + rng.below(8)) + b"</calc>")
    for span in cases:
        want = _oracle_eval(span, INT64)
        rc, got = cg.eval_calc(span)
        if isinstance(want, int):
            assert rc == cg.CG_OK and got == want, span
        else:
            assert rc == cg.CG_E_EVAL and got == want, (span, got)
    # malformed spans are parse errors
    for bad in (b"<calc>1+</calc>", b"<calc>(1</calc>", b"<calc>1)</calc>", b"<calc></calc>", b"<calc>1 2</calc>"):
        assert cg.eval_calc(bad)[0] == cg.CG_E_PARSE, bad


def test_library_walker_matches_oracle(og, vocab):
    cg = _cg()
    blob, off, toks = vocab
    g = cg.Grammar(W.spec_json(6), blob, off, host_only=True)
    rng = W.SplitMix(65)
    for i in range(400):
        data, _ = _random_member(rng, rng.below(4))
        if i % 2:
            d = bytearray(data)
            p = rng.below(len(d))
            d[p] = b"<>/ce0-_x"[rng.below(9)]
            data = bytes(d)
        assert g.try_input(data) == og.try_input(data), data
