"""String-operation spans (CPU only).

Page "Evaluator aware decoding", section "Not just arithmetic: string
operations": the same span protocol carries pure string functions -- the
page counts the r's in "strawberry" -- evaluated by the engine and injected
as the result; a small registry (count, len, reverse, upper, substr).

Pins: the page's example; the evaluators against Python's own string
methods; the grammar against a regular-expression validator on random and
mutated members; the library's evaluator and table walker against the
oracle's.
"""
import re

import pytest

from logit_masking_amd import workloads as W
from oracle import oracle as O
from tests import langref

SPEC = W.SPECS[7]
PAGE = b'The count is <strop>count("strawberry", "r")</strop>'


@pytest.fixture(scope="module")
def og():
    return O.load_spec(W.spec_json(7))


def _cg():
    import logit_masking_amd as cg
    try:
        cg.lib()
    except (ImportError, OSError) as e:
        pytest.skip(f"libcg.so not built: {e}")
    return cg


def test_page_example(og):
    row = O.Row(og, W.GEN_CAP)
    sts = [row.advance(bytes([b])) for b in PAGE]
    assert sts[-1] == O.ROW_INJECT and set(sts[:-1]) == {O.ROW_OK}
    span = PAGE[PAGE.index(b"<strop>"):]
    assert O.eval_strop(span) == b"3"
    assert row.force(b"<result>3</result>") == O.ROW_OK
    assert row.advance(b", so <end>") == O.ROW_DONE
    assert langref.calc_text_parts(SPEC, bytes(row.text))[2:4] == [("engine", b"<result>3</result>"),
                                                                   ("model", b", so ")]
    # a model may not write the result itself, and a text result is any
    # printable run without '<'
    c = og.start()
    assert og.feed(c, PAGE + b"<result>3", model=True) == len(PAGE)
    c = og.start()
    tail = b"<result>yrrebwarts and more</result>x<end>"
    assert og.feed(c, PAGE + tail) == len(PAGE) + len(tail) and og.complete(c)


def _python_eval(name, args):
    s = args[0]
    return {"count": lambda: str(s.count(args[1])), "len": lambda: str(len(s)), "reverse": lambda: s[::-1],
            "upper": lambda: s.upper(), "substr": lambda: s[args[1]:args[2]]}[name]().encode()


def _random_call(rng):
    alphabet = "abcrsy !?.-XYZ0123"
    word = lambda: "".join(alphabet[rng.below(len(alphabet))] for _ in range(rng.below(9)))
    name = ("count", "len", "reverse", "upper", "substr")[rng.below(5)]
    if name == "count":
        args = [word(), word()[:rng.below(3)]]
    elif name == "substr":
        args = [word(), rng.below(25) - 12, rng.below(25) - 12]
    else:
        args = [word()]
    text = name + "(" + ", ".join('"%s"' % a if isinstance(a, str) else str(a) for a in args) + ")"
    return name, args, ("<strop>" + text + "</strop>").encode()


def test_evaluators_against_python():
    cg = _cg()
    rng = W.SplitMix(0x57)
    for i in range(3000):
        name, args, span = _random_call(rng)
        want = _python_eval(name, args)
        assert O.eval_strop(span) == want, span
        rc, got = cg.eval_strop(span)
        assert rc == cg.CG_OK and got == want, (span, got, want)
    for bad in (b'<strop>count("a")</strop>', b'<strop>len(a)</strop>', b'<strop>upper("a",)</strop>',
                b'<strop>nope("a")</strop>', b'<strop>substr("a", 1)</strop>'):
        assert cg.eval_strop(bad)[0] == cg.CG_E_PARSE, bad


def _member(rng):
    segs = W.calc_text_script(rng, SPEC, 1 + rng.below(3))
    out = b""
    for s in segs[:-1]:
        if s.endswith(b"</strop>"):
            res = b"<result>" + O.eval_strop(s[s.rindex(b"<strop>"):]) + b"</result>"
        else:
            try:
                res = b"<result>%d</result>" % O.eval_calc(s[s.rindex(b"<calc>"):], O.INT64_RANGE)
            except O.CalcError as e:
                res = b"<result_error>" + str(e).encode() + b"</result_error>"
        out += s + res
    return out + segs[-1]


def test_members_and_mutations(og):
    cg = _cg()
    blob, off = W.make_vocab(7, 4096)
    lg = cg.Grammar(W.spec_json(7), blob, off, host_only=True)
    rng = W.SplitMix(0x58)
    alphabet = b'<>/strop()"count,len -0123456789ablr\n'
    n_in = n_out = 0
    for i in range(1500):
        d = bytearray(_member(rng))
        if i % 3:
            for _ in range(1 + rng.below(2)):
                p = rng.below(len(d) + 1)
                if rng.uniform() < 0.5 and p < len(d):
                    d[p] = alphabet[rng.below(len(alphabet))]
                else:
                    d.insert(p, alphabet[rng.below(len(alphabet))])
        d = bytes(d)
        want = langref.member(SPEC, d)
        k, complete = og.try_input(d)
        assert complete == want, d
        assert lg.try_input(d) == (k, complete), d
        n_in += want
        n_out += not want
    assert n_in > 400 and n_out > 400


def test_calc_only_text_refuses_strop():
    g6 = O.load_spec(W.spec_json(6))
    assert g6.try_input(PAGE)[0] == PAGE.index(b"<strop>") + 1
