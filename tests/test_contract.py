"""The integer-string contract (CPU only).

Page "Constrained Decoding Under Matched Conditions", section "The system
boundary I am testing": the external answer is a canonical signed-integer
string; the model writes a native JSON integer under a separate
model-facing schema; an exact inverse turns each integer back into a
string of its own digits (arbitrary precision) and the result is validated
against the original schema.  No repair: a boolean is rejected, and +26,
00026, 26.0 and 2.6e1 are not guessed into the accepted language.

Pins: the page's example and rules; the full-string validator and Python's
regex engine on the external side; a plain Python reference in the oracle
that the library's C++ transform must match byte for byte.
"""
import json
import re

import numpy as np
import pytest

from logit_masking_amd import workloads as W
from oracle import oracle as O
from tests import langref

PATTERN = O.INT_STRING_PATTERN
INT_STR = {"type": "string", "pattern": PATTERN}


def _spec(schema, ws_max=0, digits=20):
    return {"kind": "json_schema", "ws_max": ws_max, "open_string_cap": 256, "open_int_digits": digits,
            "depth_cap": 16, "schema": schema}


# the page's contract: reasoning text, then the answer as an integer string
ANSWER = _spec(W._obj([("reasoning", W._strn(2000)), ("answer", INT_STR)]))
NESTED = _spec(W._obj([
    ("id", INT_STR),
    ("totals", {"type": "array", "items": INT_STR, "maxItems": 5}),
    ("maybe", {"anyOf": [INT_STR, {"type": "null"}]}),
    ("inner", W._obj([("n", INT_STR), ("label", W._strn(10)), ("x", {"type": "number"})])),
]), ws_max=2, digits=12)  # four open integers of 20 digits would exceed the 60 KiB table


def _cg():
    import logit_masking_amd as cg
    try:
        cg.lib()
    except (ImportError, OSError) as e:
        pytest.skip(f"libcg.so not built: {e}")
    return cg


def test_page_example():
    model, n = O.contract_model_spec(ANSWER)
    assert n == 1 and model["schema"]["properties"]["answer"] == {"type": "integer"}
    assert model["schema"]["properties"]["reasoning"] == ANSWER["schema"]["properties"]["reasoning"]
    # the model writes a native integer; the inverse gives the caller's string
    ok, out, _ = O.contract_reverse(ANSWER, b'{"reasoning":"...","answer":18000}')
    assert ok and out == b'{"reasoning":"...","answer":"18000"}'
    assert json.loads(out)["answer"] == "18000"
    ok, out, _ = O.contract_reverse(ANSWER, b'{"reasoning":"...","answer":-14}')
    assert ok and json.loads(out)["answer"] == "-14"
    # a boolean is rejected even though Python treats it as an integer
    assert not O.contract_reverse(ANSWER, b'{"reasoning":"...","answer":true}')[0]
    # no guessing: these are refused by the model-facing grammar, and the
    # inverse does not accept their number forms either
    mg = O.load_spec(model)
    for bad in (b"+26", b"00026", b"26.0", b"2.6e1"):
        text = b'{"reasoning":"...","answer":' + bad + b"}"
        assert not mg.try_input(text)[1]
        if bad in (b"26.0", b"2.6e1"):
            assert not O.contract_reverse(ANSWER, text)[0]
    # on the external side the same spellings fail the pattern
    eg = O.load_spec(ANSWER)
    for bad in ("+26", "00026", "26.0", "2.6e1", ""):
        text = ('{"reasoning":"...","answer":"%s"}' % bad).encode()
        assert not eg.try_input(text)[1] and not langref.member(ANSWER, text)
        assert not re.fullmatch(PATTERN, bad)


def test_external_pattern_against_regex():
    """The external grammar's integer strings are exactly Python's regex
    matches of the pattern (with the open-integer digit cap)."""
    eg = O.load_spec(ANSWER)
    rng = W.SplitMix(0xC0)
    alphabet = "0123456789-+.e "
    for i in range(4000):
        s = "".join(alphabet[rng.below(len(alphabet))] for _ in range(rng.below(24)))
        if i % 3 == 0:
            s = str(rng.below(10 ** rng.below(22)) * (-1 if rng.uniform() < 0.5 else 1))
        text = ('{"reasoning":"","answer":"%s"}' % s).encode()
        want = bool(re.fullmatch(PATTERN, s)) and len(s.lstrip("-")) <= 20
        assert eg.try_input(text)[1] == want, s
        assert langref.member(ANSWER, text) == want, s


def _model_members(spec, n, seed):
    """Complete generations under the model-facing schema (oracle rows over
    a JSON-ish vocabulary, leaning to digits and structure)."""
    model, _ = O.contract_model_spec(spec)
    g = O.load_spec(model)
    blob, off = W.make_vocab(4, 4096)
    toks = [blob[off[i]:off[i + 1]] for i in range(len(off) - 1)]
    rng = W.SplitMix(seed)
    out = []
    while len(out) < n:
        row = O.Row(g, gen_cap=400)
        while not row.done:
            bits = O.unpack_mask(g.mask(row.conf, blob, off), len(toks))
            allowed = np.nonzero(bits)[0]
            pref = [t for t in allowed if len(toks[t]) > 1 and any(c in toks[t] for c in b'",}]0123456789')]
            pool = pref if pref and rng.uniform() < 0.8 else list(allowed)
            row.advance(toks[int(pool[rng.below(len(pool))])])
        if row.complete:
            out.append(bytes(row.text))
    return out


@pytest.mark.parametrize("spec", [ANSWER, NESTED], ids=["answer", "nested"])
def test_reverse_of_generations(spec):
    """Every generation under the model-facing schema maps back onto the
    external schema; the strings hold the integers' exact digits."""
    for text in _model_members(spec, 12, seed=len(json.dumps(spec))):
        ok, out, msg = O.contract_reverse(spec, text)
        assert ok, (text, msg)
        assert langref.member(spec, out)
        src = json.loads(text, parse_int=str)
        dst = json.loads(out)

        def check(a, b, sch):
            if sch == INT_STR:
                assert isinstance(b, str) and b == a
            elif "anyOf" in sch:
                check(a, b, INT_STR if isinstance(b, str) else {"type": "null"})
            elif sch.get("type") == "object":
                for k in a:
                    check(a[k], b[k], sch["properties"][k])
            elif sch.get("type") == "array":
                for x, y in zip(a, b):
                    check(x, y, sch["items"])

        check(src, dst, spec["schema"])


def test_library_matches_oracle():
    cg = _cg()
    for spec in (ANSWER, NESTED):
        sj = json.dumps(spec)
        model_lib, n = cg.contract_model_spec(sj)
        model_or, n_or = O.contract_model_spec(spec)
        assert n == n_or and json.loads(model_lib) == model_or
        texts = _model_members(spec, 8, seed=7 + len(sj))
        texts += [b'{"reasoning":"x","answer":true}', b'{"reasoning":"x","answer":2.5}', b"[1]", b"nope",
                  b'{"reasoning":"x","answer":123456789012345678901234567890}',
                  b'{"reasoning":"tab\\there \\u0001 \\"q\\"","answer":0}']
        for t in texts:
            rc, out, msg = cg.contract_reverse(sj, t)
            ok, want, _ = O.contract_reverse(spec, t)
            assert (rc == cg.CG_OK) == ok, (t, msg)
            if want is not None and rc == cg.CG_OK:
                assert out == want, (t, out, want)


def test_unsupported_fails_closed():
    cg = _cg()
    # an integer string beside an integer alternative: the model-facing anyOf
    # would not be LL(1) -- refused, with its path
    bad = _spec({"anyOf": [INT_STR, {"type": "integer"}]})
    with pytest.raises(cg.CgError) as e:
        cg.contract_model_spec(json.dumps(bad))
    assert e.value.code == cg.CG_E_UNSUPPORTED
    # any other pattern is refused by the compiler
    other = _spec(W._obj([("a", {"type": "string", "pattern": "^[a-z]+$"})]))
    blob, off = W.make_vocab(4, 4096)
    with pytest.raises(cg.CgError) as e:
        cg.Grammar(json.dumps(other), blob, off, host_only=True)
    assert e.value.code == cg.CG_E_UNSUPPORTED
    with pytest.raises(O.Unsupported):
        O.load_spec(other)
