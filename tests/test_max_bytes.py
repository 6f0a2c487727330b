"""The longest member of a finite language (CPU only).

The compiler reports max_bytes from the longest path of its packed automaton
(cg_grammar_info); the oracle computes it by recursion over its schema tree
and returns a witness ("Constrained decoding", "A valid call also has to
end": how long a constrained output can get).  Pins of the oracle's value:
the witness is a member (the oracle's recognizer and the independent
full-string validator in tests/langref.py both accept it, so the value is
reached), and no member of the exactly enumerated tiny languages is longer;
on alphabets that can spell the longest forms (escapes, whitespace, the
longest integers) the enumerated maximum equals it.  The compiler's value must
then equal the oracle's on every workload and tiny language, with "infinite"
(-1 / None) exactly where the language has no bound.
"""
import json

import pytest

import logit_masking_amd as cg
from logit_masking_amd import workloads as W
from oracle import oracle as O
from tests import langref
from tests.test_oracle_pins import TINY

# tiny languages whose alphabets can spell a longest member: a six-byte
# escape (\u0000), whitespace runs at ws_max, both ends of integer ranges
SPELLABLE = [
    ("str-ws1", {"kind": "json_schema", "ws_max": 1, "schema": {
        "type": "object", "properties": {"a": {"type": "string", "maxLength": 1}},
        "required": ["a"], "additionalProperties": False}},
     b'{}":,a \\u0', 40),
    ("int-enum", {"kind": "json_schema", "ws_max": 0, "schema": {
        "type": "object", "properties": {
            "b": {"type": "integer", "minimum": -12, "maximum": 3},
            "c": {"enum": ["x", "yy"]}},
        "required": ["b"], "additionalProperties": False}},
     b'{}":,bcxy-0123', 40),
    ("array-ws2", {"kind": "json_schema", "ws_max": 2, "schema": {
        "type": "array", "items": {"enum": ["p", "qq"]}, "maxItems": 2}},
     b'[]",pq ', 40),
    ("tools-shared-prefix", TINY[4][1], TINY[4][2], TINY[4][3]),
    ("depth-cap", TINY[6][1], TINY[6][2], TINY[6][3]),
    ("nested-anyof", TINY[2][1], TINY[2][2], TINY[2][3]),
]

_VOCAB = (bytes(range(256)), list(range(257)))


def _compiler_max(spec):
    g = cg.Grammar(json.dumps(spec).encode(), *_VOCAB, host_only=True)
    return g.info()["max_bytes"]


@pytest.mark.parametrize("name,spec,sigma,budget", TINY + SPELLABLE, ids=[t[0] for t in TINY + SPELLABLE])
def test_oracle_longest_member_bounds_the_enumeration(name, spec, sigma, budget):
    g = O.load_spec(spec)
    n, w = g.longest_member()
    assert n is not None and len(w) == n
    assert g.try_input(w) == (n, True) and langref.member(spec, w), w
    M = langref.Enumerator(spec, sigma, budget).members()
    assert M and max(len(m) for m in M) <= n
    if (name, spec, sigma, budget) in SPELLABLE:
        assert max(len(m) for m in M) == n


def test_oracle_longest_member_closed_forms():
    # compact {"reasoning": string of at most 2000 code points, "answer": integer}:
    # 13 + (2 + 6 x 2000) + 10 + ("-" + 20 digits) + 1
    n, w = O.load_spec(W.spec_json(4)).longest_member()
    assert n == 13 + 2 + 6 * 2000 + 10 + 21 + 1 == len(w)
    # unbounded: calc expressions, a number, an array without maxItems, any value, an uncapped string
    for spec in ({"kind": "calc"},
                 {"kind": "json_schema", "schema": {"type": "array", "items": {"type": "number"}, "maxItems": 1}},
                 {"kind": "json_schema", "schema": {"type": "array", "items": {"type": "boolean"}}},
                 {"kind": "json_schema", "schema": {"type": "object", "properties": {"v": {}},
                                                    "additionalProperties": False}},
                 {"kind": "json_schema", "open_string_cap": None, "schema": {"type": "string"}}):
        assert O.load_spec(spec).longest_member() == (None, None), spec


@pytest.mark.parametrize("cfg", sorted(W.SPECS))
def test_compiler_max_bytes_equals_oracle(cfg):
    spec = json.loads(W.spec_json(cfg))
    n, _ = O.load_spec(spec).longest_member()
    assert _compiler_max(spec) == (-1 if n is None else n)


@pytest.mark.parametrize("name,spec,sigma,budget", TINY + SPELLABLE, ids=[t[0] for t in TINY + SPELLABLE])
def test_compiler_max_bytes_tiny(name, spec, sigma, budget):
    assert _compiler_max(spec) == O.load_spec(spec).longest_member()[0]


def test_compiler_max_bytes_schemas():
    """The page's design schemas and one-sided integer bounds, strings at
    their caps, optional keys, nesting at the depth cap."""
    specs = [{"kind": "json_schema", "schema": s} for s in W.DESIGN_SCHEMAS.values()]
    for lo, hi in ((None, None), (5, None), (-7, None), (None, 40), (None, -3), (-100, 99)):
        b = {"type": "integer"}
        if lo is not None:
            b["minimum"] = lo
        if hi is not None:
            b["maximum"] = hi
        specs.append({"kind": "json_schema", "ws_max": 1, "open_int_digits": 7, "schema": {
            "type": "object", "properties": {"i": b, "s": {"type": "string"}}, "required": ["i"],
            "additionalProperties": False}})
    specs.append({"kind": "json_schema", "depth_cap": 3, "ws_max": 0, "schema": {
        "type": "object", "properties": {"a": {"type": "array", "maxItems": 2, "items": {
            "type": "object", "properties": {"b": {"type": "object", "properties": {},
                                                   "additionalProperties": False}},
            "additionalProperties": False}}}, "additionalProperties": False}})
    checked = 0
    for spec in specs:
        n, w = O.load_spec(spec).longest_member()
        assert _compiler_max(spec) == (-1 if n is None else n), spec
        if w is not None:
            assert langref.member(spec, w), w
            checked += 1
    assert checked >= 7
