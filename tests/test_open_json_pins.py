"""Pins of the oracle's open (any-JSON) values, CPU only: the recursive-JSON
grammar (objects / arrays as the root, any value inside, depth-capped) and
`{}` values inside a schema.

Every check compares the oracle with something other than itself: the JSON
grammar of RFC 8259 (hand-derived refusal offsets, tests/golden/
open_json.json), Python's json module, and brute force over tiny languages
generated from the grammar's productions (tests/langref.py).  "Constrained
decoding", "The guarantee": malformed JSON cannot be generated.
"""
import json
import os

import numpy as np
import pytest

from logit_masking_amd import workloads as W
from oracle import oracle as O
from tests import langref
from tests.test_oracle_pins import _check_tiny

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "open_json.json")
CFG = 5  # recursive JSON: object or array root, depth cap 32, whitespace runs <= 4


@pytest.fixture(scope="module")
def g5():
    return O.load_spec(W.spec_json(CFG))


def _strict_loads(data: bytes):
    def no_constant(name):
        raise ValueError(name)
    return json.loads(data.decode("utf-8"), parse_constant=no_constant)


def _depth(v):
    if isinstance(v, dict):
        return 1 + max((_depth(x) for x in v.values()), default=0)
    if isinstance(v, list):
        return 1 + max((_depth(x) for x in v), default=0)
    return 0


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["input"][:24])
def test_open_json_golden(g5, case):
    data = case["input"].encode()
    want = len(data) if case["refused_at"] is None else case["refused_at"]
    assert g5.try_input(data) == (want, case["complete"]), case["cite"]
    # the independent full-string validator and Python's parser agree on membership
    assert langref.member(W.SPECS[CFG], data) == case["complete"]
    if case["complete"]:
        assert _depth(_strict_loads(data)) <= 32


def _deep_cases():
    """Containers nested to the cap (32, the root counting as 1) and one past
    it; the refusal offset is where the construction opens container 33."""
    obj = b'{"a":'
    mixed = b""
    for d in range(32):
        mixed += b'{"k":' if d % 2 == 0 else b"["
    closes = b"".join(b"}" if d % 2 == 0 else b"]" for d in reversed(range(32)))
    return [
        (b"[" * 32 + b"]" * 32, None, True),
        (b"[" * 33, 32, False),
        (b"[" * 32 + b'1,"a",{}' + b"]" * 32, 32 + len(b'1,"a",'), False),
        (b"[" * 32 + b'1,"a",true' + b"]" * 32, None, True),
        (obj * 32 + b"null" + b"}" * 32, None, True),
        (obj * 32 + b"[]" + b"}" * 32, 32 * len(obj), False),
        (obj * 31 + b"{}" + b"}" * 31, None, True),
        (mixed + b"0" + closes, None, True),
        (mixed + b"[" , len(mixed), False),
        # the cap holds after containers close: depth goes back down and up again
        (b"[" * 31 + b"[]" + b",[]" + b"]" * 31, None, True),
        (b"[" * 31 + b"[]" + b",[[" , 31 + 2 + 2, False),
        # whitespace runs inside the root up to 4 at the deepest level
        (b"[" * 32 + b"    1    " + b"]" * 32, None, True),
    ]


@pytest.mark.parametrize("data,refused_at,complete", _deep_cases(), ids=lambda x: str(x)[:16])
def test_open_json_depth_cap(g5, data, refused_at, complete):
    want = len(data) if refused_at is None else refused_at
    assert g5.try_input(data) == (want, complete)
    assert langref.member(W.SPECS[CFG], data) == complete
    if complete:
        assert _depth(_strict_loads(data)) == 32


# ---------------------------------------------------------------------------
# Brute force: open values under tiny caps.  The enumerator builds the
# language from RFC 8259's productions (tests/langref.py: any_values,
# open_array, open_object, numbers); the oracle's viable next bytes after
# every prefix that leaves room for its longest shortest completion
# (min_room) must be exactly the bytes that keep it a prefix of a member.
# ---------------------------------------------------------------------------
OPEN = {"anyOf": [{"type": "object"}, {"type": "array"}]}
OPEN_TINY = [
    # structure: keys, colons, commas, nesting to the cap of 2, no whitespace;
    # the longest shortest completion is 6 ('[{"":1,' + '"":1}]')
    ("structure", {"kind": "json_schema", "ws_max": 0, "open_string_cap": 1, "depth_cap": 2, "schema": OPEN},
     b'[]{}",:1', 16, 6),
    # the same with whitespace runs of one byte around structural bytes
    ("whitespace", {"kind": "json_schema", "ws_max": 1, "open_string_cap": 1, "depth_cap": 2, "schema": OPEN},
     b'[]{}",:1 ', 12, 6),
    # numbers (RFC 8259 section 6) as array items, no nesting ('[-' + '0]')
    ("numbers-e", {"kind": "json_schema", "ws_max": 0, "open_string_cap": 0, "depth_cap": 1,
                   "schema": {"type": "array"}}, b"[],-01.e+", 10, 2),
    ("numbers-E", {"kind": "json_schema", "ws_max": 0, "open_string_cap": 0, "depth_cap": 1,
                   "schema": {"type": "array"}}, b"[],-0.1E-", 10, 2),
    # the literal names (RFC 8259 section 3); after '[f' the completion is 'alse]'
    ("literals", {"kind": "json_schema", "ws_max": 0, "open_string_cap": 0, "depth_cap": 1,
                  "schema": {"type": "array"}}, b"[],truefalsn", 22, 5),
    # an open value as a declared property's schema ({} inside an object,
    # as store_record's value of the tool-call grammar)
    ("property", {"kind": "json_schema", "ws_max": 0, "open_string_cap": 1, "depth_cap": 2, "schema": {
        "type": "object", "properties": {"v": {}}, "required": ["v"], "additionalProperties": False}},
     b'{}[]":,v1', 17, 6),
]


@pytest.mark.parametrize("name,spec,sigma,budget,room", OPEN_TINY, ids=[t[0] for t in OPEN_TINY])
def test_open_values_bruteforce(name, spec, sigma, budget, room):
    assert _check_tiny(spec, sigma, budget, min_room=room) > 20


def test_open_values_enumerator_matches_python_json():
    """The enumerator itself against Python's parser: over the alphabet of the
    structure case, every byte string of length <= 6 is a member iff
    json.loads takes it as an object or array nested at most twice."""
    import itertools
    spec, sigma = OPEN_TINY[0][1], OPEN_TINY[0][2]
    members = langref.Enumerator(spec, sigma, 6).members()
    n = 0
    for k in range(1, 7):
        for t in itertools.product(sigma, repeat=k):
            s = bytes(t)
            try:
                v = _strict_loads(s)
                ok = isinstance(v, (dict, list)) and _depth(v) <= 2 and all(
                    len(key) <= 1 for key in _keys(v)) and all(len(x) <= 1 for x in _strs(v))
                ok = ok and b" " not in s
            except ValueError:
                ok = False
            assert (s in members) == ok, s
            n += ok
    assert n > 20


def _keys(v):
    if isinstance(v, dict):
        for k, x in v.items():
            yield k
            yield from _keys(x)
    elif isinstance(v, list):
        for x in v:
            yield from _keys(x)


def _strs(v):
    if isinstance(v, str):
        yield v
    elif isinstance(v, dict):
        for x in v.values():
            yield from _strs(x)
    elif isinstance(v, list):
        for x in v:
            yield from _strs(x)


def test_open_json_outputs_parse():
    """Rows of the recursive-JSON grammar driven to completion over a 4096-token
    vocabulary of the workload: every finished text is a member (validator),
    parses with Python's json module and nests at most 32 deep."""
    g = O.load_spec(W.spec_json(CFG))
    blob, off = W.make_vocab(CFG, 4096)
    V = len(off) - 1
    toks = [blob[off[i]:off[i + 1]] for i in range(V)]
    rng = W.SplitMix(505)
    finished = 0
    for trial in range(8):
        row = O.Row(g, gen_cap=W.GEN_CAP)
        while not row.done:
            bits = O.unpack_mask(g.mask(row.conf, blob, off), V)
            allowed = np.nonzero(bits)[0]
            assert len(allowed) > 0
            # lean toward closing tokens and deep nesting in turn, so rows both
            # reach the cap region and finish
            close = [t for t in allowed if toks[t][-1:] in (b"]", b"}")]
            deep = [t for t in allowed if toks[t][-1:] in (b"[", b"{")]
            u = rng.uniform()
            pool = (deep if trial % 2 and row.step < 200 and u < 0.5 else close if u < 0.6 else []) or allowed
            row.advance(toks[int(pool[rng.below(len(pool))])])
        if row.complete:
            finished += 1
            text = bytes(row.text)
            assert langref.member(W.SPECS[CFG], text)
            assert _depth(_strict_loads(text)) <= 32
    assert finished >= 6
