"""Decision-schema designs 2-5 as compile targets (CPU only).

Page "Guided Decoding & Structured-Output Reliability", sections "Designs
2-4 -- making the schema show its working" and "Design 5 -- the pipeline":
fields ahead of the decision (free-text calculation and a band; a boolean
gate with a nullable tier; one field per predicate, with a native integer
and a number), or an extraction schema with no decision fields (a nullable
integer, an array of at most 10 numbers, nullable capped strings).

Pins: hand-written members and near-members from the page's field lists,
the full-string validator (tests/langref.py) and Python's json module on
finished outputs; then the library's table walker against the oracle.
"""
import json

import numpy as np
import pytest

from logit_masking_amd import workloads as W
from oracle import oracle as O
from tests import langref

DESIGNS = sorted(W.DESIGN_SCHEMAS)

DECISION_TAIL = ('"eligibility":{"criteria_met":true,"reason_code":"eligible"},"action":"book_appointment",'
                 '"appointment":{"date":"2024-05-01","time":"10:00"},"response_text":"Booked."}')

MEMBERS = {
    2: ['{"calculation":"3 x 1500 = 4500","within_limit_banding":"within_limit",' + DECISION_TAIL,
        '{"calculation":"","within_limit_banding":"over_limit",' + DECISION_TAIL.replace(
            '{"date":"2024-05-01","time":"10:00"}', "null")],
    3: ['{"exceeds_value_limit":false,"over_limit_tier":null,' + DECISION_TAIL,
        '{"exceeds_value_limit":true,"over_limit_tier":"hard_decline",' + DECISION_TAIL],
    4: ['{"customer_age":34,"age_within_18_to_70":true,"total_requested_value":10450.5,'
        '"total_at_most_10000":false,"total_at_most_12000":true,' + DECISION_TAIL,
        '{"customer_age":-1,"age_within_18_to_70":false,"total_requested_value":1e4,'
        '"total_at_most_10000":true,"total_at_most_12000":true,' + DECISION_TAIL],
    5: ['{"customer_age":null,"price_components":[],"requested_date":null,"requested_time":null}',
        '{"customer_age":71,"price_components":[1200,350.75,1e2],"requested_date":"next Tuesday",'
        '"requested_time":"9am"}',
        '{"customer_age": 20, "price_components": [1, 2, 3, 4, 5, 6, 7, 8, 9, 10], '
        '"requested_date": null, "requested_time": "10:30"}'],
}

# (design, text, first refused byte): values the schemas rule out
REFUSED = [
    (3, '{"exceeds_value_limit":true,"over_limit_tier":"soft"', len('{"exceeds_value_limit":true,"over_limit_tier":"')),
    (3, '{"exceeds_value_limit":1', len('{"exceeds_value_limit":')),
    (4, '{"customer_age":"34"', len('{"customer_age":')),
    (4, '{"customer_age":34.5', len('{"customer_age":34')),
    (4, '{"customer_age":34,"age_within_18_to_70":true,"total_requested_value":01',
     len('{"customer_age":34,"age_within_18_to_70":true,"total_requested_value":0')),
    (5, '{"customer_age":null,"price_components":[1,2,3,4,5,6,7,8,9,10,11',
     len('{"customer_age":null,"price_components":[1,2,3,4,5,6,7,8,9,10')),
    (5, '{"customer_age":null,"price_components":["1"', len('{"customer_age":null,"price_components":[')),
    (5, '{"eligibility"', len('{"')),
    (2, '{"within_limit_banding"', len('{"')),
]


@pytest.fixture(scope="module")
def grammars():
    return {d: O.load_spec(W.design_spec_json(d)) for d in DESIGNS}


@pytest.mark.parametrize("design", DESIGNS)
def test_members(grammars, design):
    g = grammars[design]
    spec = json.loads(W.design_spec_json(design))
    for text in MEMBERS[design]:
        data = text.encode()
        assert g.try_input(data) == (len(data), True), text
        assert langref.member(spec, data)
        obj = json.loads(text)
        assert list(obj) == list(W.DESIGN_SCHEMAS[design]["properties"])


@pytest.mark.parametrize("design,text,at", REFUSED)
def test_refused(grammars, design, text, at):
    k, complete = grammars[design].try_input(text.encode())
    assert (k, complete) == (at, False), text


@pytest.mark.parametrize("design", DESIGNS)
def test_random_outputs_are_members(grammars, design):
    """Rows driven to completion with the oracle's masks: every finished
    output is a member (validator), parses as JSON with the declared key
    order, and keeps the schema's value types."""
    blob, off = W.make_vocab(2, 4096)
    toks = [blob[off[i]:off[i + 1]] for i in range(len(off) - 1)]
    g = grammars[design]
    spec = json.loads(W.design_spec_json(design))
    rng = W.SplitMix(0xDE5 + design)
    done = 0
    for trial in range(5):
        row = O.Row(g, gen_cap=1500)
        while not row.done:
            bits = O.unpack_mask(g.mask(row.conf, blob, off), len(toks))
            allowed = np.nonzero(bits)[0]
            assert len(allowed)
            short = [t for t in allowed if len(toks[t]) > 1 and (b'"' in toks[t] or b"," in toks[t])]
            pool = short if short and rng.uniform() < 0.75 else list(allowed)
            row.advance(toks[int(pool[rng.below(len(pool))])])
        if not row.complete:
            continue
        done += 1
        text = bytes(row.text)
        assert langref.member(spec, text)
        obj = json.loads(text.decode())
        assert list(obj) == list(W.DESIGN_SCHEMAS[design]["properties"])
        if design == 5:
            assert isinstance(obj["price_components"], list) and len(obj["price_components"]) <= 10
            assert all(isinstance(x, (int, float)) and not isinstance(x, bool) for x in obj["price_components"])
            assert obj["customer_age"] is None or (isinstance(obj["customer_age"], int)
                                                   and not isinstance(obj["customer_age"], bool))
        if design == 3:
            assert obj["over_limit_tier"] in (None, "reduced_scope", "hard_decline")
    assert done >= 1


@pytest.mark.parametrize("design", DESIGNS)
def test_library_walker_matches_oracle(grammars, design):
    import logit_masking_amd as cg
    try:
        cg.lib()
    except (ImportError, OSError) as e:
        pytest.skip(f"libcg.so not built: {e}")
    blob, off = W.make_vocab(2, 4096)
    lg = cg.Grammar(W.design_spec_json(design), blob, off, host_only=True)
    g = grammars[design]
    rng = W.SplitMix(0xDE9 + design)
    alphabet = b'{}[]",:0123456789.-+eE ntrufals_abcdxyz'
    texts = [m.encode() for m in MEMBERS[design]] + [t.encode() for d, t, _ in REFUSED if d == design]
    for i in range(400):
        d = bytearray(texts[rng.below(len(texts))])
        for _ in range(1 + rng.below(3)):
            p = rng.below(len(d) + 1)
            if rng.uniform() < 0.5 and p < len(d):
                d[p] = alphabet[rng.below(len(alphabet))]
            else:
                d.insert(p, alphabet[rng.below(len(alphabet))])
        d = bytes(d)
        assert lg.try_input(d) == g.try_input(d), d
