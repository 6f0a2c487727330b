"""CPU tests of the C ABI library: exports, decoupling, the host compiler and
its table walker (cg_try_input) against the oracle.  No device calls."""
import json
import os
import re
import subprocess

import numpy as np
import pytest

import logit_masking_amd as cg
from logit_masking_amd import workloads as W
from oracle import oracle as O
from tests import langref
from tests.test_oracle_pins import TINY

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    src = open(os.path.join(ROOT, "include", "cg.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(cg_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    declared = _header_functions()
    assert set(declared) == set(cg.EXPORTS)
    out = subprocess.check_output(["nm", "-D", "--defined-only", cg.LIB_PATH], text=True)
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for name in declared:
        assert name in exported, name
    L = cg.lib()
    for name in declared:
        assert hasattr(L, name)


def test_library_names_no_framework():
    """The contract names no model, tokenizer or framework: the library links
    only the HIP runtime and the C/C++ runtime ("Constrained decoding", "The
    guarantee is not tied to this engine")."""
    out = subprocess.check_output(["ldd", cg.LIB_PATH], text=True)
    # the library names and paths, not the load addresses (random hex digits)
    names = [w for l in out.splitlines() for w in l.split() if not w.startswith("(0x")]
    assert any("amdhip64" in n for n in names), names
    for bad in ("torch", "python", "c10"):
        assert not any(bad in n.lower() for n in names), names


def test_floor_library_is_apart():
    """The bench's read-only reference kernel lives in a library of its own:
    one export, not linked by libcg (whose exports stay those of cg.h)."""
    floor = os.path.join(ROOT, "logit_masking_amd", "libcg_floor.so")
    if not os.path.exists(floor):
        pytest.skip("libcg_floor.so is built by logit_masking_amd/build.py")
    out = subprocess.check_output(["nm", "-D", "--defined-only", floor], text=True)
    assert {l.split()[-1] for l in out.splitlines() if " T " in l} == {"cg_floor_read_rows"}
    assert "libcg_floor" not in subprocess.check_output(["ldd", cg.LIB_PATH], text=True)


@pytest.fixture(scope="module")
def small_vocabs():
    return {c: (W.make_vocab(c, 4096) if c != 1 else W.make_vocab(1)) for c in W.SPECS}


@pytest.mark.parametrize("cfg", sorted(W.SPECS))
def test_compile_all_configs(cfg, small_vocabs):
    blob, off = small_vocabs[cfg]
    g = cg.Grammar(W.spec_json(cfg), blob, off, host_only=True)
    info = g.info()
    assert info["n_states"] > 0 and info["table_bytes"] <= 64 * 1024
    assert info["vocab_size"] == len(off) - 1


def test_full_vocab_compile_config3():
    blob, off = W.make_vocab(3)
    g = cg.Grammar(W.spec_json(3), blob, off, host_only=True)
    assert g.info()["max_token_len"] <= 24


def _host(spec, blob=b"ab", off=(0, 1, 2)):
    import json
    return cg.Grammar(json.dumps(spec).encode(), blob, list(off), host_only=True)


REFUSALS = [
    ({"$ref": "#/x"}, "$.schema"),
    ({"type": "string", "pattern": "a+"}, "$.schema"),
    ({"type": "string", "format": "date"}, "$.schema"),
    ({"oneOf": [{"type": "null"}]}, "$.schema"),
    ({"allOf": [{"type": "null"}]}, "$.schema"),
    ({"type": "object", "properties": {"a": {"type": "null"}}}, "$.schema"),
    ({"type": "object", "patternProperties": {}}, "$.schema"),
    ({"type": "array", "minItems": 1}, "$.schema"),
    ({"type": "integer", "multipleOf": 2}, "$.schema"),
    ({"anyOf": [{"type": "integer"}, {"type": "number"}]}, "$.schema"),
    ({"anyOf": [{"type": "string"}, {"enum": ["a"]}]}, "$.schema"),
    ({"type": "object", "properties": {"a": {"type": "string", "minLength": 1}}, "required": [],
      "additionalProperties": False}, "$.schema/properties/a"),
    ({"type": "integer", "minimum": 5, "maximum": 4}, "$.schema"),
    ({"type": "integer"}, "$.schema"),
    ({}, "$.schema"),
    # a negative bound is refused, not read as "no bound" (fail closed)
    ({"type": "array", "items": {"type": "null"}, "maxItems": -1}, "$.schema"),
    ({"type": "array", "maxItems": -1}, "$.schema"),
    ({"type": "object", "properties": {"a": {"type": "array", "maxItems": -3}}, "required": [],
      "additionalProperties": False}, "$.schema/properties/a"),
]


@pytest.mark.parametrize("schema,path", REFUSALS)
def test_refusals_match_oracle(schema, path):
    spec = {"kind": "json_schema", "schema": schema}
    with pytest.raises(O.Unsupported) as e:
        O.load_spec(spec)
    assert e.value.path == path
    with pytest.raises(cg.CgError) as e2:
        _host(spec)
    assert e2.value.code == cg.CG_E_UNSUPPORTED
    assert str(e2.value).split("] ", 1)[1].startswith(path + ":")


def test_bad_json_and_vocab():
    with pytest.raises(cg.CgError) as e:
        cg.Grammar(b"{not json", b"a", [0, 1], host_only=True)
    assert e.value.code == cg.CG_E_PARSE
    with pytest.raises(cg.CgError) as e:
        cg.Grammar(W.spec_json(1), b"ab", [0, 2, 1], host_only=True)
    assert e.value.code == cg.CG_E_VOCAB
    with pytest.raises(cg.CgError) as e:
        cg.Grammar(W.spec_json(1), b"a" * 33, [0, 33], host_only=True)
    assert e.value.code == cg.CG_E_LIMIT
    with pytest.raises(cg.CgError) as e:
        cg.Grammar(b'{"kind":"nope"}', b"a", [0, 1], host_only=True)
    assert e.value.code == cg.CG_E_UNSUPPORTED


def test_host_only_grammar_refuses_device_calls():
    g = cg.Grammar(W.spec_json(1), *W.make_vocab(1), host_only=True)
    import ctypes
    rc = cg.lib().cg_init_state(g._h, ctypes.c_void_p(0), 0, ctypes.c_void_p(0))
    assert rc == cg.CG_E_ARG


# ---------------------------------------------------------------------------
# try_input (packed table, host walker) == oracle
# ---------------------------------------------------------------------------
def _agree(og, hg, s):
    assert hg.try_input(s) == og.try_input(s), s


@pytest.mark.parametrize("case", __import__("tests.test_oracle_pins", fromlist=["x"])._page_cases()["cases"],
                         ids=lambda c: c["input"][:40])
def test_page_examples_host(case, small_vocabs):
    blob, off = small_vocabs[case["cfg"]]
    hg = cg.Grammar(W.spec_json(case["cfg"]), blob, off, host_only=True)
    data = case["input"].encode()
    k, complete = hg.try_input(data)
    assert k == (len(data) if case["refused_at"] is None else case["refused_at"])
    assert complete == case["complete"]


@pytest.mark.parametrize("name,spec,sigma,budget", TINY, ids=[t[0] for t in TINY])
def test_tiny_languages_host(name, spec, sigma, budget):
    import json
    og = O.load_spec(spec)
    hg = cg.Grammar(json.dumps(spec).encode(), b"a", [0, 1], host_only=True)
    M = langref.Enumerator(spec, sigma, budget).members()
    P = sorted(langref.prefixes(M))
    if len(P) > 3000:
        rng = W.SplitMix(len(P))
        P = [P[rng.below(len(P))] for _ in range(3000)]
    for p in P:
        for b in set(sigma) | {0xFF, 0x20}:
            _agree(og, hg, p + bytes([b]))


def _open_json_cases():
    from tests import test_open_json_pins as P
    cases = [(c["input"].encode(), c["refused_at"], c["complete"]) for c in P._golden()]
    return cases + P._deep_cases()


@pytest.mark.parametrize("data,refused_at,complete", _open_json_cases(), ids=lambda x: str(x)[:16])
def test_open_json_host(data, refused_at, complete, small_vocabs):
    """The library's table walker on the recursive-JSON pins (RFC 8259 offsets,
    the depth cap of 32)."""
    blob, off = small_vocabs[5]
    hg = cg.Grammar(W.spec_json(5), blob, off, host_only=True)
    assert hg.try_input(data) == (len(data) if refused_at is None else refused_at, complete)


@pytest.mark.parametrize("case", __import__("tests.test_open_json_pins", fromlist=["x"]).OPEN_TINY,
                         ids=lambda c: c[0] if isinstance(c, tuple) else None)
def test_open_tiny_languages_host(case):
    """Open values under tiny caps: the table walker against the exact
    prefix set of the enumerated language (every prefix with room for its
    completion, each alphabet byte appended; bytes outside the alphabet
    against the oracle)."""
    name, spec, sigma, budget, room = case
    hg = cg.Grammar(json.dumps(spec).encode(), b"a", [0, 1], host_only=True)
    og = O.load_spec(spec)
    M = langref.Enumerator(spec, sigma, budget).members()
    P = langref.prefixes(M)
    Ps = sorted(p for p in P if len(p) + 1 + room <= budget)
    if len(Ps) > 3000:
        rng = W.SplitMix(len(Ps))
        Ps = [Ps[rng.below(len(Ps))] for _ in range(3000)]
    for p in Ps:
        assert hg.try_input(p) == (len(p), p in M), p
        for b in set(sigma):
            q = p + bytes([b])
            assert (hg.try_input(q)[0] == len(q)) == (q in P), q
        for b in {0xFF, 0x20, ord("x")} - set(sigma):  # outside the alphabet: the oracle
            _agree(og, hg, p + bytes([b]))


@pytest.mark.parametrize("cfg", sorted(W.SPECS))
def test_random_walks_host(cfg, small_vocabs):
    """Random viable walks chosen by the oracle, each extended by every token
    of a 4096-token vocabulary: the host walker agrees on where each
    candidate is refused and whether it is complete."""
    blob, off = small_vocabs[cfg]
    toks = [blob[off[i]:off[i + 1]] for i in range(len(off) - 1)]
    og = O.load_spec(W.spec_json(cfg))
    hg = cg.Grammar(W.spec_json(cfg), blob, off, host_only=True)
    rng = W.SplitMix(1000 + cfg)
    for walk in range(6):
        conf = og.start()
        text = b""
        for step in range(rng.below(60) + 1):
            nb = sorted(og.next_bytes(conf))
            if not nb:
                break
            b = bytes([nb[rng.below(len(nb))]])
            og.feed(conf, b)
            text += b
        words = og.mask(conf, blob, off)
        bits = O.unpack_mask(words, len(toks))
        for t in range(0, len(toks), 3):
            k, _ = hg.try_input(text + toks[t])
            assert (k == len(text) + len(toks[t])) == bits[t], (text, toks[t])
        for t in range(0, len(toks), 97):
            _agree(og, hg, text + toks[t])


def test_generation_strings_host():
    """Long members with every construct: deep open JSON, escapes, caps."""
    import json
    og5 = O.load_spec(W.spec_json(5))
    hg5 = cg.Grammar(W.spec_json(5), b"a", [0, 1], host_only=True)
    deep = b"[" * 32 + b"]" * 32
    _agree(og5, hg5, deep)
    _agree(og5, hg5, b"[" * 33)
    _agree(og5, hg5, b'{"a":[1,-0.5e+3,true,{"b":null}],"c":"\\u00e9\\n\xf0\x9f\x98\x80"}')
    og3 = O.load_spec(W.spec_json(3))
    hg3 = cg.Grammar(W.spec_json(3), b"a", [0, 1], host_only=True)
    s = b'store_record({"key":"k","value":' + b"[" * 15 + b"]" * 15 + b',"ttl":-1})'
    _agree(og3, hg3, s)
    _agree(og3, hg3, b'store_record({"key":"k","value":' + b"[" * 16)
    _agree(og3, hg3, b'store_record({"key":"k","value":{"a":' + b"[" * 14 + b"{")
    _agree(og3, hg3, b'calendar({"action":"list","date":"d","time":"t","duration_minutes":480,"notify":true})')
    _agree(og3, hg3, b'calendar({"action":"list","date":"d","time":"t","duration_minutes":481')
    _agree(og3, hg3, b'set_timer({"seconds":86400,"label":"' + b"x" * 41)
    _agree(og3, hg3, b'read_document({"path":"a"})')
    _agree(og3, hg3, b'read_document({"path":"a","max_pages":0')


def test_grammar_cache():
    """Identical compiles share one handle; any difference in spec text,
    vocabulary or options builds a new one; idle handles stay cached up to a
    bound and cache_clear releases them."""
    import gc
    import logit_masking_amd as cg
    cg.cache_clear()
    e0, h0, m0 = cg.cache_stats()
    blob, off = W.make_vocab(2, 4096)
    spec = W.spec_json(2)
    a = cg.Grammar(spec, blob, off, host_only=True)
    b = cg.Grammar(spec, blob, off, host_only=True)
    assert a._h.value == b._h.value
    e, h, m = cg.cache_stats()
    assert (h - h0, m - m0) == (1, 1)
    c = cg.Grammar(spec, blob, off, gen_cap=100, host_only=True)      # options differ
    blob2 = bytes(blob[:-1]) + bytes([blob[-1] ^ 1])                 # one byte of the vocabulary differs
    d = cg.Grammar(spec, blob2, off, host_only=True)
    f = cg.Grammar(spec + b" ", blob, off, host_only=True)            # spec text differs
    assert len({a._h.value, c._h.value, d._h.value, f._h.value}) == 4
    assert a.try_input(b'{"eligibility"')[0] == 14
    del a
    gc.collect()
    assert b.try_input(b'{"eligibility"')[0] == 14                  # still held by b
    del b, c, d, f
    gc.collect()
    e, h, m = cg.cache_stats()
    assert e == e0 + 4                                               # all idle, all kept
    g2 = cg.Grammar(spec, blob, off, host_only=True)                 # answered from the cache
    assert cg.cache_stats()[1] == h + 1
    del g2
    gc.collect()
    # more idle grammars than the cache keeps: the oldest go
    keep = [cg.Grammar(json.dumps({"kind": "calc", "int_max": 10 + i}), blob, off, host_only=True) for i in range(12)]
    del keep
    gc.collect()
    assert cg.cache_stats()[0] <= e0 + 8
    cg.cache_clear()
    assert cg.cache_stats()[0] == e0


def test_noalloc_scratch_constant():
    """The binding's scratch size is the header's."""
    src = open(os.path.join(ROOT, "include", "cg.h")).read()
    m = re.search(r"#define CG_FILL_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == cg.FILL_NOALLOC_SCRATCH_BYTES
