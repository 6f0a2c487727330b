"""Run in a child process by tests/test_sanitizers.py with the sanitizer
runtime preloaded: the host paths of the library (spec compiler, table
walker, contract and evaluators) and the oracle's recognizer, both built
with AddressSanitizer and UBSan, driven through the page examples, tiny
languages, random walks, and mutated specs.  Any sanitizer report aborts
the process (halt_on_error); results are also checked for agreement.

usage: sanitize_run.py <sanitized libcg.so> <sanitized recognizer .so>
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import logit_masking_amd as cg  # noqa: E402
from logit_masking_amd import workloads as W  # noqa: E402
from oracle import oracle as O  # noqa: E402

cg.LIB_PATH = sys.argv[1]
O.SO_PATH = sys.argv[2]
from tests import langref  # noqa: E402
from tests.test_oracle_pins import TINY  # noqa: E402
from tests.test_open_json_pins import OPEN_TINY, _deep_cases  # noqa: E402

n = 0


def host(spec):
    return cg.Grammar(json.dumps(spec).encode() if isinstance(spec, dict) else spec, b"a", [0, 1], host_only=True)


def agree(hg, og, data):
    global n
    n += 1
    a, b = hg.try_input(data), og.try_input(data)
    assert a == b, (data, a, b)


# page examples and the recursive-JSON pins
gold = json.load(open(os.path.join(ROOT, "tests", "golden", "page_examples.json")))["cases"]
oj = json.load(open(os.path.join(ROOT, "tests", "golden", "open_json.json")))["cases"]
cases = [(c["cfg"], c["input"].encode(), c["refused_at"], c["complete"]) for c in gold]
cases += [(5, c["input"].encode(), c["refused_at"], c["complete"]) for c in oj]
cases += [(5, d, r, cpl) for d, r, cpl in _deep_cases()]
for cfg, data, ra, cpl in cases:
    hg, og = host(W.SPECS[cfg]), O.load_spec(W.spec_json(cfg))
    want = (len(data) if ra is None else ra, cpl)
    assert hg.try_input(data) == want and og.try_input(data) == want, (cfg, data)
    n += 1

# tiny languages: every prefix of the enumerated language, with each
# alphabet byte and two bytes outside it appended
for item in TINY + [t[:4] for t in OPEN_TINY]:
    name, spec, sigma, budget = item[:4]
    budget = min(budget, 11)
    hg, og = host(spec), O.load_spec(spec)
    P = sorted(langref.prefixes(langref.Enumerator(spec, sigma, budget).members()))[:1500]
    for p in P:
        for b in set(sigma) | {0xFF, 0x20}:
            agree(hg, og, p + bytes([b]))

# random walks on small vocabularies: the oracle's masks (threaded) pick
# legal tokens; every prefix of the text through both walkers
for cfg in sorted(W.SPECS):
    blob, off = W.make_vocab(cfg, 4096) if cfg != 1 else W.make_vocab(1)
    V = len(off) - 1
    toks = [blob[off[i]:off[i + 1]] for i in range(V)]
    og = O.load_spec(W.spec_json(cfg))
    hg = cg.Grammar(W.spec_json(cfg), blob, off, host_only=True)
    rng = W.SplitMix(1000 + cfg)
    for trial in range(3):
        row = O.Row(og, 300)
        for step in range(60):
            if row.done:
                break
            words, _ = og.mask_rows([row.conf], [False], blob, off, 4)
            allowed = np.nonzero(O.unpack_mask(words[0], V))[0]
            if len(allowed) == 0:
                break
            row.advance(toks[int(allowed[rng.below(len(allowed))])])
        text = bytes(row.text)
        for k in range(0, len(text) + 1, max(1, len(text) // 40)):
            agree(hg, og, text[:k])

# mutated specs: the compiler parses untrusted JSON; whatever it answers,
# no sanitizer report (the oracle's reader is Python's json module)
rng = W.SplitMix(77)
for cfg in sorted(W.SPECS):
    base = W.spec_json(cfg)
    for _ in range(150):
        s = bytearray(base)
        for _ in range(1 + rng.below(4)):
            op, i = rng.below(4), rng.below(len(s) + 1)
            if op == 0 and i < len(s):
                s[i] = rng.below(256)
            elif op == 1:
                alpha = b'{}[]":,0-9a\\'
                s[i:i] = alpha[rng.below(len(alpha)):][:1]
            elif op == 2:
                del s[i:i + 1 + rng.below(8)]
            else:
                s = s[:i]
        try:
            g = host(bytes(s))
            g.try_input(b'{"a":1}')
        except cg.CgError:
            pass
        n += 1

# contract transform and evaluators
for d in sorted(W.DESIGN_SCHEMAS) if hasattr(W, "DESIGN_SCHEMAS") else []:
    spec = W.design_spec_json(d)
    try:
        cg.contract_model_spec(spec)
    except cg.CgError:
        pass
for span in (b"<calc>17 * 23 + 91</calc>", b"<calc>1/0</calc>", b"<calc>(((1)))*9223372036854775807</calc>",
             b"<calc>", b"", b"<calc>1+</calc>"):
    cg.eval_calc(span)
for span in (b'<strop>count("strawberry", "r")</strop>', b'<strop>substr("abc", -9, 99)</strop>',
             b'<strop>upper("")</strop>', b"<strop>len(</strop>", b""):
    cg.eval_strop(span)
print("sanitized runs ok:", n, "checks")
