"""Seeded synthetic workloads for the constrained-decoding hot path.

This module is shared by the tests, the benchmark and the smoke check.  It
holds the six grammar specs, the vocabulary generators, per-row seeds and
the logits recipe -- inputs only.  It performs none of the method's
arithmetic (no automaton, no masking, no sampling).

The workloads restate the pages' settings:
  * calc span grammar ("Evaluator aware decoding", "This is a grammar
    problem"): ints 0-999, bounded whitespace, parentheses.
  * decision schema ("Guided Decoding & Structured-Output Reliability",
    "Design 1 -- base schema, validators-first ordering"), T = 0.7 and a
    400-token cap ("The ten conditions").
  * tool call ``name(args)`` ("Constrained decoding", "Where it arms, and
    therefore where it stops" / "Reading the grammar for a tool"), with the
    whitespace bound, the open-field cap and the 2048 engine cap ("A valid
    call also has to end"), 256-token bench runs ("What it is worth").
  * integer-answer contract ("Constrained Decoding Under Matched Conditions",
    "The system boundary I am testing"), compact separators ("What the audit
    found"), greedy decoding ("The protocol was frozen before the cloud run").
  * a recursive-JSON stress grammar capped at 2048 tokens.
  * text with evaluated calc spans ("Evaluator aware decoding", "A concrete
    prototype on llama.cpp"): the model writes prose and <calc> spans, the
    engine writes <result> / <result_error> blocks; and the same with
    string-operation spans too ("Not just arithmetic: string operations").

Random numbers come from splitmix64 written in plain Python so that every
vocabulary is byte-identical across numpy versions.
"""
from __future__ import annotations

import functools
import hashlib
import json
import math

MASK64 = (1 << 64) - 1


def splitmix64(x: int) -> int:
    """One splitmix64 output for state ``x`` (Steele, Lea, Flood, OOPSLA'14)."""
    z = (x + 0x9E3779B97F4A7C15) & MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


class SplitMix:
    """Counter-mode splitmix64 stream: output k is splitmix64(seed + k*golden)."""

    def __init__(self, seed: int):
        self.state = seed & MASK64

    def next(self) -> int:
        self.state = (self.state + 0x9E3779B97F4A7C15) & MASK64
        z = self.state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
        return z ^ (z >> 31)

    def uniform(self) -> float:
        """Uniform double in [0, 1) from the top 53 bits."""
        return (self.next() >> 11) * (1.0 / (1 << 53))

    def below(self, n: int) -> int:
        return self.next() % n

    def choice(self, seq):
        return seq[self.below(len(seq))]

    def poisson(self, lam: float) -> int:
        """Knuth's multiplicative Poisson sampler (small lambda)."""
        L = math.exp(-lam)
        k, p = 0, 1.0
        while True:
            p *= self.uniform()
            if p <= L:
                return k
            k += 1


# ---------------------------------------------------------------------------
# Grammar specs (the input format of cg_compile_grammar).
# ---------------------------------------------------------------------------

def _obj(props, required=None):
    """A closed JSON-Schema object: declared order, no extra keys."""
    return {
        "type": "object",
        "properties": dict(props),
        "required": list(required if required is not None else [k for k, _ in props]),
        "additionalProperties": False,
    }


STR = {"type": "string"}


def _strn(n):
    return {"type": "string", "maxLength": n}


def _int(lo, hi):
    return {"type": "integer", "minimum": lo, "maximum": hi}


def _enum(*vals):
    return {"type": "string", "enum": list(vals)}


BOOL = {"type": "boolean"}

# Decision schema of design 1; the elided eligibility/appointment bodies are
# read as fully required closed objects, appointment = {date<=20, time<=10}.
DECISION_SCHEMA = _obj([
    ("eligibility", _obj([
        ("criteria_met", BOOL),
        ("reason_code", _enum("eligible", "under_age", "over_limit", "insufficient_info")),
    ])),
    ("action", _enum("book_appointment", "decline", "offer_alternative", "escalate_human")),
    ("appointment", {"anyOf": [_obj([("date", _strn(20)), ("time", _strn(10))]), {"type": "null"}]}),
    ("response_text", _strn(700)),
])

# Designs 2-5 of the same page ("Designs 2-4 -- making the schema show its
# working", "Design 5 -- the pipeline"): fields ahead of the decision, or an
# extraction schema with no decision at all.  "..." on the page is read as
# the rest of design 1's object.
_DECISION_PROPS = list(DECISION_SCHEMA["properties"].items())
DESIGN_SCHEMAS = {
    2: _obj([("calculation", _strn(400)),
             ("within_limit_banding", _enum("within_limit", "reduced_scope_band", "over_limit"))] + _DECISION_PROPS),
    3: _obj([("exceeds_value_limit", BOOL),
             ("over_limit_tier", {"anyOf": [_enum("reduced_scope", "hard_decline"), {"type": "null"}]})]
            + _DECISION_PROPS),
    4: _obj([("customer_age", {"type": "integer"}), ("age_within_18_to_70", BOOL),
             ("total_requested_value", {"type": "number"}), ("total_at_most_10000", BOOL),
             ("total_at_most_12000", BOOL)] + _DECISION_PROPS),
    5: _obj([("customer_age", {"anyOf": [{"type": "integer"}, {"type": "null"}]}),
             ("price_components", {"type": "array", "items": {"type": "number"}, "maxItems": 10}),
             ("requested_date", {"anyOf": [_strn(20), {"type": "null"}]}),
             ("requested_time", {"anyOf": [_strn(10), {"type": "null"}]})]),
}


def design_spec_json(design: int) -> bytes:
    return json.dumps({"kind": "json_schema", "ws_max": 4, "open_string_cap": 256, "depth_cap": 32,
                       "schema": DESIGN_SCHEMAS[design]}, separators=(",", ":")).encode()


# Eight tools with 1-5 typed arguments; ``?`` marks an optional argument.
TOOLS = [
    ("calculate", [("expression", STR)]),
    ("read_document", [("path", STR), ("max_pages?", _int(1, 500))]),
    ("calendar", [("action", _enum("create", "list", "delete")), ("date", _strn(20)),
                  ("time", _strn(10)), ("duration_minutes", _int(5, 480)), ("notify?", BOOL)]),
    ("send_email", [("to", STR), ("subject", _strn(100)), ("body", STR),
                    ("priority", _enum("low", "normal", "high"))]),
    ("get_weather", [("city", STR), ("units", _enum("celsius", "fahrenheit"))]),
    ("set_timer", [("seconds", _int(1, 86400)), ("label?", _strn(40))]),
    ("search_web", [("query", STR), ("top_k", _int(1, 20)), ("safe", BOOL)]),
    ("store_record", [("key", _strn(64)), ("value", {}), ("ttl", _int(-1, 1000000))]),
]


def _tool(name, args):
    props = [(k.rstrip("?"), v) for k, v in args]
    req = [k for k, _ in args if not k.endswith("?")]
    return {"name": name, "parameters": _obj(props, req)}


SPECS = {
    1: {"kind": "calc", "int_min": 0, "int_max": 999, "ws_max": 2, "depth_cap": 16},
    2: {"kind": "json_schema", "ws_max": 4, "open_string_cap": 256, "depth_cap": 32,
        "schema": DECISION_SCHEMA},
    3: {"kind": "tool_call", "ws_max": 4, "open_string_cap": 256, "depth_cap": 16,
        "tools": [_tool(n, a) for n, a in TOOLS]},
    4: {"kind": "json_schema", "ws_max": 0, "open_string_cap": 256, "open_int_digits": 20,
        "depth_cap": 16,
        "schema": _obj([("reasoning", _strn(2000)), ("answer", {"type": "integer"})])},
    5: {"kind": "json_schema", "ws_max": 4, "open_string_cap": None, "depth_cap": 32,
        "schema": {"anyOf": [{"type": "object"}, {"type": "array"}]}},
    6: {"kind": "calc_text", "int_min": 0, "int_max": 999, "ws_max": 2, "depth_cap": 16},
    7: {"kind": "calc_text", "evaluators": ["calc", "strop"], "int_min": 0, "int_max": 999, "ws_max": 2,
        "depth_cap": 16},
}


def spec_json(cfg: int) -> bytes:
    return json.dumps(SPECS[cfg], separators=(",", ":")).encode()


# ---------------------------------------------------------------------------
# Workload table.
# ---------------------------------------------------------------------------

CONFIGS = {
    1: dict(name="calc-span", B=4, V=512, dtype="f32", logits="normal", sigma=1.0,
            T=0.0, steps=1, maxlen=6, seed=0xC0F1),
    2: dict(name="decision-schema", B=64, V=32000, dtype="f32", logits="normal", sigma=2.0,
            T=0.7, steps=400, maxlen=16, mean=6.0, seed=0xC0F2),
    3: dict(name="tool-call", B=256, V=128256, dtype="bf16", logits="normal", sigma=3.0,
            T=0.7, steps=256, maxlen=24, mean=6.0, seed=0xC0F3),
    4: dict(name="integer-answer", B=1024, V=151936, dtype="bf16", logits="normal", sigma=1.0,
            T=0.0, steps=400, maxlen=24, mean=6.0, seed=0xC0F4),
    5: dict(name="stress-json", B=512, V=256000, dtype="bf16", logits="student_t3", sigma=1.0,
            T=1.0, steps=2048, maxlen=32, mean=7.0, seed=0xC0F5),
    6: dict(name="calc-text", B=256, V=128256, dtype="bf16", logits="normal", sigma=3.0,
            T=0.7, steps=256, maxlen=16, mean=5.0, seed=0xC0F6),
    7: dict(name="eval-text", B=256, V=128256, dtype="bf16", logits="normal", sigma=3.0,
            T=0.7, steps=256, maxlen=16, mean=5.0, seed=0xC0F7),
}

GEN_CAP = 2048  # engine cap on one constrained generation, in tokens


def row_seeds(cfg: int, B: int | None = None):
    """Per-request seeds: seed_r = splitmix64(seed_c xor r)."""
    c = CONFIGS[cfg]
    n = c["B"] if B is None else B
    return [splitmix64(c["seed"] ^ r) for r in range(n)]


# ---------------------------------------------------------------------------
# Vocabularies: ids 0-255 are the single bytes; the rest are unique strings.
# ---------------------------------------------------------------------------

_CALC_ALPHA = b"0123456789+-*/() <>/calc"
_PRINTABLE = bytes(range(0x20, 0x7F))

_GLUE = ['{"', '":', '","', '"}', '": "', '", "', '":{"', '"},"', '},{', '[{', '}]',
         '":[', '],"', ', ', ': ', '{}', '[]', 'true', 'false', 'null', '\\n', '\\"',
         '\\u00e9', '"', ',', ':', '{', '}', '[', ']', ' ', '\n', '\t']

_FRAGS = {
    2: ["eligibility", "criteria_met", "reason_code", "eligible", "under_age", "over_limit",
        "insufficient_info", "action", "book_appointment", "decline", "offer_alternative",
        "escalate_human", "appointment", "date", "time", "response_text"],
    3: ["calculate", "expression", "read_document", "path", "max_pages", "calendar", "action",
        "create", "list", "delete", "date", "time", "duration_minutes", "notify", "send_email",
        "to", "subject", "body", "priority", "low", "normal", "high", "get_weather", "city",
        "units", "celsius", "fahrenheit", "set_timer", "seconds", "label", "search_web",
        "query", "top_k", "safe", "store_record", "key", "value", "ttl", "({\"", "\"})", "})",
        "(", ")"],
    4: ["reasoning", "answer", '{"reasoning":"', '","answer":', "-", "}", "total", "sum",
        "each", "so", "the"],
    5: ["id", "name", "items", "type", "value", "data", "list", "key", "x", "y", "e", "E", ".",
        "-", "+", "0.5", "1e9", "-3", "1.25e-3"],
}

_TEXT_FRAGS = ["<calc>", "</calc>", "<result>", "</result>", "<result_error>", "</result_error>", "<end>",
               "<", ">", "</", "calc", "result", " + ", " - ", " * ", " / ", "+", "-", "*", "/", "(", ")",
               " (", ") ", " = ", "=", " is", " the", " answer", " total", ".", ",", "\n", " "]

_STROP_FRAGS = ["<strop>", "</strop>", "count(", "len(", "reverse(", "upper(", "substr(", '"', '", "', '")',
                '", ', ", ", ")</strop>", "(", ")", "strawberry", "r", "hello", "abc"]
_CALC_BYTES = b"0123456789+-*/() "
_TEXT_PUNCT = b".,;:!?'\"\n\t <>"
_LETTERS = b"abcdefghijklmnopqrstuvwxyz"
_UTF8_RANGES = [(0xA0, 0x24F), (0x370, 0x3FF), (0x400, 0x4FF), (0x4E00, 0x9FFF),
                (0x1F300, 0x1F64F), (0xAC00, 0xD7A3)]


def _utf8_piece(rng: SplitMix) -> bytes:
    lo, hi = _UTF8_RANGES[rng.below(len(_UTF8_RANGES))]
    return chr(lo + rng.below(hi - lo + 1)).encode("utf-8")


def _gen_text_token(rng: SplitMix, L: int, strop: bool = False) -> bytes:
    """One candidate token of exactly L bytes for text with evaluated spans."""
    u = rng.uniform()
    out = bytearray()
    if u < 0.30:  # tags, operators and glue
        frags = _TEXT_FRAGS + _STROP_FRAGS if strop else _TEXT_FRAGS
        while len(out) < L:
            piece = rng.choice(frags).encode()
            if not out and len(piece) > 1 and rng.uniform() < 0.4:
                piece = piece[rng.below(len(piece)):]
            out += piece
    elif u < 0.65:  # words, usually with a leading space
        if rng.uniform() < 0.7:
            out += b" "
        while len(out) < L:
            out.append(_LETTERS[rng.below(26)])
    elif u < 0.85:  # digits, operators, spaces, parentheses
        while len(out) < L:
            out.append(_CALC_BYTES[rng.below(len(_CALC_BYTES))] if rng.uniform() < 0.7 else 0x30 + rng.below(10))
    elif u < 0.95:  # punctuation and whitespace
        while len(out) < L:
            out.append(_TEXT_PUNCT[rng.below(len(_TEXT_PUNCT))])
    else:  # raw bytes
        while len(out) < L:
            out.append(rng.below(256))
    return bytes(out[:L])


def _gen_token(rng: SplitMix, cfg: int, L: int) -> bytes:
    """One candidate token of exactly L bytes (configs 2-5)."""
    u = rng.uniform()
    out = bytearray()
    if u < 0.30:  # schema / JSON fragments with glue
        pool = _FRAGS[cfg] + _GLUE
        while len(out) < L:
            piece = rng.choice(pool).encode()
            if not out and len(piece) > 1 and rng.uniform() < 0.5:
                piece = piece[rng.below(len(piece)):]
            out += piece
    elif u < 0.65:  # words, usually with a leading space
        if rng.uniform() < 0.7:
            out += b" "
        while len(out) < L:
            c = _LETTERS[rng.below(26)]
            if not out.strip() and rng.uniform() < 0.2:
                c = ord(chr(c).upper())
            out.append(c)
    elif u < 0.75:  # numbers
        if rng.uniform() < 0.2:
            out += b"-"
        while len(out) < L:
            r = rng.uniform()
            out += b"0123456789"[rng.below(10):][:1] if r < 0.85 else rng.choice([b".", b"e", b"E", b"-", b"+"])
    elif u < 0.85:  # punctuation and whitespace mixes
        while len(out) < L:
            out += rng.choice([b"{", b"}", b"[", b"]", b'"', b":", b",", b".", b" ", b"\n", b"\t",
                               b"\\", b"(", b")", b"'", b"!", b"?", b"/"])
    elif u < 0.95:  # multi-byte UTF-8, sometimes cut mid-character
        while len(out) < L:
            out += _utf8_piece(rng)
        if rng.uniform() < 0.2:
            return bytes(out[:L])
        # keep whole characters where possible
        cut = bytes(out[:L])
        return cut
    else:  # raw bytes
        while len(out) < L:
            out.append(rng.below(256))
    return bytes(out[:L])


@functools.lru_cache(maxsize=8)
def make_vocab(cfg: int, V: int | None = None):
    """Return (blob: bytes, offsets: list[int]) for the config's vocabulary.

    Ids 0-255 are the single bytes 0x00-0xFF (byte fallback); ids >= 256 are
    distinct strings of 2..maxlen bytes with lengths 2 + Poisson(mean - 2).
    """
    c = CONFIGS[cfg]
    V = c["V"] if V is None else V
    rng = SplitMix(c["seed"] * 0x100000001B3)
    toks = [bytes([i]) for i in range(min(256, V))]
    seen = set(toks)
    while len(toks) < V:
        if cfg == 1:
            L = 2 + rng.below(5)
            t = bytes((_CALC_ALPHA[rng.below(len(_CALC_ALPHA))] if rng.uniform() < 0.8
                       else _PRINTABLE[rng.below(len(_PRINTABLE))]) for _ in range(L))
        elif cfg in (6, 7):
            L = min(c["maxlen"], 2 + rng.poisson(c["mean"] - 2.0))
            t = _gen_text_token(rng, L, strop=cfg == 7)
        else:
            L = min(c["maxlen"], 2 + rng.poisson(c["mean"] - 2.0))
            t = _gen_token(rng, cfg, L)
        if len(t) < 2 or t in seen:
            continue
        seen.add(t)
        toks.append(t)
    offsets = [0]
    for t in toks:
        offsets.append(offsets[-1] + len(t))
    return b"".join(toks), offsets


def vocab_tokens(cfg: int, V: int | None = None):
    blob, off = make_vocab(cfg, V)
    return [blob[off[i]:off[i + 1]] for i in range(len(off) - 1)]


def vocab_sha256(cfg: int) -> str:
    blob, off = make_vocab(cfg)
    h = hashlib.sha256(blob)
    h.update(b"".join(o.to_bytes(4, "little") for o in off))
    return h.hexdigest()


# ---------------------------------------------------------------------------
# Logits (device-side, untimed).  torch is imported lazily.
# ---------------------------------------------------------------------------

def logits_seed(cfg: int, step: int) -> int:
    return CONFIGS[cfg]["seed"] * 1_000_003 + step


def make_logits(cfg: int, step: int, B: int, V: int, device, row_stride: int | None = None):
    """Seeded logits for one step: N(0, sigma^2), or Student-t with 3 degrees
    of freedom as z / sqrt(chi2_3 / 3), cast to the config's dtype."""
    import torch
    c = CONFIGS[cfg]
    g = torch.Generator(device=device)
    g.manual_seed(logits_seed(cfg, step))
    stride = V if row_stride is None else row_stride
    if c["logits"] == "normal":
        x = torch.randn((B, stride), generator=g, device=device, dtype=torch.float32) * c["sigma"]
    else:
        z = torch.randn((B, stride), generator=g, device=device, dtype=torch.float32)
        chi = torch.randn((3, B, stride), generator=g, device=device, dtype=torch.float32)
        x = z / torch.sqrt((chi * chi).sum(0) / 3.0) * c["sigma"]
    dt = torch.bfloat16 if c["dtype"] == "bf16" else torch.float32
    return x.to(dt)


# ---------------------------------------------------------------------------
# Scripts for text with calc spans: what a row's model writes, segment by
# segment.  Each segment but the last ends with a closed <calc> span (the
# engine writes the result after it); the last ends with "<end>".  Inputs
# only: nothing here evaluates a span.
# ---------------------------------------------------------------------------
_PROSE_WORDS = [b"the", b"total", b"is", b"so", b"we", b"get", b"then", b"each", b"and", b"of", b"price",
                b"items", b"sum", b"answer", b"left", b"per", b"box"]


def calc_expr(rng: SplitMix, spec, depth: int = 0, budget: int = 6) -> bytes:
    """A random expression of the calc span grammar of `spec` (ints within
    [int_min, int_max], + - * /, parentheses under depth_cap, whitespace
    runs within ws_max).  Sometimes divides by zero or multiplies large
    numbers so that evaluation fails."""
    lo, hi = spec.get("int_min", 0), spec.get("int_max", 999)
    wsm, dcap = spec.get("ws_max", 4), spec.get("depth_cap", 16)

    def ws():
        return b" " * rng.below(wsm + 1) if wsm else b""

    def term(d, budget):
        if d < dcap and budget > 1 and rng.uniform() < 0.2:
            return b"(" + ws() + expr(d + 1, budget - 1) + ws() + b")"
        r = rng.uniform()
        v = lo if r < 0.08 else hi if r < 0.2 else lo + rng.below(hi - lo + 1)
        return str(v).encode()

    def expr(d, budget):
        out = term(d, budget)
        n = rng.below(max(1, min(4, budget)))
        for _ in range(n):
            out += ws() + bytes([b"+-*/"[rng.below(4)]]) + ws() + term(d, budget - n)
        return out

    return expr(depth, budget)


_STROP_WORDS = ["strawberry", "r", "hello world", "abc", "", "banana", "an", "racecar", "Mixed Case 12"]


def strop_call(rng: SplitMix, spec) -> bytes:
    """A random string-operation span body: NAME(ARGS) with whitespace runs
    within ws_max after the commas."""
    wsm = spec.get("ws_max", 4)

    def ws():
        return b" " * rng.below(wsm + 1) if wsm else b""

    def s():
        return b'"' + rng.choice(_STROP_WORDS).encode() + b'"'

    def i():
        return str(rng.below(25) - 8).encode()

    k = rng.below(5)
    if k == 0:
        return b"count(" + s() + b"," + ws() + s() + b")"
    if k == 4:
        return b"substr(" + s() + b"," + ws() + i() + b"," + ws() + i() + b")"
    return (b"len(", b"reverse(", b"upper(")[k - 1] + s() + b")"


def calc_text_script(rng: SplitMix, spec, n_spans: int) -> list:
    """Model segments of one row: prose, then a closed span ("<calc>" EXPR
    "</calc>", or "<strop>" CALL "</strop>" when the spec has that
    evaluator), n_spans times, then prose and "<end>"."""
    def prose():
        words = [rng.choice(_PROSE_WORDS) for _ in range(rng.below(6))]
        text = b" ".join(words)
        if text and rng.uniform() < 0.3:
            text += b"\n"
        return text + (b" " if text else b"")

    segs = []
    strop = "strop" in spec.get("evaluators", ["calc"])
    for _ in range(n_spans):
        if strop and rng.uniform() < 0.5:
            segs.append(prose() + b"<strop>" + strop_call(rng, spec) + b"</strop>")
            continue
        w = spec.get("ws_max", 4)
        lead = b" " * rng.below(w + 1) if w else b""
        tail = b" " * rng.below(w + 1) if w else b""
        segs.append(prose() + b"<calc>" + lead + calc_expr(rng, spec) + tail + b"</calc>")
    segs.append(prose() + b"<end>")
    return segs


class ScriptTokens:
    """The vocabulary token that spells the next bytes of a script: the
    longest token that is a prefix of the remaining bytes (how the scripted
    runs lean the logits toward a row's script; an input recipe, not a
    tokenizer of the method)."""

    def __init__(self, toks):
        self.by = {t: i for i, t in enumerate(toks)}
        self.maxlen = max(len(t) for t in toks)

    def longest(self, rest: bytes, rng: SplitMix | None = None) -> int:
        cands = [self.by[rest[:k]] for k in range(1, min(len(rest), self.maxlen) + 1) if rest[:k] in self.by]
        if rng is not None and len(cands) > 1 and rng.uniform() < 0.3:
            return cands[rng.below(len(cands))]
        return cands[-1]

    def count(self, data: bytes) -> int:
        """Tokens of a greedy longest-match spelling of `data`."""
        n = pos = 0
        while pos < len(data):
            pos += len(self.longest_bytes(data[pos:]))
            n += 1
        return n

    def longest_bytes(self, rest: bytes) -> bytes:
        for k in range(min(len(rest), self.maxlen), 0, -1):
            if rest[:k] in self.by:
                return rest[:k]
        raise ValueError("byte not in the vocabulary")
