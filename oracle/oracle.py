"""The oracle -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct CPU implementation of the constrained
decoding step, used only by tests/, the smoke check and the benchmark's
CPU-baseline leg.  The product path (the HIP library and its binding) never
imports, links or runs anything from this directory, and this module imports
nothing from the product package.

Parts:
  * load_spec(): reads a grammar spec (calc span, JSON schema or tool call)
    with Python's json module into a schema tree interpreted by the C
    recognizer in recognizer.c (frame stack, no tables).
  * masks: bit t of a row is set iff the row is not finished and its bytes so
    far followed by the bytes of token t are a viable prefix of the grammar's
    language -- "a pushdown automaton masks the logits at every step"
    (page "Constrained decoding", section "The guarantee").
  * sampling after masking ("Sampling runs after masking", same section), in
    float64: greedy argmax with lowest-id ties, or two-level Gumbel-max over
    2048-id chunks driven by Philox4x32-10 (Salmon, Moraes, Dror, Shaw,
    "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11).
  * advance: append the chosen token's bytes; a forced token is a transition
    the model did not choose (page "Evaluator aware decoding", section "A
    concrete prototype on llama.cpp"); the engine caps one constrained
    generation at gen_cap tokens (page "Constrained decoding", section "A
    valid call also has to end").
  * eval_calc(): the calc-span evaluator (page "Evaluator aware decoding",
    section "The core idea").
"""
from __future__ import annotations

import ctypes
import json
import math
import os
import re
import subprocess
import threading
from fractions import Fraction

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SO_PATH = os.path.join(HERE, "_recognizer.so")
SRC_PATH = os.path.join(HERE, "recognizer.c")


def build(force: bool = False) -> str:
    """Compile recognizer.c with gcc (plain C11, -O2)."""
    if force or not os.path.exists(SO_PATH) or os.path.getmtime(SO_PATH) < os.path.getmtime(SRC_PATH):
        tmp = SO_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-std=gnu11", "-O2", "-Wall", "-shared", "-fPIC", "-o", tmp, SRC_PATH,
                               "-lpthread"])
        os.replace(tmp, SO_PATH)
    return SO_PATH


_lib = None
_lib_lock = threading.Lock()


class ONode(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("first", ctypes.c_int32), ("count", ctypes.c_int32),
                ("cap", ctypes.c_int32), ("open", ctypes.c_int32), ("item", ctypes.c_int32),
                ("any_kinds", ctypes.c_int32), ("maxdigits", ctypes.c_int32),
                ("lo", ctypes.c_int64), ("hi", ctypes.c_int64),
                ("has_lo", ctypes.c_int32), ("has_hi", ctypes.c_int32)]


class OProp(ctypes.Structure):
    _fields_ = [("lit_off", ctypes.c_int32), ("lit_len", ctypes.c_int32), ("node", ctypes.c_int32),
                ("required", ctypes.c_int32)]


class OG(ctypes.Structure):
    _fields_ = [("gkind", ctypes.c_int32), ("root", ctypes.c_int32), ("tools_first", ctypes.c_int32),
                ("tools_count", ctypes.c_int32), ("ws_max", ctypes.c_int32), ("depth_cap", ctypes.c_int32),
                ("open_cap", ctypes.c_int32), ("calc_min", ctypes.c_int32), ("calc_max", ctypes.c_int32),
                ("open_obj", ctypes.c_int32), ("open_arr", ctypes.c_int32),
                ("nodes", ctypes.POINTER(ONode)), ("props", ctypes.POINTER(OProp)),
                ("pool", ctypes.POINTER(ctypes.c_uint8)), ("evaluators", ctypes.c_int32)]


def lib():
    global _lib
    with _lib_lock:
        if _lib is None:
            build()
            L = ctypes.CDLL(SO_PATH)
            vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
            L.oc_size.restype = ctypes.c_int
            L.oc_start.argtypes = [vp, vp]
            L.oc_feed.argtypes = [vp, vp, vp, i32]
            L.oc_feed.restype = ctypes.c_int
            L.oc_feed_model.argtypes = [vp, vp, vp, i32]
            L.oc_feed_model.restype = ctypes.c_int
            L.oc_in_engine.argtypes = [vp, vp]
            L.oc_in_engine.restype = ctypes.c_int
            L.oc_complete.argtypes = [vp, vp]
            L.oc_complete.restype = ctypes.c_int
            L.oc_mask.argtypes = [vp, vp, vp, vp, i32, vp]
            L.oc_mask.restype = i64
            L.oc_mask_rows.argtypes = [vp, vp, vp, i32, vp, vp, i32, vp, i32]
            L.oc_mask_rows.restype = i64
            L.oc_next_bytes.argtypes = [vp, vp, vp]
            L.og_sat.argtypes = [vp, i32, i32]
            L.og_sat.restype = ctypes.c_int
            _lib = L
    return _lib


# ---------------------------------------------------------------------------
# Spec reading
# ---------------------------------------------------------------------------
K_OBJ, K_ARR, K_STR, K_INT, K_NUM, K_BOOL, K_NULL, K_ENUM, K_ANYOF, K_ANY, K_INTSTR = range(1, 12)
# The one string pattern read: a canonical signed decimal integer (the external
# side of the integer-string contract, page "Constrained Decoding Under Matched
# Conditions", section "The system boundary I am testing").
INT_STRING_PATTERN = "^-?(0|[1-9][0-9]*)$"
G_CALC, G_JSON, G_TOOL, G_TEXT = 1, 2, 3, 4
AK_ALL = 31

# Defaults of a spec that leaves a setting out.
DEFAULTS = dict(ws_max=4, open_string_cap=256, open_int_digits=20, depth_cap=16, int_min=0, int_max=999)

_ANNOTATIONS = {"title", "description", "$comment", "examples", "default"}


class Unsupported(ValueError):
    """A construct outside the supported subset (refused, fail closed)."""

    def __init__(self, path, msg):
        super().__init__(f"{path}: {msg}")
        self.path = path


def json_spelling(s: str) -> bytes:
    """The one accepted spelling of a key or enum value: a JSON string with
    only the escapes JSON requires (quote, backslash, control characters;
    \\b \\f \\n \\r \\t short forms, other controls as lowercase \\u00XX)."""
    out = ['"']
    short = {'"': '\\"', '\\': '\\\\', '\b': '\\b', '\f': '\\f', '\n': '\\n', '\r': '\\r', '\t': '\\t'}
    for ch in s:
        if ch in short:
            out.append(short[ch])
        elif ord(ch) < 0x20:
            out.append('\\u%04x' % ord(ch))
        else:
            out.append(ch)
    out.append('"')
    try:
        return "".join(out).encode("utf-8")
    except UnicodeEncodeError:
        raise Unsupported("$", "string with a lone surrogate")


def _first_classes(node, nodes, props):
    """Conservative set of first-byte classes of a node (the LL(1) rule of
    anyOf): '{', '[', '"', 'num' (minus or digit), 't', 'f', 'n'."""
    n = nodes[node]
    k = n["kind"]
    if k == K_OBJ:
        return {"{"}
    if k == K_ARR:
        return {"["}
    if k in (K_STR, K_ENUM, K_INTSTR):
        return {'"'}
    if k in (K_INT, K_NUM):
        return {"num"}
    if k == K_BOOL:
        return {"t", "f"}
    if k == K_NULL:
        return {"n"}
    if k == K_ANY:
        return {"{", "[", '"', "num", "t", "f", "n"}
    s = set()
    for i in range(n["count"]):
        s |= _first_classes(props[n["first"] + i]["node"], nodes, props)
    return s


class _Builder:
    def __init__(self, settings):
        self.nodes = []
        self.props = []
        self.pool = bytearray()
        self.s = settings

    def lit(self, b: bytes):
        off = len(self.pool)
        self.pool += b
        return off, len(b)

    def add(self, **kw):
        d = dict(kind=0, first=0, count=0, cap=-1, open=0, item=-1, any_kinds=0, maxdigits=0, lo=0, hi=0,
                 has_lo=0, has_hi=0)
        d.update(kw)
        self.nodes.append(d)
        return len(self.nodes) - 1

    def add_props(self, entries):
        first = len(self.props)
        self.props.extend(entries)
        return first

    def schema(self, sch, path, depth):
        if not isinstance(sch, dict):
            raise Unsupported(path, "schema must be an object")
        keys = set(sch) - _ANNOTATIONS
        if not keys:
            return self.add(kind=K_ANY, any_kinds=AK_ALL)
        if "anyOf" in keys:
            if keys != {"anyOf"}:
                raise Unsupported(path, "anyOf mixed with other keywords")
            alts = sch["anyOf"]
            if not isinstance(alts, list) or not alts:
                raise Unsupported(path, "anyOf must be a non-empty list")
            kids = [self.schema(a, f"{path}/anyOf/{i}", depth) for i, a in enumerate(alts)]
            seen = set()
            for kid in kids:
                fc = _first_classes(kid, self.nodes, self.props)
                if fc & seen:
                    raise Unsupported(path, "anyOf alternatives share a first byte")
                seen |= fc
            first = self.add_props([dict(lit_off=0, lit_len=0, node=k, required=0) for k in kids])
            return self.add(kind=K_ANYOF, first=first, count=len(kids))
        if "enum" in keys:
            if not keys <= {"enum", "type"} or sch.get("type", "string") != "string":
                raise Unsupported(path, "only plain string enums are supported")
            vals = sch["enum"]
            if not isinstance(vals, list) or not vals or not all(isinstance(v, str) for v in vals):
                raise Unsupported(path, "enum must list strings")
            if len(set(vals)) != len(vals) or len(vals) > 64:
                raise Unsupported(path, "enum values must be distinct (at most 64)")
            ents = []
            for v in vals:
                off, ln = self.lit(json_spelling(v))
                ents.append(dict(lit_off=off, lit_len=ln, node=-1, required=0))
            first = self.add_props(ents)
            return self.add(kind=K_ENUM, first=first, count=len(vals))
        t = sch.get("type")
        if not isinstance(t, str):
            raise Unsupported(path, "missing or non-string type")
        if t == "object":
            if not keys <= {"type", "properties", "required", "additionalProperties"}:
                raise Unsupported(path, f"unsupported keywords {sorted(keys - {'type', 'properties', 'required', 'additionalProperties'})}")
            props = sch.get("properties")
            addl = sch.get("additionalProperties", True)
            req = sch.get("required", [])
            if props is None:
                if req:
                    raise Unsupported(path, "required without properties")
                if addl is True:
                    return self.add(kind=K_OBJ, open=1)
                if addl is False:
                    return self.add(kind=K_OBJ, open=0, count=0)
                raise Unsupported(path, "additionalProperties must be a boolean")
            if addl is not False:
                raise Unsupported(path, "properties need additionalProperties: false")
            if not isinstance(props, dict) or len(props) > 64:
                raise Unsupported(path, "properties must be an object of at most 64 keys")
            if not isinstance(req, list) or len(set(req)) != len(req) or any(r not in props for r in req):
                raise Unsupported(path, "required must list distinct declared properties")
            ents = []
            for k, v in props.items():
                kid = self.schema(v, f"{path}/properties/{k}", depth + 1)
                off, ln = self.lit(json_spelling(k))
                ents.append(dict(lit_off=off, lit_len=ln, node=kid, required=int(k in req)))
            first = self.add_props(ents)
            return self.add(kind=K_OBJ, first=first, count=len(ents))
        if t == "array":
            if not keys <= {"type", "items", "maxItems"}:
                raise Unsupported(path, f"unsupported keywords {sorted(keys - {'type', 'items', 'maxItems'})}")
            mi = sch.get("maxItems", -1)  # absent: no bound
            if "maxItems" in sch and (not isinstance(mi, int) or isinstance(mi, bool) or mi < 0):
                raise Unsupported(path, "maxItems must be a non-negative integer")
            if "items" in sch:
                item = self.schema(sch["items"], f"{path}/items", depth + 1)
                return self.add(kind=K_ARR, item=item, cap=mi)
            return self.add(kind=K_ARR, open=1, cap=mi)
        if t == "string" and "pattern" in sch:
            if not keys <= {"type", "pattern"}:
                raise Unsupported(path, f"unsupported keywords {sorted(keys - {'type', 'pattern'})}")
            if sch["pattern"] != INT_STRING_PATTERN:
                raise Unsupported(path, "the only pattern supported is the canonical signed integer")
            return self.add(kind=K_INTSTR, maxdigits=self.s["open_int_digits"])
        if t == "string":
            if not keys <= {"type", "maxLength"}:
                raise Unsupported(path, f"unsupported keywords {sorted(keys - {'type', 'maxLength'})}")
            if "maxLength" in sch:
                ml = sch["maxLength"]
                if not isinstance(ml, int) or isinstance(ml, bool) or ml < 0:
                    raise Unsupported(path, "maxLength must be a non-negative integer")
                return self.add(kind=K_STR, cap=ml)
            return self.add(kind=K_STR, cap=self.s["open_cap"])
        if t == "integer":
            if not keys <= {"type", "minimum", "maximum"}:
                raise Unsupported(path, f"unsupported keywords {sorted(keys - {'type', 'minimum', 'maximum'})}")
            lo, hi = sch.get("minimum"), sch.get("maximum")
            for b in (lo, hi):
                if b is not None and (not isinstance(b, int) or isinstance(b, bool) or not -(1 << 63) <= b < (1 << 63)):
                    raise Unsupported(path, "integer bounds must be 64-bit integers")
            if lo is not None and hi is not None and lo > hi:
                raise Unsupported(path, "empty integer range")
            both = lo is not None and hi is not None
            return self.add(kind=K_INT, maxdigits=19 if both else self.s["open_int_digits"],
                            lo=lo or 0, hi=hi or 0, has_lo=int(lo is not None), has_hi=int(hi is not None))
        if keys != {"type"}:
            raise Unsupported(path, f"unsupported keywords {sorted(keys - {'type'})}")
        if t == "number":
            return self.add(kind=K_NUM)
        if t == "boolean":
            return self.add(kind=K_BOOL)
        if t == "null":
            return self.add(kind=K_NULL)
        raise Unsupported(path, f"unknown type {t!r}")


def _setting(spec, name, lo, hi, allow_none=False):
    v = spec.get(name, DEFAULTS.get(name))
    if v is None and allow_none:
        return -1
    if not isinstance(v, int) or isinstance(v, bool) or not lo <= v <= hi:
        raise Unsupported("$", f"{name} out of range")
    return v


class Grammar:
    """A loaded spec: the schema tree the recognizer interprets."""

    def __init__(self, spec):
        if isinstance(spec, (bytes, str)):
            spec = json.loads(spec)
        self.spec = spec
        kind = spec.get("kind")
        s = dict(ws_max=_setting(spec, "ws_max", 0, 64), depth_cap=_setting(spec, "depth_cap", 1, 64),
                 open_cap=_setting(spec, "open_string_cap", 0, (1 << 24), allow_none=True),
                 open_int_digits=_setting(spec, "open_int_digits", 1, 20))
        b = _Builder(s)
        og = OG()
        og.ws_max, og.depth_cap, og.open_cap = s["ws_max"], s["depth_cap"], s["open_cap"]
        og.root, og.tools_first, og.tools_count = -1, 0, 0
        og.evaluators = 1
        if kind in ("calc", "calc_text"):
            og.gkind = G_CALC if kind == "calc" else G_TEXT
            if "evaluators" in spec:
                ev = spec["evaluators"]
                if kind != "calc_text" or not isinstance(ev, list) or not ev or \
                        not all(e in ("calc", "strop") for e in ev):
                    raise Unsupported("$.evaluators", "evaluators are 'calc' and 'strop' (calc_text only)")
                og.evaluators = (1 if "calc" in ev else 0) | (2 if "strop" in ev else 0)
            og.calc_min = _setting(spec, "int_min", 0, 10**9)
            og.calc_max = _setting(spec, "int_max", 0, 10**9)
            if og.calc_min > og.calc_max:
                raise Unsupported("$", "empty integer range")
        elif kind == "json_schema":
            og.gkind = G_JSON
            og.root = b.schema(spec.get("schema"), "$.schema", 0)
            # prefix-free languages only: a number at the root has no end
            if "num" in _first_classes(og.root, b.nodes, b.props):
                raise Unsupported("$.schema", "the root value must end by itself (object, array, string, literal)")
        elif kind == "tool_call":
            og.gkind = G_TOOL
            tools = spec.get("tools")
            if not isinstance(tools, list) or not tools or len(tools) > 64:
                raise Unsupported("$.tools", "tools must be a list of 1-64 tools")
            names = [t.get("name") for t in tools]
            ents = []
            for i, t in enumerate(tools):
                nm = t.get("name")
                if not isinstance(nm, str) or not nm or not all(c.isascii() and (c.isalnum() or c in "_.-") for c in nm):
                    raise Unsupported(f"$.tools/{i}", "tool names are non-empty [A-Za-z0-9_.-]")
                if names.count(nm) > 1:
                    raise Unsupported(f"$.tools/{i}", "duplicate tool name")
                params = t.get("parameters")
                if not isinstance(params, dict) or params.get("type") != "object":
                    raise Unsupported(f"$.tools/{i}", "parameters must be an object schema")
                node = b.schema(params, f"$.tools/{i}/parameters", 0)
                off, ln = b.lit(nm.encode() + b"(")
                ents.append(dict(lit_off=off, lit_len=ln, node=node, required=1))
            og.tools_first = b.add_props(ents)
            og.tools_count = len(ents)
        else:
            raise Unsupported("$.kind", f"unknown grammar kind {kind!r}")
        og.open_obj = b.add(kind=K_OBJ, open=1)
        og.open_arr = b.add(kind=K_ARR, open=1)
        self._tree = (b.nodes, b.props, bytes(b.pool))
        self.settings = s
        self.gkind = og.gkind
        n = max(1, len(b.nodes))
        self._nodes = (ONode * n)(*[ONode(**d) for d in b.nodes])
        p = max(1, len(b.props))
        self._props = (OProp * p)(*[OProp(**d) for d in b.props])
        self._pool = (ctypes.c_uint8 * max(1, len(b.pool))).from_buffer_copy(bytes(b.pool) or b"\0")
        og.nodes = self._nodes
        og.props = self._props
        og.pool = self._pool
        self._og = og
        self._L = lib()
        self.conf_size = self._L.oc_size()
        # the language must not be empty
        if og.gkind == G_JSON and not self._L.og_sat(ctypes.byref(og), og.root, 0):
            raise Unsupported("$", "grammar accepts no string")
        if og.gkind == G_TOOL and not any(self._L.og_sat(ctypes.byref(og), b.props[og.tools_first + i]["node"], 0)
                                          for i in range(og.tools_count)):
            raise Unsupported("$", "grammar accepts no string")

    # -- the longest member --------------------------------------------------
    def longest_member(self):
        """The language's longest member as (length, witness), or (None, None)
        when the language is infinite (page "Constrained decoding", section "A
        valid call also has to end": how long a constrained output can get).
        A recursion over the schema tree under the recognizer's rules: every
        optional key present, every whitespace slot filled to ws_max (after
        '{' '[' ',' and around ':' and after each member), every capped string
        at its cap with each code point spelled as the longest escape
        (\\u0041, six bytes), each integer at its longest canonical spelling
        within its bounds and digit limit, containers only where the depth cap
        allows them.  Uncapped strings, arrays without maxItems, numbers,
        any-JSON values and calc expressions are unbounded."""
        nodes, props, pool = self._tree
        W = b" " * self.settings["ws_max"]
        cap = self.settings["depth_cap"]

        class _Inf(Exception):
            pass

        def lit(p):
            return pool[p["lit_off"]:p["lit_off"] + p["lit_len"]]

        def kids(n):
            return [props[n["first"] + j] for j in range(n["count"])]

        def sat(i, d):  # the recognizer's satisfiability under the depth cap
            n = nodes[i]
            k = n["kind"]
            if k == K_OBJ:
                return d + 1 <= cap and (n["open"] or all(sat(p["node"], d + 1) for p in kids(n) if p["required"]))
            if k == K_ARR:
                return d + 1 <= cap
            if k == K_ANYOF:
                return any(sat(p["node"], d) for p in kids(n))
            return True

        def longest(i, d) -> bytes:  # a longest spelling of node i nested in d containers
            n = nodes[i]
            k = n["kind"]
            if k == K_OBJ:
                if n["open"]:
                    raise _Inf
                members = [lit(p) + W + b":" + W + longest(p["node"], d + 1) + W
                           for p in kids(n) if sat(p["node"], d + 1)]
                return b"{" + W + (b"," + W).join(members) + b"}"
            if k == K_ARR:
                if n["open"]:
                    raise _Inf
                if not sat(n["item"], d + 1) or n["cap"] == 0:
                    return b"[" + W + b"]"
                if n["cap"] < 0:
                    raise _Inf
                item = longest(n["item"], d + 1) + W
                return b"[" + W + (b"," + W).join([item] * n["cap"]) + b"]"
            if k == K_STR:
                if n["cap"] < 0:
                    raise _Inf
                return b'"' + b"\\u0041" * n["cap"] + b'"'
            if k == K_INT:
                md = n["maxdigits"]
                if n["has_lo"] and n["has_hi"]:
                    c = [str(n["lo"]), str(n["hi"])]
                else:
                    c = []
                    if not n["has_hi"]:
                        c.append("9" * md)
                    elif n["hi"] >= 0:
                        c.append(str(n["hi"]))
                    if not n["has_lo"]:
                        c.append("-" + "9" * md)
                    elif n["lo"] < 0:
                        c.append(str(n["lo"]))
                return max(c, key=len).encode()
            if k == K_INTSTR:
                return b'"-' + b"9" * n["maxdigits"] + b'"'
            if k == K_BOOL:
                return b"false"
            if k == K_NULL:
                return b"null"
            if k == K_ENUM:
                return max((lit(p) for p in kids(n)), key=len)
            if k == K_ANYOF:
                return max((longest(p["node"], d) for p in kids(n) if sat(p["node"], d)), key=len)
            raise _Inf  # numbers, any-JSON values

        try:
            if self.gkind == G_JSON:
                w = longest(self._og.root, 0)
            elif self.gkind == G_TOOL:
                tools = [props[self._og.tools_first + i] for i in range(self._og.tools_count)]
                w = max((lit(t) + longest(t["node"], 0) + b")" for t in tools if sat(t["node"], 0)), key=len)
            else:
                raise _Inf  # calc expressions and text
        except _Inf:
            return None, None
        return len(w), w

    # -- configurations --------------------------------------------------
    def start(self):
        c = ctypes.create_string_buffer(self.conf_size)
        self._L.oc_start(ctypes.byref(self._og), c)
        return c

    @staticmethod
    def clone(conf):
        c = ctypes.create_string_buffer(len(conf))
        ctypes.memmove(c, conf, len(conf))
        return c

    def feed(self, conf, data: bytes, model: bool = False) -> int:
        """Feed bytes; returns how many were accepted (len(data) if all).
        model=True: the bytes are the model's, refused where the engine
        writes (the result region of calc_text)."""
        if not data:
            return 0
        buf = (ctypes.c_uint8 * len(data)).from_buffer_copy(data)
        fn = self._L.oc_feed_model if model else self._L.oc_feed
        return fn(ctypes.byref(self._og), conf, buf, len(data))

    def in_engine(self, conf) -> bool:
        """Is the next byte one the engine writes?"""
        return bool(self._L.oc_in_engine(ctypes.byref(self._og), conf))

    def complete(self, conf) -> bool:
        return bool(self._L.oc_complete(ctypes.byref(self._og), conf))

    def try_input(self, data: bytes):
        """(refused_at, complete): where the candidate string is refused
        (len(data) if never) and whether it is a full member -- the
        try-input diagnostic of page "Constrained decoding", section
        "Reading the grammar for a tool"."""
        c = self.start()
        k = self.feed(c, data)
        return k, (k == len(data) and self.complete(c))

    def viable(self, data: bytes) -> bool:
        return self.try_input(data)[0] == len(data)

    def next_bytes(self, conf):
        out = (ctypes.c_uint64 * 4)()
        self._L.oc_next_bytes(ctypes.byref(self._og), conf, out)
        return {b for b in range(256) if (out[b >> 6] >> (b & 63)) & 1}

    def mask(self, conf, blob: bytes, offsets) -> np.ndarray:
        V = len(offsets) - 1
        W = (V + 63) // 64
        words = np.zeros(W, dtype=np.uint64)
        bl, off = _vocab_arrays(blob, offsets)
        self._L.oc_mask(ctypes.byref(self._og), conf, bl.ctypes.data, off.ctypes.data, V, words.ctypes.data)
        return words

    def mask_rows(self, confs, done, blob: bytes, offsets, nthreads: int = 1):
        """Masks of many rows; returns (words[B, W] uint64, bytes walked)."""
        V = len(offsets) - 1
        W = (V + 63) // 64
        B = len(confs)
        arr = np.zeros((max(1, B), self.conf_size), dtype=np.uint8)
        for i, c in enumerate(confs):
            arr[i] = np.frombuffer(c.raw, dtype=np.uint8)
        dn = np.ascontiguousarray(np.asarray(done, dtype=np.uint8).reshape(-1)) if B else np.zeros(1, np.uint8)
        words = np.zeros((max(1, B), W), dtype=np.uint64)
        bl, off = _vocab_arrays(blob, offsets)
        walked = self._L.oc_mask_rows(ctypes.byref(self._og), arr.ctypes.data, dn.ctypes.data, B,
                                      bl.ctypes.data, off.ctypes.data, V, words.ctypes.data, nthreads)
        return words[:B], walked


_vocab_cache = {}


def _vocab_arrays(blob, offsets):
    key = (id(blob), len(blob), len(offsets))
    hit = _vocab_cache.get(key)
    if hit is not None and hit[0] is blob:
        return hit[1], hit[2]
    bl = np.frombuffer(blob if blob else b"\0", dtype=np.uint8).copy()
    off = np.asarray(offsets, dtype=np.uint32)
    _vocab_cache.clear()
    _vocab_cache[key] = (blob, bl, off)
    return bl, off


def load_spec(spec) -> Grammar:
    return Grammar(spec)


# ---------------------------------------------------------------------------
# Rows: state + step counter + the engine cap.
# ---------------------------------------------------------------------------
ROW_OK, ROW_DONE, ROW_CAPPED, ROW_REJECTED, ROW_NOOP, ROW_INJECT = 0, 1, 2, 3, 4, 5


class Row:
    """One sequence: accepted bytes (as a recognizer configuration), tokens
    accepted so far, and whether it is finished.  done = the bytes form a
    complete member, or step >= gen_cap."""

    def __init__(self, g: Grammar, gen_cap: int):
        self.g = g
        self.conf = g.start()
        self.step = 0
        self.gen_cap = gen_cap
        self.complete = False
        self.capped = gen_cap <= 0
        self.text = bytearray()

    @property
    def done(self):
        return self.complete or self.capped

    def advance(self, tok: bytes | None) -> int:
        """A token the model chose (or a forced token id): every byte must be
        the model's to write."""
        if tok is None:
            return ROW_NOOP
        return self._take(tok, model=True)

    def force(self, data: bytes) -> int:
        """Bytes the engine writes -- an evaluated result injected into the
        stream, a transition the model did not choose (page "Evaluator aware
        decoding", section "A concrete prototype on llama.cpp").  Not a
        generation step: the step count and the cap are untouched.  Empty is
        a no-op."""
        if not data:
            return ROW_NOOP
        return self._take(data, model=False)

    def _take(self, data: bytes, model: bool) -> int:
        if self.done or not data:
            return ROW_REJECTED
        c = self.g.clone(self.conf)
        if self.g.feed(c, data, model=model) != len(data):
            return ROW_REJECTED
        self.conf = c
        self.text += data
        self.complete = self.g.complete(c)
        if model:
            self.step += 1
            if self.step >= self.gen_cap:
                self.capped = True
        if self.complete:
            return ROW_DONE
        if self.capped:
            return ROW_CAPPED
        if self.g.in_engine(c):
            return ROW_INJECT
        return ROW_OK


# ---------------------------------------------------------------------------
# Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11), vectorised in numpy.
# ---------------------------------------------------------------------------
PHILOX_M0, PHILOX_M1 = 0xD2511F53, 0xCD9E8D57
PHILOX_W0, PHILOX_W1 = 0x9E3779B9, 0xBB67AE85
U32 = 0xFFFFFFFF


def philox4x32_10(ctr, key):
    """ctr: uint32 array [..., 4]; key: (k0, k1).  Returns uint32 [..., 4].

    Ten rounds; each round multiplies words 0 and 2 by M0 and M1 into 64-bit
    products and recombines:  (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0),
    with the key bumped by the Weyl constants (W0, W1) between rounds."""
    c = np.asarray(ctr, dtype=np.uint64) & U32
    c0, c1, c2, c3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
    k0, k1 = np.uint64(key[0] & U32), np.uint64(key[1] & U32)
    for r in range(10):
        p0 = c0 * np.uint64(PHILOX_M0)
        p1 = c2 * np.uint64(PHILOX_M1)
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(U32)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(U32)
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
        k0 = (k0 + np.uint64(PHILOX_W0)) & np.uint64(U32)
        k1 = (k1 + np.uint64(PHILOX_W1)) & np.uint64(U32)
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def philox_words(seed: int, step: int, lvl: int, idx) -> np.ndarray:
    """Word for element i of the shared stream: out[i & 3] of the block at
    counter (i >> 2, step, lvl, 0), key = (seed lo32, seed hi32)."""
    idx = np.asarray(idx, dtype=np.int64)
    j = (idx >> 2).astype(np.uint64)
    ctr = np.stack([j, np.full_like(j, step & U32), np.full_like(j, lvl), np.zeros_like(j)], axis=-1)
    out = philox4x32_10(ctr, (seed & U32, (seed >> 32) & U32))
    return out[np.arange(len(idx)), idx & 3]


def gumbel(words) -> np.ndarray:
    """u = (w + 1/2) 2^-32 (exact in float64, inside (0,1)); g = -ln(-ln u)."""
    u = (np.asarray(words, dtype=np.float64) + 0.5) * 2.0 ** -32
    return -np.log(-np.log(u))


CHUNK = 2048


def _lse(v):
    m = np.max(v)
    if not np.isfinite(m):
        return -math.inf
    return float(m + np.log(np.sum(np.exp(v - m))))


def sample_row(x, allowed, T, seed, step, chunk=CHUNK):
    """Pick one token from stored logits x (exact values, any float dtype)
    restricted to `allowed`, in float64.  Returns (id, logprob, info).

    T == 0: greedy argmax (lowest id on ties), logprob at temperature 1.
    T > 0 : two-level Gumbel-max: chunk c of `chunk` ids gets log-mass
    LSE_c = logsumexp_{i in c, allowed} x_i/T; c* = argmax_c LSE_c + g(u_c)
    (stream level 1, element c); then id = argmax_{i in c*} x_i/T + g(u_i)
    (level 0, element i).  P(id) = P(c*) P(id | c*) = softmax(x/T) on the
    mask.  logprob = x_id/T - logsumexp_{allowed} x/T.
    info: top-2 score margins at each level (inf when there is one candidate).
    An allowed token whose logit is -inf carries no probability; with no
    allowed token of finite logit there is nothing to draw: (-1, 0).
    """
    x = np.asarray(x, dtype=np.float64)
    allowed = np.asarray(allowed, dtype=bool) & (x > -np.inf)
    V = len(x)
    info = {"margin_chunk": math.inf, "margin_token": math.inf}
    if not allowed.any():
        return -1, 0.0, info
    if T == 0:
        xm = np.where(allowed, x, -np.inf)
        i = int(np.argmax(xm))
        top = np.sort(xm[allowed])[::-1]
        if len(top) > 1:
            info["margin_token"] = float(top[0] - top[1])
        return i, float(x[i] - _lse(x[allowed])), info
    T = float(np.float32(T))  # the temperature as the device holds it
    z = x / T
    K = (V + chunk - 1) // chunk
    lse_c = np.full(K, -np.inf)
    for c in range(K):
        a = allowed[c * chunk:(c + 1) * chunk]
        if a.any():
            lse_c[c] = _lse(z[c * chunk:(c + 1) * chunk][a])
    gc = gumbel(philox_words(seed, step, 1, np.arange(K)))
    sc = lse_c + gc
    cs = int(np.argmax(sc))
    fin = np.sort(sc[np.isfinite(sc)])[::-1]
    if len(fin) > 1:
        info["margin_chunk"] = float(fin[0] - fin[1])
    lo = cs * chunk
    hi = min(V, lo + chunk)
    ids = np.arange(lo, hi)
    a = allowed[lo:hi]
    gt = gumbel(philox_words(seed, step, 0, ids))
    st = np.where(a, z[lo:hi] + gt, -np.inf)
    k = int(np.argmax(st))
    fin = np.sort(st[a])[::-1]
    if len(fin) > 1:
        info["margin_token"] = float(fin[0] - fin[1])
    i = lo + k
    return i, float(z[i] - _lse(z[allowed])), info


def unpack_mask(words, V):
    """uint64 words -> bool[V], bit t & 63 of word t >> 6."""
    w = np.ascontiguousarray(np.asarray(words, dtype=np.uint64))
    bits = np.unpackbits(w.view(np.uint8), bitorder="little")
    return bits[:V].astype(bool)


# ---------------------------------------------------------------------------
# Calc-span evaluator: exact integers, * and / before + and -, left to
# right, / truncating toward zero, division by zero an error (page "Evaluator
# aware decoding", sections "The core idea" and "A concrete prototype on
# llama.cpp": a small local parser evaluates the closed span).  bound=(lo,
# hi): also an error when a literal or any intermediate result leaves
# [lo, hi] -- a fixed-width engine's range.
# ---------------------------------------------------------------------------
class CalcError(ValueError):
    pass


INT64_RANGE = (-(1 << 63), (1 << 63) - 1)


def eval_calc(span: bytes, bound=None) -> int:
    s = span.decode("ascii")
    if not (s.startswith("<calc>") and s.endswith("</calc>")):
        raise CalcError("not a calc span")

    def within(v):
        if bound is not None and not bound[0] <= v <= bound[1]:
            raise CalcError("out of range")
        return v

    toks = []
    body = s[6:-7]
    i = 0
    while i < len(body):
        ch = body[i]
        if ch in " \t\n\r":
            i += 1
        elif ch.isdigit():
            j = i
            while j < len(body) and body[j].isdigit():
                j += 1
            toks.append(int(body[i:j]))
            i = j
        elif ch in "+-*/()":
            toks.append(ch)
            i += 1
        else:
            raise CalcError(f"bad byte {ch!r}")
    pos = 0

    def peek():
        return toks[pos] if pos < len(toks) else None

    def term():
        nonlocal pos
        t = peek()
        pos += 1
        if t == "(":
            v = expr()
            if peek() != ")":
                raise CalcError("missing )")
            pos += 1
            return v
        if isinstance(t, int):
            return within(t)
        raise CalcError("expected a term")

    def prod():
        nonlocal pos
        v = term()
        while peek() in ("*", "/"):
            op = peek()
            pos += 1
            r = term()
            if op == "*":
                v = v * r
            else:
                if r == 0:
                    raise CalcError("division by zero")
                q = abs(v) // abs(r)
                v = q if (v >= 0) == (r >= 0) else -q
            within(v)
        return v

    def expr():
        nonlocal pos
        v = prod()
        while peek() in ("+", "-"):
            op = peek()
            pos += 1
            r = prod()
            v = v + r if op == "+" else v - r
            within(v)
        return v

    v = expr()
    if pos != len(toks):
        raise CalcError("trailing input")
    return v


# ---------------------------------------------------------------------------
# The integer-string contract (page "Constrained Decoding Under Matched
# Conditions", section "The system boundary I am testing"): external
# canonical signed-integer strings become native JSON integers for the
# model; after one generation each such integer goes back to a string of its
# own base-10 text, and the result is validated against the external schema.
# ---------------------------------------------------------------------------
class _RawNum(str):
    """A JSON number kept as its source text."""


class ContractError(ValueError):
    pass


def _is_int_string(sch):
    return isinstance(sch, dict) and sch.get("type") == "string" and sch.get("pattern") == INT_STRING_PATTERN


def contract_model_spec(spec: dict) -> tuple:
    """(model-facing spec, number of replaced fields)."""
    n = 0

    def conv(s):
        nonlocal n
        if _is_int_string(s):
            n += 1
            return {"type": "integer"}
        if not isinstance(s, dict):
            return s
        out = {}
        for k, v in s.items():
            if k == "properties" and isinstance(v, dict):
                out[k] = {pk: conv(pv) for pk, pv in v.items()}
            elif k == "items":
                out[k] = conv(v)
            elif k == "anyOf" and isinstance(v, list):
                out[k] = [conv(a) for a in v]
            else:
                out[k] = v
        return out

    model = dict(spec)
    model["schema"] = conv(spec["schema"])
    return model, n


def _dump(v) -> str:
    if v is None:
        return "null"
    if v is True:
        return "true"
    if v is False:
        return "false"
    if isinstance(v, _RawNum):
        return str.__str__(v)
    if isinstance(v, str):
        return json.dumps(v, ensure_ascii=False)
    if isinstance(v, list):
        return "[" + ",".join(_dump(x) for x in v) + "]"
    return "{" + ",".join(json.dumps(k, ensure_ascii=False) + ":" + _dump(x) for k, x in v.items()) + "}"


def _integer_text(v):
    return isinstance(v, _RawNum) and all(c in "-0123456789" for c in v)


def _fits(sch, v):
    if _is_int_string(sch):
        return _integer_text(v)
    t = sch.get("type") if isinstance(sch, dict) else None
    if not isinstance(t, str):
        return True
    if v is None:
        return t == "null"
    if isinstance(v, bool):
        return t == "boolean"
    if isinstance(v, _RawNum):
        return t == "number" or (t == "integer" and _integer_text(v))
    if isinstance(v, str):
        return t == "string"
    if isinstance(v, list):
        return t == "array"
    return t == "object"


def contract_reverse(spec: dict, text: bytes):
    """(ok, output text or None, message).  ok: the output maps onto the
    external schema and the external grammar accepts it in full."""
    try:
        v = json.loads(text.decode("utf-8"), parse_int=_RawNum, parse_float=_RawNum,
                       parse_constant=_RawNum)
    except (ValueError, UnicodeDecodeError) as e:
        return False, None, f"generated text: {e}"

    def rev(sch, v):
        if _is_int_string(sch):
            if not _integer_text(v):
                raise ContractError("expected an integer")
            return str(str.__str__(v))
        if not isinstance(sch, dict):
            return v
        if "anyOf" in sch:
            for alt in sch["anyOf"]:
                if _fits(alt, v):
                    return rev(alt, v)
            return v
        if isinstance(v, dict) and isinstance(sch.get("properties"), dict):
            return {k: (rev(sch["properties"][k], x) if k in sch["properties"] else x) for k, x in v.items()}
        if isinstance(v, list) and "items" in sch:
            return [rev(sch["items"], x) for x in v]
        return v

    try:
        out = _dump(rev(spec["schema"], v)).encode("utf-8")
    except ContractError as e:
        return False, None, str(e)
    k, complete = Grammar(spec).try_input(out)
    return complete, out, "" if complete else f"refused at byte {k}"


# ---------------------------------------------------------------------------
# String operations (page "Evaluator aware decoding", section "Not just
# arithmetic: string operations"): a small registry of pure functions over
# the span's arguments.  count = non-overlapping occurrences scanning left to
# right (an empty pattern occurs len + 1 times), len = characters, reverse,
# upper = ASCII letters upper-cased, substr(s, i, j) = the characters from i
# up to j, negative positions counting from the end, clamped to the string.
# Integer results are written as decimal text, string results as they are.
# ---------------------------------------------------------------------------
def _count(s, t):
    if not t:
        return len(s) + 1
    n = i = 0
    while True:
        k = s.find(t, i)
        if k < 0:
            return n
        n += 1
        i = k + len(t)


def _slice(s, i, j):
    n = len(s)

    def norm(x):
        x = x + n if x < 0 else x
        return min(max(x, 0), n)

    a, b = norm(i), norm(j)
    return s[a:b] if a < b else ""


def eval_strop(span: bytes) -> bytes:
    s = span.decode("ascii")
    m = re.fullmatch(r'<strop>(count|len|reverse|upper|substr)\((.*)\)</strop>', s, re.S)
    if not m:
        raise CalcError("not a string-operation span")
    name, rest = m.group(1), m.group(2)
    args = []
    i = 0
    while i < len(rest):
        ch = rest[i]
        if ch in " \t\n\r,":
            i += 1
        elif ch == '"':
            j = rest.index('"', i + 1)
            args.append(rest[i + 1:j])
            i = j + 1
        else:
            j = i + 1
            while j < len(rest) and rest[j].isdigit():
                j += 1
            args.append(int(rest[i:j]))
            i = j
    if name == "count":
        out = str(_count(args[0], args[1]))
    elif name == "len":
        out = str(len(args[0]))
    elif name == "reverse":
        out = args[0][::-1]
    elif name == "upper":
        out = "".join(chr(ord(c) - 32) if "a" <= c <= "z" else c for c in args[0])
    else:
        out = _slice(args[0], args[1], args[2])
    return out.encode("ascii")
