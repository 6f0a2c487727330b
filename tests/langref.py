"""Independent references used to pin the oracle (tests only).

* member(spec, data): a full-string recursive-descent validator.  It reads a
  complete candidate at once (no incremental state), validates UTF-8 with
  Python's strict codec, integers with int(), keys/enums against
  json.dumps spellings -- a different construction from the oracle's
  incremental frame stack.
* enumerate_members(spec, sigma, budget): every member of the language whose
  bytes all lie in `sigma`, generated from the spec (generative, not
  recognising), for tiny specs.
* closed_chars(sigma): every JSON string character (raw UTF-8 scalar or
  escape) spelled with bytes of `sigma`.
"""
from __future__ import annotations

import itertools
import json
import re

WS = b" \t\n\r"
_INT_RE = re.compile(rb"-?(0|[1-9][0-9]*)")
_NUM_RE = re.compile(rb"-?(0|[1-9][0-9]*)(\.[0-9]+)?([eE][+-]?[0-9]+)?")
_SHORT_ESC = set(b'"\\/bfnrt')

DEFAULTS = dict(ws_max=4, open_string_cap=256, open_int_digits=20, depth_cap=16, int_min=0, int_max=999)


def _get(spec, k):
    return spec.get(k, DEFAULTS[k])


class _Fail(Exception):
    pass


class _P:
    """Recursive-descent reader over a complete byte string."""

    def __init__(self, spec, data):
        self.s = data
        self.i = 0
        self.ws_max = _get(spec, "ws_max")
        self.cap = spec.get("open_string_cap", DEFAULTS["open_string_cap"])
        self.digits = _get(spec, "open_int_digits")
        self.depth_cap = _get(spec, "depth_cap")
        self.depth = 0

    def peek(self):
        return self.s[self.i] if self.i < len(self.s) else None

    def lit(self, b):
        if not self.s.startswith(b, self.i):
            raise _Fail
        self.i += len(b)

    def ws(self):
        j = self.i
        while j < len(self.s) and self.s[j] in WS:
            j += 1
        if j - self.i > self.ws_max:
            raise _Fail
        self.i = j

    def string(self, cap):
        if self.peek() != 0x22:
            raise _Fail
        j = self.i + 1
        chars = 0
        while True:
            if j >= len(self.s):
                raise _Fail
            c = self.s[j]
            if c == 0x22:
                break
            if c == 0x5C:
                if j + 1 >= len(self.s):
                    raise _Fail
                e = self.s[j + 1]
                if e == ord("u"):
                    h = self.s[j + 2:j + 6]
                    if len(h) != 4 or not all(chr(x) in "0123456789abcdefABCDEF" for x in h):
                        raise _Fail
                    if 0xD800 <= int(h, 16) <= 0xDFFF:
                        raise _Fail
                    j += 6
                elif e in _SHORT_ESC:
                    j += 2
                else:
                    raise _Fail
                chars += 1
                continue
            if c < 0x20:
                raise _Fail
            # one UTF-8 scalar: try 1..4 bytes with the strict codec
            for n in (1, 2, 3, 4):
                try:
                    ch = self.s[j:j + n].decode("utf-8")
                except UnicodeDecodeError:
                    continue
                if len(ch) == 1:
                    break
            else:
                raise _Fail
            j += n
            chars += 1
        if cap is not None and cap >= 0 and chars > cap:
            raise _Fail
        self.i = j + 1

    def value(self, sch):
        if sch is None:
            return self.any_value()
        keys = set(sch) - {"title", "description", "$comment", "examples", "default"}
        if not keys:
            return self.any_value()
        if "anyOf" in sch:
            start = self.i
            ok = 0
            for alt in sch["anyOf"]:
                self.i = start
                d0 = self.depth
                try:
                    self.value(alt)
                    ok += 1
                    end = self.i
                except _Fail:
                    self.depth = d0
            if ok != 1:
                raise _Fail
            self.i = end
            return
        if "enum" in sch:
            for v in sch["enum"]:
                sp = json.dumps(v, ensure_ascii=False).encode()
                if self.s.startswith(sp, self.i):
                    self.i += len(sp)
                    return
            raise _Fail
        t = sch["type"]
        if t == "object":
            return self.obj(sch)
        if t == "array":
            return self.arr(sch)
        if t == "string" and "pattern" in sch:
            # the canonical signed-integer string: Python's regex engine on the
            # string's raw content (no escapes spell a digit)
            start = self.i
            self.string(-1)
            content = self.s[start + 1:self.i - 1].decode("utf-8")
            if not re.fullmatch(sch["pattern"], content) or len(content.lstrip("-")) > self.digits:
                raise _Fail
            return
        if t == "string":
            return self.string(sch.get("maxLength", self.cap if self.cap is not None else -1))
        if t == "integer":
            m = _INT_RE.match(self.s, self.i)
            if not m:
                raise _Fail
            txt = m.group(0)
            if txt == b"-0":
                raise _Fail
            mag = txt.lstrip(b"-")
            both = "minimum" in sch and "maximum" in sch
            if len(mag) > (19 if both else self.digits):
                raise _Fail
            v = int(txt)
            lim = 10 ** self.digits - 1
            if v < sch.get("minimum", -lim) or v > sch.get("maximum", lim):
                raise _Fail
            self.i = m.end()
            return
        if t == "number":
            m = _NUM_RE.match(self.s, self.i)
            if not m:
                raise _Fail
            self.i = m.end()
            return
        if t == "boolean":
            for b in (b"true", b"false"):
                if self.s.startswith(b, self.i):
                    self.i += len(b)
                    return
            raise _Fail
        if t == "null":
            return self.lit(b"null")
        raise _Fail

    def enter(self):
        self.depth += 1
        if self.depth > self.depth_cap:
            raise _Fail

    def obj(self, sch):
        props = sch.get("properties")
        req = set(sch.get("required", []))
        self.lit(b"{")
        self.enter()
        self.ws()
        order = list(props) if props is not None else None
        seen = []
        if self.peek() == ord("}"):
            self.i += 1
        else:
            while True:
                if order is None:
                    self.string(self.cap if self.cap is not None else -1)
                    vs = None
                else:
                    for k in order:
                        sp = json.dumps(k, ensure_ascii=False).encode()
                        if self.s.startswith(sp, self.i):
                            break
                    else:
                        raise _Fail
                    # declared order, no repeats
                    if seen and order.index(k) <= order.index(seen[-1]):
                        raise _Fail
                    seen.append(k)
                    self.i += len(sp)
                    vs = props[k]
                self.ws()
                self.lit(b":")
                self.ws()
                self.value(vs)
                self.ws()
                c = self.peek()
                if c == ord(","):
                    self.i += 1
                    self.ws()
                    continue
                if c == ord("}"):
                    self.i += 1
                    break
                raise _Fail
        if order is not None and not req <= set(seen):
            raise _Fail
        self.depth -= 1

    def arr(self, sch):
        item = sch.get("items")
        mi = sch.get("maxItems")
        self.lit(b"[")
        self.enter()
        self.ws()
        n = 0
        if self.peek() == ord("]"):
            self.i += 1
        else:
            while True:
                self.value(item)
                n += 1
                self.ws()
                c = self.peek()
                if c == ord(","):
                    self.i += 1
                    self.ws()
                    continue
                if c == ord("]"):
                    self.i += 1
                    break
                raise _Fail
        if mi is not None and n > mi:
            raise _Fail
        self.depth -= 1

    def any_value(self):
        c = self.peek()
        if c == ord("{"):
            return self.obj({"type": "object"})
        if c == ord("["):
            return self.arr({"type": "array"})
        if c == ord('"'):
            return self.string(self.cap if self.cap is not None else -1)
        if c is not None and (c == ord("-") or 0x30 <= c <= 0x39):
            return self.value({"type": "number"})
        for b in (b"true", b"false", b"null"):
            if self.s.startswith(b, self.i):
                self.i += len(b)
                return
        raise _Fail


def _calc_member(spec, s):
    lo, hi = _get(spec, "int_min"), _get(spec, "int_max")
    wsm, dcap = _get(spec, "ws_max"), _get(spec, "depth_cap")
    if not (s.startswith(b"<calc>") and s.endswith(b"</calc>")):
        return False
    body = s[6:-7]
    i = 0

    def ws():
        nonlocal i
        j = i
        while j < len(body) and body[j] in WS:
            j += 1
        if j - i > wsm:
            raise _Fail
        i = j

    def term(d):
        nonlocal i
        if i < len(body) and body[i] == ord("("):
            if d + 1 > dcap:
                raise _Fail
            i += 1
            ws()
            expr(d + 1)
            ws()
            if i >= len(body) or body[i] != ord(")"):
                raise _Fail
            i += 1
            return
        m = re.compile(rb"0|[1-9][0-9]*").match(body, i)
        if not m or not lo <= int(m.group(0)) <= hi:
            raise _Fail
        i = m.end()

    def expr(d):
        nonlocal i
        term(d)
        while True:
            save = i
            try:
                ws()
                if i < len(body) and body[i] in b"+-*/":
                    i += 1
                    ws()
                    term(d)
                    continue
            except _Fail:
                pass
            i = save
            return

    try:
        ws()
        expr(0)
        ws()
    except _Fail:
        return False
    return i == len(body)


_RESULT_RE = re.compile(rb"<result>-?[0-9]{1,20}</result>|<result_error>[\x20-\x3b\x3d-\x7e]*</result_error>")
_TEXT_RESULT_RE = re.compile(rb"<result>[\x20-\x3b\x3d-\x7e]*</result>|<result_error>[\x20-\x3b\x3d-\x7e]*</result_error>")


def _strop_re(ws_max):
    w = rb"[ \t\n\r]{0,%d}" % ws_max
    s = rb'"[\x20\x21\x23-\x3b\x3d-\x5b\x5d-\x7e]*"'
    i = rb"-?[0-9]{1,6}"
    c = w + rb"," + w
    body = (rb"count\(" + w + s + c + s + w + rb"\)|(?:len|reverse|upper)\(" + w + s + w + rb"\)|substr\(" + w + s + c
            + i + c + i + w + rb"\)")
    return re.compile(rb"<strop>(?:" + body + rb")</strop>")
_TEXT_RE = re.compile(rb"[\n\x20-\x3b\x3d-\x7e]*")


def calc_text_parts(spec, data: bytes):
    """Split a complete calc_text member into (who, bytes) pieces, who =
    "model" or "engine"; None if `data` is not a member.  Reads the text
    left to right with regular expressions and the calc-span validator."""
    evaluators = spec.get("evaluators", ["calc"])
    strop_re = _strop_re(_get(spec, "ws_max"))
    parts = []
    i = 0
    while True:
        m = _TEXT_RE.match(data, i)
        if m.end() > i:
            parts.append(("model", data[i:m.end()]))
        i = m.end()
        if data[i:] == b"<end>":
            parts.append(("model", b"<end>"))
            return parts
        if "calc" in evaluators and data.startswith(b"<calc>", i):
            j = data.find(b"</calc>", i)
            if j < 0 or not _calc_member(spec, data[i:j + 7]):
                return None
            end, result_re = j + 7, _RESULT_RE
        elif "strop" in evaluators and data.startswith(b"<strop>", i):
            s = strop_re.match(data, i)
            if not s:
                return None
            end, result_re = s.end(), _TEXT_RESULT_RE
        else:
            return None
        parts.append(("model", data[i:end]))
        i = end
        r = result_re.match(data, i)
        if not r:
            return None
        parts.append(("engine", r.group(0)))
        i = r.end()


def member(spec, data: bytes) -> bool:
    """Is `data` (complete) in the language of `spec`?"""
    kind = spec["kind"]
    if kind == "calc":
        return _calc_member(spec, data)
    if kind == "calc_text":
        return calc_text_parts(spec, data) is not None
    p = _P(spec, data)
    try:
        if kind == "json_schema":
            p.value(spec["schema"])
        else:
            for t in spec["tools"]:
                nm = t["name"].encode() + b"("
                if data.startswith(nm):
                    p.i = len(nm)
                    p.value(t["parameters"])
                    p.lit(b")")
                    break
            else:
                return False
    except _Fail:
        return False
    return p.i == len(data)


# ---------------------------------------------------------------------------
# Generative enumeration for tiny specs.
# ---------------------------------------------------------------------------

def closed_chars(sigma: bytes):
    """All JSON string characters whose spelling uses only bytes of sigma."""
    sig = set(sigma)
    out = []
    for b in sig:
        if 0x20 <= b < 0x80 and b not in (0x22, 0x5C):
            out.append(bytes([b]))
    if 0x5C in sig:
        for e in _SHORT_ESC:
            if e in sig:
                out.append(bytes([0x5C, e]))
        if ord("u") in sig:
            hexd = [x for x in sig if chr(x) in "0123456789abcdefABCDEF"]
            for h in itertools.product(hexd, repeat=4):
                if not 0xD800 <= int(bytes(h), 16) <= 0xDFFF:
                    out.append(b"\\u" + bytes(h))
    hi = sorted(x for x in sig if x >= 0x80)
    for n in (2, 3, 4):
        for seq in itertools.product(hi, repeat=n):
            try:
                ch = bytes(seq).decode("utf-8")
            except UnicodeDecodeError:
                continue
            if len(ch) == 1:
                out.append(bytes(seq))
    return sorted(set(out))


def _ws_runs(k, sigma):
    ws = [bytes([c]) for c in WS if c in sigma]
    out = []
    for n in range(k + 1):
        out.extend(b"".join(p) for p in itertools.product(ws, repeat=n))
    return out


def _cat(parts_lists, budget):
    """All concatenations (one from each list) of total length <= budget."""
    res = [b""]
    for lst in parts_lists:
        lst = sorted(lst, key=len)
        nxt = []
        for a in res:
            room = budget - len(a)
            for b in lst:
                if len(b) > room:
                    break
                nxt.append(a + b)
        res = nxt
        if not res:
            break
    return res


class Enumerator:
    def __init__(self, spec, sigma: bytes, budget: int):
        self.spec = spec
        self.sigma = set(sigma)
        self.budget = budget
        self.ws = _ws_runs(_get(spec, "ws_max"), self.sigma)
        self.chars = closed_chars(sigma)
        self.cap = spec.get("open_string_cap", DEFAULTS["open_string_cap"])
        self.digits = _get(spec, "open_int_digits")
        self._memo = {}

    def ok(self, b):
        return all(c in self.sigma for c in b)

    def strings(self, cap, budget):
        """Every string of at most `cap` characters (None or < 0: any
        number) spelled within `budget` bytes."""
        if cap is None or cap < 0:
            cap = budget
        out = [b'"' + b'"']
        cur = [b""]
        for _ in range(cap):
            cur = [a + c for a in cur for c in self.chars if len(a) + len(c) + 2 <= budget]
            if not cur:
                break
            out.extend(b'"' + a + b'"' for a in cur)
        return [s for s in out if len(s) <= budget]

    # ---- open JSON values (RFC 8259), written from the grammar's productions:
    # value = object / array / string / number / true / false / null;
    # containers count against depth_cap (the root container is depth 1).
    def numbers(self, budget):
        """number = [ "-" ] int [ frac ] [ exp ]; int = "0" / [1-9] *DIGIT;
        frac = "." 1*DIGIT; exp = ("e" / "E") [ "+" / "-" ] 1*DIGIT --
        every spelling within `budget` bytes over the alphabet."""
        sig = self.sigma
        digits = [bytes([d]) for d in b"0123456789" if d in sig]
        runs, cur = [], [b""]
        while True:  # 1*DIGIT
            cur = [a + d for a in cur for d in digits if len(a) + 1 <= budget]
            if not cur:
                break
            runs += cur
        ints = [b"0"] if b"0" in digits else []
        ints += [r for r in runs if r[:1] != b"0"]
        signs = [b""] + ([b"-"] if ord("-") in sig else [])
        fracs = [b""] + ([b"." + r for r in runs] if ord(".") in sig else [])
        exps = [b""]
        for e in b"eE":
            if e in sig:
                for s in [b""] + [bytes([c]) for c in b"+-" if c in sig]:
                    exps += [bytes([e]) + s + r for r in runs]
        return _cat([signs, ints, fracs, exps], budget)

    def any_values(self, budget, depth):
        key = ("any", budget, depth)
        if key in self._memo:
            return self._memo[key]
        out = self.strings(self.cap, budget) + self.numbers(budget)
        out += [b for b in (b"true", b"false", b"null") if self.ok(b) and len(b) <= budget]
        out += self.open_array(budget, depth) + self.open_object(budget, depth)
        self._memo[key] = out
        return out

    def _members(self, first, budget):
        """`first` (W member W) followed by any number of ("," W member W),
        within `budget` bytes: the inside of a container."""
        out, cur = list(first), list(first)
        while cur:
            nxt = []
            for a in cur:
                nxt += [a + b for b in _cat([[b","], first], budget - len(a))]
            out += nxt
            cur = nxt
        return out

    def open_array(self, budget, depth):
        if depth + 1 > _get(self.spec, "depth_cap") or budget < 2:
            return []
        W = self.ws
        out = _cat([[b"["], W, [b"]"]], budget)
        elem = _cat([W, self.any_values(budget - 2, depth + 1), W], budget - 2)
        out += [b"[" + s + b"]" for s in self._members(elem, budget - 2)]
        return out

    def open_object(self, budget, depth):
        if depth + 1 > _get(self.spec, "depth_cap") or budget < 2:
            return []
        W = self.ws
        out = _cat([[b"{"], W, [b"}"]], budget)
        keys = self.strings(self.cap, budget - 2)
        pair = _cat([W, keys, W, [b":"], W, self.any_values(budget - 2, depth + 1), W], budget - 2)
        out += [b"{" + s + b"}" for s in self._members(pair, budget - 2)]
        return out

    def values(self, sch, budget, depth=0):
        keys = set(sch) - {"title", "description"}
        if not keys:
            return self.any_values(budget, depth)
        if keys == {"type"} and sch["type"] == "array":
            return self.open_array(budget, depth)
        if keys == {"type"} and sch["type"] == "object":
            return self.open_object(budget, depth)
        if "anyOf" in sch:
            out = []
            for a in sch["anyOf"]:
                out += self.values(a, budget, depth)
            return out
        if "enum" in sch:
            return [sp for sp in (json.dumps(v, ensure_ascii=False).encode() for v in sch["enum"])
                    if len(sp) <= budget and self.ok(sp)]
        t = sch["type"]
        if t == "string":
            return self.strings(sch.get("maxLength", self.cap), budget)
        if t == "integer":
            lo, hi = sch["minimum"], sch["maximum"]
            return [s for s in (str(v).encode() for v in range(lo, hi + 1)) if len(s) <= budget and self.ok(s)]
        if t == "boolean":
            return [b for b in (b"true", b"false") if self.ok(b) and len(b) <= budget]
        if t == "null":
            return [b"null"] if self.ok(b"null") and len(b"null") <= budget else []
        if t in ("array", "object") and depth + 1 > _get(self.spec, "depth_cap"):
            return []
        if t == "array":
            item = sch["items"]
            mi = sch.get("maxItems", 3)
            W = self.ws
            out = _cat([[b"["], W, [b"]"]], budget)
            vals = self.values(item, budget, depth + 1)
            seqs = [[b"["], W, vals, W]
            for n in range(1, mi + 1):
                out += _cat(seqs + [[b"]"]], budget)
                seqs = seqs + [[b","], W, vals, W]
            return out
        if t == "object":
            props = list(sch["properties"].items())
            req = set(sch.get("required", []))
            W = self.ws
            out = []
            for mask in range(1 << len(props)):
                chosen = [props[i] for i in range(len(props)) if mask >> i & 1]
                if not req <= {k for k, _ in chosen}:
                    continue
                if not chosen:
                    out += _cat([[b"{"], W, [b"}"]], budget)
                    continue
                parts = [[b"{"], W]
                for j, (k, v) in enumerate(chosen):
                    if j:
                        parts += [[b","], W]
                    parts += [[json.dumps(k, ensure_ascii=False).encode()], W, [b":"], W,
                              self.values(v, budget, depth + 1), W]
                parts += [[b"}"]]
                out += _cat(parts, budget)
            return out
        raise ValueError(t)

    def members(self):
        spec, B = self.spec, self.budget
        kind = spec["kind"]
        if kind == "json_schema":
            res = self.values(spec["schema"], B)
        elif kind == "tool_call":
            res = []
            for t in spec["tools"]:
                nm = t["name"].encode() + b"("
                res += [nm + a + b")" for a in self.values(t["parameters"], B - len(nm) - 1)]
        else:
            res = self.calc()
        return {r for r in res if len(r) <= B and self.ok(r)}

    def calc(self):
        lo, hi = _get(self.spec, "int_min"), _get(self.spec, "int_max")
        dcap = _get(self.spec, "depth_cap")
        W = self.ws
        ints = [s for s in (str(v).encode() for v in range(lo, hi + 1)) if self.ok(s)]
        ops = [bytes([c]) for c in b"+-*/" if c in self.sigma]
        B = self.budget - 13
        memo = {}

        def E(d, budget):
            key = ("E", d, budget)
            if key in memo:
                return memo[key]
            out = []
            frontier = list(T(d, budget))
            out += frontier
            while frontier:
                nxt = []
                for a in frontier:
                    for tail in _cat([W, ops, W], budget - len(a)):
                        for t in T(d, budget - len(a) - len(tail)):
                            nxt.append(a + tail + t)
                out += nxt
                frontier = nxt
            memo[key] = out
            return out

        def T(d, budget):
            key = ("T", d, budget)
            if key in memo:
                return memo[key]
            out = [i for i in ints if len(i) <= budget]
            if d < dcap and budget >= 3 and b"(" in [bytes([c]) for c in self.sigma] + [b""]:
                for w1 in W:
                    for w2 in W:
                        room = budget - 2 - len(w1) - len(w2)
                        if room <= 0:
                            continue
                        for e in E(d + 1, room):
                            out.append(b"(" + w1 + e + w2 + b")")
            memo[key] = out
            return out

        res = []
        for w1 in W:
            for w2 in W:
                for e in E(0, B - len(w1) - len(w2)):
                    res.append(b"<calc>" + w1 + e + w2 + b"</calc>")
        return res


def prefixes(members):
    P = set()
    for m in members:
        for i in range(len(m) + 1):
            P.add(m[:i])
    return P
