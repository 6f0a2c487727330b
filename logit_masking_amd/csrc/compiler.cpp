// compiler.cpp -- grammar spec -> byte-level pushdown automaton -> packed table.
//
// Three spec kinds: an arithmetic span ("Evaluator aware decoding", "This is
// a grammar problem"), a JSON schema ("Guided Decoding & Structured-Output
// Reliability", "Design 1"), and a tool call name(args) ("Constrained
// decoding", "Where it arms, and therefore where it stops").
//
// Construction is by continuation: value(n, C, d) makes a fresh state whose
// bytes start a value of schema n (with d containers already open) and whose
// completion continues in state C.  Self-delimiting values end with a byte
// edge into C; numbers end where C's bytes begin, so their accepting states
// take a copy of C's edges.  Everything a schema fixes (key order, enums,
// integer ranges, nesting of schema objects) lives in control states; only
// open JSON ({} / untyped containers) uses the object/array bit stack.
// Whitespace runs (ws_max) and string code points (caps) are registers.
//
// After construction every state that cannot reach the accepting state is
// trimmed, so "the byte is accepted" equals "the prefix can still be
// completed" -- a malformed call, an unknown key, an out-of-range number or
// a missing required key becomes unrepresentable ("Constrained decoding",
// "The guarantee").
#include <stdarg.h>
#include <string.h>

#include <algorithm>
#include <chrono>
#include <functional>
#include <map>
#include <set>
#include <string>
#include <unordered_map>
#include <vector>

#include "cg_internal.hpp"
#include "json.hpp"

namespace cg {

// The one string pattern accepted: a canonical signed decimal integer (the
// external side of the integer-string contract, "Constrained Decoding Under
// Matched Conditions", "The system boundary I am testing").  Any other
// pattern is refused.
extern const char *const kIntStringPattern;
const char *const kIntStringPattern = "^-?(0|[1-9][0-9]*)$";

static thread_local std::string g_err;

void set_error(const char *fmt, ...) {
    char buf[1024];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
}

const char *last_error() { return g_err.c_str(); }

namespace {

struct CompileError {
    int code;
    std::string msg;
};

[[noreturn]] void refuse(const std::string &path, const std::string &msg) {
    throw CompileError{CG_E_UNSUPPORTED, path + ": " + msg};
}

using u128 = unsigned __int128;
using i128 = __int128;

// ---------------------------------------------------------------------------
// Spec reading -> IR
// ---------------------------------------------------------------------------
enum Kind { K_OBJ, K_ARR, K_STR, K_INT, K_NUM, K_BOOL, K_NULL, K_ENUM, K_ANYOF, K_ANY, K_INTSTR };


enum { AK_OBJ = 1, AK_ARR = 2, AK_STR = 4, AK_NUM = 8, AK_LIT = 16, AK_ALL = 31, AK_SCALAR = 28 };

struct Node {
    Kind kind = K_ANY;
    std::vector<std::string> lits; // OBJ: key spellings; ENUM: value spellings (quoted JSON)
    std::vector<int> kids;         // OBJ: property values; ANYOF: alternatives
    std::vector<bool> req;         // OBJ
    int item = -1;                 // ARR
    int64_t max_items = -1;        // ARR (-1 none)
    int64_t cap = -1;              // STR code points (-1 none)
    bool has_lo = false, has_hi = false;
    int64_t lo = 0, hi = 0;        // INT
    int maxdigits = 0;             // INT
    int any_kinds = AK_ALL;        // ANY
    // first-byte classes of the construct as written (anyOf rule)
    unsigned first = 0;
};

// first-byte classes: '{', '[', '"', number, 't', 'f', 'n'
enum { FC_OBJ = 1, FC_ARR = 2, FC_STR = 4, FC_NUM = 8, FC_T = 16, FC_F = 32, FC_N = 64, FC_ALL = 127 };

struct Settings {
    int ws_max = 4;
    int depth_cap = 16;
    int64_t open_cap = 256;  // -1 uncapped
    int open_int_digits = 20;
    int64_t calc_min = 0, calc_max = 999;
    bool calc = true, strop = false;  // evaluators whose spans a text may hold
};

bool is_annotation(const std::string &k) {
    return k == "title" || k == "description" || k == "$comment" || k == "examples" || k == "default";
}

// The one accepted spelling of a key or enum value: JSON string with the
// escapes JSON requires and nothing else (short forms for \b \f \n \r \t,
// lowercase \u00XX for other control characters).
std::string spelling(const Json &s, const std::string &path) {
    if (s.lone_surrogate) refuse(path, "string with a lone surrogate");
    static const char *hexd = "0123456789abcdef";
    std::string o = "\"";
    for (unsigned char c : s.s) {
        switch (c) {
        case '"': o += "\\\""; break;
        case '\\': o += "\\\\"; break;
        case '\b': o += "\\b"; break;
        case '\f': o += "\\f"; break;
        case '\n': o += "\\n"; break;
        case '\r': o += "\\r"; break;
        case '\t': o += "\\t"; break;
        default:
            if (c < 0x20) {
                o += "\\u00";
                o += hexd[c >> 4];
                o += hexd[c & 15];
            } else {
                o += (char)c;
            }
        }
    }
    o += '"';
    return o;
}

bool is_plain_int(const Json *v) { return v && v->t == Json::NUM && v->is_int; }

struct Reader {
    Settings S;
    std::vector<Node> nodes;

    int add(Node n) {
        nodes.push_back(std::move(n));
        return (int)nodes.size() - 1;
    }

    std::string keylist(const Json &sch, const std::set<std::string> &allowed) {
        std::string out;
        for (auto &kv : sch.o)
            if (!is_annotation(kv.first) && !allowed.count(kv.first)) out += (out.empty() ? "" : ", ") + kv.first;
        return out;
    }

    int schema(const Json *sch, const std::string &path) {
        if (!sch || sch->t != Json::OBJ) refuse(path, "schema must be an object");
        std::set<std::string> keys;
        for (auto &kv : sch->o)
            if (!is_annotation(kv.first)) keys.insert(kv.first);
        Node n;
        if (keys.empty()) {
            n.kind = K_ANY;
            n.any_kinds = AK_ALL;
            n.first = FC_ALL;
            return add(n);
        }
        if (keys.count("anyOf")) {
            if (keys.size() != 1) refuse(path, "anyOf mixed with other keywords");
            const Json *alts = sch->get("anyOf");
            if (alts->t != Json::ARR || alts->a.empty()) refuse(path, "anyOf must be a non-empty list");
            n.kind = K_ANYOF;
            unsigned seen = 0;
            for (size_t i = 0; i < alts->a.size(); i++) {
                int k = schema(&alts->a[i], path + "/anyOf/" + std::to_string(i));
                n.kids.push_back(k);
            }
            for (int k : n.kids) {
                if (nodes[k].first & seen) refuse(path, "anyOf alternatives share a first byte");
                seen |= nodes[k].first;
            }
            n.first = seen;
            return add(n);
        }
        if (keys.count("enum")) {
            const Json *ty = sch->get("type");
            bool ok = true;
            for (auto &k : keys)
                if (k != "enum" && k != "type") ok = false;
            if (!ok || (ty && !(ty->t == Json::STR && ty->s == "string")))
                refuse(path, "only plain string enums are supported");
            const Json *vals = sch->get("enum");
            if (vals->t != Json::ARR || vals->a.empty()) refuse(path, "enum must list strings");
            for (auto &v : vals->a)
                if (v.t != Json::STR) refuse(path, "enum must list strings");
            std::set<std::string> distinct;
            for (auto &v : vals->a) distinct.insert(v.s + (v.lone_surrogate ? std::string("\x01\xff") : ""));
            if (distinct.size() != vals->a.size() || vals->a.size() > 64)
                refuse(path, "enum values must be distinct (at most 64)");
            n.kind = K_ENUM;
            for (auto &v : vals->a) n.lits.push_back(spelling(v, path));
            n.first = FC_STR;
            return add(n);
        }
        const Json *ty = sch->get("type");
        if (!ty || ty->t != Json::STR) refuse(path, "missing or non-string type");
        const std::string &t = ty->s;
        if (t == "object") {
            std::string extra = keylist(*sch, {"type", "properties", "required", "additionalProperties"});
            if (!extra.empty()) refuse(path, "unsupported keywords " + extra);
            const Json *props = sch->get("properties");
            const Json *addl = sch->get("additionalProperties");
            const Json *req = sch->get("required");
            n.first = FC_OBJ;
            if (!props || props->t == Json::NUL) {
                if (req && req->truthy()) refuse(path, "required without properties");
                if (!addl || (addl->t == Json::BOOL && addl->b)) {
                    n.kind = K_ANY;
                    n.any_kinds = AK_OBJ;
                    return add(n);
                }
                if (addl->t == Json::BOOL && !addl->b) {
                    n.kind = K_OBJ;
                    return add(n);
                }
                refuse(path, "additionalProperties must be a boolean");
            }
            if (!addl || !(addl->t == Json::BOOL && !addl->b))
                refuse(path, "properties need additionalProperties: false");
            if (props->t != Json::OBJ || props->o.size() > 64)
                refuse(path, "properties must be an object of at most 64 keys");
            std::set<std::string> reqset;
            if (req) {
                bool ok = req->t == Json::ARR;
                if (ok)
                    for (auto &r : req->a) {
                        if (r.t != Json::STR || reqset.count(r.s) || !props->get(r.s)) ok = false;
                        else reqset.insert(r.s);
                    }
                if (!ok) refuse(path, "required must list distinct declared properties");
            }
            n.kind = K_OBJ;
            for (auto &kv : props->o) {
                int k = schema(&kv.second, path + "/properties/" + kv.first);
                Json key;
                key.t = Json::STR;
                key.s = kv.first;
                n.lits.push_back(spelling(key, path));
                n.kids.push_back(k);
                n.req.push_back(reqset.count(kv.first) > 0);
            }
            return add(n);
        }
        if (t == "array") {
            std::string extra = keylist(*sch, {"type", "items", "maxItems"});
            if (!extra.empty()) refuse(path, "unsupported keywords " + extra);
            const Json *mi = sch->get("maxItems");
            int64_t m = -1;
            if (mi) {
                if (!is_plain_int(mi) || mi->i < 0) refuse(path, "maxItems must be a non-negative integer");
                m = mi->i;
            }
            n.first = FC_ARR;
            const Json *items = sch->get("items");
            if (items) {
                n.kind = K_ARR;
                n.item = schema(items, path + "/items");
                n.max_items = m;
                return add(n);
            }
            if (m < 0) {
                n.kind = K_ANY;
                n.any_kinds = AK_ARR;
                return add(n);
            }
            Node anyv;
            anyv.kind = K_ANY;
            anyv.any_kinds = AK_ALL;
            anyv.first = FC_ALL;
            n.kind = K_ARR;
            n.item = add(anyv);
            n.max_items = m;
            return add(n);
        }
        if (t == "string") {
            const Json *pat = sch->get("pattern");
            if (pat) {
                std::string extra = keylist(*sch, {"type", "pattern"});
                if (!extra.empty()) refuse(path, "unsupported keywords " + extra);
                if (pat->t != Json::STR || pat->s != kIntStringPattern)
                    refuse(path, "the only pattern supported is the canonical signed integer " +
                                     std::string(kIntStringPattern));
                n.kind = K_INTSTR;
                n.first = FC_STR;
                n.maxdigits = S.open_int_digits;
                return add(n);
            }
            std::string extra = keylist(*sch, {"type", "maxLength"});
            if (!extra.empty()) refuse(path, "unsupported keywords " + extra);
            n.kind = K_STR;
            n.first = FC_STR;
            const Json *ml = sch->get("maxLength");
            if (ml) {
                if (!is_plain_int(ml) || ml->i < 0) refuse(path, "maxLength must be a non-negative integer");
                n.cap = ml->i;
            } else {
                n.cap = S.open_cap;
            }
            return add(n);
        }
        if (t == "integer") {
            std::string extra = keylist(*sch, {"type", "minimum", "maximum"});
            if (!extra.empty()) refuse(path, "unsupported keywords " + extra);
            const Json *lo = sch->get("minimum"), *hi = sch->get("maximum");
            for (const Json *b : {lo, hi})
                if (b && b->t != Json::NUL && !is_plain_int(b)) refuse(path, "integer bounds must be 64-bit integers");
            n.kind = K_INT;
            n.first = FC_NUM;
            n.has_lo = lo && lo->t != Json::NUL;
            n.has_hi = hi && hi->t != Json::NUL;
            n.lo = n.has_lo ? lo->i : 0;
            n.hi = n.has_hi ? hi->i : 0;
            if (n.has_lo && n.has_hi && n.lo > n.hi) refuse(path, "empty integer range");
            n.maxdigits = (n.has_lo && n.has_hi) ? 19 : S.open_int_digits;
            return add(n);
        }
        {
            std::string extra = keylist(*sch, {"type"});
            if (!extra.empty()) refuse(path, "unsupported keywords " + extra);
        }
        if (t == "number") {
            n.kind = K_NUM;
            n.first = FC_NUM;
            return add(n);
        }
        if (t == "boolean") {
            n.kind = K_BOOL;
            n.first = FC_T | FC_F;
            return add(n);
        }
        if (t == "null") {
            n.kind = K_NULL;
            n.first = FC_N;
            return add(n);
        }
        refuse(path, "unknown type '" + t + "'");
    }
};

int64_t setting(const Json &spec, const char *name, int64_t dflt, int64_t lo, int64_t hi, bool allow_null,
                bool *is_null = nullptr) {
    const Json *v = spec.get(name);
    if (is_null) *is_null = false;
    if (!v) return dflt;
    if (v->t == Json::NUL && allow_null) {
        if (is_null) *is_null = true;
        return -1;
    }
    if (!is_plain_int(v) || v->i < lo || v->i > hi) refuse("$", std::string(name) + " out of range");
    return v->i;
}

// ---------------------------------------------------------------------------
// Automaton under construction
// ---------------------------------------------------------------------------
struct Edge {
    int lo, hi;
    uint32_t op, arg;
    int to;            // next state (POP: target when the stack empties; STR_OPEN: resume state)
    int to_obj = -1;   // POP: target inside an object
    int to_arr = -1;   // POP: target inside an array
};

struct BState {
    std::vector<Edge> e;
    bool string_state = false;
    bool trie_node = false;  // interior node made by trie()
    bool forced = false;     // inside a region only the engine writes
};

struct Builder {
    Settings S;
    const std::vector<Node> &N;
    std::vector<BState> st;
    int accept = -1, s_body = -1, start = -1;
    bool need_strings = false;

    Builder(const Settings &s, const std::vector<Node> &nodes) : S(s), N(nodes) {}

    int add() {
        st.emplace_back();
        return (int)st.size() - 1;
    }

    void edge(int s, int lo, int hi, uint32_t op, uint32_t arg, int to, int to_obj = -1, int to_arr = -1) {
        for (auto &x : st[s].e) {
            if (hi < x.lo || lo > x.hi) continue;
            if (x.lo == lo && x.hi == hi && x.op == op && x.arg == arg && x.to == to && x.to_obj == to_obj &&
                x.to_arr == to_arr)
                return;
            throw CompileError{CG_E_UNSUPPORTED, "$: ambiguous grammar (two continuations share a byte)"};
        }
        st[s].e.push_back(Edge{lo, hi, op, arg, to, to_obj, to_arr});
    }

    void ws_loop(int s) {
        if (S.ws_max <= 0) return;
        for (int b : {' ', '\t', '\n', '\r'}) edge(s, b, b, OP_WS, 0, s);
    }

    void copy_from(int dst, int src) {
        std::vector<Edge> es = st[src].e;  // st may grow
        for (auto &x : es) edge(dst, x.lo, x.hi, x.op, x.arg, x.to, x.to_obj, x.to_arr);
    }

    // literal alternatives from s; the last byte of each goes to `to`
    void trie(int s, const std::vector<std::string> &words, int to) {
        for (auto &w : words) {
            int cur = s;
            for (size_t i = 0; i < w.size(); i++) {
                int b = (unsigned char)w[i];
                bool last = i + 1 == w.size();
                if (last) {
                    edge(cur, b, b, OP_NONE, 0, to);
                    break;
                }
                int nxt = -1;
                for (auto &x : st[cur].e)
                    if (x.lo == b && x.hi == b && x.op == OP_NONE && st[x.to].trie_node) nxt = x.to;
                if (nxt < 0) {
                    nxt = add();
                    st[nxt].trie_node = true;
                    edge(cur, b, b, OP_NONE, 0, nxt);
                }
                cur = nxt;
            }
        }
    }

    uint32_t cap_arg(int64_t cap) const {
        if (cap < 0 || cap >= (int64_t)kUncapped) return kUncapped;
        return (uint32_t)cap;
    }

    void str_open(int s, int64_t cap, int resume) {
        need_strings = true;
        edge(s, '"', '"', OP_STR_OPEN, cap_arg(cap), resume);
    }

    // Can a value of node n be completed with `depth` containers open?
    bool sat(int n, int depth) const {
        const Node &x = N[n];
        switch (x.kind) {
        case K_OBJ:
            if (depth + 1 > S.depth_cap) return false;
            for (size_t j = 0; j < x.kids.size(); j++)
                if (x.req[j] && !sat(x.kids[j], depth + 1)) return false;
            return true;
        case K_ARR:
            return depth + 1 <= S.depth_cap;
        case K_ANYOF:
            for (int k : x.kids)
                if (sat(k, depth)) return true;
            return false;
        case K_ANY:
            if (x.any_kinds & AK_SCALAR) return true;
            return depth + 1 <= S.depth_cap;
        default:
            return true;
        }
    }

    // ---- values -------------------------------------------------------
    int value(int n, int C, int depth) {
        if (!sat(n, depth)) return -1;
        const Node &x = N[n];
        int s = add();
        switch (x.kind) {
        case K_STR: str_open(s, x.cap, C); break;
        case K_ENUM: trie(s, x.lits, C); break;
        case K_BOOL: trie(s, {"true", "false"}, C); break;
        case K_NULL: trie(s, {"null"}, C); break;
        case K_INT: integer(s, x, C); break;
        case K_INTSTR: {
            // '"' -?(0|[1-9][0-9]*) '"' with at most maxdigits digits (the
            // pattern itself admits "-0")
            const int I = add(), M = add(), Z = add();
            edge(s, '"', '"', OP_NONE, 0, I);
            edge(I, '-', '-', OP_NONE, 0, M);
            std::vector<int> D(x.maxdigits + 1);
            for (int k = 1; k <= x.maxdigits; k++) D[k] = add();
            for (int from : {I, M}) {
                edge(from, '0', '0', OP_NONE, 0, Z);
                edge(from, '1', '9', OP_NONE, 0, D[1]);
            }
            for (int k = 1; k < x.maxdigits; k++) edge(D[k], '0', '9', OP_NONE, 0, D[k + 1]);
            edge(Z, '"', '"', OP_NONE, 0, C);
            for (int k = 1; k <= x.maxdigits; k++) edge(D[k], '"', '"', OP_NONE, 0, C);
            break;
        }
        case K_NUM: number(s, C); break;
        case K_ANYOF:
            for (int k : x.kids) {
                int a = value(k, C, depth);
                if (a >= 0) copy_from(s, a);
            }
            break;
        case K_OBJ: object(s, x, C, depth); break;
        case K_ARR: array(s, x, C, depth); break;
        case K_ANY: any_json(s, x.any_kinds, C, depth); break;
        }
        return s;
    }

    // closed object: keys in declared order, optional keys may be skipped
    void object(int s, const Node &x, int C, int depth) {
        const int d1 = depth + 1, n = (int)x.kids.size();
        std::vector<bool> ok(n);
        for (int j = 0; j < n; j++) ok[j] = sat(x.kids[j], d1);
        auto cands = [&](int i) {
            std::vector<int> c;
            for (int j = i + 1; j < n; j++) {
                if (ok[j]) c.push_back(j);
                if (x.req[j]) break;
            }
            return c;
        };
        auto may_close = [&](int i) {
            for (int j = i + 1; j < n; j++)
                if (x.req[j]) return false;
            return true;
        };
        std::vector<int> AV(n, -1), AX(n, -1), AK(n, -1), AC(n, -1);
        for (int j = 0; j < n; j++)
            if (ok[j]) {
                AV[j] = add();
                AX[j] = add();
                AK[j] = add();
            }
        std::map<std::vector<int>, int> tries;
        auto trie_for = [&](const std::vector<int> &c) {
            auto it = tries.find(c);
            if (it != tries.end()) return it->second;
            int root = add();
            for (int j : c) trie(root, {x.lits[j].substr(1)}, AK[j]);
            tries[c] = root;
            return root;
        };
        int P0 = add();
        edge(s, '{', '{', OP_NONE, 0, P0);
        ws_loop(P0);
        {
            auto c = cands(-1);
            if (!c.empty()) edge(P0, '"', '"', OP_NONE, 0, trie_for(c));
            if (may_close(-1)) edge(P0, '}', '}', OP_NONE, 0, C);
        }
        for (int j = 0; j < n; j++) {
            if (!ok[j]) continue;
            ws_loop(AV[j]);
            auto c = cands(j);
            if (!c.empty()) {
                edge(AV[j], ',', ',', OP_NONE, 0, AX[j]);
                ws_loop(AX[j]);
                edge(AX[j], '"', '"', OP_NONE, 0, trie_for(c));
            }
            if (may_close(j)) edge(AV[j], '}', '}', OP_NONE, 0, C);
        }
        for (int j = 0; j < n; j++) {
            if (!ok[j]) continue;
            AC[j] = value(x.kids[j], AV[j], d1);
            ws_loop(AC[j]);
            ws_loop(AK[j]);
            edge(AK[j], ':', ':', OP_NONE, 0, AC[j]);
        }
    }

    void array(int s, const Node &x, int C, int depth) {
        const int d1 = depth + 1;
        int P0 = add();
        edge(s, '[', '[', OP_NONE, 0, P0);
        ws_loop(P0);
        edge(P0, ']', ']', OP_NONE, 0, C);
        if (x.max_items == 0 || !sat(x.item, d1)) return;
        if (x.max_items < 0) {
            int AV = add(), AX = add();
            ws_loop(AV);
            edge(AV, ',', ',', OP_NONE, 0, AX);
            edge(AV, ']', ']', OP_NONE, 0, C);
            int I = value(x.item, AV, d1);
            copy_from(P0, I);
            ws_loop(AX);
            copy_from(AX, I);
            return;
        }
        const int64_t m = x.max_items;
        if (m > 256) throw CompileError{CG_E_LIMIT, "$: maxItems above 256"};
        std::vector<int> AV(m);
        for (int64_t k = 0; k < m; k++) AV[k] = add();
        std::vector<int> AX(m, -1);
        for (int64_t k = 0; k < m; k++) {
            ws_loop(AV[k]);
            if (k + 1 < m) {
                AX[k] = add();
                edge(AV[k], ',', ',', OP_NONE, 0, AX[k]);
            }
            edge(AV[k], ']', ']', OP_NONE, 0, C);
        }
        copy_from(P0, value(x.item, AV[0], d1));
        for (int64_t k = 1; k < m; k++) {
            ws_loop(AX[k - 1]);
            copy_from(AX[k - 1], value(x.item, AV[k], d1));
        }
    }

    // RFC 8259 number; accepting states continue with C's bytes
    void number(int s, int C) {
        int NM = add(), NZ = add(), NI = add(), ND = add(), NF = add(), NE = add(), NS = add(), NX = add();
        edge(s, '-', '-', OP_NONE, 0, NM);
        edge(s, '0', '0', OP_NONE, 0, NZ);
        edge(s, '1', '9', OP_NONE, 0, NI);
        edge(NM, '0', '0', OP_NONE, 0, NZ);
        edge(NM, '1', '9', OP_NONE, 0, NI);
        for (int q : {NZ, NI}) {
            edge(q, '.', '.', OP_NONE, 0, ND);
            edge(q, 'e', 'e', OP_NONE, 0, NE);
            edge(q, 'E', 'E', OP_NONE, 0, NE);
        }
        edge(NI, '0', '9', OP_NONE, 0, NI);
        edge(ND, '0', '9', OP_NONE, 0, NF);
        edge(NF, '0', '9', OP_NONE, 0, NF);
        edge(NF, 'e', 'e', OP_NONE, 0, NE);
        edge(NF, 'E', 'E', OP_NONE, 0, NE);
        edge(NE, '+', '+', OP_NONE, 0, NS);
        edge(NE, '-', '-', OP_NONE, 0, NS);
        edge(NE, '0', '9', OP_NONE, 0, NX);
        edge(NS, '0', '9', OP_NONE, 0, NX);
        edge(NX, '0', '9', OP_NONE, 0, NX);
        for (int q : {NZ, NI, NF, NX}) copy_from(q, C);
    }

    // Canonical decimal magnitudes in [a, b] (at most D digits), as a DFA
    // whose states are the sets of digit suffixes that still complete a
    // value: per suffix length k, an interval of k-digit suffixes.
    void magnitude(int root, u128 a, u128 b, int D, int C) {
        typedef std::vector<std::pair<u128, u128>> Sig;  // (lo, hi+1); lo == hi+1 means empty
        auto pw = [](int k) {
            u128 r = 1;
            while (k-- > 0) r *= 10;
            return r;
        };
        auto sig_of = [&](u128 p, int L, bool zero) {
            Sig s;
            for (int k = 0; k + L <= D; k++) {
                if (zero && k > 0) break;
                u128 lo = p * pw(k), hi = (p + 1) * pw(k) - 1;
                u128 x = std::max(lo, a), y = std::min(hi, b);
                if (x > y) s.push_back({0, 0});
                else s.push_back({x - lo, y - lo + 1});
            }
            while (!s.empty() && s.back().first == s.back().second) s.pop_back();
            return s;
        };
        std::map<Sig, int> ids;
        struct Item {
            int id;
            u128 p;
            int L;
            bool zero;
        };
        std::vector<Item> work;
        auto get = [&](u128 p, int L, bool zero, bool *fresh) {
            Sig s = sig_of(p, L, zero);
            if (s.empty()) return -1;
            auto it = ids.find(s);
            if (it != ids.end()) {
                *fresh = false;
                return it->second;
            }
            int id = add();
            ids[s] = id;
            *fresh = true;
            if (s[0].first != s[0].second) copy_from(id, C);  // the digits so far are a value
            work.push_back({id, p, L, zero});
            return id;
        };
        for (int d = 0; d <= 9; d++) {
            bool fresh;
            int c = get((u128)d, 1, d == 0, &fresh);
            if (c >= 0) edge(root, '0' + d, '0' + d, OP_NONE, 0, c);
        }
        for (size_t w = 0; w < work.size(); w++) {
            Item it = work[w];
            if (it.zero || it.L >= D) continue;
            for (int d = 0; d <= 9; d++) {
                bool fresh;
                int c = get(it.p * 10 + (u128)d, it.L + 1, false, &fresh);
                if (c >= 0) edge(it.id, '0' + d, '0' + d, OP_NONE, 0, c);
            }
        }
    }

    void integer(int s, const Node &x, int C) {
        i128 big = 1;
        for (int k = 0; k < x.maxdigits; k++) big *= 10;
        big -= 1;
        i128 lo = x.has_lo ? (i128)x.lo : -big, hi = x.has_hi ? (i128)x.hi : big;
        if (hi >= 0) magnitude(s, (u128)std::max<i128>(lo, 0), (u128)hi, x.maxdigits, C);
        if (lo < 0) {
            i128 a = std::max<i128>(1, -hi), b = -lo;
            if (a <= b) {
                int M = add();
                edge(s, '-', '-', OP_NONE, 0, M);
                magnitude(M, (u128)a, (u128)b, x.maxdigits, C);
            }
        }
    }

    // scalar or container value of open JSON at state X, continuing in T
    void any_start(int X, int kinds, int T, int cap, int OB, int AR) {
        if (kinds & AK_STR) str_open(X, S.open_cap, T);
        if (kinds & AK_NUM) number(X, T);
        if (kinds & AK_LIT) trie(X, {"true", "false", "null"}, T);
        if (cap >= 1 && (kinds & AK_OBJ)) edge(X, '{', '{', OP_PUSH, ((uint32_t)cap << 1) | 0u, OB);
        if (cap >= 1 && (kinds & AK_ARR)) edge(X, '[', '[', OP_PUSH, ((uint32_t)cap << 1) | 1u, AR);
    }

    // open JSON value (RFC 8259) with containers on the bit stack; at most
    // depth_cap - depth containers may be open inside it
    void any_json(int s, int kinds, int C, int depth) {
        const int cap = S.depth_cap - depth;
        if (cap < 1 || !(kinds & (AK_OBJ | AK_ARR))) {
            any_start(s, kinds & AK_SCALAR, C, 0, -1, -1);
            return;
        }
        int OB = add(), AKo = add(), ACo = add(), AVo = add(), AXo = add();
        int AR = add(), AVa = add(), AXa = add();
        auto pop = [&](int q, int b) { edge(q, b, b, OP_POP, 0, C, AVo, AVa); };
        ws_loop(OB);
        str_open(OB, S.open_cap, AKo);
        pop(OB, '}');
        ws_loop(AKo);
        edge(AKo, ':', ':', OP_NONE, 0, ACo);
        ws_loop(AVo);
        edge(AVo, ',', ',', OP_NONE, 0, AXo);
        pop(AVo, '}');
        ws_loop(AXo);
        str_open(AXo, S.open_cap, AKo);
        ws_loop(AVa);
        edge(AVa, ',', ',', OP_NONE, 0, AXa);
        pop(AVa, ']');
        ws_loop(ACo);
        any_start(ACo, AK_ALL, AVo, cap, OB, AR);
        ws_loop(AR);
        pop(AR, ']');
        any_start(AR, AK_ALL, AVa, cap, OB, AR);
        ws_loop(AXa);
        any_start(AXa, AK_ALL, AVa, cap, OB, AR);
        any_start(s, kinds, C, cap, OB, AR);
    }

    // ---- string body (shared by every string; the resume state is a register)
    void strings() {
        int SB = add(), T1 = add(), T2 = add(), T2a = add(), T2d = add(), T3 = add(), T3a = add(), T3d = add();
        int SE = add(), U0 = add(), U1 = add(), U1d = add(), U2 = add(), U3 = add();
        for (int q : {SB, T1, T2, T2a, T2d, T3, T3a, T3d, SE, U0, U1, U1d, U2, U3}) st[q].string_state = true;
        s_body = SB;
        edge(SB, '"', '"', OP_STR_CLOSE, 0, SB);
        edge(SB, '\\', '\\', OP_CHAR, 0, SE);
        edge(SB, 0x20, 0x21, OP_CHAR, 0, SB);
        edge(SB, 0x23, 0x5B, OP_CHAR, 0, SB);
        edge(SB, 0x5D, 0x7F, OP_CHAR, 0, SB);
        // well-formed UTF-8 (Unicode Table 3-7): the lead byte counts the code point
        edge(SB, 0xC2, 0xDF, OP_CHAR, 0, T1);
        edge(SB, 0xE0, 0xE0, OP_CHAR, 0, T2a);
        edge(SB, 0xE1, 0xEC, OP_CHAR, 0, T2);
        edge(SB, 0xED, 0xED, OP_CHAR, 0, T2d);
        edge(SB, 0xEE, 0xEF, OP_CHAR, 0, T2);
        edge(SB, 0xF0, 0xF0, OP_CHAR, 0, T3a);
        edge(SB, 0xF1, 0xF3, OP_CHAR, 0, T3);
        edge(SB, 0xF4, 0xF4, OP_CHAR, 0, T3d);
        edge(T1, 0x80, 0xBF, OP_NONE, 0, SB);
        edge(T2, 0x80, 0xBF, OP_NONE, 0, T1);
        edge(T2a, 0xA0, 0xBF, OP_NONE, 0, T1);
        edge(T2d, 0x80, 0x9F, OP_NONE, 0, T1);
        edge(T3, 0x80, 0xBF, OP_NONE, 0, T2);
        edge(T3a, 0x90, 0xBF, OP_NONE, 0, T2);
        edge(T3d, 0x80, 0x8F, OP_NONE, 0, T2);
        for (int b : {'"', '\\', '/', 'b', 'f', 'n', 'r', 't'}) edge(SE, b, b, OP_NONE, 0, SB);
        edge(SE, 'u', 'u', OP_NONE, 0, U0);
        // \uXXXX outside the surrogate block D800-DFFF
        auto hex = [&](int q, int to, bool no_d, bool low_only) {
            if (low_only) {
                edge(q, '0', '7', OP_NONE, 0, to);
                return;
            }
            edge(q, '0', '9', OP_NONE, 0, to);
            edge(q, 'a', no_d ? 'c' : 'f', OP_NONE, 0, to);
            edge(q, 'A', no_d ? 'C' : 'F', OP_NONE, 0, to);
            if (no_d) {
                edge(q, 'e', 'f', OP_NONE, 0, to);
                edge(q, 'E', 'F', OP_NONE, 0, to);
            }
        };
        hex(U0, U1, true, false);
        edge(U0, 'd', 'd', OP_NONE, 0, U1d);
        edge(U0, 'D', 'D', OP_NONE, 0, U1d);
        hex(U1, U2, false, false);
        hex(U1d, U2, false, true);
        hex(U2, U3, false, false);
        hex(U3, SB, false, false);
    }

    // ---- whole grammars -----------------------------------------------
    // "<calc>" W E W "</calc>" from state `from` to state `to`
    void calc_span(int from, int to) {
        int ETt = add(), ETi = add(), ATt = add(), ATi = add();
        for (int q : {ETt, ETi, ATt, ATi}) ws_loop(q);
        for (int op : {'+', '-', '*', '/'}) {
            edge(ATt, op, op, OP_NONE, 0, ETt);
            edge(ATi, op, op, OP_NONE, 0, ETi);
        }
        trie(ATt, {"</calc>"}, to);
        edge(ATi, ')', ')', OP_POP, 0, ATt, ATi, ATi);
        const uint32_t push = ((uint32_t)S.depth_cap << 1);
        edge(ETt, '(', '(', OP_PUSH, push, ETi);
        edge(ETi, '(', '(', OP_PUSH, push, ETi);
        magnitude(ETt, (u128)S.calc_min, (u128)S.calc_max, 19, ATt);
        magnitude(ETi, (u128)S.calc_min, (u128)S.calc_max, 19, ATi);
        trie(from, {"<calc>"}, ETt);
    }

    void calc() {
        start = add();
        calc_span(start, accept);
    }

    // A string-operation span ("Evaluator aware decoding", "Not just
    // arithmetic: string operations"): "<strop>" NAME "(" W ARGS W ")"
    // "</strop>" with NAME(ARGS) one of count(S, S), len(S), reverse(S),
    // upper(S), substr(S, I, I); arguments separated by W "," W; S = '"'
    // (printable ASCII other than '"', '\\' and '<')* '"'; I = "-"? digit{1,6}.
    void strop_span(int from, int to) {
        const int NS = add();
        trie(from, {"<strop>"}, NS);
        const int T = add();
        trie(T, {"</strop>"}, to);
        auto str_arg = [&](int s) {
            const int Bd = add(), E = add();
            edge(s, '"', '"', OP_NONE, 0, Bd);
            edge(Bd, 0x20, 0x21, OP_NONE, 0, Bd);
            edge(Bd, 0x23, 0x3B, OP_NONE, 0, Bd);
            edge(Bd, 0x3D, 0x5B, OP_NONE, 0, Bd);
            edge(Bd, 0x5D, 0x7E, OP_NONE, 0, Bd);
            edge(Bd, '"', '"', OP_NONE, 0, E);
            return E;
        };
        const struct {
            const char *name;
            const char *args;  // S: string, I: integer
        } ops[] = {{"count(", "SS"}, {"len(", "S"}, {"reverse(", "S"}, {"upper(", "S"}, {"substr(", "SII"}};
        for (const auto &op : ops) {
            int q = add();
            trie(NS, {op.name}, q);
            ws_loop(q);
            const int n = (int)strlen(op.args);
            for (int i = 0; i < n; i++) {
                const bool last = i + 1 == n;
                // what follows an argument: whitespace, then ',' and the next argument, or ')'
                const int J = add(), N = last ? -1 : add();
                ws_loop(J);
                if (last) edge(J, ')', ')', OP_NONE, 0, T);
                else edge(J, ',', ',', OP_NONE, 0, N);
                if (op.args[i] == 'S') {
                    copy_from(str_arg(q), J);
                } else {
                    const int M = add();
                    int D[7];
                    for (int k = 1; k <= 6; k++) D[k] = add();
                    edge(q, '-', '-', OP_NONE, 0, M);
                    edge(q, '0', '9', OP_NONE, 0, D[1]);
                    edge(M, '0', '9', OP_NONE, 0, D[1]);
                    for (int k = 1; k < 6; k++) edge(D[k], '0', '9', OP_NONE, 0, D[k + 1]);
                    for (int k = 1; k <= 6; k++) copy_from(D[k], J);
                }
                if (!last) {
                    ws_loop(N);
                    q = N;
                }
            }
        }
    }

    // Text with evaluated spans: TEXT* (SPAN RESULT TEXT*)* "<end>", TEXT = LF
    // or printable ASCII other than '<', SPAN a calc span and/or a string
    // operation (the evaluators the spec names).  RESULT is written by the
    // engine, never sampled, so its states are marked forced: after a calc
    // span "<result>" "-"? digit{1,20} "</result>", after a string operation
    // "<result>" TEXT' "</result>" (TEXT' = printable ASCII other than '<'),
    // or after either "<result_error>" MSG "</result_error>" for a failed
    // evaluation, MSG = printable ASCII other than '<'.
    void calc_text() {
        const int TX = start = add();
        edge(TX, '\n', '\n', OP_NONE, 0, TX);
        edge(TX, 0x20, '<' - 1, OP_NONE, 0, TX);
        edge(TX, '<' + 1, 0x7E, OP_NONE, 0, TX);
        const int R0 = S.calc ? add() : -1, R1 = S.strop ? add() : -1;
        if (S.calc) calc_span(TX, R0);
        if (S.strop) strop_span(TX, R1);
        trie(TX, {"<end>"}, accept);
        const int first_forced = (int)st.size();
        const int RM = add();
        edge(RM, 0x20, '<' - 1, OP_NONE, 0, RM);
        edge(RM, '<' + 1, 0x7E, OP_NONE, 0, RM);
        trie(RM, {"</result_error>"}, TX);
        if (S.calc) {
            const int RV = add(), RN = add();
            int RD[21];
            for (int d = 1; d <= 20; d++) RD[d] = add();
            trie(R0, {"<result>"}, RV);
            trie(R0, {"<result_error>"}, RM);
            edge(RV, '-', '-', OP_NONE, 0, RN);
            edge(RV, '0', '9', OP_NONE, 0, RD[1]);
            edge(RN, '0', '9', OP_NONE, 0, RD[1]);
            for (int d = 1; d <= 20; d++) {
                if (d < 20) edge(RD[d], '0', '9', OP_NONE, 0, RD[d + 1]);
                trie(RD[d], {"</result>"}, TX);
            }
            st[R0].forced = true;
        }
        if (S.strop) {
            const int RT = add();
            trie(R1, {"<result>"}, RT);
            trie(R1, {"<result_error>"}, RM);
            edge(RT, 0x20, '<' - 1, OP_NONE, 0, RT);
            edge(RT, '<' + 1, 0x7E, OP_NONE, 0, RT);
            trie(RT, {"</result>"}, TX);
            st[R1].forced = true;
        }
        for (int q = first_forced; q < (int)st.size(); q++) st[q].forced = true;
    }
};

// ---------------------------------------------------------------------------
// Trim, pack
// ---------------------------------------------------------------------------
void trim_and_pack(Builder &B, cg_grammar *g) {
    const int n = (int)B.st.size();
    // live = can reach the accepting state (string states always can: a
    // string may close at any code-point boundary and resumes in `ret`)
    std::vector<bool> live(n, false);
    live[B.accept] = true;
    for (int q = 0; q < n; q++)
        if (B.st[q].string_state) live[q] = true;
    auto edge_live = [&](const Edge &e) {
        if (e.op == OP_STR_CLOSE) return true;
        if (e.op == OP_POP) return (bool)live[e.to];  // inside, the targets live iff the exit does
        return (bool)live[e.to];
    };
    for (bool changed = true; changed;) {
        changed = false;
        for (int q = 0; q < n; q++) {
            if (live[q]) continue;
            for (auto &e : B.st[q].e)
                if (edge_live(e)) {
                    live[q] = true;
                    changed = true;
                    break;
                }
        }
    }
    if (!live[B.start]) throw CompileError{CG_E_UNSUPPORTED, "$: grammar accepts no string"};
    for (int q = 0; q < n; q++) {
        auto &es = B.st[q].e;
        es.erase(std::remove_if(es.begin(), es.end(), [&](const Edge &e) { return !edge_live(e); }), es.end());
    }
    // reachable from the start
    std::vector<bool> reach(n, false);
    std::vector<int> stack{B.start};
    reach[B.start] = true;
    auto visit = [&](int q) {
        if (q >= 0 && !reach[q]) {
            reach[q] = true;
            stack.push_back(q);
        }
    };
    while (!stack.empty()) {
        int q = stack.back();
        stack.pop_back();
        for (auto &e : B.st[q].e) {
            if (e.op == OP_STR_OPEN) visit(B.s_body);
            if (e.op != OP_STR_CLOSE) visit(e.to);
            visit(e.to_obj);
            visit(e.to_arr);
        }
    }
    reach[B.accept] = true;
    if (B.s_body >= 0 && reach[B.s_body])
        for (int q = 0; q < n; q++)
            if (B.st[q].string_state) reach[q] = true;
    // row displacement: densest rows first, first fit
    std::vector<int> order;
    for (int q = 0; q < n; q++)
        if (reach[q]) order.push_back(q);
    auto width = [&](int q) {
        int w = 0;
        for (auto &e : B.st[q].e) w += e.hi - e.lo + 1;
        return w;
    };
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return width(a) > width(b); });
    std::vector<char> used;   // slot occupied
    std::vector<char> isbase; // base taken
    std::vector<int> base(n, -1);
    int max_base = 0;
    for (int q : order) {
        std::vector<int> bytes;
        for (auto &e : B.st[q].e)
            for (int b = e.lo; b <= e.hi; b++) bytes.push_back(b);
        for (int bs = 0;; bs++) {
            if ((size_t)bs + 256 > used.size()) {
                used.resize(bs + 512, 0);
                isbase.resize(bs + 512, 0);
            }
            if (isbase[bs]) continue;
            bool fits = true;
            for (int b : bytes)
                if (used[bs + b]) {
                    fits = false;
                    break;
                }
            if (!fits) continue;
            for (int b : bytes) used[bs + b] = 1;
            isbase[bs] = 1;
            base[q] = bs;
            max_base = std::max(max_base, bs);
            break;
        }
    }
    if (max_base > (int)kMaxStateId)
        throw CompileError{CG_E_LIMIT, "$: automaton too large (" + std::to_string(order.size()) + " states)"};
    const uint32_t comb_len = (uint32_t)max_base + 1 + 256;
    if (comb_len * sizeof(uint64_t) > 60 * 1024)
        throw CompileError{CG_E_LIMIT, "$: transition table of " + std::to_string(comb_len * 8) +
                                           " bytes exceeds the 60 KiB staged in LDS"};
    uint64_t *comb = (uint64_t *)malloc(sizeof(uint64_t) * comb_len);
    const uint32_t start_id = (uint32_t)base[B.start];
    for (uint32_t i = 0; i < comb_len; i++) comb[i] = (uint64_t)kEmptyOwner | ((uint64_t)start_id << 16);
    for (int q : order) {
        for (auto &e : B.st[q].e) {
            uint32_t next = 0, arg = e.arg;
            if (e.op == OP_STR_CLOSE) next = start_id;
            else next = (uint32_t)base[e.to];
            if (e.op == OP_POP) arg = (uint32_t)base[e.to_obj] | ((uint32_t)base[e.to_arr] << 14);
            for (int b = e.lo; b <= e.hi; b++) {
                const uint32_t owner = (uint32_t)base[q] | (B.st[q].forced ? kEngineOwner : 0u);
                uint64_t lo32 = (uint64_t)owner | ((uint64_t)next << 16);
                uint64_t hi32 = (uint64_t)e.op | ((uint64_t)arg << 4);
                comb[base[q] + b] = lo32 | (hi32 << 32);
            }
        }
    }
    g->host_forced.assign(((size_t)max_base + 1 + 31) / 32, 0u);
    for (int q : order)
        if (B.st[q].forced) g->host_forced[base[q] >> 5] |= 1u << (base[q] & 31);
    g->has_forced = std::any_of(order.begin(), order.end(), [&](int q) { return B.st[q].forced; });
    g->plain_q.clear();
    for (int q : order)
        if (!B.st[q].string_state && !B.st[q].forced && q != B.accept) g->plain_q.push_back((uint32_t)base[q]);
    std::sort(g->plain_q.begin(), g->plain_q.end());
    g->host_comb = comb;
    g->comb_len = comb_len;
    g->n_states = (int)order.size();
    g->k.start = start_id;
    g->k.accept = (uint32_t)base[B.accept];
    g->k.s_body = (B.s_body >= 0 && reach[B.s_body]) ? (uint32_t)base[B.s_body] : 0xFFFFu;
    g->k.ws_max = (uint32_t)B.S.ws_max;
    g->k.q_limit = (uint32_t)max_base + 1;
}

// ---- the longest member ------------------------------------------------
// The language's longest member in bytes, or -1 when the language is
// infinite: the longest path from the start configuration to the accepting
// state in the configuration graph of the packed automaton (the walker's
// rules, step_byte).  Outside strings a configuration is (state, whitespace
// run, container stack); a string, from its opening quote to its closing
// one, is a single edge of 2 + cap x P bytes, where P is the longest path of
// the string machine from its body state back to it (one code point: each
// such path starts with the one OP_CHAR that spends the budget).  A cycle
// through a configuration that can still reach the accepting state, or a
// string with no cap, makes the language infinite.
struct LongestMember {
    const uint64_t *comb;
    WalkConsts k;
    static constexpr int64_t kDead = INT64_MIN / 4;
    struct Cfg {
        uint32_t q, ws, depth;
        uint64_t stk;
        bool operator==(const Cfg &o) const { return q == o.q && ws == o.ws && depth == o.depth && stk == o.stk; }
    };
    struct Hash {
        size_t operator()(const Cfg &c) const {
            return std::hash<uint64_t>()(c.stk * 0x9E3779B97F4A7C15ull ^ ((uint64_t)c.q << 24 | c.ws << 16 | c.depth));
        }
    };
    struct Infinite {};
    std::unordered_map<Cfg, int64_t, Hash> memo;  // kGray while on the search path
    static constexpr int64_t kGray = INT64_MIN / 2;
    int64_t code_point = 0;  // P

    // the edges of a configuration outside strings: (next, bytes); false if
    // the byte is refused there
    bool step(const Cfg &c, uint32_t b, Cfg &n, int64_t &w) const {
        const uint64_t e = comb[c.q + b];
        const uint32_t lo = (uint32_t)e, hi = (uint32_t)(e >> 32);
        if ((lo & 0x7FFFu) != c.q) return false;  // the engine's bytes belong to the output too
        const uint32_t op = hi & 0xFu, arg = hi >> 4;
        n = c;
        n.q = lo >> 16;
        n.ws = op == OP_WS ? c.ws + 1 : 0;
        if (n.ws > k.ws_max) return false;
        w = 1;
        switch (op) {
        case OP_STR_OPEN:
            if (arg == kUncapped) throw Infinite{};
            w = 2 + (int64_t)arg * code_point;  // the body from state k.s_body, then the closing quote
            return true;
        case OP_PUSH:
            if (c.depth >= (arg >> 1)) return false;
            n.stk = (c.stk << 1) | (arg & 1u);
            n.depth = c.depth + 1;
            return true;
        case OP_POP:
            if (c.depth == 0) return false;
            n.stk = c.stk >> 1;
            n.depth = c.depth - 1;
            n.q = n.depth == 0 ? n.q : ((n.stk & 1u) ? (arg >> 14) : (arg & 0x3FFFu));
            return true;
        case OP_NONE:
        case OP_WS:
            return true;
        default:  // code points and closing quotes occur only inside the string machine
            return false;
        }
    }

    // breadth first, so the nearest way out is found first
    bool reaches_accept(const Cfg &from) const {
        std::unordered_map<Cfg, char, Hash> seen;
        std::vector<Cfg> todo{from};
        seen[from] = 1;
        for (size_t i = 0; i < todo.size(); i++) {
            const Cfg c = todo[i];
            if (c.q == k.accept) return true;
            if (seen.size() > (1u << 22)) return true;  // (not reached by these grammars)
            for (uint32_t b = 0; b < 256; b++) {
                Cfg n;
                int64_t w;
                if (step(c, b, n, w) && seen.emplace(n, 1).second) todo.push_back(n);
            }
        }
        return false;
    }

    int64_t longest(const Cfg &c) {
        if (c.q == k.accept) return 0;
        auto it = memo.find(c);
        if (it != memo.end()) {
            if (it->second != kGray) return it->second;
            if (reaches_accept(c)) throw Infinite{};
            return kDead;  // a cycle that cannot end
        }
        memo[c] = kGray;
        int64_t best = kDead;
        for (uint32_t b = 0; b < 256; b++) {
            Cfg n;
            int64_t w;
            if (!step(c, b, n, w)) continue;
            const int64_t v = longest(n);
            if (v != kDead) best = std::max(best, w + v);
        }
        memo[c] = best;
        return best;
    }

    // P: the longest code point of the string machine, each path from the
    // body state back to it holding exactly one OP_CHAR (its first edge)
    int64_t string_body() const {
        if (k.s_body >= k.q_limit) return 0;
        std::unordered_map<uint32_t, int64_t> f;  // longest path from a state inside a code point back to the body
        std::function<int64_t(uint32_t)> back = [&](uint32_t q) -> int64_t {
            if (q == k.s_body) return 0;
            auto it = f.find(q);
            if (it != f.end()) {
                if (it->second == kGray) throw Infinite{};
                return it->second;
            }
            f[q] = kGray;
            int64_t best = kDead;
            for (uint32_t b = 0; b < 256; b++) {
                const uint64_t e = comb[q + b];
                if (((uint32_t)e & 0xFFFFu) != q) continue;
                // (inside a code point every edge is a plain move)
                const int64_t v = back(((uint32_t)e >> 16) & 0xFFFFu);
                if (v != kDead) best = std::max(best, 1 + v);
            }
            f[q] = best;
            return best;
        };
        int64_t p = 0;
        for (uint32_t b = 0; b < 256; b++) {
            const uint64_t e = comb[k.s_body + b];
            if (((uint32_t)e & 0xFFFFu) != k.s_body) continue;
            const uint32_t op = (uint32_t)(e >> 32) & 0xFu;
            if (op != OP_CHAR) continue;  // the closing quote
            const int64_t v = back(((uint32_t)e >> 16) & 0xFFFFu);
            if (v != kDead) p = std::max(p, 1 + v);
        }
        return p;
    }

    int64_t run() {
        try {
            code_point = string_body();
            const int64_t v = longest(Cfg{k.start, 0, 0, 0});
            return v < 0 ? -1 : v;
        } catch (const Infinite &) {
            return -1;
        }
    }
};

}  // namespace

int compile_spec(const char *spec, size_t len, cg_grammar *g) {
    auto t0 = std::chrono::steady_clock::now();
    try {
        Json root;
        try {
            root = JsonReader(spec, len).parse();
        } catch (const JsonError &e) {
            set_error("spec is not valid JSON: %s", e.msg.c_str());
            return CG_E_PARSE;
        }
        if (root.t != Json::OBJ) {
            set_error("spec must be a JSON object");
            return CG_E_PARSE;
        }
        Settings S;
        S.ws_max = (int)setting(root, "ws_max", 4, 0, 64, false);
        S.depth_cap = (int)setting(root, "depth_cap", 16, 1, 64, false);
        S.open_cap = setting(root, "open_string_cap", 256, 0, (int64_t)1 << 24, true);
        S.open_int_digits = (int)setting(root, "open_int_digits", 20, 1, 20, false);
        const Json *kind = root.get("kind");
        std::string k = (kind && kind->t == Json::STR) ? kind->s : "";
        Reader R;
        R.S = S;
        int json_root = -1;
        std::vector<std::pair<std::string, int>> tools;
        if (k == "calc" || k == "calc_text") {
            S.calc_min = setting(root, "int_min", 0, 0, 1000000000, false);
            S.calc_max = setting(root, "int_max", 999, 0, 1000000000, false);
            if (S.calc_min > S.calc_max) refuse("$", "empty integer range");
            if (const Json *ev = root.get("evaluators")) {
                if (k != "calc_text" || ev->t != Json::ARR || ev->a.empty())
                    refuse("$.evaluators", "evaluators must be a non-empty list (calc_text only)");
                S.calc = S.strop = false;
                for (auto &e : ev->a) {
                    if (e.t == Json::STR && e.s == "calc") S.calc = true;
                    else if (e.t == Json::STR && e.s == "strop") S.strop = true;
                    else refuse("$.evaluators", "evaluators are \"calc\" and \"strop\"");
                }
            }
        } else if (k == "json_schema") {
            json_root = R.schema(root.get("schema"), "$.schema");
            if (R.nodes[json_root].first & FC_NUM)
                refuse("$.schema", "the root value must end by itself (object, array, string, literal)");
        } else if (k == "tool_call") {
            const Json *ts = root.get("tools");
            if (!ts || ts->t != Json::ARR || ts->a.empty() || ts->a.size() > 64)
                refuse("$.tools", "tools must be a list of 1-64 tools");
            std::vector<std::string> names;
            for (auto &t : ts->a) {
                const Json *nm = t.t == Json::OBJ ? t.get("name") : nullptr;
                names.push_back(nm && nm->t == Json::STR ? nm->s : std::string("\x01"));
            }
            for (size_t i = 0; i < ts->a.size(); i++) {
                const std::string p = "$.tools/" + std::to_string(i);
                const std::string &nm = names[i];
                bool ok = !nm.empty() && nm != "\x01";
                for (unsigned char c : nm)
                    if (!(isalnum(c) || c == '_' || c == '.' || c == '-') || c >= 0x80) ok = false;
                if (!ok) refuse(p, "tool names are non-empty [A-Za-z0-9_.-]");
                if (std::count(names.begin(), names.end(), nm) > 1) refuse(p, "duplicate tool name");
                const Json *params = ts->a[i].get("parameters");
                const Json *pt = params && params->t == Json::OBJ ? params->get("type") : nullptr;
                if (!pt || pt->t != Json::STR || pt->s != "object") refuse(p, "parameters must be an object schema");
                tools.push_back({nm + "(", R.schema(params, p + "/parameters")});
            }
        } else {
            refuse("$.kind", "unknown grammar kind");
        }
        Builder B(S, R.nodes);
        B.accept = B.add();
        if (k == "calc") {
            B.calc();
        } else if (k == "calc_text") {
            B.calc_text();
        } else if (k == "json_schema") {
            B.start = B.value(json_root, B.accept, 0);
            if (B.start < 0) refuse("$", "grammar accepts no string");
        } else {
            B.start = B.add();
            for (auto &t : tools) {
                int close = B.add();
                B.edge(close, ')', ')', OP_NONE, 0, B.accept);
                int args = B.value(t.second, close, 0);
                if (args >= 0) B.trie(B.start, {t.first}, args);
            }
        }
        if (B.need_strings) B.strings();
        trim_and_pack(B, g);
        g->max_bytes = LongestMember{g->host_comb, g->k}.run();
    } catch (const CompileError &e) {
        set_error("%s", e.msg.c_str());
        return e.code;
    } catch (const std::bad_alloc &) {
        set_error("out of host memory");
        return CG_E_LIMIT;
    }
    g->compile_ms = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
    return CG_OK;
}

}  // namespace cg
