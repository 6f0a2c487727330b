// contract.cpp -- the integer-string contract transform (host).
//
// "Constrained Decoding Under Matched Conditions", "The system boundary I am
// testing": the caller's contract asks for a canonical signed-integer
// string; the model is better aligned with a native JSON integer.  The
// contract is not weakened: a separate model-facing schema is made (every
// such string becomes an integer), one constrained generation runs under
// it, an exact inverse maps the generated integers back to strings (their
// base-10 text, which for a canonical JSON integer is the digits as written
// -- no parsing, any length), and the result is validated against the
// original schema.  Nothing is repaired or guessed: a field that is not an
// integer where one is expected fails, and so does a final object the
// original schema refuses.
#include <stdio.h>
#include <string.h>

#include <string>

#include "cg_internal.hpp"
#include "json.hpp"

namespace cg {
const char *last_error();
int compile_spec(const char *spec, size_t len, cg_grammar *g);
extern const char *const kIntStringPattern;

namespace {

struct Fail {
    int code;
    std::string msg;
};

void dump(const Json &v, std::string &o) {
    switch (v.t) {
    case Json::NUL: o += "null"; break;
    case Json::BOOL: o += v.b ? "true" : "false"; break;
    case Json::NUM: o += v.s; break;
    case Json::STR: {
        o += '"';
        for (unsigned char c : v.s) {
            if (c == '"') o += "\\\"";
            else if (c == '\\') o += "\\\\";
            else if (c == '\n') o += "\\n";
            else if (c == '\r') o += "\\r";
            else if (c == '\t') o += "\\t";
            else if (c == '\b') o += "\\b";
            else if (c == '\f') o += "\\f";
            else if (c < 0x20) {
                char buf[8];
                snprintf(buf, sizeof buf, "\\u%04x", c);
                o += buf;
            } else o += (char)c;
        }
        o += '"';
        break;
    }
    case Json::ARR:
        o += '[';
        for (size_t i = 0; i < v.a.size(); i++) {
            if (i) o += ',';
            dump(v.a[i], o);
        }
        o += ']';
        break;
    case Json::OBJ:
        o += '{';
        for (size_t i = 0; i < v.o.size(); i++) {
            if (i) o += ',';
            Json k;
            k.t = Json::STR;
            k.s = v.o[i].first;
            dump(k, o);
            o += ':';
            dump(v.o[i].second, o);
        }
        o += '}';
        break;
    }
}

bool is_int_string(const Json &sch) {
    if (sch.t != Json::OBJ) return false;
    const Json *t = sch.get("type"), *p = sch.get("pattern");
    return t && t->t == Json::STR && t->s == "string" && p && p->t == Json::STR && p->s == kIntStringPattern;
}

bool is_integer_text(const Json &v) {
    if (v.t != Json::NUM) return false;
    return v.s.find_first_of(".eE") == std::string::npos && v.s.find_first_not_of("-0123456789") == std::string::npos;
}

// external schema -> model-facing schema: each integer string becomes an integer
Json to_model(const Json &sch, int &n) {
    if (is_int_string(sch)) {
        Json out;
        out.t = Json::OBJ;
        Json ty;
        ty.t = Json::STR;
        ty.s = "integer";
        out.o.emplace_back("type", ty);
        n++;
        return out;
    }
    if (sch.t != Json::OBJ) return sch;
    Json out = sch;
    for (auto &kv : out.o) {
        if (kv.first == "properties" && kv.second.t == Json::OBJ) {
            for (auto &p : kv.second.o) p.second = to_model(p.second, n);
        } else if (kv.first == "items") {
            kv.second = to_model(kv.second, n);
        } else if (kv.first == "anyOf" && kv.second.t == Json::ARR) {
            for (auto &a : kv.second.a) a = to_model(a, n);
        }
    }
    return out;
}

// the JSON type names a value satisfies
bool type_fits(const Json &sch, const Json &v) {
    const Json *t = sch.t == Json::OBJ ? sch.get("type") : nullptr;
    if (is_int_string(sch)) return is_integer_text(v);
    if (!t || t->t != Json::STR) return true;
    const std::string &s = t->s;
    switch (v.t) {
    case Json::NUL: return s == "null";
    case Json::BOOL: return s == "boolean";
    case Json::NUM: return s == "number" || (s == "integer" && is_integer_text(v));
    case Json::STR: return s == "string";
    case Json::ARR: return s == "array";
    case Json::OBJ: return s == "object";
    }
    return false;
}

// generated value (under the model-facing schema) -> value for the external schema
void reverse(const Json &sch, Json &v, const std::string &path) {
    if (is_int_string(sch)) {
        if (!is_integer_text(v)) throw Fail{CG_E_INVALID, path + ": expected an integer"};
        const std::string txt = v.s;
        v = Json();
        v.t = Json::STR;
        v.s = txt;  // the integer's own base-10 text, every digit kept
        return;
    }
    if (sch.t != Json::OBJ) return;
    if (const Json *any = sch.get("anyOf")) {
        if (any->t != Json::ARR) return;
        for (const Json &alt : any->a)
            if (type_fits(alt, v)) {
                reverse(alt, v, path);
                return;
            }
        return;
    }
    if (v.t == Json::OBJ) {
        if (const Json *props = sch.get("properties"))
            for (auto &kv : v.o)
                if (const Json *ps = props->get(kv.first)) reverse(*ps, kv.second, path + "/" + kv.first);
    } else if (v.t == Json::ARR) {
        if (const Json *items = sch.get("items"))
            for (size_t i = 0; i < v.a.size(); i++) reverse(*items, v.a[i], path + "/" + std::to_string(i));
    }
}

Json parse_spec(const char *spec, size_t len) {
    try {
        Json root = JsonReader(spec, len).parse();
        if (root.t != Json::OBJ || !root.get("schema")) throw Fail{CG_E_PARSE, "spec is not a json_schema spec"};
        const Json *k = root.get("kind");
        if (!k || k->t != Json::STR || k->s != "json_schema") throw Fail{CG_E_PARSE, "spec kind must be json_schema"};
        return root;
    } catch (const JsonError &e) {
        throw Fail{CG_E_PARSE, "spec: " + e.msg};
    }
}

int put(const std::string &s, char *out, size_t cap, size_t *out_len) {
    *out_len = s.size();
    if (s.size() + 1 > cap) {
        set_error("output needs %zu bytes (with the terminating zero)", s.size() + 1);
        return CG_E_LIMIT;
    }
    memcpy(out, s.data(), s.size());
    out[s.size()] = 0;
    return CG_OK;
}

}  // namespace
}  // namespace cg

using namespace cg;

extern "C" {

int cg_contract_model_spec(const char *ext_spec, size_t len, char *out, size_t cap, size_t *out_len,
                           int32_t *n_fields) {
    if (!ext_spec || !out_len || (cap && !out)) {
        set_error("NULL argument");
        return CG_E_ARG;
    }
    try {
        Json root = parse_spec(ext_spec, len);
        int n = 0;
        for (auto &kv : root.o)
            if (kv.first == "schema") kv.second = to_model(kv.second, n);
        std::string s;
        dump(root, s);
        // the model-facing spec must compile (fail closed, e.g. an integer
        // string beside another numeric alternative of an anyOf)
        cg_grammar probe;
        const int rc = compile_spec(s.data(), s.size(), &probe);
        free(probe.host_comb);
        if (rc != CG_OK) return rc;
        if (n_fields) *n_fields = n;
        return put(s, out, cap, out_len);
    } catch (const Fail &f) {
        set_error("%s", f.msg.c_str());
        return f.code;
    }
}

int cg_contract_reverse(const char *ext_spec, size_t len, const uint8_t *text, size_t text_len, char *out,
                        size_t cap, size_t *out_len) {
    if (!ext_spec || !out_len || (text_len && !text) || (cap && !out)) {
        set_error("NULL argument");
        return CG_E_ARG;
    }
    try {
        Json root = parse_spec(ext_spec, len);
        Json v;
        try {
            v = JsonReader((const char *)text, text_len).parse();
        } catch (const JsonError &e) {
            throw Fail{CG_E_INVALID, "generated text: " + e.msg};
        }
        reverse(*root.get("schema"), v, "$");
        std::string s;
        dump(v, s);
        // validation against the original schema, on its own automaton
        cg_grammar ext;
        const int rc = compile_spec(ext_spec, len, &ext);
        if (rc != CG_OK) {
            free(ext.host_comb);
            return rc;
        }
        Walker w;
        w.q = ext.k.start;
        w.ret = ext.k.start;
        w.cnt = 0;
        w.ws = 0;
        w.depth = 0;
        w.stk = 0;
        size_t i = 0;
        for (; i < s.size(); i++)
            if (!step_byte<true>(w, (uint8_t)s[i], ext.host_comb, ext.k)) break;
        const bool ok = i == s.size() && w.q == ext.k.accept;
        free(ext.host_comb);
        const int prc = put(s, out, cap, out_len);
        if (prc != CG_OK) return prc;
        if (!ok) {
            set_error("the original schema refuses the result at byte %zu", i);
            return CG_E_INVALID;
        }
        return CG_OK;
    } catch (const Fail &f) {
        set_error("%s", f.msg.c_str());
        return f.code;
    }
}

}  // extern "C"
