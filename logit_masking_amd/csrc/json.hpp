// json.hpp -- a small JSON reader for grammar specs.
//
// Numbers keep their text; integers (no fraction, no exponent) also carry
// their value when it fits in 64 bits.  Objects keep key order; a repeated
// key keeps its first position and takes the last value.  NaN, Infinity and
// -Infinity are read as non-integer numbers.  Strings are decoded to UTF-8;
// an unpaired \uD800-\uDFFF escape sets `lone_surrogate`.
#pragma once
#include <stdint.h>

#include <string>
#include <utility>
#include <vector>

namespace cg {

struct Json {
    enum Type { NUL, BOOL, NUM, STR, ARR, OBJ } t = NUL;
    bool b = false;
    bool is_int = false;  // integer literal that fits int64
    bool big_int = false; // integer literal outside int64
    int64_t i = 0;
    std::string s;        // STR (UTF-8) / NUM (text)
    bool lone_surrogate = false;
    std::vector<Json> a;
    std::vector<std::pair<std::string, Json>> o;

    const Json *get(const std::string &k) const {
        for (auto &kv : o)
            if (kv.first == k) return &kv.second;
        return nullptr;
    }
    bool has(const std::string &k) const { return get(k) != nullptr; }
    // Python truthiness
    bool truthy() const {
        switch (t) {
        case NUL: return false;
        case BOOL: return b;
        case NUM: return !(is_int && i == 0) && s != "0.0" && s != "-0.0" && s != "0" && s != "-0";
        case STR: return !s.empty();
        case ARR: return !a.empty();
        case OBJ: return !o.empty();
        }
        return false;
    }
};

struct JsonError {
    std::string msg;
};

class JsonReader {
  public:
    JsonReader(const char *p, size_t n) : p_(p), n_(n) {}

    Json parse() {
        ws();
        Json v = value(0);
        ws();
        if (i_ != n_) err("trailing data");
        return v;
    }

  private:
    const char *p_;
    size_t n_, i_ = 0;

    [[noreturn]] void err(const char *m) { throw JsonError{std::string(m) + " at offset " + std::to_string(i_)}; }
    int peek() const { return i_ < n_ ? (unsigned char)p_[i_] : -1; }
    void ws() {
        while (i_ < n_ && (p_[i_] == ' ' || p_[i_] == '\t' || p_[i_] == '\n' || p_[i_] == '\r')) i_++;
    }
    bool lit(const char *s) {
        size_t k = 0;
        while (s[k]) k++;
        if (i_ + k <= n_ && std::string(p_ + i_, k) == s) {
            i_ += k;
            return true;
        }
        return false;
    }

    Json value(int depth) {
        if (depth > 512) err("nesting too deep");
        int c = peek();
        Json v;
        if (c == '{') {
            i_++;
            v.t = Json::OBJ;
            ws();
            if (peek() == '}') {
                i_++;
                return v;
            }
            for (;;) {
                ws();
                if (peek() != '"') err("expected key");
                Json k = str();
                ws();
                if (peek() != ':') err("expected ':'");
                i_++;
                ws();
                Json val = value(depth + 1);
                bool found = false;
                for (auto &kv : v.o)
                    if (kv.first == k.s) {
                        kv.second = std::move(val);
                        found = true;
                        break;
                    }
                if (!found) v.o.emplace_back(k.s, std::move(val));
                ws();
                if (peek() == ',') {
                    i_++;
                    continue;
                }
                if (peek() == '}') {
                    i_++;
                    return v;
                }
                err("expected ',' or '}'");
            }
        }
        if (c == '[') {
            i_++;
            v.t = Json::ARR;
            ws();
            if (peek() == ']') {
                i_++;
                return v;
            }
            for (;;) {
                ws();
                v.a.push_back(value(depth + 1));
                ws();
                if (peek() == ',') {
                    i_++;
                    continue;
                }
                if (peek() == ']') {
                    i_++;
                    return v;
                }
                err("expected ',' or ']'");
            }
        }
        if (c == '"') return str();
        if (lit("null")) return v;
        if (lit("true")) {
            v.t = Json::BOOL;
            v.b = true;
            return v;
        }
        if (lit("false")) {
            v.t = Json::BOOL;
            return v;
        }
        if (lit("NaN") || lit("Infinity") || lit("-Infinity")) {
            v.t = Json::NUM;
            v.s = "nan";
            return v;
        }
        if (c == '-' || (c >= '0' && c <= '9')) return num();
        err("unexpected character");
    }

    Json num() {
        size_t st = i_;
        bool integer = true;
        if (peek() == '-') i_++;
        if (peek() == '0') {
            i_++;
        } else if (peek() >= '1' && peek() <= '9') {
            while (peek() >= '0' && peek() <= '9') i_++;
        } else {
            err("bad number");
        }
        if (peek() == '.') {
            integer = false;
            i_++;
            if (!(peek() >= '0' && peek() <= '9')) err("bad number");
            while (peek() >= '0' && peek() <= '9') i_++;
        }
        if (peek() == 'e' || peek() == 'E') {
            integer = false;
            i_++;
            if (peek() == '+' || peek() == '-') i_++;
            if (!(peek() >= '0' && peek() <= '9')) err("bad number");
            while (peek() >= '0' && peek() <= '9') i_++;
        }
        Json v;
        v.t = Json::NUM;
        v.s.assign(p_ + st, i_ - st);
        if (integer) {
            // exact value with overflow detection
            bool neg = v.s[0] == '-';
            unsigned __int128 m = 0;
            bool over = false;
            for (size_t k = neg ? 1 : 0; k < v.s.size(); k++) {
                m = m * 10 + (unsigned)(v.s[k] - '0');
                if (m > ((unsigned __int128)1 << 64)) over = true;
            }
            unsigned __int128 lim = neg ? ((unsigned __int128)1 << 63) : (((unsigned __int128)1 << 63) - 1);
            if (over || m > lim) {
                v.big_int = true;
            } else {
                v.is_int = true;
                v.i = neg ? (int64_t)(-(__int128)m) : (int64_t)m;
            }
        }
        return v;
    }

    static void put_utf8(std::string &o, uint32_t cp) {
        if (cp < 0x80) {
            o += (char)cp;
        } else if (cp < 0x800) {
            o += (char)(0xC0 | (cp >> 6));
            o += (char)(0x80 | (cp & 0x3F));
        } else if (cp < 0x10000) {
            o += (char)(0xE0 | (cp >> 12));
            o += (char)(0x80 | ((cp >> 6) & 0x3F));
            o += (char)(0x80 | (cp & 0x3F));
        } else {
            o += (char)(0xF0 | (cp >> 18));
            o += (char)(0x80 | ((cp >> 12) & 0x3F));
            o += (char)(0x80 | ((cp >> 6) & 0x3F));
            o += (char)(0x80 | (cp & 0x3F));
        }
    }

    int hex4(uint32_t &out) {
        if (i_ + 4 > n_) return 0;
        uint32_t v = 0;
        for (int k = 0; k < 4; k++) {
            int c = (unsigned char)p_[i_ + k], h;
            if (c >= '0' && c <= '9') h = c - '0';
            else if (c >= 'a' && c <= 'f') h = c - 'a' + 10;
            else if (c >= 'A' && c <= 'F') h = c - 'A' + 10;
            else return 0;
            v = v * 16 + (uint32_t)h;
        }
        out = v;
        i_ += 4;
        return 1;
    }

    Json str() {
        Json v;
        v.t = Json::STR;
        i_++;  // opening quote
        for (;;) {
            if (i_ >= n_) err("unterminated string");
            unsigned char c = (unsigned char)p_[i_];
            if (c == '"') {
                i_++;
                return v;
            }
            if (c < 0x20) err("control character in string");
            if (c != '\\') {
                v.s += (char)c;
                i_++;
                continue;
            }
            i_++;
            int e = peek();
            i_++;
            switch (e) {
            case '"': v.s += '"'; break;
            case '\\': v.s += '\\'; break;
            case '/': v.s += '/'; break;
            case 'b': v.s += '\b'; break;
            case 'f': v.s += '\f'; break;
            case 'n': v.s += '\n'; break;
            case 'r': v.s += '\r'; break;
            case 't': v.s += '\t'; break;
            case 'u': {
                uint32_t u;
                if (!hex4(u)) err("bad \\u escape");
                if (u >= 0xD800 && u <= 0xDBFF && i_ + 6 <= n_ && p_[i_] == '\\' && p_[i_ + 1] == 'u') {
                    size_t save = i_;
                    i_ += 2;
                    uint32_t lo;
                    if (hex4(lo) && lo >= 0xDC00 && lo <= 0xDFFF) {
                        put_utf8(v.s, 0x10000 + ((u - 0xD800) << 10) + (lo - 0xDC00));
                        break;
                    }
                    i_ = save;
                }
                if (u >= 0xD800 && u <= 0xDFFF) {
                    v.lone_surrogate = true;
                    put_utf8(v.s, 0xFFFD);
                } else {
                    put_utf8(v.s, u);
                }
                break;
            }
            default: err("bad escape");
            }
        }
    }
};

}  // namespace cg
