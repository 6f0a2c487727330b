/*
 * oracle/recognizer.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, schema-interpreting incremental recognizer used as the
 * oracle for grammar-constrained decoding.  Only tests/, the smoke check and
 * the benchmark's CPU-baseline leg may load it; the product path never does.
 * It shares no code, header or table with the HIP library.
 *
 * What it decides (the definition the GPU path must reproduce):
 *   a byte string p is a viable prefix of the grammar's language L iff some
 *   continuation s makes p.s a member of L.  A pushdown automaton masks the
 *   logits so that only viable continuations can be generated ("Constrained
 *   decoding", section "The guarantee").  Every grammar here is prefix-free,
 *   so once p is complete no byte may follow.
 *
 * How: a stack of frames, one per open syntactic construct (root, object,
 * array, string, integer, number, literal, enum, calc span).  feed() hands a
 * byte to the innermost frame.  A frame either takes it, refuses it, or
 * finishes -- consuming the byte (closing quote, brace) or leaving it for its
 * parent (a number ends at the first byte that cannot extend it).  Every
 * refusal is taken at the first byte after which no completion exists:
 *   - integers: arithmetic over the interval of values that the digits so
 *     far can still reach (canonical spelling, inclusive bounds);
 *   - UTF-8: the contiguous code-point interval that the bytes so far can
 *     still reach, intersected with the well-formed scalars of that length;
 *   - \u escapes: the interval of the remaining hex completions minus the
 *     surrogate block;
 *   - keys and enums: literal spellings still matching the bytes so far.
 *
 * Whitespace: runs of SP/HT/LF/CR of length <= ws_max, only at the marked
 * positions ("A valid call also has to end": the grammar bounds consecutive
 * whitespace).  Open strings are capped in code points ("the length of a field
 * the schema leaves open").
 */
#include <stdint.h>
#include <string.h>
#include <stdlib.h>
#include <pthread.h>

typedef __int128 i128;

/* ---- schema description, filled in by oracle.py ---------------------- */
enum { K_OBJ = 1, K_ARR, K_STR, K_INT, K_NUM, K_BOOL, K_NULL, K_ENUM, K_ANYOF, K_ANY, K_INTSTR };
enum { G_CALC = 1, G_JSON = 2, G_TOOL = 3, G_TEXT = 4 };
/* K_ANY kinds that may start a value */
enum { AK_OBJ = 1, AK_ARR = 2, AK_STR = 4, AK_NUM = 8, AK_LIT = 16 };

typedef struct {
    int32_t kind;
    int32_t first, count; /* OBJ: props; ENUM: literals; ANYOF: alternatives */
    int32_t cap;          /* STR: code-point cap (-1 none); ARR: maxItems (-1 none) */
    int32_t open;         /* OBJ/ARR: keys/items unconstrained */
    int32_t item;         /* ARR: items node (-1 = any JSON value) */
    int32_t any_kinds;    /* ANY: AK_* mask */
    int32_t maxdigits;    /* INT: digits excluding the sign */
    int64_t lo, hi;       /* INT: inclusive bounds (used if has_lo / has_hi) */
    int32_t has_lo, has_hi;
} onode;

typedef struct {
    int32_t lit_off, lit_len; /* spelling in the literal pool */
    int32_t node;             /* value schema (props, tools, anyOf alternatives) */
    int32_t required;
} oprop;

typedef struct {
    int32_t gkind;
    int32_t root;            /* JSON root node */
    int32_t tools_first, tools_count; /* TOOL: props whose literal is "name(" */
    int32_t ws_max, depth_cap, open_cap; /* open_cap -1 = uncapped */
    int32_t calc_min, calc_max;
    int32_t open_obj, open_arr; /* nodes of an unconstrained object / array */
    const onode *nodes;
    const oprop *props;
    const uint8_t *pool;
    int32_t evaluators;      /* TEXT: 1 calc spans, 2 string-operation spans */
} og;

/* ---- configuration ---------------------------------------------------- */
enum { F_ROOT = 1, F_OBJ, F_ARR, F_STR, F_INT, F_NUM, F_LIT, F_ENUM, F_CALC, F_TEXT, F_STROP };
#define MAXF 48

typedef struct {
    int8_t kind, phase, ws, aux; /* aux: INT sign / STR utf8 length / NUM phase */
    int32_t node;
    int32_t a;     /* per kind: see below */
    int32_t b;
    uint64_t cand; /* candidate literal set */
    i128 v;        /* INT magnitude prefix; STR hex value or utf8 bytes */
} ofr;

typedef struct {
    int32_t n;
    int32_t pad;
    ofr f[MAXF];
} oconf;

/* results of one frame step */
enum { R_OK = 0, R_DEAD, R_DONE_TOOK, R_DONE_LEFT };

static int is_ws(int c) { return c == ' ' || c == '\t' || c == '\n' || c == '\r'; }
static int is_digit(int c) { return c >= '0' && c <= '9'; }

/* whitespace at a position that allows it: 1 taken, -1 over the bound, 0 not ws */
static int take_ws(const og *g, ofr *f, int c) {
    if (!is_ws(c)) return 0;
    if (f->ws >= g->ws_max) return -1;
    f->ws++;
    return 1;
}

static i128 pow10i(int n) { i128 r = 1; while (n-- > 0) r *= 10; return r; }

/* ---- integer viability (plain interval arithmetic) --------------------- */
/* Bounds of a K_INT node, or of the calc span's integers. */
static void int_bounds(const og *g, int node, i128 *lo, i128 *hi, int *maxd) {
    if (node < 0) { *lo = g->calc_min; *hi = g->calc_max; *maxd = 19; return; }
    const onode *n = &g->nodes[node];
    i128 big = pow10i(n->maxdigits) - 1;
    *lo = n->has_lo ? (i128)n->lo : -big;
    *hi = n->has_hi ? (i128)n->hi : big;
    *maxd = n->maxdigits;
}

/*
 * Can the canonical integer whose spelling starts with sign `neg` and the
 * digits d[0..L) be completed (by appending digits) to a value in [lo, hi]?
 * Canonical: no '+', no leading zero unless the magnitude is "0", no "-0".
 */
static int int_viable(int neg, const char *d, int L, i128 lo, i128 hi, int maxd) {
    if (L > maxd) return 0;
    if (L >= 2 && d[0] == '0') return 0;
    i128 p = 0;
    for (int i = 0; i < L; i++) p = p * 10 + (d[i] - '0');
    for (int n = (L > 0 ? L : 1); n <= maxd; n++) {
        i128 mlo, mhi;
        if (L == 0) {
            mlo = (n == 1) ? 0 : pow10i(n - 1);
            mhi = pow10i(n) - 1;
        } else {
            if (d[0] == '0' && n > 1) break; /* "0" cannot be extended */
            i128 s = pow10i(n - L);
            mlo = p * s;
            mhi = (p + 1) * s - 1;
        }
        if (neg) {
            if (mlo < 1) mlo = 1;
            if (mlo > mhi) continue;
            /* values [-mhi, -mlo] */
            if (-mlo >= lo && -mhi <= hi) return 1;
        } else {
            if (mhi >= lo && mlo <= hi) return 1;
        }
    }
    return 0;
}

static int int_complete(int neg, const char *d, int L, i128 lo, i128 hi, int maxd) {
    if (L == 0 || L > maxd) return 0;
    if (L >= 2 && d[0] == '0') return 0;
    i128 p = 0;
    for (int i = 0; i < L; i++) p = p * 10 + (d[i] - '0');
    if (neg && p == 0) return 0;
    i128 v = neg ? -p : p;
    return v >= lo && v <= hi;
}

/* ---- UTF-8 and escape viability ---------------------------------------- */
/* Expected sequence length from a lead byte, 0 if it can never lead. */
static int utf8_len(int b) {
    if (b >= 0xC0 && b <= 0xDF) return 2;
    if (b >= 0xE0 && b <= 0xEF) return 3;
    if (b >= 0xF0 && b <= 0xF7) return 4;
    return 0;
}

/*
 * The bytes s[0..k) (lead + continuations) of an n-byte sequence: the code
 * points reachable by completing it form the interval obtained by filling
 * the missing continuations with 0x80 and with 0xBF.  Viable iff that
 * interval meets the well-formed scalars of length n (shortest form, not a
 * surrogate, at most U+10FFFF).
 */
static int utf8_viable(const uint8_t *s, int k, int n) {
    for (int i = 1; i < k; i++)
        if (s[i] < 0x80 || s[i] > 0xBF) return 0;
    uint32_t lo = 0, hi = 0;
    int lead_bits = (n == 2) ? 5 : (n == 3) ? 4 : 3;
    lo = hi = s[0] & ((1u << lead_bits) - 1);
    for (int i = 1; i < n; i++) {
        uint32_t cl = (i < k) ? (s[i] & 0x3F) : 0x00;
        uint32_t ch = (i < k) ? (s[i] & 0x3F) : 0x3F;
        lo = (lo << 6) | cl;
        hi = (hi << 6) | ch;
    }
    uint32_t vmin = (n == 2) ? 0x80 : (n == 3) ? 0x800 : 0x10000;
    uint32_t vmax = (n == 2) ? 0x7FF : (n == 3) ? 0xFFFF : 0x10FFFF;
    if (lo < vmin) lo = vmin;
    if (hi > vmax) hi = vmax;
    if (lo > hi) return 0;
    if (lo >= 0xD800 && hi <= 0xDFFF) return 0; /* only surrogates remain */
    return 1;
}

/* k hex digits with value v: is some completion outside D800..DFFF? */
static int hex_viable(uint32_t v, int k) {
    uint32_t s = 1u << (4 * (4 - k));
    uint32_t lo = v * s, hi = (v + 1) * s - 1;
    return !(lo >= 0xD800 && hi <= 0xDFFF);
}

static int hexval(int c) {
    if (c >= '0' && c <= '9') return c - '0';
    if (c >= 'a' && c <= 'f') return c - 'a' + 10;
    if (c >= 'A' && c <= 'F') return c - 'A' + 10;
    return -1;
}

/* ---- literal candidate matching ---------------------------------------- */
/* Narrow the candidate set (props[first..first+count)) on byte c at pos.
 * Returns the index of a fully matched literal, -1 if still partial, -2 dead. */
static int lit_step(const og *g, int first, int count, uint64_t *cand, int pos, int c) {
    uint64_t keep = 0;
    int full = -1;
    for (int i = 0; i < count; i++) {
        if (!((*cand >> i) & 1)) continue;
        const oprop *p = &g->props[first + i];
        if (pos < p->lit_len && g->pool[p->lit_off + pos] == c) {
            keep |= 1ull << i;
            if (pos + 1 == p->lit_len) full = i;
        }
    }
    *cand = keep;
    if (!keep) return -2;
    return full;
}

/* ---- frames ------------------------------------------------------------ */
static int depth_of(const oconf *c) {
    int d = 0;
    for (int i = 0; i < c->n; i++)
        if (c->f[i].kind == F_OBJ || c->f[i].kind == F_ARR) d++;
    return d;
}

static ofr *push(oconf *c, int kind, int node) {
    if (c->n >= MAXF) abort();
    ofr *f = &c->f[c->n++];
    memset(f, 0, sizeof *f);
    f->kind = (int8_t)kind;
    f->node = node;
    return f;
}

static int start_value(const og *g, oconf *c, int node, int kinds, int byte);

/* object phases */
enum { O_OPEN = 0, O_KEY, O_KEYSTR, O_COLON, O_VALUE, O_INVAL, O_AFTER, O_COMMA };
/* array phases */
enum { A_OPEN = 0, A_INVAL, A_AFTER, A_COMMA };
/* string phases */
enum { S_BODY = 0, S_ESC, S_HEX, S_UTF };
/* number phases (RFC 8259) */
enum { N_MINUS = 0, N_ZERO, N_INT, N_DOT, N_FRAC, N_E, N_ESIGN, N_EXP };
/* calc phases */
enum { C_OPEN = 0, C_ET, C_INT, C_AT, C_CLOSE, C_DONE };
/* root phases */
enum { RT_NAME = 0, RT_VALUE, RT_INVAL, RT_CLOSE, RT_DONE };
/* text phases; inside X_RES the engine writes every byte */
enum { X_TEXT = 0, X_LT, X_END, X_CALC, X_RES, X_DONE };

/*
 * Can a value of schema `node` be completed when `depth` containers are
 * already open?  A container needs room under the depth cap, and a closed
 * object also needs every required property to be completable one level
 * deeper.  (A value that cannot be completed must not be started: the
 * prefix would not be viable.)
 */
static int sat(const og *g, int node, int depth) {
    const onode *o = &g->nodes[node];
    switch (o->kind) {
    case K_OBJ:
        if (depth + 1 > g->depth_cap) return 0;
        if (o->open) return 1;
        for (int j = 0; j < o->count; j++)
            if (g->props[o->first + j].required && !sat(g, g->props[o->first + j].node, depth + 1)) return 0;
        return 1;
    case K_ARR:
        return depth + 1 <= g->depth_cap;
    case K_ANYOF:
        for (int j = 0; j < o->count; j++)
            if (sat(g, g->props[o->first + j].node, depth)) return 1;
        return 0;
    case K_ANY:
        if (o->any_kinds & (AK_STR | AK_NUM | AK_LIT)) return 1;
        return depth + 1 <= g->depth_cap;
    default:
        return 1;
    }
}

/* Properties of object node o (open at `depth`) that may come next after
 * property `last`: every later completable property up to and including the
 * first required one. */
static uint64_t obj_candidates(const og *g, const onode *o, int last, int depth) {
    uint64_t m = 0;
    for (int j = last + 1; j < o->count; j++) {
        const oprop *p = &g->props[o->first + j];
        if (sat(g, p->node, depth)) m |= 1ull << j;
        if (p->required) break;
    }
    return m;
}

static int obj_may_close(const og *g, const onode *o, int last) {
    for (int j = last + 1; j < o->count; j++)
        if (g->props[o->first + j].required) return 0;
    return 1;
}

static int step_obj(const og *g, oconf *c, ofr *f, int ch) {
    const onode *o = &g->nodes[f->node];
    int w;
    switch (f->phase) {
    case O_OPEN:
    case O_COMMA:
        if ((w = take_ws(g, f, ch))) return w > 0 ? R_OK : R_DEAD;
        if (ch == '}' && f->phase == O_OPEN) {
            if (o->open || obj_may_close(g, o, f->a)) return R_DONE_TOOK;
            return R_DEAD;
        }
        if (ch != '"') return R_DEAD;
        f->ws = 0;
        if (o->open) {
            f->phase = O_KEYSTR;
            ofr *s = push(c, F_STR, -1);
            s->b = g->open_cap; /* cap */
            return R_OK;
        }
        f->cand = obj_candidates(g, o, f->a, depth_of(c));
        if (!f->cand) return R_DEAD;
        f->phase = O_KEY;
        f->b = 1; /* bytes of the quoted key matched */
        return R_OK;
    case O_KEY: {
        int full = lit_step(g, o->first, o->count, &f->cand, f->b, ch);
        if (full == -2) return R_DEAD;
        f->b++;
        if (full >= 0) { f->a = full; f->phase = O_COLON; f->ws = 0; }
        return R_OK;
    }
    case O_COLON:
        if ((w = take_ws(g, f, ch))) return w > 0 ? R_OK : R_DEAD;
        if (ch != ':') return R_DEAD;
        f->phase = O_VALUE;
        f->ws = 0;
        return R_OK;
    case O_VALUE: {
        if ((w = take_ws(g, f, ch))) return w > 0 ? R_OK : R_DEAD;
        f->ws = 0;
        f->phase = O_INVAL;
        int vnode = o->open ? -1 : g->props[o->first + f->a].node;
        return start_value(g, c, vnode, AK_OBJ | AK_ARR | AK_STR | AK_NUM | AK_LIT, ch) ? R_OK : R_DEAD;
    }
    case O_AFTER:
        if ((w = take_ws(g, f, ch))) return w > 0 ? R_OK : R_DEAD;
        if (ch == '}') {
            if (o->open || obj_may_close(g, o, f->a)) return R_DONE_TOOK;
            return R_DEAD;
        }
        if (ch == ',') {
            if (!o->open && !obj_candidates(g, o, f->a, depth_of(c))) return R_DEAD;
            f->phase = O_COMMA;
            f->ws = 0;
            return R_OK;
        }
        return R_DEAD;
    }
    return R_DEAD;
}

static int step_arr(const og *g, oconf *c, ofr *f, int ch) {
    const onode *o = &g->nodes[f->node];
    int w;
    switch (f->phase) {
    case A_OPEN:
    case A_COMMA:
        if ((w = take_ws(g, f, ch))) return w > 0 ? R_OK : R_DEAD;
        if (ch == ']' && f->phase == A_OPEN) return R_DONE_TOOK;
        if (o->cap >= 0 && f->a >= o->cap) return R_DEAD;
        if (!o->open && !sat(g, o->item, depth_of(c))) return R_DEAD;
        f->a++;
        f->ws = 0;
        f->phase = A_INVAL;
        return start_value(g, c, o->open ? -1 : o->item, AK_OBJ | AK_ARR | AK_STR | AK_NUM | AK_LIT, ch)
                   ? R_OK : R_DEAD;
    case A_AFTER:
        if ((w = take_ws(g, f, ch))) return w > 0 ? R_OK : R_DEAD;
        if (ch == ']') return R_DONE_TOOK;
        if (ch == ',') {
            if (o->cap >= 0 && f->a >= o->cap) return R_DEAD;
            if (!o->open && !sat(g, o->item, depth_of(c))) return R_DEAD;
            f->phase = A_COMMA;
            f->ws = 0;
            return R_OK;
        }
        return R_DEAD;
    }
    return R_DEAD;
}

/* string frame: a = code points so far, b = cap (-1 none), v = hex value /
 * pending utf8 bytes, aux = utf8 sequence length, ws = bytes of it seen */
static int count_char(ofr *f) {
    if (f->b >= 0 && f->a >= f->b) return 0;
    f->a++;
    return 1;
}

static int step_str(ofr *f, int ch) {
    switch (f->phase) {
    case S_BODY:
        if (ch == '"') return R_DONE_TOOK;
        if (ch == '\\') {
            if (!count_char(f)) return R_DEAD;
            f->phase = S_ESC;
            return R_OK;
        }
        if (ch < 0x20) return R_DEAD;
        if (ch < 0x80) return count_char(f) ? R_OK : R_DEAD;
        {
            int n = utf8_len(ch);
            uint8_t s[4] = {(uint8_t)ch, 0, 0, 0};
            if (!n || !utf8_viable(s, 1, n)) return R_DEAD;
            if (!count_char(f)) return R_DEAD;
            f->aux = (int8_t)n;
            f->ws = 1;
            f->v = ch;
            f->phase = S_UTF;
            return R_OK;
        }
    case S_UTF: {
        uint8_t s[4];
        int k = f->ws;
        for (int i = 0; i < k; i++) s[i] = (uint8_t)(f->v >> (8 * i));
        s[k] = (uint8_t)ch;
        if (!utf8_viable(s, k + 1, f->aux)) return R_DEAD;
        f->v |= (i128)ch << (8 * k);
        f->ws = (int8_t)(k + 1);
        if (f->ws == f->aux) { f->phase = S_BODY; f->ws = 0; f->v = 0; }
        return R_OK;
    }
    case S_ESC:
        if (ch == 'u') { f->phase = S_HEX; f->ws = 0; f->v = 0; return R_OK; }
        if (ch == '"' || ch == '\\' || ch == '/' || ch == 'b' || ch == 'f' || ch == 'n' || ch == 'r' ||
            ch == 't') {
            f->phase = S_BODY;
            return R_OK;
        }
        return R_DEAD;
    case S_HEX: {
        int h = hexval(ch);
        if (h < 0) return R_DEAD;
        uint32_t v = (uint32_t)f->v * 16 + (uint32_t)h;
        int k = f->ws + 1;
        if (!hex_viable(v, k)) return R_DEAD;
        f->v = v;
        f->ws = (int8_t)k;
        if (k == 4) { f->phase = S_BODY; f->ws = 0; f->v = 0; }
        return R_OK;
    }
    }
    return R_DEAD;
}

/* integer frame: aux = minus seen, a = digits so far, digits kept in v as a
 * little base-16 stack of decimal digits (max 21) -> decode for checks.
 * phase 1: the content of a string with the signed-integer pattern; it ends
 * by taking the closing quote. */
static void int_digits(const ofr *f, char *d) {
    for (int i = 0; i < f->a; i++) d[i] = (char)('0' + (int)((f->v >> (4 * i)) & 0xF));
}

static int step_int(const og *g, ofr *f, int ch) {
    i128 lo, hi;
    int maxd;
    int_bounds(g, f->node, &lo, &hi, &maxd);
    char d[40];
    int_digits(f, d);
    if (f->phase == 1) {
        /* the pattern -?(0|[1-9][0-9]*), at most maxd digits ("-0" matches it) */
        if (ch == '"') return f->a > 0 ? R_DONE_TOOK : R_DEAD;
        if (ch == '-') {
            if (f->a > 0 || f->aux) return R_DEAD;
            f->aux = 1;
            return R_OK;
        }
        if (!is_digit(ch) || f->a >= maxd || (f->a > 0 && d[0] == '0')) return R_DEAD;
        f->v |= (i128)(ch - '0') << (4 * f->a);
        f->a++;
        return R_OK;
    }
    if (is_digit(ch)) {
        d[f->a] = (char)ch;
        if (!int_viable(f->aux, d, f->a + 1, lo, hi, maxd)) return R_DEAD;
        f->v |= (i128)(ch - '0') << (4 * f->a);
        f->a++;
        return R_OK;
    }
    return int_complete(f->aux, d, f->a, lo, hi, maxd) ? R_DONE_LEFT : R_DEAD;
}

static int step_num(ofr *f, int ch) {
    int dg = is_digit(ch);
    switch (f->phase) {
    case N_MINUS:
        if (ch == '0') { f->phase = N_ZERO; return R_OK; }
        if (dg) { f->phase = N_INT; return R_OK; }
        return R_DEAD;
    case N_ZERO:
    case N_INT:
        if (dg && f->phase == N_INT) return R_OK;
        if (ch == '.') { f->phase = N_DOT; return R_OK; }
        if (ch == 'e' || ch == 'E') { f->phase = N_E; return R_OK; }
        return R_DONE_LEFT;
    case N_DOT:
        if (dg) { f->phase = N_FRAC; return R_OK; }
        return R_DEAD;
    case N_FRAC:
        if (dg) return R_OK;
        if (ch == 'e' || ch == 'E') { f->phase = N_E; return R_OK; }
        return R_DONE_LEFT;
    case N_E:
        if (ch == '+' || ch == '-') { f->phase = N_ESIGN; return R_OK; }
        if (dg) { f->phase = N_EXP; return R_OK; }
        return R_DEAD;
    case N_ESIGN:
        if (dg) { f->phase = N_EXP; return R_OK; }
        return R_DEAD;
    case N_EXP:
        if (dg) return R_OK;
        return R_DONE_LEFT;
    }
    return R_DEAD;
}

/* literal frame (true / false / null): a = bytes matched, node = literal id */
static const char *LITS[3] = {"true", "false", "null"};

static int step_lit(ofr *f, int ch) {
    const char *s = LITS[f->b];
    if (ch != (uint8_t)s[f->a]) return R_DEAD;
    f->a++;
    return s[f->a] == 0 ? R_DONE_TOOK : R_OK;
}

static int step_enum(const og *g, ofr *f, int ch) {
    const onode *o = &g->nodes[f->node];
    int full = lit_step(g, o->first, o->count, &f->cand, f->a, ch);
    if (full == -2) return R_DEAD;
    f->a++;
    return full >= 0 ? R_DONE_TOOK : R_OK;
}

/* calc span:  "<calc>" W E W "</calc>",  E := T (W op W T)*,
 * T := INT | "(" W E W ")"  with the depth of open parentheses capped. */
static const char CALC_OPEN[] = "<calc>";
static const char CALC_CLOSE[] = "</calc>";

static int step_calc(const og *g, ofr *f, int ch) {
    int w;
    /* a = paren depth, b = literal position, v = digits (base 16), aux = ndigits */
    for (;;) {
        switch (f->phase) {
        case C_OPEN:
            if (ch != CALC_OPEN[f->b]) return R_DEAD;
            if (++f->b == 6) { f->phase = C_ET; f->ws = 0; }
            return R_OK;
        case C_ET:
            if ((w = take_ws(g, f, ch))) return w > 0 ? R_OK : R_DEAD;
            if (ch == '(') {
                if (f->a >= g->depth_cap) return R_DEAD;
                f->a++;
                f->ws = 0;
                return R_OK;
            }
            if (is_digit(ch)) {
                char d[1] = {(char)ch};
                if (!int_viable(0, d, 1, g->calc_min, g->calc_max, 19)) return R_DEAD;
                f->v = ch - '0';
                f->aux = 1;
                f->phase = C_INT;
                return R_OK;
            }
            return R_DEAD;
        case C_INT: {
            char d[24];
            for (int i = 0; i < f->aux; i++) d[i] = (char)('0' + (int)((f->v >> (4 * i)) & 0xF));
            if (is_digit(ch)) {
                d[(int)f->aux] = (char)ch;
                if (!int_viable(0, d, f->aux + 1, g->calc_min, g->calc_max, 19)) return R_DEAD;
                f->v |= (i128)(ch - '0') << (4 * f->aux);
                f->aux++;
                return R_OK;
            }
            if (!int_complete(0, d, f->aux, g->calc_min, g->calc_max, 19)) return R_DEAD;
            f->phase = C_AT;
            f->ws = 0;
            continue; /* the byte belongs to what follows the term */
        }
        case C_AT:
            if ((w = take_ws(g, f, ch))) return w > 0 ? R_OK : R_DEAD;
            if (ch == '+' || ch == '-' || ch == '*' || ch == '/') {
                f->phase = C_ET;
                f->ws = 0;
                return R_OK;
            }
            if (ch == ')') {
                if (f->a == 0) return R_DEAD;
                f->a--;
                f->ws = 0;
                return R_OK;
            }
            if (ch == '<') {
                if (f->a != 0) return R_DEAD;
                f->phase = C_CLOSE;
                f->b = 1;
                return R_OK;
            }
            return R_DEAD;
        case C_CLOSE:
            if (ch != CALC_CLOSE[f->b]) return R_DEAD;
            if (++f->b == 7) {
                if (g->gkind == G_TEXT) return R_DONE_TOOK; /* a span inside text */
                f->phase = C_DONE;
            }
            return R_OK;
        default:
            return R_DEAD;
        }
    }
}

/* string-operation span (page "Evaluator aware decoding", "Not just
 * arithmetic: string operations"): "<strop>" NAME "(" W ARGS W ")" "</strop>",
 * NAME(ARGS) one of count(S, S), len(S), reverse(S), upper(S), substr(S, I, I),
 * arguments separated by W "," W; S = '"' (printable ASCII but '"', '\\',
 * '<')* '"'; I = "-"? digit{1,6}.  a = the operation, b = position in a
 * literal or the argument index, aux = digits of an integer, cand = names
 * still matching. */
enum { S_TAG = 0, S_NAME, S_ARG, S_STR, S_INT, S_AFTER, S_CLOSE };
static const char STROP_OPEN[] = "<strop>";
static const char STROP_CLOSE[] = "</strop>";
static const char *const STROP_NAMES[5] = {"count(", "len(", "reverse(", "upper(", "substr("};
static const char *const STROP_ARGS[5] = {"SS", "S", "S", "S", "SII"};

static int step_strop(const og *g, ofr *f, int ch) {
    int w;
    for (;;) {
        switch (f->phase) {
        case S_TAG:
            if (ch != STROP_OPEN[f->b]) return R_DEAD;
            if (++f->b == 7) { f->phase = S_NAME; f->b = 0; f->cand = 31; }
            return R_OK;
        case S_NAME: {
            uint64_t nc = 0;
            for (int i = 0; i < 5; i++)
                if (((f->cand >> i) & 1) && STROP_NAMES[i][f->b] == ch) nc |= 1ull << i;
            if (!nc) return R_DEAD;
            f->cand = nc;
            f->b++;
            for (int i = 0; i < 5; i++)
                if (((nc >> i) & 1) && STROP_NAMES[i][f->b] == 0) {
                    f->a = i;
                    f->phase = S_ARG;
                    f->b = 0;
                    f->ws = 0;
                }
            return R_OK;
        }
        case S_ARG:
            if ((w = take_ws(g, f, ch))) return w > 0 ? R_OK : R_DEAD;
            if (STROP_ARGS[f->a][f->b] == 'S') {
                if (ch != '"') return R_DEAD;
                f->phase = S_STR;
                return R_OK;
            }
            if (ch != '-' && !is_digit(ch)) return R_DEAD;
            f->phase = S_INT;
            f->aux = is_digit(ch) ? 1 : 0;
            return R_OK;
        case S_STR:
            if (ch == '"') { f->phase = S_AFTER; f->ws = 0; return R_OK; }
            return (ch >= 0x20 && ch <= 0x7E && ch != '\\' && ch != '<') ? R_OK : R_DEAD;
        case S_INT:
            if (is_digit(ch)) {
                if (f->aux >= 6) return R_DEAD;
                f->aux++;
                return R_OK;
            }
            if (f->aux == 0) return R_DEAD;
            f->phase = S_AFTER;
            f->ws = 0;
            continue; /* the byte belongs to what follows the integer */
        case S_AFTER: {
            if ((w = take_ws(g, f, ch))) return w > 0 ? R_OK : R_DEAD;
            const int last = STROP_ARGS[f->a][f->b + 1] == 0;
            if (!last && ch == ',') { f->b++; f->phase = S_ARG; f->ws = 0; return R_OK; }
            if (last && ch == ')') { f->phase = S_CLOSE; f->b = 0; return R_OK; }
            return R_DEAD;
        }
        case S_CLOSE:
            if (ch != STROP_CLOSE[f->b]) return R_DEAD;
            return ++f->b == 8 ? R_DONE_TOOK : R_OK;
        default:
            return R_DEAD;
        }
    }
}

/* text with evaluated spans (page "Evaluator aware decoding", "A concrete
 * prototype on llama.cpp": the model writes a span, the engine evaluates it
 * and writes the result, or an error the model can recover from, back):
 *   X* ("<calc>" ... "</calc>" RESULT X*)* "<end>",
 *   X = LF or printable ASCII other than '<',
 *   RESULT = "<result>" "-"? digit{1,20} "</result>"
 *          | "<result_error>" M* "</result_error>",  M = printable ASCII but '<'.
 * In X_RES, a = position in RESULT: 0 "<result" (b bytes matched), 1 value
 * start, 2 after '-', 3 digits (aux of them), 4 "</result>" (b matched),
 * 5 "_error>" (b matched), 6 message, 7 "</result_error>" (b matched). */
static const char END_TAG[] = "<end>";
static const char RES_OPEN[] = "<result";
static const char RES_CLOSE[] = "</result>";
static const char ERR_OPEN[] = "_error>";
static const char ERR_CLOSE[] = "</result_error>";

static int printable(int ch) { return ch >= 0x20 && ch <= 0x7E; }

static int step_text(const og *g, oconf *c, ofr *f, int ch) {
    switch (f->phase) {
    case X_TEXT:
        if (ch == '<') { f->phase = X_LT; return R_OK; }
        return (ch == '\n' || printable(ch)) ? R_OK : R_DEAD;
    case X_LT:
        if (ch == 'e') { f->phase = X_END; f->b = 2; return R_OK; }
        if (ch == 'c' && (g->evaluators & 1)) {
            ofr *k = push(c, F_CALC, -1);
            k->phase = C_OPEN;
            k->b = 2; /* "<c" matched */
            f->phase = X_CALC;
            f->aux = 0;
            return R_OK;
        }
        if (ch == 's' && (g->evaluators & 2)) {
            ofr *k = push(c, F_STROP, -1);
            k->phase = S_TAG;
            k->b = 2; /* "<s" matched */
            f->phase = X_CALC;
            f->aux = 1;
            return R_OK;
        }
        return R_DEAD;
    case X_END:
        if (ch != END_TAG[f->b]) return R_DEAD;
        if (++f->b == 5) f->phase = X_DONE;
        return R_OK;
    case X_RES:
        switch (f->a) {
        case 0:
            if (f->b < 7) {
                if (ch != RES_OPEN[f->b]) return R_DEAD;
                f->b++;
                return R_OK;
            }
            if (ch == '>') { f->a = f->aux ? 8 : 1; return R_OK; }
            if (ch == '_') { f->a = 5; f->b = 1; return R_OK; }
            return R_DEAD;
        case 1:
        case 2:
            if (f->a == 1 && ch == '-') { f->a = 2; return R_OK; }
            if (!is_digit(ch)) return R_DEAD;
            f->a = 3;
            f->aux = 1;
            return R_OK;
        case 3:
            if (is_digit(ch)) {
                if (f->aux >= 20) return R_DEAD;
                f->aux++;
                return R_OK;
            }
            if (ch != '<') return R_DEAD;
            f->a = 4;
            f->b = 1;
            return R_OK;
        case 4:
            if (ch != RES_CLOSE[f->b]) return R_DEAD;
            if (++f->b == 9) f->phase = X_TEXT;
            return R_OK;
        case 5:
            if (ch != ERR_OPEN[f->b]) return R_DEAD;
            if (++f->b == 7) f->a = 6;
            return R_OK;
        case 6:
            if (ch == '<') { f->a = 7; f->b = 1; return R_OK; }
            return printable(ch) ? R_OK : R_DEAD;
        case 7:
            if (ch != ERR_CLOSE[f->b]) return R_DEAD;
            if (++f->b == 15) f->phase = X_TEXT;
            return R_OK;
        case 8: /* a string operation's result: text up to "</result>" */
            if (ch == '<') { f->a = 4; f->b = 1; return R_OK; }
            return printable(ch) ? R_OK : R_DEAD;
        }
        return R_DEAD;
    default:
        return R_DEAD;
    }
}

/* ---- value dispatch ---------------------------------------------------- */
/* Start a value of schema `node` (-1 = any JSON value limited to `kinds`)
 * whose first byte is `ch`. */
static int start_value(const og *g, oconf *c, int node, int kinds, int ch) {
    if (node >= 0) {
        const onode *o = &g->nodes[node];
        switch (o->kind) {
        case K_ANY:
            return start_value(g, c, -1, o->any_kinds, ch);
        case K_ANYOF: {
            /* alternatives are told apart by their first byte */
            oconf trial;
            int found = -1;
            for (int i = 0; i < o->count; i++) {
                oconf t = *c;
                if (start_value(g, &t, g->props[o->first + i].node, kinds, ch)) {
                    if (found >= 0) abort(); /* ambiguous: refused at load time */
                    found = i;
                    trial = t;
                }
            }
            if (found < 0) return 0;
            *c = trial;
            return 1;
        }
        case K_OBJ:
        case K_ARR: {
            if (ch != (o->kind == K_OBJ ? '{' : '[')) return 0;
            if (!sat(g, node, depth_of(c))) return 0;
            ofr *f = push(c, o->kind == K_OBJ ? F_OBJ : F_ARR, node);
            f->a = (o->kind == K_OBJ) ? -1 : 0;
            return 1;
        }
        case K_STR: {
            if (ch != '"') return 0;
            ofr *f = push(c, F_STR, node);
            f->b = o->cap;
            return 1;
        }
        case K_INT: {
            ofr *f = push(c, F_INT, node);
            if (ch == '-') {
                i128 lo, hi;
                int maxd;
                int_bounds(g, node, &lo, &hi, &maxd);
                f->aux = 1;
                return int_viable(1, "", 0, lo, hi, maxd);
            }
            if (!is_digit(ch)) return 0;
            return step_int(g, f, ch) == R_OK;
        }
        case K_INTSTR: {
            if (ch != '"') return 0;
            ofr *f = push(c, F_INT, node);
            f->phase = 1;
            return 1;
        }
        case K_NUM: {
            if (ch != '-' && !is_digit(ch)) return 0;
            ofr *f = push(c, F_NUM, node);
            f->phase = N_MINUS;
            if (ch == '-') return 1;
            return step_num(f, ch) == R_OK;
        }
        case K_BOOL:
        case K_NULL: {
            int id = (o->kind == K_NULL) ? 2 : (ch == 't' ? 0 : 1);
            if (o->kind == K_BOOL && ch != 't' && ch != 'f') return 0;
            ofr *f = push(c, F_LIT, node);
            f->b = id;
            return step_lit(f, ch) == R_OK;
        }
        case K_ENUM: {
            ofr *f = push(c, F_ENUM, node);
            f->cand = (o->count >= 64) ? ~0ull : ((1ull << o->count) - 1);
            return step_enum(g, f, ch) == R_OK;
        }
        }
        return 0;
    }
    /* any JSON value */
    if (ch == '{' && (kinds & AK_OBJ)) {
        if (depth_of(c) + 1 > g->depth_cap) return 0;
        ofr *f = push(c, F_OBJ, g->open_obj);
        f->a = -1;
        return 1;
    }
    if (ch == '[' && (kinds & AK_ARR)) {
        if (depth_of(c) + 1 > g->depth_cap) return 0;
        push(c, F_ARR, g->open_arr);
        return 1;
    }
    if (ch == '"' && (kinds & AK_STR)) {
        ofr *f = push(c, F_STR, -1);
        f->b = g->open_cap;
        return 1;
    }
    if ((ch == '-' || is_digit(ch)) && (kinds & AK_NUM)) {
        ofr *f = push(c, F_NUM, -1);
        f->phase = N_MINUS;
        if (ch == '-') return 1;
        return step_num(f, ch) == R_OK;
    }
    if ((ch == 't' || ch == 'f' || ch == 'n') && (kinds & AK_LIT)) {
        ofr *f = push(c, F_LIT, -1);
        f->b = ch == 't' ? 0 : ch == 'f' ? 1 : 2;
        return step_lit(f, ch) == R_OK;
    }
    return 0;
}

static int step_frame(const og *g, oconf *c, ofr *f, int ch);

static int step_root(const og *g, oconf *c, ofr *f, int ch) {
    switch (f->phase) {
    case RT_NAME: {
        int full = lit_step(g, g->tools_first, g->tools_count, &f->cand, f->a, ch);
        if (full == -2) return R_DEAD;
        f->a++;
        if (full >= 0) { f->b = full; f->phase = RT_VALUE; }
        return R_OK;
    }
    case RT_VALUE: {
        int node = (g->gkind == G_TOOL) ? g->props[g->tools_first + f->b].node : g->root;
        f->phase = RT_INVAL;
        return start_value(g, c, node, AK_OBJ | AK_ARR | AK_STR | AK_NUM | AK_LIT, ch) ? R_OK : R_DEAD;
    }
    case RT_CLOSE:
        if (ch != ')') return R_DEAD;
        f->phase = RT_DONE;
        return R_OK;
    default:
        return R_DEAD;
    }
}

/* a child frame finished: advance the parent's phase */
static void child_done(const og *g, ofr *p) {
    switch (p->kind) {
    case F_ROOT:
        p->phase = (g->gkind == G_TOOL) ? RT_CLOSE : RT_DONE;
        break;
    case F_OBJ:
        if (p->phase == O_KEYSTR) p->phase = O_COLON;
        else p->phase = O_AFTER;
        p->ws = 0;
        break;
    case F_ARR:
        p->phase = A_AFTER;
        p->ws = 0;
        break;
    case F_TEXT: /* a calc span closed: the engine's result comes next */
        p->phase = X_RES;
        p->a = 0;
        p->b = 0;
        break;
    default:
        abort();
    }
}

static int step_frame(const og *g, oconf *c, ofr *f, int ch) {
    switch (f->kind) {
    case F_ROOT: return step_root(g, c, f, ch);
    case F_OBJ: return step_obj(g, c, f, ch);
    case F_ARR: return step_arr(g, c, f, ch);
    case F_STR: return step_str(f, ch);
    case F_INT: return step_int(g, f, ch);
    case F_NUM: return step_num(f, ch);
    case F_LIT: return step_lit(f, ch);
    case F_ENUM: return step_enum(g, f, ch);
    case F_CALC: return step_calc(g, f, ch);
    case F_TEXT: return step_text(g, c, f, ch);
    case F_STROP: return step_strop(g, f, ch);
    }
    return R_DEAD;
}

/* ---- public API --------------------------------------------------------- */
int og_sat(const og *g, int node, int depth) { return sat(g, node, depth); }

int oc_size(void) { return (int)sizeof(oconf); }

void oc_start(const og *g, oconf *c) {
    memset(c, 0, sizeof *c);
    if (g->gkind == G_CALC) {
        push(c, F_CALC, -1);
        return;
    }
    if (g->gkind == G_TEXT) {
        push(c, F_TEXT, -1);
        return;
    }
    ofr *r = push(c, F_ROOT, -1);
    if (g->gkind == G_TOOL) {
        /* tools whose arguments can be completed */
        r->phase = RT_NAME;
        r->cand = 0;
        for (int i = 0; i < g->tools_count; i++)
            if (sat(g, g->props[g->tools_first + i].node, 0)) r->cand |= 1ull << i;
    } else {
        r->phase = RT_VALUE;
    }
}

static int feed1(const og *g, oconf *c, int ch) {
    for (;;) {
        ofr *f = &c->f[c->n - 1];
        int r = step_frame(g, c, f, ch);
        if (r == R_OK) return 1;
        if (r == R_DEAD) return 0;
        /* the frame finished */
        c->n--;
        child_done(g, &c->f[c->n - 1]);
        if (r == R_DONE_TOOK) return 1;
        /* R_DONE_LEFT: the parent sees the same byte */
    }
}

/* Is the next byte one the engine writes (not the model)? */
int oc_in_engine(const og *g, const oconf *c) {
    return g->gkind == G_TEXT && c->n == 1 && c->f[0].phase == X_RES;
}

/* Feed n bytes of the language (engine-written ones included); returns how
 * many were accepted before the first refusal (n if all were).  After a
 * refusal the configuration is unspecified. */
int oc_feed(const og *g, oconf *c, const uint8_t *s, int n) {
    for (int i = 0; i < n; i++)
        if (!feed1(g, c, s[i])) return i;
    return n;
}

/* The same for bytes the model writes: a byte where the engine writes is
 * refused (a model token may end where the engine's region begins). */
int oc_feed_model(const og *g, oconf *c, const uint8_t *s, int n) {
    for (int i = 0; i < n; i++)
        if (oc_in_engine(g, c) || !feed1(g, c, s[i])) return i;
    return n;
}

/* Is the byte string fed so far a member of the language? */
int oc_complete(const og *g, const oconf *c) {
    const ofr *f = &c->f[0];
    if (g->gkind == G_CALC) return f->phase == C_DONE;
    if (g->gkind == G_TEXT) return c->n == 1 && f->phase == X_DONE;
    return c->n == 1 && f->phase == RT_DONE;
}

static void copy_conf(oconf *dst, const oconf *src) {
    dst->n = src->n;
    memcpy(dst->f, src->f, sizeof(ofr) * (size_t)src->n);
}

/*
 * Token mask for one configuration: bit t is set iff every byte of token t
 * is accepted from the configuration as a byte the model writes, i.e.
 * p.b(t) is a viable prefix reached without writing into the engine's part.
 * Bit t&63 of word t>>6.  Returns the number of bytes walked.
 */
int64_t oc_mask(const og *g, const oconf *c, const uint8_t *blob, const uint32_t *off, int V,
                uint64_t *words) {
    int W = (V + 63) / 64;
    memset(words, 0, sizeof(uint64_t) * (size_t)W);
    int64_t walked = 0;
    oconf t;
    for (int tok = 0; tok < V; tok++) {
        uint32_t a = off[tok], b = off[tok + 1];
        if (b == a) continue; /* empty tokens are never allowed */
        copy_conf(&t, c);
        int k = oc_feed_model(g, &t, blob + a, (int)(b - a));
        walked += (k < (int)(b - a)) ? k + 1 : k;
        if (k == (int)(b - a)) words[tok >> 6] |= 1ull << (tok & 63);
    }
    return walked;
}

/* rows in parallel over nthreads; done[r] != 0 gives an all-zero row */
typedef struct {
    const og *g;
    const oconf *confs;
    const uint8_t *done;
    const uint8_t *blob;
    const uint32_t *off;
    int V, r0, r1;
    uint64_t *words;
    int64_t walked;
} mask_job;

static void *mask_worker(void *p) {
    mask_job *j = (mask_job *)p;
    int W = (j->V + 63) / 64;
    for (int r = j->r0; r < j->r1; r++) {
        if (j->done && j->done[r]) {
            memset(j->words + (size_t)r * W, 0, sizeof(uint64_t) * (size_t)W);
            continue;
        }
        j->walked += oc_mask(j->g, &j->confs[r], j->blob, j->off, j->V, j->words + (size_t)r * W);
    }
    return NULL;
}

int64_t oc_mask_rows(const og *g, const oconf *confs, const uint8_t *done, int rows, const uint8_t *blob,
                     const uint32_t *off, int V, uint64_t *words, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > rows) nthreads = rows > 0 ? rows : 1;
    pthread_t th[256];
    mask_job jobs[256];
    if (nthreads > 256) nthreads = 256;
    for (int i = 0; i < nthreads; i++) {
        jobs[i] = (mask_job){g, confs, done, blob, off, V, rows * i / nthreads, rows * (i + 1) / nthreads,
                             words, 0};
        pthread_create(&th[i], NULL, mask_worker, &jobs[i]);
    }
    int64_t walked = 0;
    for (int i = 0; i < nthreads; i++) {
        pthread_join(th[i], NULL);
        walked += jobs[i].walked;
    }
    return walked;
}

/* bytes allowed next (a 256-bit set as 4 words): the "boundary trace" */
void oc_next_bytes(const og *g, const oconf *c, uint64_t *set4) {
    memset(set4, 0, 32);
    oconf t;
    for (int b = 0; b < 256; b++) {
        copy_conf(&t, c);
        uint8_t s = (uint8_t)b;
        if (oc_feed_model(g, &t, &s, 1) == 1) set4[b >> 6] |= 1ull << (b & 63);
    }
}
