// capi.cpp -- the C ABI (include/cg.h): argument checks, device upload, and
// the host walker behind cg_try_input.
#include <string.h>

#include <algorithm>
#include <chrono>
#include <functional>
#include <mutex>
#include <string>
#include <vector>

#include "cg_internal.hpp"
#include "fill_plan.hpp"

namespace cg {
const char *last_error();
int launch_init(const cg_grammar *g, cg_state *states, int B, hipStream_t st);
int launch_advance(const cg_grammar *g, cg_state *states, int B, const int32_t *ids, int32_t *steps,
                   int32_t *status, hipStream_t st);
int launch_force(const cg_grammar *g, cg_state *states, int B, const uint8_t *bytes, uint64_t n_bytes,
                 const uint32_t *offsets, int32_t *status, hipStream_t st);
int launch_fill(const cg_grammar *g, const cg_state *states, int B, uint64_t *mask, int wpr, void *ws,
                hipStream_t st);
int noalloc_setup(int dev);
int launch_fill_noalloc(const cg_grammar *g, const cg_state *states, int B, uint64_t *mask, int wpr,
                        hipStream_t st);
int launch_draft(const cg_grammar *g, const cg_state *states, const int32_t *steps, int B, const int32_t *draft,
                 int kd, cg_state *path, int32_t *accept_len, hipStream_t st);
int fill_plan_stride(const cg_grammar *g);
int launch_mask_and(uint64_t *rows, const uint8_t *need, const uint64_t *m, int n, int Wv, hipStream_t st);
size_t sample_workspace_bytes(int B, int V);
size_t fill_lds_bytes(const cg_grammar *g, int items_per_row);
int launch_sample(const void *logits, int dt, int B, int V, int64_t stride, const uint64_t *mask, int wpr,
                  const float *temp, const uint64_t *seed, const int32_t *step, void *ws, int32_t *out_id,
                  float *out_lp, const cg_grammar *g, cg_state *states, int32_t *steps_rw, int32_t *status,
                  hipStream_t st, const FillArgs *plan = nullptr);
FillArgs make_fill_args(const cg_grammar *g, const cg_state *states, int B, uint64_t *mask, int wpr, void *ws);
int fill_check(const cg_grammar *g, int B);
int launch_fill_walk(const cg_grammar *g, const FillArgs &a, hipStream_t st);
}  // namespace cg

using namespace cg;

namespace {

int arg_error(const char *msg) {
    set_error("%s", msg);
    return CG_E_ARG;
}

template <class T>
int upload(T **dst, const T *src, size_t n) {
    if (hipMalloc((void **)dst, std::max<size_t>(n, 1) * sizeof(T)) != hipSuccess) return CG_E_DEVICE;
    if (n && hipMemcpy(*dst, src, n * sizeof(T), hipMemcpyHostToDevice) != hipSuccess) return CG_E_DEVICE;
    return CG_OK;
}

void release(cg_grammar *g) {
    if (!g) return;
    if (g->device >= 0) {
        int cur = 0;
        (void)hipGetDevice(&cur);
        (void)hipSetDevice(g->device);
        (void)hipFree(g->dev.comb);
        (void)hipFree(g->dev.tokw);
        (void)hipFree(g->dev.tokinfo);
        (void)hipFree(g->dev.legal);
        (void)hipFree(g->dev.forced);
        (void)hipFree(g->dev.state_mask);
        (void)hipFree(g->dev.closebits);
        (void)hipFree(g->dev.c_idlen);
        (void)hipFree(g->dev.c_jump);
        (void)hipFree(g->dev.c_w);
        (void)hipFree(g->dev.c_tile);
        (void)hipFree(g->dev.retmask2);
        (void)hipFree(g->dev.qc_idlen);
        (void)hipFree(g->dev.qc_jump);
        (void)hipFree(g->dev.qc_w);
        (void)hipFree(g->dev.qc_tile);
        (void)hipFree(g->dev.retmask);
        (void)hipFree(g->dev.rq_idx);
        (void)hipFree(g->dev.smask_idx);
        (void)hipFree(g->dev.lex_idlen);
        (void)hipFree(g->dev.lex_jump);
        (void)hipFree(g->dev.lex_w);
        (void)hipFree(g->dev.lex_tile);
        (void)hipFree(g->dev.q_idlen);
        (void)hipFree(g->dev.q_jump);
        (void)hipFree(g->dev.q_w);
        (void)hipFree(g->dev.q_tile);
        (void)hipFree(g->dev.strbits);
        (void)hipSetDevice(cur);
    }
    free(g->host_comb);
    delete g;
}

bool on_device(const cg_grammar *g) { return g && g->device >= 0; }

// Walk a token through the string body from a code-point boundary with the
// same table the kernels use; see tokinfo in cg_internal.hpp.
uint32_t string_summary(const cg_grammar *g, const uint8_t *s, uint32_t n) {
    if (g->k.s_body >= g->k.q_limit) return STR_DEAD << 8;
    uint32_t q = g->k.s_body, chars = 0;
    for (uint32_t i = 0; i < n; i++) {
        const uint64_t e = g->host_comb[q + s[i]];
        const uint32_t lo = (uint32_t)e, op = (uint32_t)(e >> 32) & 0xFu;
        if ((lo & 0xFFFFu) != q) return STR_DEAD << 8;
        if (op == OP_STR_CLOSE) return (STR_QUOTE << 8) | (chars << 10) | (i << 16);
        if (op == OP_CHAR) chars++;
        q = lo >> 16;
    }
    return (STR_IN << 8) | (chars << 10);
}

// Candidate tables of the fill kernel (see DeviceTables).  In lexicographic
// order, tokens sharing their first bytes sit in the same 64-token tiles: a
// row then visits only tiles holding a key it can accept.
constexpr size_t kCloseMaskBudget = 64ull << 20;  // bytes of per-resume-state closing masks

struct FillHost {
    std::vector<uint64_t> legal, strbits, closebits, retmask;
    std::vector<int32_t> rq_idx;
    std::vector<uint64_t> s0;  // tokens that stay inside the container a row is in (bit per id)
    std::vector<uint64_t> retmask2;  // [resume][kind of the open container][Wv]
    std::vector<uint32_t> qc_idlen, qc_jump, qc_w;
    std::vector<uint2> qc_tile;
    std::vector<uint32_t> c_idlen, c_jump, c_w;
    std::vector<uint2> c_tile;
    std::vector<uint32_t> lex_idlen, lex_jump, lex_w, q_idlen, q_jump, q_w;
    std::vector<uint2> lex_tile, q_tile;
};

// Brackets of a token read from outside a string: R = the deepest level at
// or below the start that a closing bracket lands on (-1: none), H = the
// highest level an opening bracket opens from (-1: none).  Brackets inside
// JSON strings are content when the grammar has strings.  The automaton's
// pushes and pops happen only on these bytes, so R and H never under-count
// what a walk of the token does.
void bracket_profile(const uint8_t *b, uint32_t n, bool json_strings, int &R, int &H) {
    int lvl = 0;
    bool in_str = false, esc = false;
    R = -1;
    H = -1;
    for (uint32_t i = 0; i < n; i++) {
        const uint8_t c = b[i];
        if (in_str) {
            if (esc) esc = false;
            else if (c == '\\') esc = true;
            else if (c == '"') in_str = false;
            continue;
        }
        if (json_strings && c == '"') {
            in_str = true;
        } else if (c == '{' || c == '[' || c == '(') {
            H = std::max(H, lvl);
            lvl++;
        } else if (c == '}' || c == ']' || c == ')') {
            lvl--;
            if (lvl <= 0) R = std::max(R, -lvl);
        }
    }
}

void build_fill_tables(const cg_grammar *g, const uint8_t *tok_bytes, const uint32_t *tok_offsets,
                       const std::vector<uint32_t> &tokinfo, FillHost &f) {
    constexpr uint32_t kPad = 0xFFFFFFFFu;
    const uint32_t V = (uint32_t)g->V, nw = (uint32_t)g->nw, Wv = (V + 63) / 64;
    auto bytes = [&](uint32_t t) { return tok_bytes + tok_offsets[t]; };
    auto len = [&](uint32_t t) { return tok_offsets[t + 1] - tok_offsets[t]; };
    auto less_from = [&](uint32_t a, uint32_t oa, uint32_t b, uint32_t ob) {
        const uint32_t na = len(a) - oa, nb = len(b) - ob;
        const int c = memcmp(bytes(a) + oa, bytes(b) + ob, std::min(na, nb));
        if (c != 0) return c < 0;
        if (na != nb) return na < nb;
        return a < b;
    };
    // bytes with a transition out of each state
    f.legal.assign((size_t)g->k.q_limit * 4, 0ull);
    for (uint32_t q = 0; q < g->k.q_limit; q++)
        for (uint32_t b = 0; b < 256; b++)
            if ((g->host_comb[q + b] & 0xFFFFu) == q) f.legal[(size_t)q * 4 + (b >> 6)] |= 1ull << (b & 63);
    auto pad = [&](std::vector<uint32_t> &order) { order.resize((order.size() + kTile - 1) / kTile * kTile, kPad); };
    // a list's walk data: per token, id | bytes to walk << 24 | 1 << 31 (0 marks
    // padding) and those bytes, from(t) on, nw words per token
    auto pack = [&](const std::vector<uint32_t> &order, std::vector<uint32_t> &idlen, std::vector<uint32_t> &w,
                    auto from) {
        const size_t n = order.size();
        idlen.assign(std::max<size_t>(n, 1), 0u);
        w.assign(std::max<size_t>(nw * n, 1), 0u);
        for (size_t i = 0; i < n; i++) {
            const uint32_t t = order[i];
            if (t == kPad) continue;
            const uint32_t f0 = from(t);
            idlen[i] = t | (len(t) - f0) << 24 | 1u << 31;
            for (uint32_t j = f0; j < len(t); j++)
                w[((j - f0) >> 2) * n + i] |= (uint32_t)bytes(t)[j] << (8 * ((j - f0) & 3));
        }
    };
    auto whole = [](uint32_t) { return 0u; };
    // key span of each tile over its real tokens (keys never decrease along a list)
    auto spans = [&](const std::vector<uint32_t> &order, auto key, std::vector<uint2> &tile) {
        tile.clear();
        for (size_t i = 0; i < order.size(); i += kTile) {
            size_t j = i + kTile - 1;
            while (order[j] == kPad) j--;
            tile.push_back(make_uint2(key(order[i]), key(order[j])));
        }
        if (tile.empty()) tile.push_back(make_uint2(1, 0));  // placeholder, never read
    };
    std::vector<uint32_t> lex, q;
    for (uint32_t t = 0; t < V; t++) {
        if (len(t) == 0) continue;
        lex.push_back(t);
        if (tok_kind(tokinfo[t]) == STR_QUOTE) q.push_back(t);
    }
    auto qoff = [&](uint32_t t) { return tok_pos(tokinfo[t]) + 1; };
    std::sort(lex.begin(), lex.end(), [&](uint32_t a, uint32_t b) { return less_from(a, 0, b, 0); });
    std::sort(q.begin(), q.end(), [&](uint32_t a, uint32_t b) { return less_from(a, qoff(a), b, qoff(b)); });
    pad(lex);
    pad(q);
    pack(lex, f.lex_idlen, f.lex_w, whole);
    pack(q, f.q_idlen, f.q_w, qoff);  // the bytes after the closing quote
    spans(lex, [&](uint32_t t) { return lead_key(bytes(t)[0], len(t) > 1 ? bytes(t)[1] : 0u, len(t)); }, f.lex_tile);
    spans(q, [&](uint32_t t) { return qoff(t) == len(t) ? 0u : bytes(t)[qoff(t)] + 1u; }, f.q_tile);
    // the jump: where the token's first quote is, and how the bytes after it
    // read as string content
    // read from where the list's walk starts (from(t))
    auto jumps = [&](const std::vector<uint32_t> &order, std::vector<uint32_t> &jump, auto from) {
        jump.assign(std::max<size_t>(order.size(), 1), kNoQuote);
        for (size_t i = 0; i < order.size(); i++) {
            const uint32_t t = order[i];
            if (t == kPad || g->k.s_body >= g->k.q_limit) continue;
            const uint8_t *b = bytes(t) + from(t);
            const uint32_t n = len(t) - from(t);
            const uint8_t *qp = (const uint8_t *)memchr(b, '"', n);
            if (!qp) continue;
            const uint32_t at = (uint32_t)(qp - b);
            jump[i] = at | string_summary(g, b + at + 1, n - at - 1);
        }
    };
    // a string list's tokens also carry the code points before their closing
    // quote (bits 21..26)
    auto with_chars = [&](const std::vector<uint32_t> &order, std::vector<uint32_t> &jump) {
        for (size_t i = 0; i < order.size(); i++)
            if (order[i] != kPad) jump[i] |= tok_chars(tokinfo[order[i]]) << 21;
    };
    jumps(lex, f.lex_jump, whole);
    // tokens that stay inside the container a row is in (s0) and the rest,
    // kept as a lexicographic tile list of their own
    f.s0.assign(Wv, 0ull);
    std::vector<uint32_t> cl;
    const bool json_strings = g->k.s_body < g->k.q_limit;
    for (uint32_t t = 0; t < V; t++) {
        if (len(t) == 0) continue;
        int R, H;
        bracket_profile(bytes(t), len(t), json_strings, R, H);
        if (R <= 0 && H <= kPushLimit) f.s0[t >> 6] |= 1ull << (t & 63);
        else cl.push_back(t);
    }
    std::sort(cl.begin(), cl.end(), [&](uint32_t a, uint32_t b) { return less_from(a, 0, b, 0); });
    pad(cl);
    pack(cl, f.c_idlen, f.c_w, whole);
    spans(cl, [&](uint32_t t) { return lead_key(bytes(t)[0], len(t) > 1 ? bytes(t)[1] : 0u, len(t)); }, f.c_tile);
    jumps(cl, f.c_jump, whole);
    jumps(q, f.q_jump, qoff);
    with_chars(q, f.q_jump);
    // tokens that end inside the string, per budget
    f.strbits.assign((size_t)kStrBitsets * Wv, 0ull);
    for (uint32_t t = 0; t < V; t++) {
        if (len(t) == 0 || tok_kind(tokinfo[t]) != STR_IN) continue;
        for (uint32_t c = tok_chars(tokinfo[t]); c < (uint32_t)kStrBitsets; c++)
            f.strbits[(size_t)c * Wv + (t >> 6)] |= 1ull << (t & 63);
    }
    // Tokens that close the string: the content before the quote fits a
    // budget of c code points (closebits[c]), and the bytes after the quote
    // are accepted from resume state R with no open container (retmask[R]).
    // A row inside a string with no open container then needs no walk:
    // strbits[c] | (closebits[c] & retmask[ret]).
    f.closebits.assign((size_t)kStrBitsets * Wv, 0ull);
    f.rq_idx.assign(g->k.q_limit, -1);
    if (g->k.s_body >= g->k.q_limit) return;
    std::vector<uint32_t> closers;
    for (uint32_t t : q)
        if (t != kPad) closers.push_back(t);
    for (uint32_t t : closers)
        for (uint32_t c = tok_chars(tokinfo[t]); c < (uint32_t)kStrBitsets; c++)
            f.closebits[(size_t)c * Wv + (t >> 6)] |= 1ull << (t & 63);
    std::vector<uint32_t> resume;
    for (uint32_t i = 0; i < g->comb_len; i++) {
        const uint64_t e = g->host_comb[i];
        const uint32_t owner = (uint32_t)e & 0xFFFFu, op = (uint32_t)(e >> 32) & 0xFu;
        if (owner < g->k.q_limit && op == OP_STR_OPEN) resume.push_back(((uint32_t)e >> 16) & 0xFFFFu);
    }
    std::sort(resume.begin(), resume.end());
    resume.erase(std::unique(resume.begin(), resume.end()), resume.end());
    if (resume.size() * Wv * 8 > kCloseMaskBudget) return;
    f.retmask.assign(resume.size() * Wv, 0ull);
    for (size_t j = 0; j < resume.size(); j++) {
        f.rq_idx[resume[j]] = (int32_t)j;
        for (uint32_t t : closers) {
            Walker w;
            w.q = resume[j];
            w.ret = g->k.start;
            w.cnt = 0;
            w.ws = 0;
            w.depth = 0;
            w.stk = 0;
            bool ok = true;
            for (uint32_t i = tok_pos(tokinfo[t]) + 1; ok && i < len(t); i++)
                ok = step_byte(w, bytes(t)[i], g->host_comb, g->k);
            if (ok) f.retmask[j * Wv + (t >> 6)] |= 1ull << (t & 63);
        }
    }
    // The same inside an open container (depth 1, container kind b), for the
    // closing tokens whose bytes after the quote stay inside it and open at
    // most kPushLimit more; the other closing tokens form a list of their
    // own, in the string-closing order, walked for such rows.
    std::vector<uint32_t> qc;
    std::vector<uint32_t> stay;
    for (uint32_t t : q) {
        if (t == kPad) continue;
        int R, H;
        const uint32_t at = tok_pos(tokinfo[t]) + 1;
        bracket_profile(bytes(t) + at, len(t) - at, true, R, H);
        if (R <= 0 && H <= kPushLimit) stay.push_back(t);
        else qc.push_back(t);
    }
    if (resume.size() * 2 * Wv * 8 <= kCloseMaskBudget) {
        f.retmask2.assign(resume.size() * 2 * Wv, 0ull);
        for (size_t j = 0; j < resume.size(); j++)
            for (uint32_t b = 0; b < 2; b++)
                for (uint32_t t : stay) {
                    Walker w;
                    w.q = resume[j];
                    w.ret = g->k.start;
                    w.cnt = 0;
                    w.ws = 0;
                    w.depth = 1;
                    w.stk = b;
                    bool ok = true;
                    for (uint32_t i = tok_pos(tokinfo[t]) + 1; ok && i < len(t); i++)
                        ok = step_byte(w, bytes(t)[i], g->host_comb, g->k);
                    if (ok) f.retmask2[(j * 2 + b) * Wv + (t >> 6)] |= 1ull << (t & 63);
                }
    }
    pad(qc);
    pack(qc, f.qc_idlen, f.qc_w, qoff);
    spans(qc, [&](uint32_t t) { return qoff(t) == len(t) ? 0u : bytes(t)[qoff(t)] + 1u; }, f.qc_tile);
    jumps(qc, f.qc_jump, qoff);
    with_chars(qc, f.qc_jump);
}

}  // namespace

// Masks computed once with the fill kernels themselves, for states outside
// strings: context 0 = (state, whitespace run, no open container), the whole
// mask; contexts 1 and 2 = the same inside an open object / array at depth 1,
// kept only for the tokens in s0 (those that cannot close the container the
// row is in and open at most kPushLimit more).  A state's registers other
// than the whitespace run and the container stack are read only inside
// strings, so context 0 depends on (state, run) alone; an s0 token reads of
// the stack only the innermost container's kind and meets the depth cap
// only if depth + kPushLimit reaches the smallest cap, so for such rows
// context 1 / 2 holds exactly.  Rows above that depth walk as before.  The
// table keeps to kStateMaskBudget bytes, dropping whitespace runs, then
// open containers, when it would not fit.
constexpr size_t kStateMaskBudget = 96ull << 20;

int build_state_masks(cg_grammar *g, const FillHost &f) {
    const size_t Wv = ((size_t)g->V + 63) / 64;
    const uint32_t QL = g->k.q_limit, WD = g->k.ws_max + 1;
    // targets of whitespace bytes, and the states that can be inside an open container
    std::vector<char> ws_target(QL, 0), inside(QL, 0);
    std::vector<uint32_t> work;
    int min_cap = 0;
    for (uint32_t q = 0; q < QL; q++)
        for (uint32_t b = 0; b < 256; b++) {
            const uint64_t e = g->host_comb[q + b];
            if (((uint32_t)e & 0xFFFFu) != q) continue;
            const uint32_t op = (uint32_t)(e >> 32) & 0xFu, nx = ((uint32_t)e >> 16) & 0xFFFFu;
            if (op == OP_WS && nx < QL) ws_target[nx] = 1;
            if (op == OP_PUSH) {
                const int cap = (int)((uint32_t)(e >> 36) >> 1);
                min_cap = min_cap == 0 ? cap : std::min(min_cap, cap);
                if (nx < QL && !inside[nx]) {
                    inside[nx] = 1;
                    work.push_back(nx);
                }
            }
        }
    while (!work.empty()) {
        const uint32_t q = work.back();
        work.pop_back();
        for (uint32_t b = 0; b < 256; b++) {
            const uint64_t e = g->host_comb[q + b];
            if (((uint32_t)e & 0xFFFFu) != q) continue;
            const uint32_t op = (uint32_t)(e >> 32) & 0xFu, arg = (uint32_t)(e >> 36);
            uint32_t to[2] = {((uint32_t)e >> 16) & 0xFFFFu, 0xFFFFFFFFu};
            if (op == OP_STR_CLOSE) continue;
            if (op == OP_POP) to[0] = arg >> 14, to[1] = arg & 0x3FFFu;
            for (uint32_t t : to)
                if (t < QL && !inside[t]) {
                    inside[t] = 1;
                    work.push_back(t);
                }
        }
    }
    g->min_push_cap = min_cap;
    struct Cfg {
        uint32_t q, ws, ctx;
    };
    std::vector<Cfg> cfg;
    const size_t cap_rows = kStateMaskBudget / (Wv * 8);
    auto add_group = [&](uint32_t ws_lo, uint32_t ws_hi, bool ctx0, bool ctx12) {
        std::vector<Cfg> grp;
        for (uint32_t q : g->plain_q)
            for (uint32_t ws = ws_lo; ws <= ws_hi; ws++) {
                if (ws > 0 && !ws_target[q]) continue;
                if (ctx0) grp.push_back({q, ws, 0});
                if (ctx12 && inside[q] && min_cap > 0) {
                    grp.push_back({q, ws, 1});
                    grp.push_back({q, ws, 2});
                }
            }
        if (cfg.size() + grp.size() <= cap_rows) cfg.insert(cfg.end(), grp.begin(), grp.end());
    };
    add_group(0, 0, true, false);
    add_group(0, 0, false, true);
    if (g->k.ws_max > 0) {
        add_group(1, g->k.ws_max, true, false);
        add_group(1, g->k.ws_max, false, true);
    }
    const size_t n = cfg.size();
    if (n == 0) return CG_OK;
    std::vector<cg_state> st(n);
    std::vector<uint8_t> need(n, 0);
    std::vector<int32_t> idx((size_t)QL * WD * 3, -1);
    for (size_t i = 0; i < n; i++) {
        cg_state &c = st[i];
        memset(&c, 0, sizeof c);
        c.q = (uint16_t)cfg[i].q;
        c.ret = (uint16_t)g->k.start;
        c.ws = (uint8_t)cfg[i].ws;
        c.depth = cfg[i].ctx ? 1 : 0;
        c.stk = cfg[i].ctx == 2 ? 1u : 0u;
        need[i] = cfg[i].ctx != 0;
        idx[((size_t)cfg[i].q * WD + cfg[i].ws) * 3 + cfg[i].ctx] = (int32_t)i;
    }
    cg_state *d_st = nullptr;
    void *d_ws = nullptr;
    uint64_t *d_mask = nullptr, *d_s0 = nullptr;
    uint8_t *d_need = nullptr;
    int rc = CG_OK;
    const size_t ws_bytes = (size_t)fill_plan_stride(g) * 4 * n;
    if (upload(&d_st, st.data(), n) != CG_OK || upload(&d_need, need.data(), n) != CG_OK ||
        upload(&d_s0, f.s0.data(), f.s0.size()) != CG_OK || hipMalloc(&d_ws, ws_bytes) != hipSuccess ||
        hipMalloc((void **)&d_mask, n * Wv * 8) != hipSuccess) {
        set_error("state masks: allocation failed: %s", hipGetErrorString(hipGetLastError()));
        rc = CG_E_DEVICE;
    }
    if (rc == CG_OK) rc = launch_fill(g, d_st, (int)n, d_mask, (int)Wv, d_ws, nullptr);
    if (rc == CG_OK) rc = launch_mask_and(d_mask, d_need, d_s0, (int)n, (int)Wv, nullptr);
    if (rc == CG_OK && hipStreamSynchronize(nullptr) != hipSuccess) {
        set_error("state masks: %s", hipGetErrorString(hipGetLastError()));
        rc = CG_E_DEVICE;
    }
    if (rc == CG_OK && upload(&g->dev.smask_idx, idx.data(), idx.size()) != CG_OK) {
        set_error("state masks: upload failed");
        rc = CG_E_DEVICE;
    }
    (void)hipFree(d_st);
    (void)hipFree(d_ws);
    (void)hipFree(d_need);
    (void)hipFree(d_s0);
    if (rc != CG_OK) {
        (void)hipFree(d_mask);
        return rc;
    }
    g->dev.state_mask = d_mask;
    g->n_smask = (int32_t)n;
    return CG_OK;
}

// Compiled grammars are shared by (spec text, vocabulary, options, device):
// an identical compile returns the same read-only handle with one more
// reference ("Evaluator aware decoding", "Where XGrammar-2 could take
// this": cross-grammar caching keeps repeated grammars from blowing up
// compilation).  Up to kCacheIdle handles no one holds any more are kept
// for later identical compiles (least recently released first out).
namespace {
constexpr size_t kCacheIdle = 8;

struct CacheEntry {
    std::string spec;
    uint64_t h1, h2;  // two independent hashes of the vocabulary
    int32_t V;
    uint32_t gen_cap, flags;
    int device;
    cg_grammar *g;
    uint64_t idle_since;  // 0 while referenced
};

std::mutex g_cache_mu;
std::vector<CacheEntry> g_cache;
uint64_t g_clock = 0;
int64_t g_hits = 0, g_misses = 0;

void vocab_hash(const uint8_t *bytes, const uint32_t *off, int32_t V, uint64_t &h1, uint64_t &h2) {
    h1 = 0xcbf29ce484222325ull;  // FNV-1a, then a second FNV-style pass with another basis and prime
    h2 = 0x84222325cbf29ce4ull;
    auto mix = [&](uint8_t b) {
        h1 = (h1 ^ b) * 0x100000001b3ull;
        h2 = (h2 ^ b) * 0x00000100000001b3ull + 0x9e3779b97f4a7c15ull;
    };
    for (int32_t t = 0; t <= V; t++)
        for (int k = 0; k < 4; k++) mix((uint8_t)(off[t] >> (8 * k)));
    for (uint32_t i = 0; i < off[V]; i++) mix(bytes[i]);
}

void evict_idle() {
    size_t idle = 0;
    for (auto &e : g_cache) idle += e.g->refs == 0;
    while (idle > kCacheIdle) {
        size_t oldest = g_cache.size();
        for (size_t i = 0; i < g_cache.size(); i++)
            if (g_cache[i].g->refs == 0 && (oldest == g_cache.size() || g_cache[i].idle_since < g_cache[oldest].idle_since))
                oldest = i;
        release(g_cache[oldest].g);
        g_cache.erase(g_cache.begin() + oldest);
        idle--;
    }
}

int compile_uncached(const char *spec_json, size_t spec_len, const uint8_t *tok_bytes, const uint32_t *tok_offsets,
                     int32_t vocab_size, const cg_options *opts, cg_grammar **out) {
    *out = nullptr;
    if (!spec_json) return arg_error("spec_json is NULL");
    if (vocab_size < 1 || !tok_offsets) return arg_error("vocabulary is empty");
    if (tok_offsets[0] != 0) {
        set_error("tok_offsets[0] must be 0");
        return CG_E_VOCAB;
    }
    int max_len = 0;
    for (int32_t t = 0; t < vocab_size; t++) {
        if (tok_offsets[t + 1] < tok_offsets[t]) {
            set_error("tok_offsets decrease at token %d", t);
            return CG_E_VOCAB;
        }
        max_len = std::max<int>(max_len, (int)(tok_offsets[t + 1] - tok_offsets[t]));
    }
    if (tok_offsets[vocab_size] > 0 && !tok_bytes) return arg_error("tok_bytes is NULL");
    if (max_len > kMaxTokenLen) {
        set_error("token longer than %d bytes", kMaxTokenLen);
        return CG_E_LIMIT;
    }
    cg_grammar *g = new cg_grammar;
    int rc = compile_spec(spec_json, spec_len, g);
    if (rc != CG_OK) {
        release(g);
        return rc;
    }
    g->V = vocab_size;
    g->max_len = max_len;
    g->nw = std::max(1, (max_len + 3) / 4);
    g->gen_cap = (opts && opts->gen_cap) ? opts->gen_cap : 2048u;
    if (!(opts && (opts->flags & CG_HOST_ONLY))) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) {
            set_error("no HIP device");
            release(g);
            return CG_E_DEVICE;
        }
        g->device = dev;
        // the address of cg_fill_bitmask_noalloc's scratch array on this
        // device, taken once (a failure is reported by that call)
        (void)noalloc_setup(dev);
        if (hipDeviceGetAttribute(&g->n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || g->n_cu < 1)
            g->n_cu = 256;
        const size_t V = (size_t)vocab_size;
        std::vector<uint32_t> tokw((size_t)g->nw * V, 0u);
        std::vector<uint32_t> tokinfo(V);
        for (size_t t = 0; t < V; t++) {
            const uint32_t a = tok_offsets[t], n = tok_offsets[t + 1] - a;
            tokinfo[t] = n | string_summary(g, tok_bytes + a, n);
            for (uint32_t i = 0; i < n; i++) tokw[(size_t)(i >> 2) * V + t] |= (uint32_t)tok_bytes[a + i] << (8 * (i & 3));
        }
        int lds_max = 0;
        if (hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess &&
            lds_max > 0)
            g->lds_max = lds_max;
        FillHost f;
        build_fill_tables(g, tok_bytes, tok_offsets, tokinfo, f);
        g->lex_tiles = (int32_t)(f.lex_idlen.size() / kTile);
        g->q_tiles = (int32_t)(f.q_idlen.size() / kTile);
        g->c_tiles = (int32_t)(f.c_idlen.size() / kTile);
        g->qc_tiles = (int32_t)(f.qc_idlen.size() / kTile);
        if (fill_lds_bytes(g, 1) + 1024 > (size_t)g->lds_max) {
            set_error("transition table of %u slots needs %zu bytes of LDS in fill_bitmask, the device has %d",
                      g->comb_len, fill_lds_bytes(g, 1), g->lds_max);
            release(g);
            return CG_E_LIMIT;
        }
        if (upload(&g->dev.comb, g->host_comb, g->comb_len) || upload(&g->dev.tokw, tokw.data(), tokw.size()) ||
            upload(&g->dev.tokinfo, tokinfo.data(), V) || upload(&g->dev.legal, f.legal.data(), f.legal.size()) ||
            upload(&g->dev.lex_idlen, f.lex_idlen.data(), f.lex_idlen.size()) ||
            upload(&g->dev.lex_jump, f.lex_jump.data(), f.lex_jump.size()) ||
            upload(&g->dev.lex_w, f.lex_w.data(), f.lex_w.size()) ||
            upload(&g->dev.lex_tile, f.lex_tile.data(), f.lex_tile.size()) ||
            upload(&g->dev.q_idlen, f.q_idlen.data(), f.q_idlen.size()) ||
            upload(&g->dev.q_jump, f.q_jump.data(), f.q_jump.size()) ||
            upload(&g->dev.q_w, f.q_w.data(), f.q_w.size()) ||
            upload(&g->dev.q_tile, f.q_tile.data(), f.q_tile.size()) ||
            upload(&g->dev.strbits, f.strbits.data(), f.strbits.size()) ||
            upload(&g->dev.closebits, f.closebits.data(), f.closebits.size()) ||
            upload(&g->dev.c_idlen, f.c_idlen.data(), f.c_idlen.size()) ||
            upload(&g->dev.c_jump, f.c_jump.data(), f.c_jump.size()) ||
            upload(&g->dev.c_w, f.c_w.data(), f.c_w.size()) ||
            upload(&g->dev.c_tile, f.c_tile.data(), f.c_tile.size()) ||
            (!f.retmask2.empty() && (upload(&g->dev.retmask2, f.retmask2.data(), f.retmask2.size()) ||
                                     upload(&g->dev.qc_idlen, f.qc_idlen.data(), f.qc_idlen.size()) ||
                                     upload(&g->dev.qc_jump, f.qc_jump.data(), f.qc_jump.size()) ||
                                     upload(&g->dev.qc_w, f.qc_w.data(), f.qc_w.size()) ||
                                     upload(&g->dev.qc_tile, f.qc_tile.data(), f.qc_tile.size()))) ||
            (!f.retmask.empty() && (upload(&g->dev.retmask, f.retmask.data(), f.retmask.size()) ||
                                    upload(&g->dev.rq_idx, f.rq_idx.data(), f.rq_idx.size()))) ||
            (g->has_forced && upload(&g->dev.forced, g->host_forced.data(), g->host_forced.size()))) {
            set_error("device upload failed: %s", hipGetErrorString(hipGetLastError()));
            release(g);
            return CG_E_DEVICE;
        }
        rc = build_state_masks(g, f);
        if (rc != CG_OK) {
            release(g);
            return rc;
        }
    }
    *out = g;
    return CG_OK;
}

}  // namespace

extern "C" {

int cg_compile_grammar(const char *spec_json, size_t spec_len, const uint8_t *tok_bytes, const uint32_t *tok_offsets,
                       int32_t vocab_size, const cg_options *opts, cg_grammar **out) {
    if (!out) return arg_error("out is NULL");
    *out = nullptr;
    if (!spec_json) return arg_error("spec_json is NULL");
    if (vocab_size < 1 || !tok_offsets) return arg_error("vocabulary is empty");
    if (tok_offsets[vocab_size] > 0 && !tok_bytes) return arg_error("tok_bytes is NULL");
    const uint32_t gen_cap = (opts && opts->gen_cap) ? opts->gen_cap : 2048u;
    const uint32_t flags = opts ? opts->flags : 0u;
    int device = -1;
    if (!(flags & CG_HOST_ONLY) && hipGetDevice(&device) != hipSuccess) device = -2;
    std::lock_guard<std::mutex> lock(g_cache_mu);
    // offsets are checked by the compile below before the hash reads the bytes
    bool offsets_ok = tok_offsets[0] == 0;
    for (int32_t t = 0; offsets_ok && t < vocab_size; t++) offsets_ok = tok_offsets[t + 1] >= tok_offsets[t];
    uint64_t h1 = 0, h2 = 0;
    if (offsets_ok) {
        vocab_hash(tok_bytes, tok_offsets, vocab_size, h1, h2);
        const std::string spec(spec_json, spec_len);
        for (auto &e : g_cache)
            if (e.V == vocab_size && e.h1 == h1 && e.h2 == h2 && e.gen_cap == gen_cap && e.flags == flags &&
                e.device == device && e.spec == spec) {
                e.g->refs++;
                e.idle_since = 0;
                g_hits++;
                *out = e.g;
                return CG_OK;
            }
    }
    g_misses++;
    const auto t0 = std::chrono::steady_clock::now();
    const int rc = compile_uncached(spec_json, spec_len, tok_bytes, tok_offsets, vocab_size, opts, out);
    if (rc != CG_OK) return rc;
    (*out)->total_ms = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
    g_cache.push_back(CacheEntry{std::string(spec_json, spec_len), h1, h2, vocab_size, gen_cap, flags, device, *out, 0});
    return CG_OK;
}

void cg_free_grammar(cg_grammar *g) {
    if (!g) return;
    std::lock_guard<std::mutex> lock(g_cache_mu);
    if (--g->refs > 0) return;
    for (auto &e : g_cache)
        if (e.g == g) {
            e.idle_since = ++g_clock;  // kept for a later identical compile
            evict_idle();
            return;
        }
    release(g);
}

int cg_cache_stats(int32_t *entries, int64_t *hits, int64_t *misses) {
    std::lock_guard<std::mutex> lock(g_cache_mu);
    if (entries) *entries = (int32_t)g_cache.size();
    if (hits) *hits = g_hits;
    if (misses) *misses = g_misses;
    return CG_OK;
}

int cg_cache_clear(void) {
    std::lock_guard<std::mutex> lock(g_cache_mu);
    for (size_t i = 0; i < g_cache.size();) {
        if (g_cache[i].g->refs == 0) {
            release(g_cache[i].g);
            g_cache.erase(g_cache.begin() + i);
        } else {
            i++;
        }
    }
    return CG_OK;
}

int cg_grammar_info(const cg_grammar *g, cg_info *info) {
    if (!g || !info) return arg_error("NULL argument");
    info->vocab_size = g->V;
    info->words_per_row = (g->V + 63) / 64;
    info->max_token_len = g->max_len;
    info->n_states = g->n_states;
    info->table_entries = (int32_t)g->comb_len;
    info->table_bytes = (int32_t)(g->comb_len * sizeof(uint64_t));
    info->compile_ms = g->compile_ms;
    info->total_ms = g->total_ms;
    info->state_masks = g->n_smask;
    info->pad = 0;
    info->max_bytes = g->max_bytes;
    return CG_OK;
}

int cg_init_state(const cg_grammar *g, cg_state *d_states, int32_t batch, void *stream) {
    if (!on_device(g)) return arg_error("grammar has no device tables");
    if (batch < 0 || (batch > 0 && !d_states)) return arg_error("bad states / batch");
    return launch_init(g, d_states, batch, (hipStream_t)stream);
}

size_t cg_fill_workspace_bytes(const cg_grammar *g, int32_t batch) {
    if (!on_device(g) || batch < 1) return 0;
    return (size_t)batch * (size_t)fill_plan_stride(g) * sizeof(uint32_t);
}

int cg_fill_bitmask(const cg_grammar *g, const cg_state *d_states, int32_t batch, uint64_t *d_mask,
                    int32_t words_per_row, void *d_workspace, void *stream) {
    if (!on_device(g)) return arg_error("grammar has no device tables");
    if (batch < 0 || (batch > 0 && (!d_states || !d_mask))) return arg_error("bad states / mask / batch");
    if (words_per_row < (g->V + 63) / 64) return arg_error("words_per_row < ceil(vocab_size / 64)");
    if (batch > 0 && (!d_workspace || (uintptr_t)d_workspace % 16))
        return arg_error("workspace must be a 16-byte aligned device buffer of cg_fill_workspace_bytes bytes");
    return launch_fill(g, d_states, batch, d_mask, words_per_row, d_workspace, (hipStream_t)stream);
}

int cg_fill_bitmask_noalloc(const cg_grammar *g, const cg_state *d_states, int32_t batch, uint64_t *d_mask,
                            int32_t words_per_row, void *stream) {
    if (!on_device(g)) return arg_error("grammar has no device tables");
    if (batch < 0 || (batch > 0 && (!d_states || !d_mask))) return arg_error("bad states / mask / batch");
    if (words_per_row < (g->V + 63) / 64) return arg_error("words_per_row < ceil(vocab_size / 64)");
    return launch_fill_noalloc(g, d_states, batch, d_mask, words_per_row, (hipStream_t)stream);
}

size_t cg_draft_workspace_bytes(const cg_grammar *g, int32_t batch, int32_t k) {
    if (!on_device(g) || batch < 1 || k < 0 || k > CG_MAX_DRAFT) return 0;
    return cg_fill_workspace_bytes(g, batch * (k + 1));
}

int cg_fill_draft(const cg_grammar *g, const cg_state *d_states, const int32_t *d_step, int32_t batch,
                  const int32_t *d_draft, int32_t k, cg_state *d_path_states, uint64_t *d_masks,
                  int32_t words_per_row, int32_t *d_accept_len, void *d_workspace, void *stream) {
    if (!on_device(g)) return arg_error("grammar has no device tables");
    if (k < 0 || k > CG_MAX_DRAFT) return arg_error("k out of range");
    if (batch < 0 || (size_t)batch * (size_t)(k + 1) > (size_t)INT32_MAX) return arg_error("bad batch");
    if (batch > 0 && (!d_states || !d_path_states || !d_masks || !d_accept_len || (k > 0 && !d_draft)))
        return arg_error("bad arguments");
    if (words_per_row < (g->V + 63) / 64) return arg_error("words_per_row < ceil(vocab_size / 64)");
    if (batch > 0 && (!d_workspace || (uintptr_t)d_workspace % 16))
        return arg_error("workspace must be a 16-byte aligned device buffer of cg_draft_workspace_bytes bytes");
    hipStream_t st = (hipStream_t)stream;
    int rc = launch_draft(g, d_states, d_step, batch, d_draft, k, d_path_states, d_accept_len, st);
    if (rc != CG_OK) return rc;
    return launch_fill(g, d_path_states, batch * (k + 1), d_masks, words_per_row, d_workspace, st);
}

size_t cg_sample_workspace_bytes(int32_t batch, int32_t vocab) {
    if (batch <= 0 || vocab <= 0) return 0;
    return sample_workspace_bytes(batch, vocab);
}

int cg_apply_mask_sample(const void *d_logits, int32_t dtype, int32_t batch, int32_t vocab, int64_t row_stride,
                         const uint64_t *d_mask, int32_t words_per_row, const float *d_temperature,
                         const uint64_t *d_seed, const int32_t *d_step, void *d_workspace, int32_t *d_out_ids,
                         float *d_out_logprob, void *stream) {
    if (dtype != 0 && dtype != 1) return arg_error("dtype must be 0 (float32) or 1 (bfloat16)");
    if (batch < 0 || vocab < 1) return arg_error("bad batch / vocab");
    if (row_stride < vocab) return arg_error("row_stride < vocab");
    if (words_per_row < (vocab + 63) / 64) return arg_error("words_per_row < ceil(vocab / 64)");
    if (batch == 0) return CG_OK;
    if (!d_logits || !d_mask || !d_temperature || !d_seed || !d_step || !d_out_ids || !d_out_logprob)
        return arg_error("NULL device pointer");
    if (sample_workspace_bytes(batch, vocab) > 0 && (!d_workspace || (uintptr_t)d_workspace % 16))
        return arg_error("workspace must be a 16-byte aligned device buffer");
    return launch_sample(d_logits, dtype, batch, vocab, row_stride, d_mask, words_per_row, d_temperature, d_seed,
                         d_step, d_workspace, d_out_ids, d_out_logprob, nullptr, nullptr, nullptr, nullptr,
                         (hipStream_t)stream);
}

int cg_sample_advance(const cg_grammar *g, const void *d_logits, int32_t dtype, int32_t batch, int64_t row_stride,
                      const uint64_t *d_mask, int32_t words_per_row, const float *d_temperature,
                      const uint64_t *d_seed, int32_t *d_step, void *d_workspace, int32_t *d_out_ids,
                      float *d_out_logprob, cg_state *d_states, int32_t *d_status, void *stream) {
    if (!on_device(g)) return arg_error("grammar has no device tables");
    if (dtype != 0 && dtype != 1) return arg_error("dtype must be 0 (float32) or 1 (bfloat16)");
    if (batch < 0) return arg_error("bad batch");
    if (row_stride < g->V) return arg_error("row_stride < vocab_size");
    if (words_per_row < (g->V + 63) / 64) return arg_error("words_per_row < ceil(vocab_size / 64)");
    if (batch == 0) return CG_OK;
    if (!d_logits || !d_mask || !d_temperature || !d_seed || !d_step || !d_out_ids || !d_out_logprob || !d_states ||
        !d_status)
        return arg_error("NULL device pointer");
    if (sample_workspace_bytes(batch, g->V) > 0 && (!d_workspace || (uintptr_t)d_workspace % 16))
        return arg_error("workspace must be a 16-byte aligned device buffer");
    return launch_sample(d_logits, dtype, batch, g->V, row_stride, d_mask, words_per_row, d_temperature, d_seed,
                         d_step, d_workspace, d_out_ids, d_out_logprob, g, d_states, d_step, d_status,
                         (hipStream_t)stream);
}

namespace {
int sample_advance_next(const cg_grammar *g, const void *d_logits, int32_t dtype, int32_t batch, int64_t row_stride,
                        uint64_t *d_mask, int32_t words_per_row, const float *d_temperature, const uint64_t *d_seed,
                        int32_t *d_step, void *d_workspace, int32_t *d_out_ids, float *d_out_logprob,
                        cg_state *d_states, int32_t *d_status, void *d_fill_workspace, void *stream, bool walk) {
    if (!on_device(g)) return arg_error("grammar has no device tables");
    if (dtype != 0 && dtype != 1) return arg_error("dtype must be 0 (float32) or 1 (bfloat16)");
    if (batch < 0) return arg_error("bad batch");
    if (row_stride < g->V) return arg_error("row_stride < vocab_size");
    if (words_per_row < (g->V + 63) / 64) return arg_error("words_per_row < ceil(vocab_size / 64)");
    if (batch == 0) return CG_OK;
    if (!d_logits || !d_mask || !d_temperature || !d_seed || !d_step || !d_out_ids || !d_out_logprob || !d_states ||
        !d_status)
        return arg_error("NULL device pointer");
    if (sample_workspace_bytes(batch, g->V) > 0 && (!d_workspace || (uintptr_t)d_workspace % 16))
        return arg_error("workspace must be a 16-byte aligned device buffer");
    if (!d_fill_workspace || (uintptr_t)d_fill_workspace % 16)
        return arg_error("fill workspace must be a 16-byte aligned device buffer of cg_fill_workspace_bytes bytes");
    const int chk = fill_check(g, batch);
    if (chk != CG_OK) return chk;
    hipStream_t st = (hipStream_t)stream;
    const FillArgs a = make_fill_args(g, d_states, batch, d_mask, words_per_row, d_fill_workspace);
    const int rc = launch_sample(d_logits, dtype, batch, g->V, row_stride, d_mask, words_per_row, d_temperature,
                                 d_seed, d_step, d_workspace, d_out_ids, d_out_logprob, g, d_states, d_step, d_status,
                                 st, &a);
    if (rc != CG_OK || !walk) return rc;
    return launch_fill_walk(g, a, st);
}
}  // namespace

int cg_sample_advance_fill(const cg_grammar *g, const void *d_logits, int32_t dtype, int32_t batch,
                           int64_t row_stride, uint64_t *d_mask, int32_t words_per_row, const float *d_temperature,
                           const uint64_t *d_seed, int32_t *d_step, void *d_workspace, int32_t *d_out_ids,
                           float *d_out_logprob, cg_state *d_states, int32_t *d_status, void *d_fill_workspace,
                           void *stream) {
    return sample_advance_next(g, d_logits, dtype, batch, row_stride, d_mask, words_per_row, d_temperature, d_seed,
                               d_step, d_workspace, d_out_ids, d_out_logprob, d_states, d_status, d_fill_workspace,
                               stream, true);
}

int cg_sample_advance_plan(const cg_grammar *g, const void *d_logits, int32_t dtype, int32_t batch,
                           int64_t row_stride, uint64_t *d_mask, int32_t words_per_row, const float *d_temperature,
                           const uint64_t *d_seed, int32_t *d_step, void *d_workspace, int32_t *d_out_ids,
                           float *d_out_logprob, cg_state *d_states, int32_t *d_status, void *d_fill_workspace,
                           void *stream) {
    return sample_advance_next(g, d_logits, dtype, batch, row_stride, d_mask, words_per_row, d_temperature, d_seed,
                               d_step, d_workspace, d_out_ids, d_out_logprob, d_states, d_status, d_fill_workspace,
                               stream, false);
}

int cg_fill_walk(const cg_grammar *g, const cg_state *d_states, int32_t batch, uint64_t *d_mask,
                 int32_t words_per_row, void *d_workspace, void *stream) {
    if (!on_device(g)) return arg_error("grammar has no device tables");
    if (batch < 0 || (batch > 0 && (!d_states || !d_mask))) return arg_error("bad states / mask / batch");
    if (words_per_row < (g->V + 63) / 64) return arg_error("words_per_row < ceil(vocab_size / 64)");
    if (batch == 0) return CG_OK;
    if (!d_workspace || (uintptr_t)d_workspace % 16)
        return arg_error("workspace must be a 16-byte aligned device buffer of cg_fill_workspace_bytes bytes");
    const int chk = fill_check(g, batch);
    if (chk != CG_OK) return chk;
    return launch_fill_walk(g, make_fill_args(g, d_states, batch, d_mask, words_per_row, d_workspace),
                            (hipStream_t)stream);
}

int cg_advance(const cg_grammar *g, cg_state *d_states, int32_t batch, const int32_t *d_token_ids, int32_t *d_step,
               int32_t *d_status, void *stream) {
    if (!on_device(g)) return arg_error("grammar has no device tables");
    if (batch < 0 || (batch > 0 && (!d_states || !d_token_ids || !d_step || !d_status)))
        return arg_error("bad arguments");
    return launch_advance(g, d_states, batch, d_token_ids, d_step, d_status, (hipStream_t)stream);
}

int cg_force_bytes(const cg_grammar *g, cg_state *d_states, int32_t batch, const uint8_t *d_bytes, size_t n_bytes,
                   const uint32_t *d_offsets, int32_t *d_status, void *stream) {
    if (!on_device(g)) return arg_error("grammar has no device tables");
    if (batch < 0 || (batch > 0 && (!d_states || !d_offsets || !d_status)) || (n_bytes > 0 && !d_bytes))
        return arg_error("bad arguments");
    return launch_force(g, d_states, batch, d_bytes, (uint64_t)n_bytes, d_offsets, d_status, (hipStream_t)stream);
}

int cg_eval_calc(const uint8_t *span, size_t len, int64_t *value) {
    if (!value || (len && !span)) return arg_error("NULL argument");
    std::string s((const char *)span, len);
    if (s.size() >= 13 && s.compare(0, 6, "<calc>") == 0 && s.compare(s.size() - 7, 7, "</calc>") == 0)
        s = s.substr(6, s.size() - 13);
    size_t i = 0;
    auto skip = [&]() {
        while (i < s.size() && (s[i] == ' ' || s[i] == '\t' || s[i] == '\n' || s[i] == '\r')) i++;
    };
    struct Fail {
        int code;
        const char *msg;
    };
    // E := P (('+' | '-') P)*, P := T (('*' | '/') T)*, T := int | '(' E ')'
    std::function<int64_t()> expr;
    auto term = [&]() -> int64_t {
        skip();
        if (i < s.size() && s[i] == '(') {
            i++;
            const int64_t v = expr();
            skip();
            if (i >= s.size() || s[i] != ')') throw Fail{CG_E_PARSE, "missing )"};
            i++;
            return v;
        }
        if (i >= s.size() || s[i] < '0' || s[i] > '9') throw Fail{CG_E_PARSE, "expected an integer or ("};
        int64_t v = 0;
        while (i < s.size() && s[i] >= '0' && s[i] <= '9') {
            if (__builtin_mul_overflow(v, (int64_t)10, &v) || __builtin_add_overflow(v, (int64_t)(s[i] - '0'), &v))
                throw Fail{CG_E_EVAL, "out of range"};
            i++;
        }
        return v;
    };
    auto prod = [&]() -> int64_t {
        int64_t v = term();
        for (;;) {
            skip();
            if (i >= s.size() || (s[i] != '*' && s[i] != '/')) return v;
            const char op = s[i++];
            const int64_t r = term();
            if (op == '*') {
                if (__builtin_mul_overflow(v, r, &v)) throw Fail{CG_E_EVAL, "out of range"};
            } else {
                if (r == 0) throw Fail{CG_E_EVAL, "division by zero"};
                if (v == INT64_MIN && r == -1) throw Fail{CG_E_EVAL, "out of range"};
                v /= r;  // truncates toward zero
            }
        }
    };
    expr = [&]() -> int64_t {
        int64_t v = prod();
        for (;;) {
            skip();
            if (i >= s.size() || (s[i] != '+' && s[i] != '-')) return v;
            const char op = s[i++];
            const int64_t r = prod();
            if (op == '+' ? __builtin_add_overflow(v, r, &v) : __builtin_sub_overflow(v, r, &v))
                throw Fail{CG_E_EVAL, "out of range"};
        }
    };
    try {
        const int64_t v = expr();
        skip();
        if (i != s.size()) throw Fail{CG_E_PARSE, "trailing input"};
        *value = v;
        return CG_OK;
    } catch (const Fail &f) {
        if (f.code == CG_E_EVAL) set_error("%s", f.msg);
        else set_error("calc span: %s at byte %zu", f.msg, i);
        return f.code;
    }
}

int cg_eval_strop(const uint8_t *span, size_t len, char *out, size_t cap, size_t *out_len) {
    if (!out_len || (len && !span) || (cap && !out)) return arg_error("NULL argument");
    const std::string s((const char *)span, len);
    static const char *const kNames[5] = {"count", "len", "reverse", "upper", "substr"};
    static const char *const kArgs[5] = {"SS", "S", "S", "S", "SII"};
    auto fail = [&](const char *m) {
        set_error("strop span: %s", m);
        return CG_E_PARSE;
    };
    const std::string open = "<strop>", close = ")</strop>";
    if (s.size() < open.size() + close.size() || s.compare(0, open.size(), open) != 0 ||
        s.compare(s.size() - close.size(), close.size(), close) != 0)
        return fail("not a <strop> span");
    size_t i = open.size();
    const size_t end = s.size() - close.size();
    int op = -1;
    for (int k = 0; k < 5; k++) {
        const size_t n = strlen(kNames[k]);
        if (s.compare(i, n, kNames[k]) == 0 && i + n < end + 1 && s[i + n] == '(') {
            op = k;
            i += n + 1;
            break;
        }
    }
    if (op < 0) return fail("unknown operation");
    std::string str[2];
    long long num[2] = {0, 0};
    int ns = 0, ni = 0;
    auto skip = [&]() {
        while (i < end && (s[i] == ' ' || s[i] == '\t' || s[i] == '\n' || s[i] == '\r')) i++;
    };
    for (const char *a = kArgs[op]; *a; a++) {
        skip();
        if (a != kArgs[op]) {
            if (i >= end || s[i] != ',') return fail("expected ','");
            i++;
            skip();
        }
        if (*a == 'S') {
            if (i >= end || s[i] != '"') return fail("expected a string");
            const size_t q = s.find('"', i + 1);
            if (q == std::string::npos || q >= end) return fail("unterminated string");
            str[ns++] = s.substr(i + 1, q - i - 1);
            i = q + 1;
        } else {
            bool neg = false;
            if (i < end && s[i] == '-') neg = true, i++;
            size_t d = 0;
            long long v = 0;
            while (i < end && s[i] >= '0' && s[i] <= '9' && d < 18) v = v * 10 + (s[i++] - '0'), d++;
            if (d == 0) return fail("expected an integer");
            num[ni++] = neg ? -v : v;
        }
    }
    skip();
    if (i != end) return fail("trailing input");
    std::string r;
    const std::string &a0 = str[0];
    switch (op) {
    case 0: {  // non-overlapping occurrences, left to right; "" occurs len + 1 times
        long long n = 0;
        if (str[1].empty()) n = (long long)a0.size() + 1;
        else
            for (size_t p = a0.find(str[1]); p != std::string::npos; p = a0.find(str[1], p + str[1].size())) n++;
        r = std::to_string(n);
        break;
    }
    case 1: r = std::to_string(a0.size()); break;
    case 2: r.assign(a0.rbegin(), a0.rend()); break;
    case 3:
        r = a0;
        for (char &c : r)
            if (c >= 'a' && c <= 'z') c = (char)(c - 32);
        break;
    default: {  // positions from the end when negative, clamped to the string
        const long long n = (long long)a0.size();
        auto norm = [&](long long x) { return std::min(std::max(x < 0 ? x + n : x, 0LL), n); };
        const long long b = norm(num[0]), e = norm(num[1]);
        if (b < e) r = a0.substr((size_t)b, (size_t)(e - b));
        break;
    }
    }
    *out_len = r.size();
    if (r.size() + 1 > cap) {
        set_error("output needs %zu bytes (with the terminating zero)", r.size() + 1);
        return CG_E_LIMIT;
    }
    memcpy(out, r.data(), r.size());
    out[r.size()] = 0;
    return CG_OK;
}

int cg_try_input(const cg_grammar *g, const uint8_t *bytes, size_t len, size_t *refused_at, int *complete) {
    if (!g || !refused_at || !complete || (len && !bytes)) return arg_error("NULL argument");
    Walker w;
    w.q = g->k.start;
    w.ret = g->k.start;
    w.cnt = 0;
    w.ws = 0;
    w.depth = 0;
    w.stk = 0;
    size_t i = 0;
    for (; i < len; i++)
        if (!step_byte<true>(w, bytes[i], g->host_comb, g->k)) break;
    *refused_at = i;
    *complete = (i == len && w.q == g->k.accept) ? 1 : 0;
    return CG_OK;
}

const char *cg_last_error(void) { return last_error(); }

}  // extern "C"
