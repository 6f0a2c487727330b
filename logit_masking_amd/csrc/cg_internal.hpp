// cg_internal.hpp -- automaton table format shared by the host compiler, the
// host walker behind cg_try_input, and the gfx950 kernels.
//
// The control of the pushdown automaton is a byte-level transition table
// packed by row displacement ("comb"): a state's id is its base offset, and
// the transition of state q on byte b is the 64-bit slot comb[q + b], valid
// iff the slot's owner field equals q.  One table lookup per byte, no byte
// classes, no per-state descriptor.
//
// Slot layout (little-endian u64):
//   bits  0..15  owner   state id whose row this slot belongs to (0xFFFF:
//                        empty), plus 0x8000 when that state lies in a region
//                        only the engine writes (kEngineOwner): a model token
//                        may enter such a state but never leave it
//   bits 16..31  next    next state (see ops)
//   bits 32..35  op      what the byte does to the registers besides moving
//   bits 36..63  arg     operand (28 bits)
//
// Registers of a configuration besides the state: the open string's
// remaining code points (cnt) and resume state (ret), the whitespace run
// (ws), and a bit stack of open any-JSON containers (stk, depth) -- the
// automaton's stack alphabet is {object, array}; everything a schema fixes
// statically lives in the control states.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "../../include/cg.h"

namespace cg {

enum Op : uint32_t {
    OP_NONE = 0,      // q = next
    OP_WS = 1,        // whitespace byte: ws += 1, refused past ws_max
    OP_CHAR = 2,      // first byte of a string code point: refused when cnt == 0, cnt -= 1
    OP_STR_OPEN = 3,  // opening quote: ret = next, q = string body, cnt = arg
    OP_STR_CLOSE = 4, // closing quote: q = ret
    OP_PUSH = 5,      // open container: bit = arg & 1 (0 object, 1 array); refused if depth >= arg >> 1
    OP_POP = 6,       // close container: pop; depth == 0 ? next : (top bit ? arg >> 14 : arg & 0x3FFF)
};

constexpr uint32_t kEmptyOwner = 0xFFFF;
constexpr uint32_t kEngineOwner = 0x8000;  // owner tag of an engine-written state's slots
constexpr uint32_t kMaxStateId = 0x3FFF;   // POP packs two state ids in 28 bits
constexpr uint32_t kUncapped = 0x0FFFFFFF; // cnt of an uncapped string
constexpr int kMaxTokenLen = 32;

// Per-grammar constants needed by every walker.
struct WalkConsts {
    uint32_t s_body;   // state of a string body at a code-point boundary (0xFFFF: no strings)
    uint32_t accept;   // the single accepting state (no outgoing bytes)
    uint32_t start;    // start state
    uint32_t ws_max;   // longest whitespace run
    uint32_t q_limit;  // every valid state id is < q_limit (comb has q_limit + 256 slots)
};

// A configuration in registers.
struct Walker {
    uint32_t q, ret, cnt, ws, depth;
    uint64_t stk;
};

__host__ __device__ inline Walker load_walker(const cg_state &s) {
    Walker w;
    w.q = s.q;
    w.ret = s.ret;
    w.cnt = s.cnt;
    w.ws = s.ws;
    w.depth = s.depth;
    w.stk = s.stk;
    return w;
}

__host__ __device__ inline void store_walker(cg_state &s, const Walker &w) {
    s.q = (uint16_t)w.q;
    s.ret = (uint16_t)w.ret;
    s.cnt = w.cnt;
    s.ws = (uint8_t)w.ws;
    s.depth = (uint8_t)w.depth;
    s.stk = w.stk;
}

// One byte.  Returns false if the byte is refused (the walker is then
// unspecified but every state id in it stays < q_limit, so a dead lane may
// keep indexing the table safely).  The common ops (move, whitespace, string
// code point) are straight-line; string open/close and container push/pop
// take the rare branch.  kEngine: the engine's own bytes, which may also
// leave engine-written states (a model token's walk refuses those slots
// because their owner carries the tag).
template <bool kEngine = false>
__host__ __device__ inline bool step_byte(Walker &w, uint32_t b, const uint64_t *comb, const WalkConsts &k) {
    const uint64_t e = comb[w.q + b];
    const uint32_t lo = (uint32_t)e, hi = (uint32_t)(e >> 32);
    bool ok = (lo & (kEngine ? 0x7FFFu : 0xFFFFu)) == w.q;
    uint32_t nq = lo >> 16;
    const uint32_t op = hi & 0xFu;
    const uint32_t ws1 = (op == OP_WS) ? w.ws + 1 : 0;
    ok = ok && ws1 <= k.ws_max;
    w.ws = ws1;
    const bool ch = op == OP_CHAR;
    ok = ok && !(ch && w.cnt == 0);
    w.cnt -= ch ? 1u : 0u;
    if (op > OP_CHAR) {
        const uint32_t arg = hi >> 4;
        if (op == OP_STR_OPEN) {
            w.ret = nq;
            nq = k.s_body;
            w.cnt = arg;
        } else if (op == OP_STR_CLOSE) {
            nq = w.ret;
        } else if (op == OP_PUSH) {
            ok = ok && w.depth < (arg >> 1);
            w.stk = (w.stk << 1) | (arg & 1u);
            w.depth += 1;
        } else {
            w.stk >>= 1;
            w.depth -= 1;
            nq = (w.depth == 0) ? nq : ((w.stk & 1u) ? (arg >> 14) : (arg & 0x3FFFu));
        }
    }
    w.q = nq;
    return ok;
}

// Copy table slots [start, n) to LDS with up to 16 loads per thread in
// flight before the first store (a plain load/store loop waits out one round
// trip per slot).
__device__ inline void stage_table(uint64_t *dst, const uint64_t *__restrict__ src, uint32_t n,
                                   uint32_t start = 0) {
    constexpr int kInFlight = 16;
    for (uint32_t base = start; base < n; base += kInFlight * blockDim.x) {
        uint64_t v[kInFlight];
#pragma unroll
        for (int j = 0; j < kInFlight; j++) {
            const uint32_t i = base + j * blockDim.x + threadIdx.x;
            v[j] = i < n ? src[i] : 0ull;
        }
#pragma unroll
        for (int j = 0; j < kInFlight; j++) {
            const uint32_t i = base + j * blockDim.x + threadIdx.x;
            if (i < n) dst[i] = v[j];
        }
    }
}

// Did commit_token take the token (the row and its step count changed)?
__host__ __device__ inline bool token_taken(int res) { return res != CG_ROW_NOOP && res != CG_ROW_REJECTED; }

// Commit token `id` (its n bytes in words[], 4 per word) to a row: the
// cg_advance rules.  -1 is a no-op; an id out of range, a finished row or a
// refused byte leaves the row unchanged (REJECTED); otherwise the row takes
// the walked configuration, step + 1, and DONE / CAPPED flags, or INJECT
// when it now sits in an engine-written region.  Returns the status; `s`
// and `step` are updated only when the token is accepted.
__host__ __device__ inline bool forced_state(const uint32_t *forced, uint32_t q) {
    return forced && ((forced[q >> 5] >> (q & 31)) & 1u);
}

__host__ __device__ inline int commit_token(cg_state &s, int &step, int id, int V, uint32_t n,
                                            const uint32_t (&words)[kMaxTokenLen / 4], const uint64_t *comb,
                                            const WalkConsts &k, uint32_t gen_cap, const uint32_t *forced) {
    if (id < 0) return CG_ROW_NOOP;
    if (id >= V || (s.flags & (CG_FLAG_DONE | CG_FLAG_CAPPED)) || s.q >= k.q_limit || s.ret >= k.q_limit)
        return CG_ROW_REJECTED;
    Walker w = load_walker(s);
    bool ok = n > 0;
#pragma unroll
    for (int i = 0; i < kMaxTokenLen; i++) {  // unrolled: the word index is a constant
        if (!ok || (uint32_t)i >= n) break;
        ok = step_byte(w, (words[i >> 2] >> (8 * (i & 3))) & 0xFFu, comb, k);
    }
    if (!ok) return CG_ROW_REJECTED;
    store_walker(s, w);
    step += 1;
    int res = CG_ROW_OK;
    uint8_t fl = 0;
    if (w.q == k.accept) {
        fl |= CG_FLAG_DONE;
        res = CG_ROW_DONE;
    }
    if ((uint32_t)step >= gen_cap) {
        fl |= CG_FLAG_CAPPED;
        if (res == CG_ROW_OK) res = CG_ROW_CAPPED;
    }
    if (res == CG_ROW_OK && forced_state(forced, w.q)) res = CG_ROW_INJECT;
    s.flags = fl;
    s.pad0 = 0;
    s.pad1 = 0;
    return res;
}

// Per-token summary of a walk through a string body that starts at a
// code-point boundary (state s_body): the body's transitions depend on
// nothing but the byte and the code-point budget, so one word per token
// decides it.  Layout of tokinfo[t]:
//   bits 0..7   token length in bytes
//   bits 8..9   STR_IN (the token ends inside the string), STR_QUOTE (an
//               unescaped quote closes the string at byte `pos`), STR_DEAD
//   bits 10..15 code points the token adds to the string before it ends or
//               the quote (each needs one unit of the budget cnt)
//   bits 16..20 pos
enum : uint32_t { STR_IN = 0, STR_QUOTE = 2, STR_DEAD = 3 };

__host__ __device__ inline uint32_t tok_len(uint32_t info) { return info & 0xFFu; }
__host__ __device__ inline uint32_t tok_kind(uint32_t info) { return (info >> 8) & 3u; }
__host__ __device__ inline uint32_t tok_chars(uint32_t info) { return (info >> 10) & 63u; }
__host__ __device__ inline uint32_t tok_pos(uint32_t info) { return (info >> 16) & 31u; }

// Candidate keys of the fill.  A non-empty token's key is its first two
// bytes: b1 * 257 + (length 1 ? 0 : b2 + 1), so that in lexicographic order
// keys never decrease.  A token after the closing quote of a string is keyed
// by the byte after the quote: 0 if the quote ends the token, else byte + 1.
constexpr int kKeysPerLead = 257;
constexpr int kTile = 64;          // tokens per candidate tile (one wave)
constexpr int kStrBitsets = 33;    // in-string bitsets for budgets 0..32 code points
constexpr uint32_t kNoQuote = 63;  // jump field of a token without a quote
constexpr int kPushLimit = 6;      // containers a token may open and still take its bit from the table

__host__ __device__ inline uint32_t lead_key(uint32_t b1, uint32_t b2, uint32_t len) {
    return b1 * kKeysPerLead + (len == 1 ? 0u : b2 + 1u);
}

// Device copy of a compiled grammar.
struct DeviceTables {
    uint64_t *comb = nullptr;     // [comb_len]
    uint32_t *tokw = nullptr;     // [nw][V] token bytes, 4 per word, little-endian, zero padded
    uint32_t *tokinfo = nullptr;  // [V] length + string-body summary
    uint64_t *legal = nullptr;    // [q_limit][4] bytes with a transition out of state q (256-bit set)
    uint32_t *forced = nullptr;   // [ceil(q_limit / 32)] bit q: engine-written state (null: none)
    // Masks computed once, for a state q outside strings with whitespace run
    // ws: context 0 = no open container (the whole mask), 1 / 2 = inside an
    // open object / array (the tokens that stay inside it, see push_limit);
    // state_mask[smask_idx[(q * (ws_max + 1) + ws) * 3 + ctx]], < 0: none.
    uint64_t *state_mask = nullptr;  // [n_smask][Wv]
    int32_t *smask_idx = nullptr;    // [q_limit * (ws_max + 1) * 3]
    // Tokens whose brackets may close the container a row is in, or open
    // more than kPushLimit: walked, like the lexicographic list, for rows
    // that take context 1 / 2 from the table.
    uint32_t *c_idlen = nullptr, *c_jump = nullptr, *c_w = nullptr;
    uint2 *c_tile = nullptr;
    // String rows inside an open container: retmask2[(rq_idx[R] * 2 + kind)]
    // holds the closing tokens whose bytes after the quote stay inside it
    // (null: no table); the other closing tokens are the qc list.
    uint64_t *retmask2 = nullptr;    // [n_resume * 2][Wv]
    uint32_t *qc_idlen = nullptr, *qc_jump = nullptr, *qc_w = nullptr;
    uint2 *qc_tile = nullptr;
    // Tokens that close a string: closebits[c] = the content before the
    // quote fits a budget of c code points; retmask[rq_idx[R]] = the bytes
    // after the quote are accepted from resume state R with no open
    // container (rq_idx null: no table).
    uint64_t *closebits = nullptr;   // [kStrBitsets][Wv]
    uint64_t *retmask = nullptr;     // [n_resume][Wv]
    int32_t *rq_idx = nullptr;       // [q_limit]
    // Fill candidates: the non-empty tokens in lexicographic order, padded
    // with empty entries (idlen 0) to whole 64-token tiles.
    uint32_t *lex_idlen = nullptr;   // [lex_tiles * 64] id | len << 24 | 1 << 31 (0: padding)
    uint32_t *lex_jump = nullptr;    // [lex_tiles * 64] first quote position (kNoQuote: none) | string
                                     //       summary of the bytes after it (tokinfo layout, bits 8..20)
    uint32_t *lex_w = nullptr;       // [nw][lex_tiles * 64] token bytes
    uint2 *lex_tile = nullptr;       // [lex_tiles] first and last key of each tile
    // Tokens that close a string opened before them, sorted by the bytes
    // after the quote, padded the same way.
    uint32_t *q_idlen = nullptr;     // [q_tiles * 64] id | bytes after the quote << 24 | 1 << 31
    uint32_t *q_jump = nullptr;      // [q_tiles * 64] the first quote after the closing one, as in
                                     //       lex_jump, | code points before the closing one << 21
    uint32_t *q_w = nullptr;         // [nw][q_tiles * 64]
    uint2 *q_tile = nullptr;         // [q_tiles] first and last after-quote key of each tile
    uint64_t *strbits = nullptr;     // [33][ceil(V / 64)] tokens that stay inside a string from a
                                     //       code-point boundary within a budget of c code points
};

}  // namespace cg

struct cg_grammar {
    cg::WalkConsts k;
    uint32_t comb_len = 0;
    int32_t V = 0;
    int32_t max_len = 0;
    int32_t nw = 0;          // words per token in tokw (ceil(max_len / 4), at least 1)
    int32_t n_states = 0;
    uint32_t gen_cap = 2048;
    int device = -1;         // HIP device the tables live on (-1: host only)
    int n_cu = 256;          // compute units of that device
    int lds_max = 65536;     // LDS bytes a workgroup may use on that device
    int32_t lex_tiles = 0;   // candidate tiles of the lexicographic list
    int32_t q_tiles = 0;     // and of the string-closing list
    double compile_ms = 0;   // spec -> automaton (parse, build, trim, pack)
    double total_ms = 0;     // the whole cg_compile_grammar call that built the handle
    int64_t max_bytes = -1;  // longest member of the language in bytes; -1: infinite
    uint64_t *host_comb = nullptr;
    std::vector<uint32_t> host_forced;  // bit q: state q is inside an engine-written region
    bool has_forced = false;
    int refs = 1;                   // handles given out by cg_compile_grammar (the cache shares them)
    std::vector<uint32_t> plain_q;  // live states outside strings (candidates of the state-mask table)
    int32_t n_smask = 0;            // rows of dev.state_mask
    int32_t c_tiles = 0;            // tiles of the closing-token list
    int32_t qc_tiles = 0;           // tiles of the string-closing tokens that leave the container
    int32_t min_push_cap = 0;       // smallest depth cap of any push (0: no pushes)
    cg::DeviceTables dev;
};

namespace cg {
// compiler.cpp: parse + build + pack; fills host_comb/comb_len/k/n_states.
// Returns CG_OK or an error code (message via set_error).
int compile_spec(const char *spec, size_t len, cg_grammar *g);
void set_error(const char *fmt, ...);

// HIP launch error of the last launch, as a CG_E_DEVICE with a message.
inline int launch_status(const char *what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        set_error("%s: %s", what, hipGetErrorString(e));
        return CG_E_DEVICE;
    }
    return CG_OK;
}
}  // namespace cg
