// pda.hip -- gfx950 kernels of the automaton side of the constrained-decoding
// step ("Constrained decoding", "The guarantee": a pushdown automaton masks
// the logits at every step).
//
//   k_init        rows at the start state
//   k_advance     one lane per row walks the chosen token
//   k_fill_plan   token bitmask, part 1: per row the base words (zero, or the
//                 tokens that stay inside an open string) and the list of
//                 token tiles worth walking, chosen by the row's legal first
//                 and second bytes
//   k_fill_walk   token bitmask, part 2: one lane per listed token walks it
//                 through the transition table staged in LDS
//
// Nothing here is a dense contraction, so there is no MFMA: the work is
// table lookups, integer ALU and latency.
#include <algorithm>
#include <mutex>

#include "cg_internal.hpp"
#include "fill_plan.hpp"

namespace cg {

// ---------------------------------------------------------------------------
// init / advance
// ---------------------------------------------------------------------------
__global__ void k_init(cg_state *__restrict__ states, int B, uint32_t start) {
    int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= B) return;
    cg_state s;
    s.q = (uint16_t)start;
    s.ret = (uint16_t)start;
    s.cnt = 0;
    s.stk = 0;
    s.depth = 0;
    s.ws = 0;
    s.flags = 0;
    s.pad0 = 0;
    s.pad1 = 0;
    states[r] = s;
}

// One lane per row.  The row's id, configuration and token bytes are loaded
// first, then the transition table is staged in LDS while those loads fly,
// so the byte walk is a chain of LDS lookups, not of L2 round trips.
__global__ __launch_bounds__(256) void k_advance(const uint64_t *__restrict__ comb, uint32_t comb_len, WalkConsts k,
                                                 const uint32_t *__restrict__ tokw, const uint32_t *__restrict__ tokinfo,
                                                 int nw, int V, cg_state *__restrict__ states, int B,
                                                 const int32_t *__restrict__ ids, int32_t *__restrict__ steps,
                                                 int32_t *__restrict__ status, uint32_t gen_cap,
                                                 const uint32_t *__restrict__ forced) {
    extern __shared__ uint64_t lds_comb[];
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    const bool row = r < B;
    const int id = row ? ids[r] : -1;
    cg_state s{};
    int st0 = 0;
    if (row) {
        s = states[r];
        st0 = steps[r];
    }
    const bool valid = id >= 0 && id < V && !(s.flags & (CG_FLAG_DONE | CG_FLAG_CAPPED)) && s.q < k.q_limit &&
                       s.ret < k.q_limit;
    uint32_t n = 0;
    uint32_t words[kMaxTokenLen / 4];
#pragma unroll
    for (int j = 0; j < kMaxTokenLen / 4; j++) words[j] = 0;
    if (valid) {
        n = tok_len(tokinfo[id]);
#pragma unroll
        for (int j = 0; j < kMaxTokenLen / 4; j++)
            if (j < nw) words[j] = tokw[(size_t)j * V + id];
    }
    stage_table(lds_comb, comb, comb_len);
    __syncthreads();
    if (!row) return;
    int st = st0;
    const int res = commit_token(s, st, id, V, n, words, lds_comb, k, gen_cap, forced);
    if (token_taken(res)) {
        states[r] = s;
        steps[r] = st;
    }
    status[r] = res;
}

// One lane per row: walk the row's forced byte string (the engine writing an
// evaluated result into the text, "Evaluator aware decoding", "A concrete
// prototype on llama.cpp").  Not a generation step: the step count stays.
__global__ __launch_bounds__(256) void k_force(const uint64_t *__restrict__ comb, uint32_t comb_len, WalkConsts k,
                                               cg_state *__restrict__ states, int B, const uint8_t *__restrict__ bytes,
                                               uint64_t n_bytes, const uint32_t *__restrict__ offsets,
                                               int32_t *__restrict__ status, const uint32_t *__restrict__ forced) {
    extern __shared__ uint64_t lds_comb[];
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    const bool row = r < B;
    cg_state s{};
    uint32_t b0 = 0, b1 = 0;
    if (row) {
        s = states[r];
        b0 = offsets[r];
        b1 = offsets[r + 1];
    }
    stage_table(lds_comb, comb, comb_len);
    __syncthreads();
    if (!row) return;
    if (b1 == b0) {
        status[r] = CG_ROW_NOOP;
        return;
    }
    // offsets out of order or past the bytes: refused, nothing read
    if (b1 < b0 || b1 > n_bytes || (s.flags & (CG_FLAG_DONE | CG_FLAG_CAPPED)) || s.q >= k.q_limit ||
        s.ret >= k.q_limit) {
        status[r] = CG_ROW_REJECTED;
        return;
    }
    Walker w = load_walker(s);
    bool ok = true;
    for (uint32_t i = b0; ok && i < b1; i++) ok = step_byte<true>(w, bytes[i], lds_comb, k);
    if (!ok) {
        status[r] = CG_ROW_REJECTED;
        return;
    }
    store_walker(s, w);
    int res = CG_ROW_OK;
    s.flags = 0;
    if (w.q == k.accept) {
        s.flags = CG_FLAG_DONE;
        res = CG_ROW_DONE;
    } else if (forced_state(forced, w.q)) {
        res = CG_ROW_INJECT;
    }
    s.pad0 = 0;
    s.pad1 = 0;
    states[r] = s;
    status[r] = res;
}

// One lane per row: walk the row's k draft tokens and write the states
// along the path (position 0 = the row as it is).  The walk follows the
// cg_advance rules, caps included, from a private copy of the row and step;
// it stops at the first token that is not taken, and every later position
// gets that state marked finished, so its mask is empty.  The row itself is
// not changed.
__global__ __launch_bounds__(256) void k_draft(const uint64_t *__restrict__ comb, uint32_t comb_len, WalkConsts k,
                                               const uint32_t *__restrict__ tokw, const uint32_t *__restrict__ tokinfo,
                                               int nw, int V, const cg_state *__restrict__ states,
                                               const int32_t *__restrict__ steps, int B,
                                               const int32_t *__restrict__ draft, int kd,
                                               cg_state *__restrict__ path, int32_t *__restrict__ accept_len,
                                               uint32_t gen_cap, const uint32_t *__restrict__ forced) {
    extern __shared__ uint64_t lds_comb[];
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    const bool row = r < B;
    cg_state s{};
    int st = 0;
    if (row) {
        s = states[r];
        st = steps ? steps[r] : 0;
    }
    stage_table(lds_comb, comb, comb_len);
    __syncthreads();
    if (!row) return;
    cg_state *out = path + (size_t)r * (kd + 1);
    out[0] = s;
    int acc = 0;
    bool alive = true;
    for (int j = 0; j < kd; j++) {
        if (alive) {
            const int id = draft[(size_t)r * kd + j];
            const bool valid = id >= 0 && id < V;
            uint32_t n = 0;
            uint32_t words[kMaxTokenLen / 4];
#pragma unroll
            for (int w = 0; w < kMaxTokenLen / 4; w++) words[w] = 0;
            if (valid) {
                n = tok_len(tokinfo[id]);
#pragma unroll
                for (int w = 0; w < kMaxTokenLen / 4; w++)
                    if (w < nw) words[w] = tokw[(size_t)w * V + id];
            }
            cg_state t = s;
            int st1 = st;
            const int res = commit_token(t, st1, id, V, n, words, lds_comb, k, gen_cap, forced);
            if (token_taken(res)) {
                s = t;
                st = st1;
                acc++;
            } else {
                alive = false;
                s.flags |= CG_FLAG_DONE;  // past the draft's legal prefix: empty masks
            }
        }
        out[j + 1] = s;
    }
    accept_len[r] = acc;
}

// ---------------------------------------------------------------------------
// fill_bitmask
// ---------------------------------------------------------------------------
//
// A mask bit is the outcome of walking the token's bytes from the row's
// configuration.  Almost every token dies within its first two bytes, so the
// walk is done only where it can succeed.  Tokens are kept in lexicographic
// order cut into 64-token tiles whose key spans (first two bytes) are known.
//
//   k_fill_plan   one workgroup per row.  Writes the row's base words: zero,
//                 or for a row inside a string at a code-point boundary the
//                 precomputed set of tokens that stay inside the string
//                 within its code-point budget (decided by their count
//                 alone).  Then lists the tiles worth walking:
//     general row one lane per byte finds the legal first bytes and the
//                 state after each; a key (b1, b2) is a candidate if that
//                 state has any transition on b2 (a per-state 256-bit set);
//                 a tile is listed if its span holds a candidate key.
//     string row  the tokens whose quote closes the string, sorted by the
//                 byte after the quote; a tile is listed if that byte can
//                 follow the string.
//   k_fill_walk   (row, slice): slice s walks the listed tiles s, s + S, ...
//                 of its row, one lane per token, through the transition
//                 table staged in LDS.  A walk that opens a string at the
//                 token's first quote jumps over the string content with the
//                 token's precomputed summary of the bytes after that quote.
//                 Accepted tokens are OR-ed into the mask with 64-bit atomics.
constexpr int kWalkThreads = 1024;  // one walk workgroup per CU
constexpr int kWalkWaves = kWalkThreads / 64;

// Byte Bi of the token (compile-time index: the walk is fully unrolled, so
// the token words stay in registers with no dynamic indexing).  A lane walks
// bytes [start, end) of its token while alive; the wave leaves as soon as no
// lane has bytes left.  The step follows step_byte's rules, arranged for
// this loop: moves, whitespace and string code points take the
// straight-line path; the quotes and the container pushes and pops take the
// branch.  `jump` (kNoQuote in its low 6 bits: none) is the position of the
// first quote the walk meets and the string summary of the bytes after it:
// when that quote opens a string, the walk jumps over the string's content.
template <int Bi, int NB, int NW>
__device__ __forceinline__ void walk_bytes(Walker &wk, bool &alive, const uint32_t (&w)[NW], int &start, int &end,
                                           uint32_t jump, const uint64_t *lds_comb, const WalkConsts &k) {
    if constexpr (Bi < NB) {
        const bool left = alive && Bi < end;
        if (!__builtin_amdgcn_ballot_w64(left)) return;
        if (left && Bi >= start) {
            const uint32_t b = (w[Bi >> 2] >> ((Bi & 3) * 8)) & 0xFFu;
            const uint64_t e = lds_comb[wk.q + b];
            const uint32_t lo = (uint32_t)e, hi = (uint32_t)(e >> 32);
            bool ok = (lo & 0xFFFFu) == wk.q;
            uint32_t nq = lo >> 16;
            const uint32_t op = hi & 0xFu;
            const uint32_t is_ws = op & 1u;  // OP_WS (OP_STR_OPEN takes the branch)
            uint32_t ws1 = __umul24(is_ws, wk.ws) + is_ws;
            const bool ch = op == OP_CHAR;
            ok = ok && !(ch && wk.cnt == 0);
            wk.cnt -= ch ? 1u : 0u;
            if (op > OP_CHAR) {
                const uint32_t arg = hi >> 4;
                ws1 = 0;
                if (op == OP_STR_OPEN) {
                    wk.ret = nq;
                    nq = k.s_body;
                    wk.cnt = arg;
                    if ((jump & 63u) == (uint32_t)Bi) {
                        // the token's first quote opened the string: the rest
                        // of the token is string content up to its closing
                        // quote, if any
                        const uint32_t kind = tok_kind(jump), nch = tok_chars(jump);
                        ok = ok && kind != STR_DEAD && nch <= arg;
                        if (kind == STR_QUOTE) {
                            nq = wk.ret;
                            wk.cnt = arg - nch;
                            start = Bi + 2 + (int)tok_pos(jump);
                        } else {
                            end = 0;
                        }
                    }
                } else if (op == OP_STR_CLOSE) {
                    nq = wk.ret;
                } else if (op == OP_PUSH) {
                    ok = ok && wk.depth < (arg >> 1);
                    wk.stk = (wk.stk << 1) | (arg & 1u);
                    wk.depth += 1;
                } else {
                    wk.stk >>= 1;
                    wk.depth -= 1;
                    nq = (wk.depth == 0) ? nq : ((wk.stk & 1u) ? (arg >> 14) : (arg & 0x3FFFu));
                }
            }
            alive = ok && ws1 <= k.ws_max;
            wk.ws = ws1;
            wk.q = nq;
        }
        walk_bytes<Bi + 1, NB, NW>(wk, alive, w, start, end, jump, lds_comb, k);
    }
}

// One tile's worth of a lane: its token (or padding) and where its walk starts.
template <int NW>
struct LaneTok {
    uint32_t il, aux;  // id | bytes to walk << 24 | 1 << 31 (0: padding); jump, and in the string
                       // lists | code points before the closing quote << 21
    uint32_t w[NW];
};

template <int NW>
__device__ __forceinline__ void load_lane(LaneTok<NW> &x, uint32_t list, int i, const FillArgs &a) {
    if (list == LIST_QSTR) {
        const int n = a.q_tiles * kTile;
        x.il = a.q_idlen[i];
        x.aux = a.q_jump[i];
#pragma unroll
        for (int j = 0; j < NW; j++) x.w[j] = a.q_w[(size_t)j * n + i];
    } else if (list == LIST_QCLOSE) {
        const int n = a.qc_tiles * kTile;
        x.il = a.qc_idlen[i];
        x.aux = a.qc_jump[i];
#pragma unroll
        for (int j = 0; j < NW; j++) x.w[j] = a.qc_w[(size_t)j * n + i];
    } else if (list == LIST_CLOSE) {
        const int n = a.c_tiles * kTile;
        x.il = a.c_idlen[i];
        x.aux = a.c_jump[i];
#pragma unroll
        for (int j = 0; j < NW; j++) x.w[j] = a.c_w[(size_t)j * n + i];
    } else {
        const int n = a.lex_tiles * kTile;
        x.il = a.lex_idlen[i];
        x.aux = a.lex_jump[i];
#pragma unroll
        for (int j = 0; j < NW; j++) x.w[j] = a.lex_w[(size_t)j * n + i];
    }
}

__global__ __launch_bounds__(kPlanThreads) void k_fill_plan(FillArgs a) {
    __shared__ PlanShared sh;
    const int r = blockIdx.x;
    plan_row(a, r, a.states[r], a.comb, sh);
}

// A listed tile of some row: which row, which tile, the row's configuration.
struct TileRef {
    int r;
    uint32_t tile;
    cg_state s;
};

constexpr int kWalkRowBlock = 8192;  // rows whose tile counts are scanned at once

// Row of the g-th listed tile of the block: the last r < nb with
// prefix[r] <= g (prefix non-decreasing, prefix[0] = 0 <= g).  A 64-way
// search by the whole wave: each lane tests one boundary of the current
// span, the ballot's highest set lane narrows it (two rounds for 256 rows,
// three up to 262,144).  Every lane of the wave must be active.
__device__ __forceinline__ int row_of(const uint32_t *prefix, int nb, uint32_t g) {
    const int lane = threadIdx.x & 63;
    int lo = 0, span = nb;  // the row is in [lo, lo + span), prefix[lo] <= g
    while (span > 1) {
        const int step = (span + 63) >> 6;
        const bool ok = lane * step < span && prefix[lo + lane * step] <= g;
        const uint64_t m = __ballot(ok);  // lanes 0 .. k (lane 0 always)
        const int k = 63 - __builtin_clzll(m);
        lo += k * step;
        span = min(step, span - k * step);
    }
    return lo;
}

// Inclusive sum over the lanes of a wave with DPP: shifts by 1, 2, 4, 8
// within each row of 16 lanes, then the last lane of rows 0 / 2 into rows
// 1 / 3 and of row 1 into rows 2 and 3.  Every lane must be active.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_add(uint32_t v) {
    return v + (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v) {
    v = dpp_add<0x111, 0xF>(v);  // row_shr:1
    v = dpp_add<0x112, 0xF>(v);  // row_shr:2
    v = dpp_add<0x114, 0xF>(v);  // row_shr:4
    v = dpp_add<0x118, 0xF>(v);  // row_shr:8
    v = dpp_add<0x142, 0xA>(v);  // row_bcast:15
    v = dpp_add<0x143, 0xC>(v);  // row_bcast:31
    return v;
}

__device__ __forceinline__ void fetch_ref(TileRef &t, uint32_t g, uint32_t total, const uint32_t *prefix, int nb,
                                          int rb, const FillArgs &a) {
    if (g >= total) return;
    const int rl = __builtin_amdgcn_readfirstlane(row_of(prefix, nb, g));
    t.r = rb + rl;
    t.tile = a.plan[(size_t)t.r * a.plan_stride + 1 + (g - prefix[rl])];
    t.s = a.states[t.r];
}

// Persistent: the listed tiles of all rows form one list, dealt to waves
// round-robin, so a heavy row spreads over the whole chip.  Each wave keeps
// two tiles in flight: the next tile's tokens and the one after's row and
// tile index are loaded while the current tile is walked.
template <int NW>
__global__ __launch_bounds__(kWalkThreads) void k_fill_walk(FillArgs a) {
    extern __shared__ uint64_t lds[];
    __shared__ uint32_t wave_sum[kWalkWaves];
    uint64_t *lds_comb = lds;
    uint32_t *prefix = (uint32_t *)(lds + a.comb_len);
    const WalkConsts &k = a.k;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // the first row block's first tile count of this thread is fetched
    // before the table, so that the two round trips overlap
    const int nb0 = min(kWalkRowBlock, a.B), per0 = (nb0 + kWalkThreads - 1) / kWalkThreads;
    const uint32_t first_n = tid * per0 < nb0 ? a.plan[(size_t)(tid * per0) * a.plan_stride] : 0u;
    stage_table(lds_comb, a.comb, a.comb_len);
    for (int rb = 0; rb < a.B; rb += kWalkRowBlock) {
        const int nb = min(kWalkRowBlock, a.B - rb);
        // exclusive scan of the block's tile counts
        const int per = (nb + kWalkThreads - 1) / kWalkThreads;
        const int r0 = min(nb, tid * per), r1 = min(nb, r0 + per);
        uint32_t sum = 0;
        for (int i = r0; i < r1; i++) {
            const uint32_t n = (rb == 0 && i == r0) ? first_n : a.plan[(size_t)(rb + i) * a.plan_stride];
            prefix[i] = n;  // the count, until the scan below replaces it
            sum += n;
        }
        const uint32_t incl = wave_incl_sum(sum);
        if (lane == 63) wave_sum[wave] = incl;
        __syncthreads();
        // the totals of the waves before this one: lane w < wave reads wave
        // w's, summed across the first row of lanes
        const uint32_t before = wave_incl_sum(lane < wave ? wave_sum[lane] : 0u);
        uint32_t run = incl - sum + (uint32_t)__builtin_amdgcn_readlane((int)before, 15);
        for (int i = r0; i < r1; i++) {
            const uint32_t n = prefix[i];
            prefix[i] = run;
            run += n;
        }
        if (tid == kWalkThreads - 1) prefix[nb] = run;
        __syncthreads();
        const uint32_t total = prefix[nb];
        // tile g goes to wave g / gridDim.x of workgroup g % gridDim.x: a
        // step's tiles spread over every CU, one wave per SIMD first,
        // before any CU walks several at once
        const uint32_t stride = gridDim.x * kWalkWaves;
        uint32_t g = wave * gridDim.x + blockIdx.x;
        TileRef t0{}, t1{}, t2{};
        LaneTok<NW> cur{}, nxt{};
        fetch_ref(t0, g, total, prefix, nb, rb, a);
        fetch_ref(t1, g + stride, total, prefix, nb, rb, a);
        if (g < total) load_lane(cur, t0.tile >> 30, (int)(t0.tile & kTileMask) * kTile + lane, a);
        for (; g < total; g += stride) {
            fetch_ref(t2, g + 2 * stride, total, prefix, nb, rb, a);
            if (g + stride < total) load_lane(nxt, t1.tile >> 30, (int)(t1.tile & kTileMask) * kTile + lane, a);
            const bool in_str = (t0.tile >> 30) >= LIST_QSTR;
            const Walker w0 = load_walker(t0.s);
            const uint32_t id = cur.il & 0xFFFFFFu;
            int end = (int)((cur.il >> 24) & 0x3Fu), start = 0;
            bool alive = (int32_t)cur.il < 0;
            Walker wk = w0;
            if (in_str) {
                // a string list holds the bytes after the closing quote
                const uint32_t nch = cur.aux >> 21;
                alive = alive && nch <= w0.cnt;
                wk.q = w0.ret;
                wk.ws = 0;
                wk.cnt = w0.cnt - nch;
            }
            const uint32_t jump = cur.aux;
            walk_bytes<0, NW * 4, NW>(wk, alive, cur.w, start, end, jump, lds_comb, k);
            if (alive) atomicOr(&a.mask[(size_t)t0.r * a.words_per_row + (id >> 6)], 1ull << (id & 63));
            cur = nxt;
            t0 = t1;
            t1 = t2;
        }
        __syncthreads();  // the block's prefix is no longer read
    }
}


// ---------------------------------------------------------------------------
// launchers (argument checks are done by the C ABI)
// ---------------------------------------------------------------------------
int launch_init(const cg_grammar *g, cg_state *states, int B, hipStream_t st) {
    if (B == 0) return CG_OK;
    hipLaunchKernelGGL(k_init, dim3((B + 255) / 256), dim3(256), 0, st, states, B, g->k.start);
    return launch_status("init_state");
}

int launch_advance(const cg_grammar *g, cg_state *states, int B, const int32_t *ids, int32_t *steps,
                   int32_t *status, hipStream_t st) {
    if (B == 0) return CG_OK;
    const size_t lds = (size_t)g->comb_len * sizeof(uint64_t);
    hipLaunchKernelGGL(k_advance, dim3((B + 255) / 256), dim3(256), lds, st, g->dev.comb, g->comb_len, g->k,
                       g->dev.tokw, g->dev.tokinfo, g->nw, g->V, states, B, ids, steps, status, g->gen_cap,
                       g->dev.forced);
    return launch_status("advance");
}

int launch_draft(const cg_grammar *g, const cg_state *states, const int32_t *steps, int B, const int32_t *draft,
                 int kd, cg_state *path, int32_t *accept_len, hipStream_t st) {
    if (B == 0) return CG_OK;
    const size_t lds = (size_t)g->comb_len * sizeof(uint64_t);
    hipLaunchKernelGGL(k_draft, dim3((B + 255) / 256), dim3(256), lds, st, g->dev.comb, g->comb_len, g->k,
                       g->dev.tokw, g->dev.tokinfo, g->nw, g->V, states, steps, B, draft, kd, path, accept_len,
                       g->gen_cap, g->dev.forced);
    return launch_status("fill_draft (path)");
}

int launch_force(const cg_grammar *g, cg_state *states, int B, const uint8_t *bytes, uint64_t n_bytes,
                 const uint32_t *offsets, int32_t *status, hipStream_t st) {
    if (B == 0) return CG_OK;
    const size_t lds = (size_t)g->comb_len * sizeof(uint64_t);
    hipLaunchKernelGGL(k_force, dim3((B + 255) / 256), dim3(256), lds, st, g->dev.comb, g->comb_len, g->k, states, B,
                       bytes, n_bytes, offsets, status, g->dev.forced);
    return launch_status("force_bytes");
}

// rows[i] &= m for the rows with need[i] (the table's context 1 / 2 rows)
__global__ __launch_bounds__(256) void k_mask_and(uint64_t *__restrict__ rows, const uint8_t *__restrict__ need,
                                                  const uint64_t *__restrict__ m, int Wv) {
    const int r = blockIdx.x;
    if (!need[r]) return;
    uint64_t *row = rows + (size_t)r * Wv;
    for (int i = threadIdx.x; i < Wv; i += blockDim.x) row[i] &= m[i];
}

int launch_mask_and(uint64_t *rows, const uint8_t *need, const uint64_t *m, int n, int Wv, hipStream_t st) {
    if (n == 0) return CG_OK;
    hipLaunchKernelGGL(k_mask_and, dim3(n), dim3(256), 0, st, rows, need, m, Wv);
    return launch_status("state masks (and)");
}

// Plan of one row: listed-tile count + up to every tile of the longer list.
int fill_plan_stride(const cg_grammar *g) {
    return (1 + std::max(1, std::max(g->lex_tiles, g->q_tiles)) + 63) / 64 * 64;
}

size_t fill_lds_bytes(const cg_grammar *g, int B) {
    return (size_t)g->comb_len * 8 + (size_t)(std::min(B, kWalkRowBlock) + 1) * 4;
}

FillArgs make_fill_args(const cg_grammar *g, const cg_state *states, int B, uint64_t *mask, int wpr, void *ws) {
    FillArgs a;
    a.comb = g->dev.comb;
    a.comb_len = g->comb_len;
    a.k = g->k;
    a.legal = g->dev.legal;
    a.lex_idlen = g->dev.lex_idlen;
    a.lex_jump = g->dev.lex_jump;
    a.lex_w = g->dev.lex_w;
    a.lex_tile = g->dev.lex_tile;
    a.lex_tiles = g->lex_tiles;
    a.q_idlen = g->dev.q_idlen;
    a.q_jump = g->dev.q_jump;
    a.q_w = g->dev.q_w;
    a.q_tile = g->dev.q_tile;
    a.q_tiles = g->q_tiles;
    a.strbits = g->dev.strbits;
    a.Wv = (g->V + 63) / 64;
    a.states = states;
    a.mask = (unsigned long long *)mask;
    a.words_per_row = wpr;
    a.forced = g->dev.forced;
    a.state_mask = g->dev.state_mask;
    a.smask_idx = g->dev.state_mask ? g->dev.smask_idx : nullptr;
    a.ws_dim = (int)g->k.ws_max + 1;
    a.push_room = g->min_push_cap - kPushLimit;
    a.c_idlen = g->dev.c_idlen;
    a.c_jump = g->dev.c_jump;
    a.c_w = g->dev.c_w;
    a.c_tile = g->dev.c_tile;
    a.c_tiles = g->c_tiles;
    a.retmask2 = g->dev.retmask ? g->dev.retmask2 : nullptr;
    a.qc_idlen = g->dev.qc_idlen;
    a.qc_jump = g->dev.qc_jump;
    a.qc_w = g->dev.qc_w;
    a.qc_tile = g->dev.qc_tile;
    a.qc_tiles = g->qc_tiles;
    a.closebits = g->dev.closebits;
    a.retmask = g->dev.retmask;
    a.rq_idx = g->dev.retmask ? g->dev.rq_idx : nullptr;
    a.plan = (uint32_t *)ws;
    a.plan_stride = fill_plan_stride(g);
    a.B = B;
    return a;
}

// persistent walk of the listed tiles: one 16-wave workgroup per CU
int fill_check(const cg_grammar *g, int B) {
    const size_t lds = fill_lds_bytes(g, B);
    if (lds + 1024 > (size_t)g->lds_max) {
        set_error("fill_bitmask: %zu bytes of LDS needed, %d available", lds, g->lds_max);
        return CG_E_LIMIT;
    }
    return CG_OK;
}

// The walk kernels' dynamic-LDS limit per device as last raised (0: the
// default): raised only when a launch needs more, so the per-step path makes
// no attribute call.
constexpr int kWalkMaxDevices = 64;
static std::mutex walk_attr_mu;
static int walk_lds_attr[kWalkMaxDevices][8];

template <int NW>
static int launch_walk_nw(const cg_grammar *g, const FillArgs &a, hipStream_t st) {
    const size_t lds = fill_lds_bytes(g, a.B);
    if (lds > 64 * 1024) {
        std::lock_guard<std::mutex> lk(walk_attr_mu);
        const bool known = g->device >= 0 && g->device < kWalkMaxDevices;
        if (!known || (size_t)walk_lds_attr[g->device][NW - 1] < lds) {
            if (hipFuncSetAttribute((const void *)k_fill_walk<NW>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                    (int)lds) != hipSuccess)
                return launch_status("fill_bitmask (LDS attribute)");
            if (known) walk_lds_attr[g->device][NW - 1] = (int)lds;
        }
    }
    hipLaunchKernelGGL(k_fill_walk<NW>, dim3(g->n_cu), dim3(kWalkThreads), lds, st, a);
    return launch_status("fill_bitmask (walk)");
}

int launch_fill_walk(const cg_grammar *g, const FillArgs &a, hipStream_t st) {
    if (a.B == 0) return CG_OK;
    switch (g->nw) {
    case 1: return launch_walk_nw<1>(g, a, st);
    case 2: return launch_walk_nw<2>(g, a, st);
    case 3: return launch_walk_nw<3>(g, a, st);
    case 4: return launch_walk_nw<4>(g, a, st);
    case 5: return launch_walk_nw<5>(g, a, st);
    case 6: return launch_walk_nw<6>(g, a, st);
    case 7: return launch_walk_nw<7>(g, a, st);
    default: return launch_walk_nw<8>(g, a, st);
    }
}

// ---------------------------------------------------------------------------
// The fill's per-row tile lists in a file-scope device array, for callers
// that cannot allocate (code under graph capture, serving loops that forbid
// allocation): cg_fill_bitmask_noalloc.  Every device the library runs on
// holds one copy for the life of the process; every call on a device shares
// it, so such calls must not overlap in time on one device.  Nothing in it
// needs clearing: the plan writes each row's count and list before the walk
// reads them.  In host code the array's name is not a device address: the
// address is taken once per device with hipGetSymbolAddress and kept.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = (size_t)CG_FILL_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint32_t scratch[kScratchBytes / sizeof(uint32_t)];

constexpr int kMaxDevices = 64;
static std::mutex scratch_mu;
static void *scratch_ptr[kMaxDevices];  // per device; null until set up
static bool scratch_tried[kMaxDevices];

// Called with device `dev` current (cg_compile_grammar uploads a grammar's
// tables there).  Returns CG_OK once the device's address is known.
int noalloc_setup(int dev) {
    if (dev < 0 || dev >= kMaxDevices) {
        set_error("fill_bitmask_noalloc: device %d out of range", dev);
        return CG_E_DEVICE;
    }
    std::lock_guard<std::mutex> lk(scratch_mu);
    if (scratch_ptr[dev]) return CG_OK;
    if (!scratch_tried[dev]) {
        scratch_tried[dev] = true;
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e == hipSuccess && p) scratch_ptr[dev] = p;
        else (void)hipGetLastError();
    }
    if (!scratch_ptr[dev]) {
        set_error("fill_bitmask_noalloc: no address for the scratch array on device %d", dev);
        return CG_E_DEVICE;
    }
    return CG_OK;
}

int launch_fill(const cg_grammar *g, const cg_state *states, int B, uint64_t *mask, int wpr, void *ws,
                hipStream_t st);

int launch_fill_noalloc(const cg_grammar *g, const cg_state *states, int B, uint64_t *mask, int wpr,
                        hipStream_t st) {
    if (B == 0) return CG_OK;
    const size_t need = (size_t)B * (size_t)fill_plan_stride(g) * sizeof(uint32_t);
    if (need > kScratchBytes) {
        set_error("fill_bitmask_noalloc: %d rows need %zu bytes of scratch, the limit is %zu (use cg_fill_bitmask "
                  "with a workspace)", B, need, kScratchBytes);
        return CG_E_LIMIT;
    }
    void *p = nullptr;
    {
        std::lock_guard<std::mutex> lk(scratch_mu);
        if (g->device >= 0 && g->device < kMaxDevices) p = scratch_ptr[g->device];
    }
    if (!p) {
        set_error("fill_bitmask_noalloc: the scratch array of device %d is not set up", g->device);
        return CG_E_DEVICE;
    }
    return launch_fill(g, states, B, mask, wpr, p, st);
}

int launch_fill(const cg_grammar *g, const cg_state *states, int B, uint64_t *mask, int wpr, void *ws,
                hipStream_t st) {
    if (B == 0) return CG_OK;
    const int chk = fill_check(g, B);
    if (chk != CG_OK) return chk;
    const FillArgs a = make_fill_args(g, states, B, mask, wpr, ws);
    hipLaunchKernelGGL(k_fill_plan, dim3(B), dim3(kPlanThreads), 0, st, a);
    const int rc = launch_status("fill_bitmask (plan)");
    if (rc != CG_OK) return rc;
    return launch_fill_walk(g, a, st);
}

}  // namespace cg
