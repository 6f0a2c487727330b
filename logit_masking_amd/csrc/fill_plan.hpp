// fill_plan.hpp -- the first part of fill_bitmask, per row: the base words
// of the row's mask and the list of token tiles worth walking.  Shared by
// the plan kernel (pda.hip) and the fused sample + advance + plan launch
// (sample.hip), which plans a row's next mask right after committing its
// token ("Evaluator aware decoding", "Why isn't this in production APIs
// yet?": the mask depends on the automaton's state alone).
#pragma once

#include "cg_internal.hpp"

namespace cg {

__device__ __forceinline__ bool row_live(const cg_state &s, const WalkConsts &k) {
    return !(s.flags & (CG_FLAG_DONE | CG_FLAG_CAPPED)) && s.q < k.q_limit && s.ret < k.q_limit;
}

struct FillArgs {
    const uint64_t *comb;
    uint32_t comb_len;
    WalkConsts k;
    const uint64_t *legal;
    const uint32_t *lex_idlen, *lex_jump, *lex_w;
    const uint2 *lex_tile;
    int lex_tiles;
    const uint32_t *q_idlen, *q_jump, *q_w;
    const uint2 *q_tile;
    int q_tiles;
    const uint64_t *strbits;
    int Wv;
    const cg_state *states;
    unsigned long long *mask;
    int words_per_row;
    const uint32_t *forced;  // engine-written states: empty mask (null: none)
    const uint64_t *state_mask;  // masks computed once (null: none), see DeviceTables
    const int32_t *smask_idx;
    int ws_dim;                  // ws_max + 1
    int push_room;               // rows at depth < push_room may use contexts 1 / 2
    const uint32_t *c_idlen, *c_jump, *c_w;  // the closing-token list
    const uint2 *c_tile;
    int c_tiles;
    const uint64_t *retmask2;                 // string rows inside a container (null: none)
    const uint32_t *qc_idlen, *qc_jump, *qc_w;
    const uint2 *qc_tile;
    int qc_tiles;
    const uint64_t *closebits, *retmask;  // string rows with no open container (rq_idx null: none)
    const int32_t *rq_idx;
    uint32_t *plan;       // per row: [0] listed tiles, [1..] their indices
    int plan_stride;      // u32 per row
    int B;
};

__device__ __forceinline__ bool bit_of(const uint64_t *words, uint32_t j) { return (words[j >> 6] >> (j & 63)) & 1u; }

// Any set bit in positions [lo, hi] of a 256-bit set.
__device__ __forceinline__ bool any_bits(const uint64_t *words, uint32_t lo, uint32_t hi) {
    for (uint32_t wi = lo >> 6; wi <= (hi >> 6); wi++) {
        uint64_t m = words[wi];
        if (wi == (lo >> 6)) m &= ~0ull << (lo & 63);
        if (wi == (hi >> 6)) m &= ~0ull >> (63 - (hi & 63));
        if (m) return true;
    }
    return false;
}

// Does the key span [kf, kl] of a tile hold a candidate key of the row?
// Key 0 of a legal lead byte (its one-byte token) always is; key j > 0 is
// if the state after the lead byte has a transition on byte j - 1 (the
// 256-bit sets of those states, one per legal lead byte, are in `second`).
__device__ __forceinline__ bool span_legal(uint32_t kf, uint32_t kl, const uint64_t *valid1,
                                           const uint64_t *second) {
    const uint32_t b_lo = kf / kKeysPerLead, b_hi = kl / kKeysPerLead;
    for (uint32_t wi = b_lo >> 6; wi <= (b_hi >> 6); wi++) {
        uint64_t m = valid1[wi];
        if (wi == (b_lo >> 6)) m &= ~0ull << (b_lo & 63);
        if (wi == (b_hi >> 6)) m &= ~0ull >> (63 - (b_hi & 63));
        while (m) {
            const uint32_t b = wi * 64 + (uint32_t)__builtin_ctzll(m);
            m &= m - 1;
            const uint32_t base = b * kKeysPerLead;
            const uint32_t lo = b == b_lo ? kf - base : 0u, hi = b == b_hi ? kl - base : kKeysPerLead - 1u;
            if (lo == 0 || any_bits(second + b * 4, lo - 1, hi - 1)) return true;
        }
    }
    return false;
}

// Append the flagged tiles of this wave to the item's tile list.
__device__ __forceinline__ void append_tiles(bool act, uint32_t t, uint32_t *list, uint32_t *count) {
    const uint64_t m = __ballot(act);
    if (m == 0) return;
    const int lane = threadIdx.x & 63;
    uint32_t base = 0;
    if (lane == 0) base = atomicAdd(count, (uint32_t)__popcll(m));
    base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);  // no LDS round trip
    if (act) list[base + __popcll(m & ((1ull << lane) - 1ull))] = t;
}

// The candidate lists a listed tile can come from (bits 30..31 of its index).
enum : uint32_t { LIST_LEX = 0, LIST_CLOSE = 1, LIST_QSTR = 2, LIST_QCLOSE = 3 };
constexpr uint32_t kTileMask = (1u << 30) - 1;

constexpr int kPlanThreads = 1024;
constexpr int kPlanKeys = 8;  // tile keys each plan thread loads up front

// The plan of row r in configuration s, by a workgroup of kPlanThreads
// threads (every thread calls it; it has barriers).  comb1: the transition
// table for the first-byte walks (global, or a copy in LDS).  sh: the
// workgroup's scratch in LDS.
struct PlanShared {
    uint64_t valid1[4];
    uint64_t second[256 * 4];
    uint32_t n_active;
};

__device__ inline void plan_row(const FillArgs &a, int r, const cg_state &s, const uint64_t *comb1, PlanShared &sh) {
    uint64_t *valid1 = sh.valid1, *second = sh.second;
    uint32_t *const n_active_p = &sh.n_active;
    const WalkConsts &k = a.k;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t *plan = a.plan + (size_t)r * a.plan_stride;
    unsigned long long *out = a.mask + (size_t)r * a.words_per_row;
    const bool live = row_live(s, k) && !forced_state(a.forced, s.q);
    const bool in_str = live && s.q == k.s_body;
    // the table's row for this configuration: context 0 = no open container
    // (the whole mask), 1 / 2 = inside an object / array within push room
    // (the tokens that stay inside it; the closing list is walked)
    int ctx = -1, sidx = -1;
    if (live && !in_str && a.smask_idx && s.ws < (uint32_t)a.ws_dim) {
        if (s.depth == 0 && s.stk == 0) ctx = 0;
        else if (s.depth >= 1 && (int)s.depth < a.push_room) ctx = 1 + (int)(s.stk & 1u);
        if (ctx >= 0) sidx = a.smask_idx[((size_t)s.q * a.ws_dim + s.ws) * 3 + ctx];
    }
    // a string row inside an open container within push room: the closing
    // tokens that stay inside it come from retmask2, the rest are walked
    const int ridx2 = (in_str && a.retmask2 && s.depth >= 1 && (int)s.depth < a.push_room) ? a.rq_idx[s.ret] : -1;
    const uint32_t list = in_str ? (ridx2 >= 0 ? LIST_QCLOSE : LIST_QSTR)
                                 : (sidx >= 0 && ctx > 0) ? LIST_CLOSE : LIST_LEX;
    const int n_all = !live                  ? 0
                      : list == LIST_QSTR    ? a.q_tiles
                      : list == LIST_QCLOSE  ? a.qc_tiles
                      : list == LIST_CLOSE   ? a.c_tiles
                                             : a.lex_tiles;
    const uint2 *tkeys = list == LIST_QSTR     ? a.q_tile
                         : list == LIST_QCLOSE ? a.qc_tile
                         : list == LIST_CLOSE  ? a.c_tile
                                               : a.lex_tile;
    uint2 kk[kPlanKeys];
#pragma unroll
    for (int i = 0; i < kPlanKeys; i++) {
        const int t = tid + i * kPlanThreads;
        kk[i] = t < n_all ? tkeys[t] : make_uint2(1, 0);
    }
    // base words: zero; inside a string, the tokens that stay inside within
    // the budget, and with no open container also the tokens that close the
    // string and go on legally (then nothing is walked); outside strings,
    // the table's row (context 0: the whole mask, nothing walked)
    const bool plain = live && s.depth == 0 && s.stk == 0;
    const int ridx = (plain && in_str && a.rq_idx) ? a.rq_idx[s.ret] : -1;
    const size_t c_off = (size_t)min(s.cnt, (uint32_t)kStrBitsets - 1u) * a.Wv;
    const uint64_t *base = in_str ? a.strbits + c_off : sidx >= 0 ? a.state_mask + (size_t)sidx * a.Wv : nullptr;
    // (non-temporal stores: this workgroup never reads the words back; the
    // walk ORs into them, on any XCD, and the next sampler reads them once)
    if (ridx >= 0 || ridx2 >= 0) {
        const uint64_t *cb = a.closebits + c_off;
        const uint64_t *rm = ridx >= 0 ? a.retmask + (size_t)ridx * a.Wv
                                       : a.retmask2 + ((size_t)ridx2 * 2 + (s.stk & 1u)) * a.Wv;
        for (int i = tid; i < a.Wv; i += kPlanThreads) __builtin_nontemporal_store(base[i] | (cb[i] & rm[i]), &out[i]);
    } else {
        for (int i = tid; i < a.Wv; i += kPlanThreads) __builtin_nontemporal_store(base ? base[i] : 0ull, &out[i]);
    }
    if (!live || (sidx >= 0 && ctx == 0) || ridx >= 0) {
        if (tid == 0) plan[0] = 0;
        return;
    }
    if (tid == 0) *n_active_p = 0;
    const Walker w0 = load_walker(s);
    uint64_t after_quote[4] = {0, 0, 0, 0};
    if (in_str) {
        // after the closing quote: bytes with a transition out of the resume state
#pragma unroll
        for (int j = 0; j < 4; j++) after_quote[j] = a.legal[(size_t)w0.ret * 4 + j];
    } else if (tid < 256) {
        // legal first bytes, and the bytes out of the state after each
        Walker w = w0;
        const bool ok = step_byte(w, (uint32_t)tid, comb1, k);
        const uint64_t m = __ballot(ok);
        if (lane == 0) valid1[wave] = m;
        if (ok) {
#pragma unroll
            for (int j = 0; j < 4; j++) second[tid * 4 + j] = a.legal[(size_t)w.q * 4 + j];
        }
    }
    __syncthreads();
    for (int c0 = 0; c0 < n_all; c0 += kPlanKeys * kPlanThreads) {
        if (c0 > 0) {
#pragma unroll
            for (int i = 0; i < kPlanKeys; i++) {
                const int t = c0 + tid + i * kPlanThreads;
                kk[i] = t < n_all ? tkeys[t] : make_uint2(1, 0);
            }
        }
#pragma unroll
        for (int i = 0; i < kPlanKeys; i++) {
            if (c0 + i * kPlanThreads >= n_all) break;  // no key of this round left (the same for every thread)
            const int t = c0 + tid + i * kPlanThreads;
            bool act = false;
            if (t < n_all) {
                act = in_str ? (kk[i].x == 0 || any_bits(after_quote, kk[i].x - 1, kk[i].y - 1))
                             : span_legal(kk[i].x, kk[i].y, valid1, second);
            }
            append_tiles(act, (uint32_t)t | (list << 30), plan + 1, n_active_p);
        }
    }
    __syncthreads();
    if (tid == 0) plan[0] = *n_active_p;
}


}  // namespace cg
