// kernels.hip -- gfx950 kernels of the constrained-decoding step.
//
//   k_init        rows at the start state
//   k_fill        token bitmask: one lane per token walks the token's bytes
//                 through the transition table staged in LDS; a wave64 ballot
//                 packs 64 verdicts into one mask word ("Constrained
//                 decoding", "The guarantee": a pushdown automaton masks the
//                 logits at every step)
//   k_sample_a    streaming pass over the logits: per 2048-id chunk the
//                 masked max/argmax and the sum of exp((x - max) / T)
//   k_sample_b    per row: log-normaliser, greedy pick, or the two-level
//                 Philox Gumbel-max draw ("Sampling runs after masking")
//   k_advance     one lane per row walks the chosen token
//
// Nothing here is a dense contraction, so there is no MFMA: the fill is
// bound by table lookups and integer ALU, the sampler by HBM bandwidth.
#include <math.h>

#include <algorithm>

#include "cg_internal.hpp"

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

__global__ void k_advance(const uint64_t *__restrict__ comb, WalkConsts k, const uint8_t *__restrict__ blob,
                          const uint32_t *__restrict__ off, int V, cg_state *__restrict__ states, int B,
                          const int32_t *__restrict__ ids, int32_t *__restrict__ steps, int32_t *__restrict__ status,
                          uint32_t gen_cap) {
    int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= B) return;
    const int id = ids[r];
    if (id < 0) {
        status[r] = CG_ROW_NOOP;
        return;
    }
    cg_state s = states[r];
    if (id >= V || (s.flags & (CG_FLAG_DONE | CG_FLAG_CAPPED)) || s.q >= k.q_limit || s.ret >= k.q_limit) {
        status[r] = CG_ROW_REJECTED;
        return;
    }
    const uint32_t a = off[id], e = off[id + 1];
    Walker w = load_walker(s);
    bool ok = a < e;
    for (uint32_t i = a; ok && i < e; i++) ok = step_byte(w, blob[i], comb, k);
    if (!ok) {
        status[r] = CG_ROW_REJECTED;
        return;
    }
    store_walker(s, w);
    const int st = steps[r] + 1;
    steps[r] = st;
    int res = CG_ROW_OK;
    uint8_t fl = 0;
    if (w.q == k.accept) {
        fl |= CG_FLAG_DONE;
        res = CG_ROW_DONE;
    }
    if ((uint32_t)st >= gen_cap) {
        fl |= CG_FLAG_CAPPED;
        if (res == CG_ROW_OK) res = CG_ROW_CAPPED;
    }
    s.flags = fl;
    states[r] = s;
    status[r] = res;
}

// ---------------------------------------------------------------------------
// fill_bitmask
// ---------------------------------------------------------------------------
__device__ inline int wave_max_i32(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
    return v;
}

// Work item = (block of 256 consecutive tokens, group of rows).  Each wave
// owns 64 tokens = one mask word per row; its lanes keep their token's bytes
// in registers while the loop runs over the rows of the item, so the
// vocabulary is read once per item, not once per row.
template <int NW>
__global__ __launch_bounds__(256) void k_fill(const uint64_t *__restrict__ comb, uint32_t comb_len,
                                              const uint32_t *__restrict__ tokw, const uint8_t *__restrict__ toklen,
                                              int V, const cg_state *__restrict__ states, int B,
                                              uint64_t *__restrict__ mask, int words_per_row, WalkConsts k,
                                              int n_tok_blocks, int rows_per_item, int n_items) {
    extern __shared__ uint64_t lds_comb[];
    for (uint32_t i = threadIdx.x; i < comb_len; i += blockDim.x) lds_comb[i] = comb[i];
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int Wv = (V + 63) >> 6;
    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int tb = item % n_tok_blocks, rg = item / n_tok_blocks;
        const int word = tb * 4 + wave;
        const int tok = word * 64 + lane;
        uint32_t w[NW];
        int len = 0;
        if (tok < V) {
            len = toklen[tok];
#pragma unroll
            for (int j = 0; j < NW; j++) w[j] = tokw[(size_t)j * V + tok];
        } else {
#pragma unroll
            for (int j = 0; j < NW; j++) w[j] = 0;
        }
        const int wmax = wave_max_i32(len);
        const int r0 = rg * rows_per_item;
        const int r1 = min(B, r0 + rows_per_item);
        for (int r = r0; r < r1; r++) {
            const cg_state s = states[r];
            uint64_t bits = 0;
            const bool live_row = !(s.flags & (CG_FLAG_DONE | CG_FLAG_CAPPED)) && s.q < k.q_limit &&
                                  s.ret < k.q_limit;
            if (live_row) {
                Walker wk = load_walker(s);
                bool alive = len > 0;
#pragma unroll
                for (int b = 0; b < NW * 4; b++) {
                    if (b >= wmax) break;
                    const bool act = alive && b < len;
                    if (!__any(act)) break;
                    if (act) {
                        const uint32_t byte = (w[b >> 2] >> ((b & 3) * 8)) & 0xFFu;
                        alive = step_byte(wk, byte, lds_comb, k);
                    }
                }
                bits = __ballot(alive);
            }
            if (lane == 0 && word < Wv) mask[(size_t)r * words_per_row + word] = bits;
        }
    }
}

// ---------------------------------------------------------------------------
// mask_softmax_sample
// ---------------------------------------------------------------------------
constexpr int kChunk = 2048;           // ids per chunk (32 mask words)
constexpr float kLog2e = 1.4426950408889634f;
constexpr double kContend = 2e-5;      // chunks whose screened score is this close to the best are recomputed

struct Partial {
    float m;   // largest allowed logit of the chunk (-inf if none)
    int idx;   // its lowest id (-1 if none)
    double s;  // sum over allowed ids of exp((x - m) / T')
};

__device__ inline float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

template <int DT>
__device__ inline float load_logit(const void *p, size_t i) {
    if (DT == 0) return ((const float *)p)[i];
    return bf16_to_f32(((const uint16_t *)p)[i]);
}

__device__ inline bool better(float v, int i, float bv, int bi) {
    // larger value wins; equal values -> lower id; any allowed id beats none
    if (bi < 0) return i >= 0;
    if (i < 0) return false;
    return v > bv || (v == bv && i < bi);
}

// One wave per (row, chunk); 4 chunks per block.  Lane l reads ids
// c*2048 + g*512 + 8l .. +7 for g = 0..3: every load instruction covers 1 KB
// (bf16) of contiguous logits across the wave, and one mask byte per group.
template <int DT, bool VEC>
__global__ __launch_bounds__(256) void k_sample_a(const void *__restrict__ logits, int V, int64_t stride,
                                                  const uint64_t *__restrict__ mask, int words_per_row,
                                                  const float *__restrict__ temp, Partial *__restrict__ part,
                                                  int K) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int c = blockIdx.x * 4 + wave, r = blockIdx.y;
    if (c >= K) return;
    const float T = temp[r];
    const float kk = T > 0.f ? kLog2e / T : kLog2e;
    const uint8_t *mrow = (const uint8_t *)(mask + (size_t)r * words_per_row);
    const size_t rowbase = (size_t)r * (size_t)stride;
    float x[32];
    uint32_t mb[4];
#pragma unroll
    for (int g = 0; g < 4; g++) {
        const int e0 = c * kChunk + g * 512 + lane * 8;
        mb[g] = (e0 < V) ? mrow[e0 >> 3] : 0u;
        if (VEC && e0 + 8 <= V) {
            if (DT == 1) {
                const uint4 v = *(const uint4 *)((const uint16_t *)logits + rowbase + e0);
                const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    x[g * 8 + 2 * j] = __uint_as_float(u[j] << 16);
                    x[g * 8 + 2 * j + 1] = __uint_as_float(u[j] & 0xFFFF0000u);
                }
            } else {
                const float4 v0 = *(const float4 *)((const float *)logits + rowbase + e0);
                const float4 v1 = *(const float4 *)((const float *)logits + rowbase + e0 + 4);
                x[g * 8 + 0] = v0.x; x[g * 8 + 1] = v0.y; x[g * 8 + 2] = v0.z; x[g * 8 + 3] = v0.w;
                x[g * 8 + 4] = v1.x; x[g * 8 + 5] = v1.y; x[g * 8 + 6] = v1.z; x[g * 8 + 7] = v1.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; j++) x[g * 8 + j] = (e0 + j < V) ? load_logit<DT>(logits, rowbase + e0 + j) : 0.f;
            if (e0 + 8 > V) mb[g] &= (e0 >= V) ? 0u : ((1u << (V - e0)) - 1u);
        }
    }
    // masked max, lowest id on ties (ids increase with g, then j)
    float m = -INFINITY;
    int mi = -1;
#pragma unroll
    for (int g = 0; g < 4; g++)
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const int e = c * kChunk + g * 512 + lane * 8 + j;
            if (((mb[g] >> j) & 1u) && better(x[g * 8 + j], e, m, mi)) {
                m = x[g * 8 + j];
                mi = e;
            }
        }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float om = __shfl_xor(m, o, 64);
        const int oi = __shfl_xor(mi, o, 64);
        if (better(om, oi, m, mi)) {
            m = om;
            mi = oi;
        }
    }
    double s = 0.0;
    if (mi >= 0 && m != -INFINITY) {
#pragma unroll
        for (int g = 0; g < 4; g++) {
            float sg = 0.f;
#pragma unroll
            for (int j = 0; j < 8; j++)
                if ((mb[g] >> j) & 1u) sg += exp2f((x[g * 8 + j] - m) * kk);
            s += (double)sg;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    if (lane == 0) {
        Partial p;
        p.m = m;
        p.idx = mi;
        p.s = s;
        part[(size_t)r * K + c] = p;
    }
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two
// 32x32->64 multiplications and a xor-recombination, key bumped by the
// Weyl increments between rounds.
__device__ inline uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int i = 0; i < 10; i++) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
        const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c;
}

__device__ inline uint32_t pick_word(uint4 v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }

// -ln(-ln u), u = (w + 1/2) 2^-32, in double
__device__ inline double gumbel(uint32_t w) {
    const double u = ((double)w + 0.5) * 2.3283064365386963e-10;
    return -log(-log(u));
}

// block-wide reductions over 256 threads (4 waves)
__device__ inline double block_max_d(double v, double *sh) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[wave] = v;
    __syncthreads();
    return fmax(fmax(sh[0], sh[1]), fmax(sh[2], sh[3]));
}

__device__ inline double block_sum_d(double v, double *sh) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[wave] = v;
    __syncthreads();
    return (sh[0] + sh[1]) + (sh[2] + sh[3]);
}

// argmax of (value, index): larger value, then lower index; index -1 = none
__device__ inline void arg_better(double &v, int &i, double ov, int oi) {
    if (oi < 0) return;
    if (i < 0 || ov > v || (ov == v && oi < i)) {
        v = ov;
        i = oi;
    }
}

__device__ inline void block_argmax_d(double &v, int &i, double *shv, int *shi) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const double ov = __shfl_xor(v, o, 64);
        const int oi = __shfl_xor(i, o, 64);
        arg_better(v, i, ov, oi);
    }
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) {
        shv[wave] = v;
        shi[wave] = i;
    }
    __syncthreads();
    v = shv[0];
    i = shi[0];
    for (int k2 = 1; k2 < 4; k2++) arg_better(v, i, shv[k2], shi[k2]);
}

// log-mass of chunk c recomputed entirely in double (contenders only)
template <int DT>
__device__ double chunk_lse_exact(const void *logits, size_t rowbase, const uint8_t *mrow, int V, int c, double T,
                                  double m, double *sh) {
    double s = 0.0;
    for (int e = c * kChunk + threadIdx.x; e < min(V, (c + 1) * kChunk); e += blockDim.x)
        if ((mrow[e >> 3] >> (e & 7)) & 1u) s += exp(((double)load_logit<DT>(logits, rowbase + e) - m) / T);
    s = block_sum_d(s, sh);
    return m / T + log(s);
}

template <int DT>
__global__ __launch_bounds__(256) void k_sample_b(const void *__restrict__ logits, int V, int64_t stride,
                                                  const uint64_t *__restrict__ mask, int words_per_row,
                                                  const float *__restrict__ temp, const uint64_t *__restrict__ seed,
                                                  const int32_t *__restrict__ step,
                                                  const Partial *__restrict__ part, int K,
                                                  int32_t *__restrict__ out_id, float *__restrict__ out_lp) {
    __shared__ double shv[4];
    __shared__ int shi[4];
    __shared__ int s_cont[8];
    __shared__ int s_ncont;
    const int r = blockIdx.x;
    const float Tf = temp[r];
    const bool greedy = !(Tf > 0.f);
    const double T = greedy ? 1.0 : (double)Tf;
    const Partial *pr = part + (size_t)r * K;
    // (1) log-normaliser over the chunks, greedy candidate
    double lse_max = -INFINITY;
    double gv = -INFINITY;
    int gi = -1;
    for (int c = threadIdx.x; c < K; c += blockDim.x) {
        const Partial p = pr[c];
        if (p.idx >= 0) {
            lse_max = fmax(lse_max, (double)p.m / T + log(p.s));
            arg_better(gv, gi, (double)p.m, p.idx);
        }
    }
    lse_max = block_max_d(lse_max, shv);
    block_argmax_d(gv, gi, shv, shi);
    if (gi < 0) {  // nothing allowed (finished row)
        if (threadIdx.x == 0) {
            out_id[r] = -1;
            out_lp[r] = 0.f;
        }
        return;
    }
    double acc = 0.0;
    for (int c = threadIdx.x; c < K; c += blockDim.x) {
        const Partial p = pr[c];
        if (p.idx >= 0) acc += exp((double)p.m / T + log(p.s) - lse_max);
    }
    const double lse_all = lse_max + log(block_sum_d(acc, shv));
    if (greedy) {
        if (threadIdx.x == 0) {
            out_id[r] = gi;
            out_lp[r] = (float)(gv - lse_all);
        }
        return;
    }
    const uint64_t sd = seed[r];
    const uint32_t k0 = (uint32_t)sd, k1 = (uint32_t)(sd >> 32);
    const uint32_t stp = (uint32_t)step[r];
    const size_t rowbase = (size_t)r * (size_t)stride;
    const uint8_t *mrow = (const uint8_t *)(mask + (size_t)r * words_per_row);
    // (2) chunk choice: L_c + G(1, c)
    double best = -INFINITY;
    int bc = -1;
    for (int c = threadIdx.x; c < K; c += blockDim.x) {
        const Partial p = pr[c];
        if (p.idx < 0) continue;
        const uint4 o = philox4x32_10(make_uint4((uint32_t)c >> 2, stp, 1u, 0u), k0, k1);
        arg_better(best, bc, (double)p.m / T + log(p.s) + gumbel(pick_word(o, c & 3)), c);
    }
    block_argmax_d(best, bc, shv, shi);
    // screened scores carry ~1e-6 of rounding: recompute close contenders exactly
    if (threadIdx.x == 0) s_ncont = 0;
    __syncthreads();
    for (int c = threadIdx.x; c < K; c += blockDim.x) {
        const Partial p = pr[c];
        if (p.idx < 0) continue;
        const uint4 o = philox4x32_10(make_uint4((uint32_t)c >> 2, stp, 1u, 0u), k0, k1);
        const double sc = (double)p.m / T + log(p.s) + gumbel(pick_word(o, c & 3));
        if (sc >= best - kContend) {
            const int slot = atomicAdd(&s_ncont, 1);
            if (slot < 8) s_cont[slot] = c;
        }
    }
    __syncthreads();
    const int ncont = min(s_ncont, 8);
    if (ncont > 1) {
        double bb = -INFINITY;
        int bbc = -1;
        for (int t = 0; t < ncont; t++) {
            const int c = s_cont[t];
            const Partial p = pr[c];
            const double l = chunk_lse_exact<DT>(logits, rowbase, mrow, V, c, T, (double)p.m, shv);
            const uint4 o = philox4x32_10(make_uint4((uint32_t)c >> 2, stp, 1u, 0u), k0, k1);
            arg_better(bb, bbc, l + gumbel(pick_word(o, c & 3)), c);
        }
        bc = bbc;
    }
    // (3) token choice inside chunk bc: x_i / T + G(0, i)
    double tv = -INFINITY;
    int ti = -1;
    {
        const int e0 = bc * kChunk + threadIdx.x * 8;
        if (e0 < V) {
            const uint32_t mbits = mrow[e0 >> 3];
            if (mbits) {
                const uint4 o0 = philox4x32_10(make_uint4((uint32_t)e0 >> 2, stp, 0u, 0u), k0, k1);
                const uint4 o1 = philox4x32_10(make_uint4(((uint32_t)e0 >> 2) + 1u, stp, 0u, 0u), k0, k1);
                for (int j = 0; j < 8 && e0 + j < V; j++) {
                    if (!((mbits >> j) & 1u)) continue;
                    const uint32_t wv = pick_word(j < 4 ? o0 : o1, j & 3);
                    const double sc = (double)load_logit<DT>(logits, rowbase + e0 + j) / T + gumbel(wv);
                    arg_better(tv, ti, sc, e0 + j);
                }
            }
        }
    }
    block_argmax_d(tv, ti, shv, shi);
    if (threadIdx.x == 0) {
        out_id[r] = ti;
        out_lp[r] = (ti >= 0) ? (float)((double)load_logit<DT>(logits, rowbase + ti) / T - lse_all) : 0.f;
    }
}

// ---------------------------------------------------------------------------
// launchers (argument checks are done by the C ABI)
// ---------------------------------------------------------------------------
static int launch_status(const char *what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        set_error("%s: %s", what, hipGetErrorString(e));
        return CG_E_DEVICE;
    }
    return CG_OK;
}

int launch_init(const cg_grammar *g, cg_state *states, int B, hipStream_t st) {
    if (B == 0) return CG_OK;
    hipLaunchKernelGGL(k_init, dim3((B + 255) / 256), dim3(256), 0, st, states, B, g->k.start);
    return launch_status("init_state");
}

int launch_advance(const cg_grammar *g, cg_state *states, int B, const int32_t *ids, int32_t *steps,
                   int32_t *status, hipStream_t st) {
    if (B == 0) return CG_OK;
    hipLaunchKernelGGL(k_advance, dim3((B + 127) / 128), dim3(128), 0, st, g->dev.comb, g->k, g->dev.blob,
                       g->dev.offsets, g->V, states, B, ids, steps, status, g->gen_cap);
    return launch_status("advance");
}

template <int NW>
static int launch_fill_nw(const cg_grammar *g, const cg_state *states, int B, uint64_t *mask, int wpr,
                          hipStream_t st) {
    const size_t lds = (size_t)g->comb_len * sizeof(uint64_t);
    static int configured_bytes = 0;
    if ((int)lds > configured_bytes) {
        if (hipFuncSetAttribute((const void *)k_fill<NW>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) !=
            hipSuccess) {
            set_error("fill_bitmask: table of %zu bytes does not fit in LDS", lds);
            return CG_E_LIMIT;
        }
        configured_bytes = (int)lds;
    }
    const int ncu = g->n_cu;
    const int per_cu = std::max(1, std::min(4, (int)((160 * 1024) / std::max<size_t>(lds, 1))));
    const int n_tok_blocks = (g->V + 255) / 256;
    const int grid_cap = ncu * per_cu;
    long long want = (long long)B * n_tok_blocks;
    int rows_per_item = (int)std::max<long long>(1, std::min<long long>(B, (want + 2LL * grid_cap - 1) / (2LL * grid_cap)));
    const int n_rg = (B + rows_per_item - 1) / rows_per_item;
    const int n_items = n_rg * n_tok_blocks;
    const int grid = std::max(1, std::min(n_items, grid_cap));
    hipLaunchKernelGGL(k_fill<NW>, dim3(grid), dim3(256), lds, st, g->dev.comb, g->comb_len, g->dev.tokw,
                       g->dev.toklen, g->V, states, B, mask, wpr, g->k, n_tok_blocks, rows_per_item, n_items);
    return launch_status("fill_bitmask");
}

int launch_fill(const cg_grammar *g, const cg_state *states, int B, uint64_t *mask, int wpr, hipStream_t st) {
    if (B == 0) return CG_OK;
    switch (g->nw) {
    case 1: return launch_fill_nw<1>(g, states, B, mask, wpr, st);
    case 2: return launch_fill_nw<2>(g, states, B, mask, wpr, st);
    case 3: return launch_fill_nw<3>(g, states, B, mask, wpr, st);
    case 4: return launch_fill_nw<4>(g, states, B, mask, wpr, st);
    case 5: return launch_fill_nw<5>(g, states, B, mask, wpr, st);
    case 6: return launch_fill_nw<6>(g, states, B, mask, wpr, st);
    case 7: return launch_fill_nw<7>(g, states, B, mask, wpr, st);
    default: return launch_fill_nw<8>(g, states, B, mask, wpr, st);
    }
}

size_t sample_workspace_bytes(int B, int V) {
    const size_t K = (size_t)(V + kChunk - 1) / kChunk;
    return (size_t)B * K * sizeof(Partial);
}

int launch_sample(const void *logits, int dt, int B, int V, int64_t stride, const uint64_t *mask, int wpr,
                  const float *temp, const uint64_t *seed, const int32_t *step, void *ws, int32_t *out_id,
                  float *out_lp, hipStream_t st) {
    if (B == 0) return CG_OK;
    const int K = (V + kChunk - 1) / kChunk;
    const int es = dt == 0 ? 4 : 2;
    const bool vec = ((uintptr_t)logits % 16 == 0) && ((stride * es) % 16 == 0);
    Partial *part = (Partial *)ws;
    dim3 ga((K + 3) / 4, B);
    if (dt == 0) {
        if (vec) hipLaunchKernelGGL((k_sample_a<0, true>), ga, dim3(256), 0, st, logits, V, stride, mask, wpr, temp, part, K);
        else hipLaunchKernelGGL((k_sample_a<0, false>), ga, dim3(256), 0, st, logits, V, stride, mask, wpr, temp, part, K);
        hipLaunchKernelGGL(k_sample_b<0>, dim3(B), dim3(256), 0, st, logits, V, stride, mask, wpr, temp, seed, step,
                           part, K, out_id, out_lp);
    } else {
        if (vec) hipLaunchKernelGGL((k_sample_a<1, true>), ga, dim3(256), 0, st, logits, V, stride, mask, wpr, temp, part, K);
        else hipLaunchKernelGGL((k_sample_a<1, false>), ga, dim3(256), 0, st, logits, V, stride, mask, wpr, temp, part, K);
        hipLaunchKernelGGL(k_sample_b<1>, dim3(B), dim3(256), 0, st, logits, V, stride, mask, wpr, temp, seed, step,
                           part, K, out_id, out_lp);
    }
    return launch_status("apply_mask_sample");
}

}  // namespace cg
