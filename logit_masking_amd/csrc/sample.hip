// sample.hip -- gfx950 kernel of the masked softmax and pick
// ("Constrained decoding", "The guarantee": sampling runs after masking).
//
//   k_sample      one workgroup per row streams the logits once: masked max
//                 and sum of exp((x - max) / T) per 2048-id chunk, then the
//                 greedy pick or the two-level Philox Gumbel-max draw; fused,
//                 also the advance over the picked token and the plan of the
//                 row's next mask
//
// Bound by HBM bandwidth and the per-logit VALU work; no MFMA (nothing here
// is a dense contraction).
#include <math.h>

#include <algorithm>
#include <mutex>

#include "cg_internal.hpp"
#include "fill_plan.hpp"

namespace cg {

// ---------------------------------------------------------------------------
// mask_softmax_sample
// ---------------------------------------------------------------------------
constexpr int kChunk = 2048;            // ids per chunk (32 mask words)
constexpr float kLog2e = 1.4426950408889634f;
// Screened chunk scores carry < 1.2e-5 of error (float noise < 1e-5, float
// chunk sums ~1e-6): a gap above this decides the chunk outright.
constexpr double kContendChunk = 5e-5;

template <int DT>
__device__ inline float load_logit(const void *p, size_t i) {
    if (DT == 0) return ((const float *)p)[i];
    return __uint_as_float((uint32_t)((const uint16_t *)p)[i] << 16);
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
__device__ inline double gumbel64(uint32_t w) {
    const double u = ((double)w + 0.5) * 2.3283064365386963e-10;
    return -log(-log(u));
}

// ---- wave reductions with DPP lane permutes ------------------------------
// Within each row of 16 lanes: swap neighbours, swap pairs, rotate by 4,
// rotate by 8 (every lane of the row then holds the row's reduction); the
// four row results are read with readlane.  No LDS round trips.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}
constexpr int kQuadSwap1 = 0xB1, kQuadSwap2 = 0x4E, kRowRor4 = 0x124, kRowRor8 = 0x128;

template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
    const long long u = __double_as_longlong(v);
    const int lo = dpp_i<CTRL>((int)u), hi = dpp_i<CTRL>((int)(u >> 32));
    return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}
__device__ __forceinline__ double readlane_d(double v, int l) {
    const long long u = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane((int)u, l), hi = __builtin_amdgcn_readlane((int)(u >> 32), l);
    return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

template <class F>
__device__ __forceinline__ double wave_reduce_d(double v, F op) {
    v = op(v, dpp_d<kQuadSwap1>(v));
    v = op(v, dpp_d<kQuadSwap2>(v));
    v = op(v, dpp_d<kRowRor4>(v));
    v = op(v, dpp_d<kRowRor8>(v));
    return op(op(readlane_d(v, 0), readlane_d(v, 16)), op(readlane_d(v, 32), readlane_d(v, 48)));
}

// Wave-wide max / sum of a float in six DPP-fused instructions: four steps
// within each 16-lane row, then two row broadcasts (lane 15 of each row into
// the next row, lane 31 into rows 2 and 3) leave the result in lane 63.
// Every lane must be active.  Two wait states before each DPP read of the
// value the previous instruction wrote.
#define CG_DPP_WAVE_REDUCE(OP)                                                    \
    "s_nop 1\n\t" OP " %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t" \
    "s_nop 1\n\t" OP " %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t" \
    "s_nop 1\n\t" OP " %0, %0, %0 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"          \
    "s_nop 1\n\t" OP " %0, %0, %0 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"          \
    "s_nop 1\n\t" OP " %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"       \
    "s_nop 1\n\t" OP " %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"       \
    "s_nop 1"
__device__ __forceinline__ float wave_max_f(float v) {
    asm(CG_DPP_WAVE_REDUCE("v_max_f32_dpp") : "+v"(v));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ inline double wave_sum_d(double v) { return wave_reduce_d(v, [](double a, double b) { return a + b; }); }
__device__ __forceinline__ float wave_sum_f(float v) {
    asm(CG_DPP_WAVE_REDUCE("v_add_f32_dpp") : "+v"(v));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ int wave_min_i_fast(int v) {
    asm(CG_DPP_WAVE_REDUCE("v_min_i32_dpp") : "+v"(v));
    return __builtin_amdgcn_readlane(v, 63);
}

// Wave max of a double: rounding to float is monotone, so the lanes that
// hold the double max hold the float max; a float max picks the candidate
// lanes and the exact max is taken among them (nearly always one lane).
__device__ __forceinline__ double wave_max_d_fast(double v) {
    const float f = (float)v;
    const float fm = wave_max_f(f);
    if (fm == -INFINITY) return -INFINITY;
    uint64_t cand = __ballot(f == fm);
    double best = -INFINITY;
    while (cand) {
        const int l = __builtin_ctzll(cand);
        cand &= cand - 1;
        const long long u = ((long long)__builtin_amdgcn_readlane((int)(__double_as_longlong(v) >> 32), l) << 32) |
                            (unsigned)__builtin_amdgcn_readlane((int)__double_as_longlong(v), l);
        best = fmax(best, __longlong_as_double(u));
    }
    return best;
}

// argmax of (value, index): larger value, then lower index; index -1 = none
__device__ inline void arg_better(double &v, int &i, double ov, int oi) {
    if (oi < 0) return;
    if (i < 0 || ov > v || (ov == v && oi < i)) {
        v = ov;
        i = oi;
    }
}
template <int CTRL>
__device__ __forceinline__ void arg_step(double &v, int &i) {
    const double ov = dpp_d<CTRL>(v);
    const int oi = dpp_i<CTRL>(i);
    arg_better(v, i, ov, oi);
}
__device__ inline void wave_argmax(double &v, int &i) {
    arg_step<kQuadSwap1>(v, i);
    arg_step<kQuadSwap2>(v, i);
    arg_step<kRowRor4>(v, i);
    arg_step<kRowRor8>(v, i);
    double bv = readlane_d(v, 0);
    int bi = __builtin_amdgcn_readlane(i, 0);
    for (int l = 16; l < 64; l += 16) arg_better(bv, bi, readlane_d(v, l), __builtin_amdgcn_readlane(i, l));
    v = bv;
    i = bi;
}

// Lane l holds, in group g = 0..3, the ids c*2048 + g*512 + 8l + j (j =
// 0..7): every load instruction covers a contiguous 1 KB (bf16) or 2 KB
// (float32, two instructions per group) of the row.  The chunk's 256 mask
// bytes come in one dword load per lane (lane l: bytes 4l .. 4l + 3), so a
// chunk in flight holds 17 (bf16) or 33 registers; group g's byte for lane
// l, 64g + l, is fetched from lane 16g + l/4 when the chunk is reduced.
template <int DT>
struct ChunkRegs {
    uint32_t d[DT == 1 ? 16 : 32];
    uint32_t mw;
};

// Bounds-checked load (rows whose storage is not 16-byte aligned): ids past
// V read as 0 with their mask bits clear.
template <int DT, bool VEC>
__device__ __forceinline__ void load_chunk(ChunkRegs<DT> &R, const void *logits, size_t rowbase,
                                           const uint8_t *mrow, int V, int c, int lane) {
    R.mw = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int f0 = c * kChunk + lane * 32 + 8 * i;  // the ids of mask byte 4 lane + i
        uint32_t b = (f0 < V) ? mrow[f0 >> 3] : 0u;
        if (f0 + 8 > V) b &= (f0 >= V) ? 0u : ((1u << (V - f0)) - 1u);
        R.mw |= b << (8 * i);
    }
#pragma unroll
    for (int g = 0; g < 4; g++) {
        const int e0 = c * kChunk + g * 512 + lane * 8;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const float x = (e0 + j < V) ? load_logit<DT>(logits, rowbase + e0 + j) : 0.f;
            if (DT == 1) {
                const uint32_t u = __float_as_uint(x) >> 16;
                if (j & 1) R.d[g * 4 + j / 2] |= u << 16;
                else R.d[g * 4 + j / 2] = u;
            } else {
                R.d[g * 8 + j] = __float_as_uint(x);
            }
        }
    }
}

// The row as two buffer resources (logits and mask): a buffer load past the
// resource's size returns zeros without touching memory, so every chunk, the
// row's partial last one included, is read with the same unguarded vector
// loads.  The logits' size is rounded up to whole dwords (a dword that holds
// the last id is read whole, from the dword-aligned row).
struct RowBufs {
    __amdgpu_buffer_rsrc_t x, m;
};
constexpr int kRsrcWord3 = 0x00020000;  // gfx9 raw buffer: 32-bit data format, no swizzle
// Cache policy of the stream's loads.  Every logit and mask word is read
// once.  A launch whose rows are large next to the memory-side cache (256 MB
// on this chip) reads them with the non-temporal hint: the stream then does
// not displace the small tables that each row's tail reads after it, and
// even a plain read of the same rows goes faster.  A smaller launch keeps
// the default policy, so rows that are read again soon stay cached.
constexpr int kPolicyCached = 0, kPolicyStream = 2;
constexpr size_t kStreamBytes = size_t(32) << 20;  // logits of a launch above this: non-temporal

template <int DT, int CP>
__device__ __forceinline__ void load_buf(ChunkRegs<DT> &R, const RowBufs &rb, int c, int lane) {
    constexpr int kEs = DT == 1 ? 2 : 4;
#pragma unroll
    for (int g = 0; g < 4; g++) {
        const int e0 = c * kChunk + g * 512 + lane * 8;
#pragma unroll
        for (int h = 0; h < (DT == 1 ? 1 : 2); h++) {
            const uint4 v =
                __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rb.x, e0 * kEs + 16 * h, 0, CP));
            uint32_t *d = &R.d[g * (DT == 1 ? 4 : 8) + 4 * h];
            d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
        }
    }
    R.mw = __builtin_amdgcn_raw_buffer_load_b32(rb.m, c * 256 + lane * 4, 0, CP);
}

// The same logit loads for a row whose mask is staged in LDS: a lane reads
// its 16 bytes of group g only when their 8 mask bits (byte g of mt, the
// lane's transposed mask dword of the chunk) hold an allowed id.  A masked
// logit never reaches a result (the reduction replaces it by -inf before
// any arithmetic, the pick skips it), so the registers of a piece not read
// may hold anything.
template <int DT, int CP>
__device__ __forceinline__ void load_buf_masked(ChunkRegs<DT> &R, const RowBufs &rb, int c, int lane, uint32_t mt) {
    constexpr int kEs = DT == 1 ? 2 : 4;
#pragma unroll
    for (int g = 0; g < 4; g++) {
        if (((mt >> (8 * g)) & 0xFFu) == 0u) continue;
        const int e0 = c * kChunk + g * 512 + lane * 8;
#pragma unroll
        for (int h = 0; h < (DT == 1 ? 1 : 2); h++) {
            const uint4 v =
                __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rb.x, e0 * kEs + 16 * h, 0, CP));
            uint32_t *d = &R.d[g * (DT == 1 ? 4 : 8) + 4 * h];
            d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
        }
    }
}

// Pieces of 16 mask bytes each thread stages for a row whose mask goes to
// LDS: K <= 64 * kMaskPieces chunks.
constexpr int kMaskPieces = 4;

// Group g's mask byte for this lane (chunk byte 64g + lane) from the lane
// that loaded it: one cross-lane read per group, no LDS memory.
__device__ __forceinline__ void mask_bytes(uint32_t mw, int lane, uint32_t (&mb)[4]) {
    const int sh = 8 * (lane & 3);
#pragma unroll
    for (int g = 0; g < 4; g++)
        mb[g] = ((uint32_t)__builtin_amdgcn_ds_bpermute(64 * g + (lane & ~3), (int)mw) >> sh) & 0xFFu;
}



// max of three floats in one instruction.  fmaxf on values made by bit
// manipulation costs an extra canonicalising instruction per operand; the
// values here are logits or -inf, never signalling NaNs.
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// float32 logit j of group g, or -inf where the mask bit is clear (a
// sign-extended 1-bit field selects between the value and -inf)
template <int DT>
__device__ __forceinline__ float masked_x(const ChunkRegs<DT> &R, const uint32_t (&mb)[4], int g, int j) {
    const uint32_t sel = (uint32_t)__builtin_amdgcn_sbfe((int)mb[g], j, 1);
    const uint32_t u = R.d[g * 8 + j];
    return __uint_as_float((sel & u) | (~sel & 0xFF800000u));
}

// Mask byte -> for each of its four bf16 pairs a 32-bit select mask (a half
// of ones per allowed id), so that one bit-select per pair masks two logits.
__device__ __forceinline__ void init_pair_lut(uint4 *lut) {
    const uint32_t v = threadIdx.x;
    if (v < 256) {
        uint32_t m[4];
#pragma unroll
        for (int p = 0; p < 4; p++)
            m[p] = (((v >> (2 * p)) & 1u) ? 0x0000FFFFu : 0u) | (((v >> (2 * p + 1)) & 1u) ? 0xFFFF0000u : 0u);
        lut[v] = make_uint4(m[0], m[1], m[2], m[3]);
    }
}

// Masked max m and sum over allowed ids of 2^((x - m) kk), kk = log2(e) / T'.
// The masked values (masked-out ids as -inf) are widened to float once and
// kept for the exponential pass.  The exponent is one fma, x kk - r(m kk),
// whose only error beyond a single rounding is the constant offset
// m kk - r(m kk); that offset is taken out of the chunk sum once.  The 64
// lane sums (each of 32 terms <= 1) are added as a tree in float: relative
// error ~1e-6.  Groups of 8 ids with no allowed id skip the exponentials
// (most of a structural row).
template <int DT>
__device__ __forceinline__ void reduce_chunk(const ChunkRegs<DT> &R, const uint32_t (&mb)[4], const uint4 *lut,
                                             float kk, float &m_out, float &s_out, bool &any_out) {
    any_out = __any(mb[0] | mb[1] | mb[2] | mb[3]);
    m_out = -INFINITY;
    s_out = 0.f;
    if (!any_out) return;
    float xm[32];
    float m = -INFINITY;
#pragma unroll
    for (int g = 0; g < 4; g++) {
        if (DT == 1) {
            // one bit-select per bf16 pair (allowed halves keep their logit,
            // the others become -inf), then one shift and one and
            const uint4 sel = lut[mb[g]];
            const uint32_t sp[4] = {sel.x, sel.y, sel.z, sel.w};
#pragma unroll
            for (int p = 0; p < 4; p++) {
                uint32_t u = (R.d[g * 4 + p] & sp[p]) | (~sp[p] & 0xFF80FF80u);
                asm("" : "+v"(u));  // one select, then two widenings (not re-derived per half)
                xm[g * 8 + 2 * p] = __uint_as_float(u << 16);
                xm[g * 8 + 2 * p + 1] = __uint_as_float(u & 0xFFFF0000u);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; j++) xm[g * 8 + j] = masked_x<DT>(R, mb, g, j);
        }
#pragma unroll
        for (int j = 0; j < 8; j += 2) m = max3f(m, xm[g * 8 + j], xm[g * 8 + j + 1]);
    }
    m = wave_max_f(m);
    m_out = m;
    if (m == -INFINITY) return;  // every allowed logit is -inf
    const float mk = m * kk;
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < 4; g++) {
        if (mb[g]) {
            float sg = 0.f;
#pragma unroll
            for (int j = 0; j < 8; j++) sg += __builtin_amdgcn_exp2f(__builtin_fmaf(xm[g * 8 + j], kk, -mk));
            s += sg;
        }
    }
    // every term carries the factor 2^off, off = m kk - r(m kk) (exact from
    // one fma, |off| <= half an ulp of m kk); divide it out
    const float off = __builtin_fmaf(m, kk, -mk);
    s_out = wave_sum_f(s) * (1.f - off * 0.69314718f);
}

// ---- block-wide reductions (kWaves waves) --------------------------------
constexpr int kWaves = 16;            // one workgroup of 1024 threads per row
static_assert(kWaves == 16, "slot reductions read one slot per lane of a 16-lane row");

// Each wave reduces in registers, lane 0 parks the result in slot[wave];
// after one barrier every wave reads the 16 slots with lanes 0..15 and
// reduces that row of lanes with DPP.  One barrier, no second pass.
__device__ __forceinline__ double slots_sum_d(const double *slot) {
    double v = slot[threadIdx.x & 15];
    v += dpp_d<kQuadSwap1>(v);
    v += dpp_d<kQuadSwap2>(v);
    v += dpp_d<kRowRor4>(v);
    v += dpp_d<kRowRor8>(v);
    return readlane_d(v, 0);
}

struct ChunkInfo {
    float s;      // sum over allowed ids of 2^((x - m) kk)
    float m;      // largest allowed logit
    float g;      // chunk noise G(1, c) in float, for screening (sampled rows)
    int any;      // the chunk has an allowed id
};

// The row's decision as the three reducing waves publish it.
struct RowDecision {
    double lse_all, cs1, cs2;
    float mv;
    int mc, c1;
};

struct Decision {
    double lse_all, cs1;
    float mv;
    int mc, chosen;
    bool exact_chunk;
};

struct Slots {
    double a[kWaves], b[kWaves];
    float f[kWaves], h[kWaves];
    int i[kWaves], j[kWaves];
};

// log-mass of chunk c recomputed entirely in double by the whole workgroup
// (kWaves waves).  Every thread's mask bytes and logits are loaded before any
// is used: one round trip, not one per id (a loop that loads the logit only
// under its mask bit waits out two dependent round trips per id).
template <int DT>
__device__ double chunk_lse_exact(const void *logits, size_t rowbase, const uint8_t *mrow, int V, int c, double T,
                                  double m, double *slot) {
    constexpr int kPer = kChunk / (kWaves * 64);
    float x[kPer];
    uint32_t mb[kPer];
#pragma unroll
    for (int j = 0; j < kPer; j++) {
        const int e = c * kChunk + (int)threadIdx.x + j * kWaves * 64;
        mb[j] = e < V ? (mrow[e >> 3] >> (e & 7)) & 1u : 0u;
        x[j] = e < V ? load_logit<DT>(logits, rowbase + e) : 0.f;
    }
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < kPer; j++)
        if (mb[j]) s += exp(((double)x[j] - m) / T);
    s = wave_sum_d(s);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) slot[threadIdx.x >> 6] = s;
    __syncthreads();
    return m / T + log(slots_sum_d(slot));
}

// G(i) in float for screening, from v_log_f32 only, without branches: -ln u
// for u <= 1/2; above, with v = 1 - u (from w): a 4-term series of
// -ln(1 - v) for v < 2^-7, else -ln(1 - v) rounded from float (relative
// error < 4e-6).  Absolute error of the result < 1e-5.  The argument of the
// first logarithm is selected before it is taken: two v_log_f32 per value.
__device__ inline float gumbel32(uint32_t w) {
    constexpr float kLn2 = 0.6931471805599453f;
    const float u = ((float)w + 0.5f) * 2.3283064365386963e-10f;
    const float v = ((float)(0xFFFFFFFFu - w) + 0.5f) * 2.3283064365386963e-10f;
    const bool lo = w < 0x80000000u;
    const float t_ser = v * (1.f + v * (0.5f + v * (0.33333334f + v * 0.25f)));
    const float t_log = -kLn2 * __builtin_amdgcn_logf(lo ? u : 1.f - v);
    const float t = (!lo && v < 0.0078125f) ? t_ser : t_log;
    return -kLn2 * __builtin_amdgcn_logf(t);
}

// top two of (value, index) with the larger value first (lower index on ties)
struct Top2 {
    float v1, v2;
    int i1;
};
__device__ __forceinline__ void top2_merge(Top2 &a, float bv1, int bi1, float bv2) {
    const bool b_first = bi1 >= 0 && (a.i1 < 0 || bv1 > a.v1 || (bv1 == a.v1 && bi1 < a.i1));
    if (b_first) {
        a.v2 = fmaxf(a.v1, bv2);
        a.v1 = bv1;
        a.i1 = bi1;
    } else {
        a.v2 = fmaxf(a.v2, bv1);
    }
}
// The same from two wave maxes: the best value, the lowest index holding it,
// then the best of everything else.
__device__ __forceinline__ Top2 top2_wave_fast(const Top2 &a) {
    Top2 r;
    r.v1 = wave_max_f(a.v1);
    r.i1 = wave_min_i_fast((a.i1 >= 0 && a.v1 == r.v1) ? a.i1 : 0x7FFFFFFF);
    if (r.i1 == 0x7FFFFFFF) r.i1 = -1;
    r.v2 = wave_max_f(a.i1 == r.i1 ? a.v2 : a.v1);
    return r;
}
// the same for chunk scores, in double (they can be large for heavy-tailed logits)
struct Top2d {
    double v1, v2;
    int i1;
};
__device__ __forceinline__ void top2d_merge(Top2d &a, double bv1, int bi1, double bv2) {
    const bool b_first = bi1 >= 0 && (a.i1 < 0 || bv1 > a.v1 || (bv1 == a.v1 && bi1 < a.i1));
    if (b_first) {
        a.v2 = fmax(a.v1, bv2);
        a.v1 = bv1;
        a.i1 = bi1;
    } else {
        a.v2 = fmax(a.v2, bv1);
    }
}
// Per-wave copy of the best chunk seen so far: the chunk's logits in id
// order (4 KB of bf16 pairs, 8 KB of float32) and each lane's four mask
// bytes, so the pick inside the chosen chunk reads LDS instead of HBM.
template <int DT>
struct Stash {
    uint32_t d[kWaves][DT == 1 ? kChunk / 2 : kChunk];
    uint32_t mb[kWaves][64];
    int c[kWaves];
};

// The grammar side of the fused sample + advance: after the pick, the
// workgroup's first thread walks the chosen token from the row's
// configuration (cg_advance's rules) through the table staged in LDS.
struct AdvanceArgs {
    const uint64_t *comb;  // null: sample only
    uint32_t comb_len;
    uint32_t comb_off;     // byte offset of the staged table in dynamic LDS
    WalkConsts k;
    const uint32_t *tokw, *tokinfo;
    int nw, V;
    cg_state *states;
    int32_t *steps;        // the same array as the sampler's step (read first, then bumped)
    int32_t *status;
    uint32_t gen_cap;
    const uint32_t *forced;
};

// byte offset of the stash in dynamic LDS: after the chunk summaries, 16-byte aligned
__host__ __device__ inline size_t stash_offset(int K) { return ((size_t)K * sizeof(ChunkInfo) + 15) / 16 * 16; }

// table slots each thread fetches into registers at the start, ahead of the
// logits (a table beyond kStageRegs * 1024 slots stages its rest after the
// stream)
constexpr int kStageRegs = 3;

// One workgroup per row.  Its 16 waves stream the row's 2048-id chunks (wave
// w starts with chunk w and then takes the next unclaimed one from a counter
// in LDS; one chunk's loads in flight per wave, the next load issued as each
// chunk is reduced) and leave
// one summary per chunk in LDS (masked max, sum of exponentials, the
// chunk's screening noise); each wave also keeps a copy of its best chunk
// so far in an LDS stash.  After one barrier three waves reduce the chunk
// summaries (log-normaliser, greedy chunk, best two chunk scores) while
// eight waves pick the token inside the chunk they choose with the same
// code, read from the stash.  No state crosses workgroups, so no
// device-wide fence is ever needed.  With the fused advance the first
// thread commits the token; with plan_next the workgroup then plans its
// row's next mask from the committed state (fill_plan.hpp), rewriting the
// row's mask words it has finished reading (mask is not restrict).
template <int DT, bool VEC, bool NT, bool SP>
__global__ __launch_bounds__(1024) void k_sample(const void *__restrict__ logits, int V, int64_t stride,
                                                 const uint64_t *mask, int words_per_row,
                                                 const float *__restrict__ temp, const uint64_t *__restrict__ seed,
                                                 const int32_t *step, int K, int use_stash, int moff,
                                                 int32_t *__restrict__ out_id, float *__restrict__ out_lp,
                                                 AdvanceArgs adv, FillArgs pa, int plan_next) {
    extern __shared__ uint64_t dyn[];
    ChunkInfo *ci = (ChunkInfo *)dyn;
    // Sparse stream (aligned rows whose mask fits in LDS): the row's mask is
    // staged in LDS at the start, transposed (dword 64 c + l of lmask holds
    // bytes l, 64 + l, 128 + l, 192 + l of chunk c: lane l's four group
    // bytes), and after its first chunk a wave reads only the 16-byte pieces
    // of logits that hold an allowed id.  Rows of a constrained step are
    // mostly sparse: their logits are mostly never read.
    constexpr bool kSparse = SP && VEC;
    uint32_t *lmask = (uint32_t *)((char *)dyn + moff);
    Stash<DT> *st = (Stash<DT> *)((char *)dyn + stash_offset(K));  // valid when use_stash
    __shared__ Slots sl[4];
    __shared__ uint4 lut[256];
    __shared__ RowDecision wdec;
    __shared__ PlanShared psh;
    __shared__ cg_state next_state;
    __shared__ int next_chunk;  // the next chunk to deal to a wave
    __shared__ uint32_t cur_w[6];  // fused: the row's state, for the wave that commits the pick
    // the wave index through readfirstlane: the compiler then knows it (and
    // every chunk index derived from it) is uniform, and branches on scalars
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = blockIdx.x;
    const uint8_t *mrow = (const uint8_t *)(mask + (size_t)r * words_per_row);
    const size_t rowbase = (size_t)r * (size_t)stride;
    // Each wave streams its chunks through a ring of NB chunk buffers (the
    // first ones wave, wave + 16, ...): the next load into a buffer is
    // issued as soon as its chunk is reduced.  One chunk per wave in flight
    // (4 KB of bf16, 8 KB of float32) keeps the memory queues shallow:
    // deeper rings (all of a 128K-id row requested at once) leave every
    // chunk waiting behind the whole chip's requests and bunch the arrivals,
    // and the reductions, at the end of the stream; a second float32 buffer
    // would also leave no registers for the stash's bookkeeping.
    // Rows whose storage is not 16-byte aligned are read one chunk at a time
    // with bounds-checked loads instead.
    constexpr int NB = 1;
    const int Kf = VEC ? K : 0;  // chunks read through buffer loads
    RowBufs rb;
    rb.x = __builtin_amdgcn_make_buffer_rsrc((void *)((const char *)logits + rowbase * (DT == 1 ? 2 : 4)), (short)0,
                                             (V * (DT == 1 ? 2 : 4) + 3) & ~3, kRsrcWord3);
    rb.m = __builtin_amdgcn_make_buffer_rsrc((void *)mrow, (short)0, words_per_row * 8, kRsrcWord3);
    // (a scheduling barrier after each chunk's loads keeps the compiler from
    // regrouping loads across chunks, which would make the first chunk wait
    // for the others)
    constexpr int CP = NT ? kPolicyStream : kPolicyCached;
    auto load_all = [&](ChunkRegs<DT> &R, int cc) {
        load_buf<DT, CP>(R, rb, min(cc, Kf), lane);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto load = [&](ChunkRegs<DT> &R, int cc) {
        if (kSparse) {
            if (cc < Kf) load_buf_masked<DT, CP>(R, rb, cc, lane, lmask[cc * 64 + lane]);
        } else {
            load_buf<DT, CP>(R, rb, min(cc, Kf), lane);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    ChunkRegs<DT> buf[NB];
    // The first loads go out before anything else is read (a scalar read of
    // the row's temperature, seed or step ahead of them would hold them back
    // for its own round trip: scalar loads are waited for all together).
    // Every wave issues them (clamped, even with no chunk of its own)
    // whenever the row has pipelined chunks at all.
    if (Kf > 0) {
#pragma unroll
        for (int b = 0; b < NB; b++) load_all(buf[b], wave + b * kWaves);
    }
    // sparse: the row's mask, 16 bytes per piece, right behind the first chunk
    uint4 mp[kMaskPieces];
    if (kSparse) {
#pragma unroll
        for (int j = 0; j < kMaskPieces; j++) {
            const int p = threadIdx.x + j * 1024;
            mp[j] = make_uint4(0u, 0u, 0u, 0u);
            if (p < K * 16) mp[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rb.m, p * 16, 0, CP));
        }
    }
    // fused: wave 0's lanes 0..5 fetch the row's 24-byte state now, and
    // leave it in LDS for the committing wave after the stream, long after
    // it has arrived
    const bool fuse = adv.comb != nullptr;
    uint32_t stw = 0;
    if (fuse && wave == 0 && lane < 6) stw = ((const uint32_t *)(adv.states + r))[lane];
    __builtin_amdgcn_sched_barrier(0);
    const float Tf = temp[r];
    const uint64_t sd = seed[r];
    const uint32_t stp = (uint32_t)step[r];
    const bool greedy = !(Tf > 0.f);
    const double T = greedy ? 1.0 : (double)Tf;
    const double invT = 1.0 / T;
    const float kk = greedy ? kLog2e : kLog2e / Tf;
    const uint32_t k0 = (uint32_t)sd, k1 = (uint32_t)(sd >> 32);
    constexpr double kLn2d = 0.6931471805599453, kLog2ed = 1.4426950408889634;
    const bool stash = use_stash != 0;
    // fused advance: the transition table is fetched into registers at the
    // start, right behind the first chunk, so its round trip is over long
    // before the stream ends; it is stored to LDS after the stream and the
    // walk of the chosen token reads it there
    uint64_t *lds_comb = (uint64_t *)((char *)dyn + adv.comb_off);
    const uint32_t tn = fuse ? adv.comb_len : 0u;
    // the pick: every exit path below leaves it here (its log-probability in
    // the thread that commits it)
    int pick = -1;
    float pick_lp = 0.f;
    Decision dc;
    const uint32_t treg = min(tn, (uint32_t)(kStageRegs * blockDim.x));
    uint64_t tv[kStageRegs];
    {
        // (indices clamped rather than guarded: a fixed number of loads
        // keeps the waits exact)
        if (fuse) {
#pragma unroll
            for (int j = 0; j < kStageRegs; j++) tv[j] = adv.comb[min(j * blockDim.x + threadIdx.x, treg - 1)];
        }
        // clears the mask bits of ids past V in the last chunk (a caller's
        // mask may carry set bits there)
        auto clear_tail = [&](uint32_t (&mb)[4]) {
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const int n = V - ((K - 1) * kChunk + g * 512 + lane * 8);
                mb[g] &= n >= 8 ? 0xFFu : n <= 0 ? 0u : ((1u << n) - 1u);
            }
        };
        int c = wave;
        if (DT == 1) init_pair_lut(lut);
        if (stash && lane == 0) st->c[wave] = -1;
        if (threadIdx.x == 0) next_chunk = NB * kWaves;
        // screening noise G(1, c) of every chunk (wave w: c = w + 16 lane +
        // 1024 j), while the loads fly; any wave may reduce any chunk
        if (!greedy)
            for (int cg = wave + kWaves * lane; cg < K; cg += kWaves * 64) {
                const uint4 o = philox4x32_10(make_uint4((uint32_t)cg >> 2, stp, 1u, 0u), k0, k1);
                ci[cg].g = gumbel32(pick_word(o, cg & 3));
            }
        // sparse: the mask pieces transposed into LDS (byte k of chunk c to
        // byte k / 64 of dword 64 c + k % 64)
        if (kSparse) {
#pragma unroll
            for (int j = 0; j < kMaskPieces; j++) {
                const int p = threadIdx.x + j * 1024;
                if (p < K * 16) {
                    const int k0 = (p & 15) * 16;
                    uint8_t *dst = (uint8_t *)lmask + (size_t)((p >> 4) * 64 + (k0 & 63)) * 4 + (k0 >> 6);
                    const uint32_t w4[4] = {mp[j].x, mp[j].y, mp[j].z, mp[j].w};
#pragma unroll
                    for (int i = 0; i < 16; i++) dst[4 * i] = (uint8_t)(w4[i >> 2] >> (8 * (i & 3)));
                }
            }
        }
        // (the loads stay in flight across the barrier: a workgroup barrier
        // waits for LDS operations, not for loads from memory)
        __syncthreads();  // the pair table, the noise, the chunk counter and (sparse) the mask
        // reduce chunk cc into its summary; the wave's best chunk so far (by
        // the chunk score in float: m for greedy rows, m/T + ln s + G(1, c)
        // for sampled ones) is copied to the stash.  A near-tie that the
        // float score orders differently from the decision's only costs
        // the pick a read of the chunk from memory.
        float best = -INFINITY;
        const float invTf = (float)invT;
        auto process = [&](ChunkRegs<DT> &R, int cc) {
            uint32_t mb[4];
            if (kSparse) {
                const uint32_t mt = lmask[cc * 64 + lane];
#pragma unroll
                for (int g = 0; g < 4; g++) mb[g] = (mt >> (8 * g)) & 0xFFu;
            } else {
                mask_bytes(R.mw, lane, mb);
            }
            if (VEC && cc == K - 1) clear_tail(mb);
            float m, s;
            bool any;
            reduce_chunk<DT>(R, mb, lut, kk, m, s, any);
            if (lane == 0) {
                ci[cc].s = s;
                ci[cc].m = m;
                ci[cc].any = any ? 1 : 0;
            }
            if (!stash || !any) return;
            const float score =
                greedy ? m : (s > 0.f ? m * invTf + 0.69314718f * __builtin_amdgcn_logf(s) + ci[cc].g : -INFINITY);
            if (score > best) {
                best = score;
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    if (DT == 1) {
                        *(uint4 *)&st->d[wave][g * 256 + lane * 4] =
                            make_uint4(R.d[g * 4], R.d[g * 4 + 1], R.d[g * 4 + 2], R.d[g * 4 + 3]);
                    } else {
#pragma unroll
                        for (int h = 0; h < 2; h++)
                            *(uint4 *)&st->d[wave][g * 512 + lane * 8 + 4 * h] =
                                make_uint4(R.d[g * 8 + 4 * h], R.d[g * 8 + 4 * h + 1], R.d[g * 8 + 4 * h + 2],
                                           R.d[g * 8 + 4 * h + 3]);
                    }
                }
                st->mb[wave][lane] = mb[0] | mb[1] << 8 | mb[2] << 16 | mb[3] << 24;
                if (lane == 0) st->c[wave] = cc;
            }
        };
        // Each wave's first NB chunks are w, w + 16, ...; after that a wave
        // takes the next chunk from the counter in LDS as it starts reducing
        // one (the ticket's round trip hides behind the reduction), so the
        // row's last chunks go to the waves that are ahead rather than
        // queueing behind a wave that drew slow loads.  (With two or more
        // buffers every path issues the same loads, past the row's end
        // included -- clamped, read as zeros without touching memory -- so
        // the compiler's waits count exactly the loads behind each chunk; a
        // single buffer waits for everything it has and skips the load past
        // the end.)
        int cur[NB];
#pragma unroll
        for (int b = 0; b < NB; b++) cur[b] = wave + b * kWaves;
        auto pending = [&]() {
            bool p = false;
#pragma unroll
            for (int b = 0; b < NB; b++) p |= cur[b] < Kf;
            return p;
        };
        while (pending()) {
#pragma unroll
            for (int b = 0; b < NB; b++) {
                if (NB > 1 && cur[b] >= Kf) continue;  // this buffer is done; the others are not
                int nxt = 0;
                if (lane == 0) nxt = atomicAdd(&next_chunk, 1);
                process(buf[b], cur[b]);
                nxt = __builtin_amdgcn_readfirstlane(nxt);
                if (NB > 1 || nxt < Kf) load(buf[b], nxt);
                cur[b] = nxt;
            }
        }
        // rows not 16-byte aligned: every chunk, bounds-checked
        for (c = Kf > 0 ? K : wave; c < K; c += kWaves) {
            load_chunk<DT, VEC>(buf[0], logits, rowbase, mrow, V, c, lane);
            process(buf[0], c);
        }
    }
    // the table to LDS, made visible by the barrier after the decision
    if (fuse) {
#pragma unroll
        for (int j = 0; j < kStageRegs; j++) {
            const uint32_t i = j * blockDim.x + threadIdx.x;
            if (i < treg) lds_comb[i] = tv[j];
        }
    }
    __syncthreads();
    // ---- the row's decision: three independent reductions over the chunk
    // summaries (lane j takes chunks j, j + 64, ...) on waves 13..15 at once:
    // (0) the log-normaliser over the chunk log-masses L_c = m/T + ln s (ln
    // from v_log_f32: the chunk sums carry ~1e-6 of float rounding anyway),
    // (1) the largest allowed logit and the lowest chunk holding it, (2) the
    // two best chunk scores L_c + G(1, c).  Meanwhile the eight token waves
    // (0..7) work out the chunk choice themselves, with the same code on the
    // same summaries ((1) for greedy rows, (2) for sampled ones), and start
    // the pick inside that chunk; the decision's barrier is also the pick's.
    // Only when the exact recheck of two close chunks moves the choice (or
    // the waves' choices differ) is the pick made again.
    constexpr int kTokWaves = kChunk / 4 / 64;  // 4 ids (one Philox block) per thread
    constexpr int kDecWave = kWaves - 3;
    static_assert(kDecWave >= kTokWaves, "the reducing waves are not token waves");
    const bool tok = wave < kTokWaves;
    const int t = threadIdx.x;
    auto lmass = [&](const ChunkInfo &x) -> double {
        return (x.any && x.s > 0.f) ? (double)x.m * invT + kLn2d * (double)__builtin_amdgcn_logf(x.s) : -INFINITY;
    };
    // (1): the largest allowed logit and the lowest chunk holding it (-1:
    // nothing allowed, or every allowed logit is -inf)
    auto chunk_max = [&](float &mv_out, int &mc_out) {
        float mv = -INFINITY;
        int mc = -1;
        for (int cc = lane; cc < K; cc += 64) {
            const ChunkInfo x = ci[cc];
            if (x.any && x.m > mv) {  // chunks in increasing order: ties keep the lowest
                mv = x.m;
                mc = cc;
            }
        }
        const float m = wave_max_f(mv);
        const int c = wave_min_i_fast((mc >= 0 && mv == m) ? mc : 0x7FFFFFFF);
        mv_out = m;
        mc_out = m > -INFINITY ? c : -1;
    };
    // (2): the best chunk score, the lowest chunk holding it, the best of the rest
    auto chunk_top2 = [&](double &v1_out, int &c1_out, double &v2_out) {
        Top2d cs{-INFINITY, -INFINITY, -1};
        for (int cc = lane; cc < K; cc += 64) {
            const double l = lmass(ci[cc]);
            if (l > -INFINITY) top2d_merge(cs, l + (double)ci[cc].g, cc, -INFINITY);
        }
        const double v1 = wave_max_d_fast(cs.v1);
        int c1 = wave_min_i_fast((cs.i1 >= 0 && cs.v1 == v1) ? cs.i1 : 0x7FFFFFFF);
        if (c1 == 0x7FFFFFFF) c1 = -1;
        v1_out = v1;
        c1_out = c1;
        v2_out = wave_max_d_fast(cs.i1 == c1 ? cs.v2 : cs.v1);
    };
    if (wave == kDecWave) {
        double lmax = -INFINITY;
        float lsum = 0.f;
        for (int cc = lane; cc < K; cc += 64) {
            const double l = lmass(ci[cc]);
            if (!(l > -INFINITY)) continue;
            if (l > lmax) {
                lsum = lsum * __builtin_amdgcn_exp2f((float)((lmax - l) * kLog2ed)) + 1.f;
                lmax = l;
            } else {
                lsum += __builtin_amdgcn_exp2f((float)((l - lmax) * kLog2ed));
            }
        }
        const double L = wave_max_d_fast(lmax);
        const float tt =
            wave_sum_f(lmax > -INFINITY ? lsum * __builtin_amdgcn_exp2f((float)((lmax - L) * kLog2ed)) : 0.f);
        if (lane == 0) wdec.lse_all = L > -INFINITY ? L + kLn2d * (double)__builtin_amdgcn_logf(tt) : -INFINITY;
    } else if (wave == kDecWave + 1) {
        float m;
        int c;
        chunk_max(m, c);
        if (lane == 0) {
            wdec.mv = m;
            wdec.mc = c;
        }
    } else if (wave == kDecWave + 2 && !greedy) {
        double v1, v2;
        int c1;
        chunk_top2(v1, c1, v2);
        if (lane == 0) {
            wdec.c1 = c1;
            wdec.cs1 = v1;
            wdec.cs2 = v2;
        }
    }
    // (3) inside a chunk: the token waves' threads take 4 ids each, e = 4t ..
    // 4t + 3 (one Philox block), from the stash of the wave that reduced the
    // chunk, else from HBM.  Eight waves, not sixteen: the Philox rounds
    // dominate and cost per wave, whatever the ids per lane.  Each token
    // wave leaves its best id (greedy: the lowest id holding the largest
    // logit mv; sampled: the top two of x/T + G(0, i) screened in float) in
    // its slot, and the chunk it worked on.
    int e = 0, ws = 0;
    // Each token wave keeps its candidate and fetches that token's bytes
    // right after the decision's barrier (lane j < nw: word j, lane
    // kInfoLane: the summary word), while the candidates are merged into
    // the pick; the wave that holds the pick then commits it with the bytes
    // in registers.  (Issued before the barrier, the fetch would be waited
    // for there.)
    constexpr int kInfoLane = kMaxTokenLen / 4;
    int pre_id = -1;
    uint32_t pre_w = 0u;
    bool from_stash = false;
    float xq[4] = {0.f, 0.f, 0.f, 0.f};
    uint32_t mb4 = 0;  // mask bits of e .. e + 3
    uint32_t wq[4] = {0u, 0u, 0u, 0u};
    const float it = greedy ? 0.f : 1.0f / Tf;
    auto tok_phase = [&](int ch, float mv) {  // token waves only
        e = ch * kChunk + 4 * t;
        // the wave whose stash holds the chunk, if any (lanes 0..15 read one
        // stash tag each)
        const uint64_t held = stash ? __ballot(lane < kWaves && st->c[lane & (kWaves - 1)] == ch) : 0ull;
        ws = held ? (int)__builtin_ctzll(held) : 0;
        from_stash = held != 0ull;
        mb4 = 0;
        if (from_stash) {
            if (DT == 1) {
                const uint2 dw = *(const uint2 *)&st->d[ws][2 * t];
                xq[0] = __uint_as_float(dw.x << 16);
                xq[1] = __uint_as_float(dw.x & 0xFFFF0000u);
                xq[2] = __uint_as_float(dw.y << 16);
                xq[3] = __uint_as_float(dw.y & 0xFFFF0000u);
            } else {
                const uint4 dw = *(const uint4 *)&st->d[ws][4 * t];
                xq[0] = __uint_as_float(dw.x);
                xq[1] = __uint_as_float(dw.y);
                xq[2] = __uint_as_float(dw.z);
                xq[3] = __uint_as_float(dw.w);
            }
            const int li = 4 * t;
            mb4 = (st->mb[ws][(li & 511) >> 3] >> (8 * (li >> 9) + (li & 7))) & 15u;
        } else {
#pragma unroll
            for (int j = 0; j < 4; j++) {
                xq[j] = 0.f;
                if (e + j < V) {
                    xq[j] = load_logit<DT>(logits, rowbase + e + j);
                    mb4 |= ((mrow[(e + j) >> 3] >> ((e + j) & 7)) & 1u) << j;
                }
            }
        }
        if (greedy) {
            int im = 0x7FFFFFFF;
#pragma unroll
            for (int j = 3; j >= 0; j--)
                if (((mb4 >> j) & 1u) && xq[j] == mv) im = e + j;
            im = wave_min_i_fast(im);
            pre_id = im;
            if (lane == 0) sl[2].i[wave] = im;
        } else {
            uint4 o = make_uint4(0, 0, 0, 0);
            if (mb4) o = philox4x32_10(make_uint4((uint32_t)e >> 2, stp, 0u, 0u), k0, k1);
            wq[0] = o.x;
            wq[1] = o.y;
            wq[2] = o.z;
            wq[3] = o.w;
            Top2 ts{-INFINITY, -INFINITY, -1};
#pragma unroll
            for (int j = 0; j < 4; j++)
                if ((mb4 >> j) & 1u) top2_merge(ts, xq[j] * it + gumbel32(wq[j]), e + j, -INFINITY);
            ts = top2_wave_fast(ts);
            pre_id = ts.i1;
            if (lane == 0) {
                sl[2].f[wave] = ts.v1;
                sl[2].h[wave] = ts.v2;
                sl[2].i[wave] = ts.i1;
            }
        }
        if (lane == 0) sl[2].j[wave] = ch;
    };
    if (tok) {
        float smv = 0.f;
        int spec;
        if (greedy) {
            chunk_max(smv, spec);
        } else {
            double v1, v2;
            chunk_top2(v1, spec, v2);
        }
        if (spec >= 0) tok_phase(spec, smv);
        else if (lane == 0) sl[2].j[wave] = -1;
    }
    if (tn > treg) stage_table(lds_comb, adv.comb, tn, treg);
    if (fuse && wave == 0 && lane < 6) cur_w[lane] = stw;  // fetched at the start
    // each lane's address of its part of the candidate's token, worked out
    // here, so that no kernel argument is read between the barrier and the
    // merge (a scalar read would share the merge's LDS wait)
    const uint32_t *pre_p = nullptr;
    if (fuse && tok && pre_id >= 0 && pre_id < adv.V)
        pre_p = lane < adv.nw ? adv.tokw + (size_t)lane * adv.V + pre_id : lane == kInfoLane ? adv.tokinfo + pre_id : nullptr;
    __syncthreads();  // the decision, the table and the token waves' slots
    dc.lse_all = wdec.lse_all;
    dc.mv = wdec.mv;
    dc.mc = wdec.mc;
    dc.chosen = greedy ? wdec.mc : wdec.c1;
    dc.exact_chunk = !greedy && wdec.c1 >= 0 && !(wdec.cs1 - wdec.cs2 > kContendChunk);
    dc.cs1 = wdec.cs1;
    // the wave that holds the pick (its 256-id part of the chosen chunk)
    // publishes and commits it; wave 0 when nothing is picked
    int cw = 0;
    do {
    if (dc.mc < 0) break;  // nothing allowed: a finished row
    if (dc.exact_chunk) {
        // two chunks within the screening window: decide on exact log-masses
        // and noise in double (rare)
        double bb = -INFINITY;
        int bbc = -1;
        for (int c = 0; c < K; c++) {
            const ChunkInfo x = ci[c];
            if (!x.any || !(x.s > 0.f)) continue;
            const double l = (double)x.m * invT + kLn2d * (double)__builtin_amdgcn_logf(x.s);
            if (l + (double)x.g < dc.cs1 - 2 * kContendChunk) continue;
            const uint4 o = philox4x32_10(make_uint4((uint32_t)c >> 2, stp, 1u, 0u), k0, k1);
            arg_better(bb, bbc,
                       chunk_lse_exact<DT>(logits, rowbase, mrow, V, c, T, (double)x.m, sl[1].a) +
                           gumbel64(pick_word(o, c & 3)),
                       c);
        }
        dc.chosen = bbc;  // every thread computed the same
    }
    const int chosen = dc.chosen;
    if (chosen < 0) break;  // every allowed logit is -inf: no distribution to draw from
    bool again = false;  // (the same for every thread: read from LDS)
#pragma unroll
    for (int k = 0; k < kTokWaves; k++) again |= sl[2].j[k] != chosen;
    if (again) {
        __syncthreads();  // every slot read above
        if (tok) tok_phase(chosen, dc.mv);
        __syncthreads();
    }
    if (again)  // the candidates were picked again
        pre_p = !(fuse && tok && pre_id >= 0 && pre_id < adv.V) ? nullptr
                : lane < adv.nw                                  ? adv.tokw + (size_t)lane * adv.V + pre_id
                : lane == kInfoLane                              ? adv.tokinfo + pre_id
                                                                 : nullptr;
    if (pre_p) pre_w = *pre_p;  // the candidate's token
    auto x_of = [&](int id) -> float {  // logit of an id of the chosen chunk (a token-wave thread)
        const int li = id - chosen * kChunk;
        if (from_stash) {
            if (DT == 0) return __uint_as_float(st->d[ws][li]);
            const uint32_t dw = st->d[ws][li >> 1];
            return __uint_as_float((li & 1) ? (dw & 0xFFFF0000u) : (dw << 16));
        }
        return load_logit<DT>(logits, rowbase + id);
    };
    auto holder = [&](int id) {
        const int li = id - chosen * kChunk;
        return (li >= 0 && li < kChunk) ? li >> 8 : 0;
    };
    if (greedy) {
        int best = sl[2].i[0];
#pragma unroll
        for (int w = 1; w < kTokWaves; w++) best = min(best, sl[2].i[w]);
        pick = best;
        pick_lp = (float)((double)dc.mv - dc.lse_all);
        cw = holder(best);
        break;
    }
    // sampled: argmax_i x_i / T + G(0, i) screened in float; the winner is
    // exact unless the best two are within the screening error (x/T rounding
    // < 1e-6 |x/T|, G < 1e-5), in which case the contenders are recomputed.
    // Every wave merges the token waves' top two (slot loads first, then the
    // merges).
    float sv1[kTokWaves], sv2[kTokWaves];
    int si1[kTokWaves];
#pragma unroll
    for (int k = 0; k < kTokWaves; k++) {
        sv1[k] = sl[2].f[k];
        sv2[k] = sl[2].h[k];
        si1[k] = sl[2].i[k];
    }
    Top2 tt{sv1[0], sv2[0], si1[0]};
#pragma unroll
    for (int k = 1; k < kTokWaves; k++) top2_merge(tt, sv1[k], si1[k], sv2[k]);
    const double win = 1e-4 + 2e-6 * fabs((double)tt.v1);
    if ((double)tt.v1 - (double)tt.v2 > win) {
        pick = tt.i1;
        cw = holder(pick);
        if ((int)threadIdx.x == cw * 64) pick_lp = (float)((double)x_of(pick) * invT - dc.lse_all);
        break;
    }
    // contenders recomputed in double (rare)
    double tv = -INFINITY;
    int ti = -1;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        if (!((mb4 >> j) & 1u)) continue;
        if ((double)(xq[j] * it + gumbel32(wq[j])) >= (double)tt.v1 - win)
            arg_better(tv, ti, (double)xq[j] / T + gumbel64(wq[j]), e + j);
    }
    if (tok) {
        wave_argmax(tv, ti);
        if (lane == 0) {
            sl[3].b[wave] = tv;
            sl[3].j[wave] = ti;
        }
    }
    __syncthreads();
    {
        double v = sl[3].b[0];
        int i = sl[3].j[0];
        for (int k = 1; k < kTokWaves; k++) arg_better(v, i, sl[3].b[k], sl[3].j[k]);
        pick = i;
        cw = holder(pick);
        if ((int)threadIdx.x == cw * 64) pick_lp = (float)((double)x_of(pick) * invT - dc.lse_all);
    }
    } while (0);
    // ---- epilogue: lane 0 of wave cw publishes the pick and, fused, commits it
    uint32_t pw[kInfoLane + 1];  // the wave's fetched token (whole waves read their lanes)
#pragma unroll
    for (int j = 0; j <= kInfoLane; j++) pw[j] = (uint32_t)__builtin_amdgcn_readlane((int)pre_w, j);
    if ((int)threadIdx.x == cw * 64) {
        out_id[r] = pick;
        out_lp[r] = pick_lp;
        if (fuse) {
            cg_state row_state;
            uint32_t w6[6];
#pragma unroll
            for (int j = 0; j < 6; j++) w6[j] = cur_w[j];
            __builtin_memcpy(&row_state, w6, sizeof(w6));
            uint32_t words[kMaxTokenLen / 4];
            uint32_t n = 0;
#pragma unroll
            for (int j = 0; j < kMaxTokenLen / 4; j++) words[j] = 0;
            if (pick >= 0 && pick < adv.V) {
                if (pick == pre_id) {  // fetched with the candidate
                    n = tok_len(pw[kInfoLane]);
#pragma unroll
                    for (int j = 0; j < kMaxTokenLen / 4; j++) words[j] = pw[j];
                } else {
                    n = tok_len(adv.tokinfo[pick]);
#pragma unroll
                    for (int j = 0; j < kMaxTokenLen / 4; j++)
                        if (j < adv.nw) words[j] = adv.tokw[(size_t)j * adv.V + pick];
                }
            }
            int stp1 = (int)stp;
            const int res =
                commit_token(row_state, stp1, pick, adv.V, n, words, lds_comb, adv.k, adv.gen_cap, adv.forced);
            if (token_taken(res)) {
                adv.states[r] = row_state;
                adv.steps[r] = stp1;
            }
            adv.status[r] = res;
            next_state = row_state;  // unchanged unless the token was taken
        }
    }
    if (!plan_next) return;
    // the next mask of this row, from the committed state; every read of
    // the row's current mask is done (the pick has been made)
    __syncthreads();
    plan_row(pa, r, next_state, lds_comb, psh);
}

// ---------------------------------------------------------------------------
// launcher (argument checks are done by the C ABI)
// ---------------------------------------------------------------------------
size_t sample_workspace_bytes(int B, int V) {
    (void)B;
    (void)V;
    return 0;  // partials live in LDS
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex dev_mu;
int dev_lds_max[kMaxDevices];         // 0: not asked yet
int sample_lds_attr[kMaxDevices][16];  // k_sample<dtype, vec, nt, sparse>'s dynamic-LDS limit as raised (0: default)

// LDS a workgroup may use on a device, asked once per device
int lds_max_of(int dev) {
    std::lock_guard<std::mutex> lk(dev_mu);
    if (dev < 0 || dev >= kMaxDevices) return 65536;
    if (!dev_lds_max[dev]) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || v <= 0)
            v = 65536;
        dev_lds_max[dev] = v;
    }
    return dev_lds_max[dev];
}

// Raise a kernel's dynamic-LDS limit on a device only when a launch needs
// more than it was last raised to (a grammar's launches all need the same
// amount): no host call on the per-step path.
int raise_lds_limit(const void *kern, int dev, int which, size_t lds) {
    std::lock_guard<std::mutex> lk(dev_mu);
    const bool known = dev >= 0 && dev < kMaxDevices;
    if (known && (size_t)sample_lds_attr[dev][which] >= lds) return CG_OK;
    if (hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return launch_status("apply_mask_sample (LDS attribute)");
    if (known) sample_lds_attr[dev][which] = (int)lds;
    return CG_OK;
}
}  // namespace

int launch_sample(const void *logits, int dt, int B, int V, int64_t stride, const uint64_t *mask, int wpr,
                  const float *temp, const uint64_t *seed, const int32_t *step, void *ws, int32_t *out_id,
                  float *out_lp, const cg_grammar *g, cg_state *states, int32_t *steps_rw, int32_t *status,
                  hipStream_t st, const FillArgs *plan) {
    (void)ws;
    if (B == 0) return CG_OK;
    const int K = (V + kChunk - 1) / kChunk;
    constexpr int kMaxChunks = 2048;  // 32 KiB of chunk summaries
    const size_t lds_ci = (size_t)K * sizeof(ChunkInfo);
    if (K > kMaxChunks) {
        set_error("apply_mask_sample: vocab above %d", kMaxChunks * kChunk);
        return CG_E_ARG;
    }
    // the device and its LDS size: the grammar's (asked when it was compiled),
    // else asked once per device
    int dev = 0, lds_max = 65536;
    if (g) {
        dev = g->device;
        lds_max = g->lds_max;
    } else {
        if (hipGetDevice(&dev) != hipSuccess) return launch_status("apply_mask_sample (device)");
        lds_max = lds_max_of(dev);
    }
    const size_t static_lds =
        4 * sizeof(Slots) + 256 * sizeof(uint4) + sizeof(RowDecision) + sizeof(PlanShared) + sizeof(cg_state) + 256;
    const size_t table = g ? (size_t)g->comb_len * 8 : 0;
    // each wave's best chunk is kept in LDS when it fits beside the table
    const size_t stash_bytes = dt == 1 ? sizeof(Stash<1>) : sizeof(Stash<0>);
    const int use_stash = stash_offset(K) + stash_bytes + table + static_lds <= (size_t)lds_max;
    const size_t base = use_stash ? stash_offset(K) + stash_bytes : (lds_ci + 15) / 16 * 16;
    const size_t lds = base + table;
    if (lds + static_lds > (size_t)lds_max) {
        set_error("sample_advance: %zu bytes of LDS needed, %d available", lds + static_lds, lds_max);
        return CG_E_LIMIT;
    }
    AdvanceArgs adv{};
    if (g) {
        adv.comb = g->dev.comb;
        adv.comb_len = g->comb_len;
        adv.comb_off = (uint32_t)base;
        adv.k = g->k;
        adv.tokw = g->dev.tokw;
        adv.tokinfo = g->dev.tokinfo;
        adv.nw = g->nw;
        adv.V = g->V;
        adv.states = states;
        adv.steps = steps_rw;
        adv.status = status;
        adv.gen_cap = g->gen_cap;
        adv.forced = g->dev.forced;
    }
    static_assert(kWaves * 64 == kPlanThreads, "the plan runs on the sampler's workgroup");
    const FillArgs pa = plan ? *plan : FillArgs{};
    const int plan_next = (plan && g) ? 1 : 0;
    const int es = dt == 0 ? 4 : 2;
    const bool vec = ((uintptr_t)logits % 16 == 0) && ((stride * es) % 16 == 0);
    const bool nt = (size_t)B * (size_t)V * (size_t)es > kStreamBytes;
    // the row's mask staged in LDS for the sparse stream: aligned rows with
    // more chunks than waves (a wave's first chunk is read whole, so with
    // fewer the staging saves nothing), when it fits after the table
    const size_t moff = (lds + 15) / 16 * 16;
    const bool sp = vec && K > kWaves && K <= 64 * kMaskPieces &&
                    moff + (size_t)K * 256 + static_lds <= (size_t)lds_max;
    const size_t lds_all = sp ? moff + (size_t)K * 256 : lds;
#define CG_LAUNCH_SAMPLE(D, VV, NN, SS)                                                                          \
    do {                                                                                                         \
        if (lds_all > 64 * 1024) {                                                                               \
            const int rc = raise_lds_limit((const void *)k_sample<D, VV, NN, SS>, dev,                           \
                                           8 * ((SS) ? 1 : 0) + 4 * ((NN) ? 1 : 0) + 2 * (D) + ((VV) ? 1 : 0),    \
                                           lds_all);                                                             \
            if (rc != CG_OK) return rc;                                                                          \
        }                                                                                                        \
        hipLaunchKernelGGL((k_sample<D, VV, NN, SS>), dim3(B), dim3(kWaves * 64), lds_all, st, logits, V,       \
                           stride, mask, wpr, temp, seed, step, K, use_stash, (int)moff, out_id, out_lp, adv, pa, \
                           plan_next);                                                                           \
    } while (0)
#define CG_LAUNCH_SAMPLE_NT(D, VV, SS)              \
    do {                                            \
        if (nt) CG_LAUNCH_SAMPLE(D, VV, true, SS);  \
        else CG_LAUNCH_SAMPLE(D, VV, false, SS);    \
    } while (0)
    if (dt == 0) {
        if (sp) CG_LAUNCH_SAMPLE_NT(0, true, true);
        else if (vec) CG_LAUNCH_SAMPLE_NT(0, true, false);
        else CG_LAUNCH_SAMPLE_NT(0, false, false);
    } else {
        if (sp) CG_LAUNCH_SAMPLE_NT(1, true, true);
        else if (vec) CG_LAUNCH_SAMPLE_NT(1, true, false);
        else CG_LAUNCH_SAMPLE_NT(1, false, false);
    }
#undef CG_LAUNCH_SAMPLE_NT
#undef CG_LAUNCH_SAMPLE
    return launch_status(g ? "sample_advance" : "apply_mask_sample");
}

}  // namespace cg
