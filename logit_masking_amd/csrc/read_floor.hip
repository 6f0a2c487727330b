// read_floor.hip -- the memory floor of the masked-sample launch, for the
// bench: the same grid (one 1024-thread workgroup per row), the same chunk
// walk (wave w streams the row's 2048-id chunks w, w + 16, ... with buffer
// loads, one dword of mask per lane per chunk) and the same bytes (every
// logit and this step's mask words read, a mask's worth of words written),
// with no arithmetic beyond folding the loaded words into one value.  Four
// chunks per wave in flight: the depth at which this pattern alone reads
// fastest (two for float32 rows, whose chunks take twice the registers).
// Built as its own library; nothing in libcg uses it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kChunk = 2048;  // ids per chunk
constexpr int kWaves = 16;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format
// the sampler's cache policy rule: logits of a launch above 32 MB are read
// with the non-temporal hint, smaller ones with the default policy
constexpr size_t kStreamBytes = size_t(32) << 20;

__device__ __forceinline__ uint32_t fold(uint4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

// Chunk c of a row: 4 KB (bf16) or 8 KB (float32) of logits in 16-byte
// pieces, lane l taking the pieces l, l + 64, ..., and the chunk's 256 mask
// bytes as one dword per lane, which is also written to the output row.
template <int ES, bool NT>
__global__ __launch_bounds__(1024) void k_read_floor(const char *logits, int V, int64_t stride,
                                                     const uint64_t *mask, int wpr, uint64_t *out_mask) {
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = blockIdx.x;
    const int K = (V + kChunk - 1) / kChunk;
    constexpr int kPieces = kChunk * ES / 16 / 64;  // 16-byte pieces per lane per chunk
    constexpr int kInFlight = ES == 2 ? 4 : 2;
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc((void *)(logits + (size_t)r * stride * ES), (short)0, (V * ES + 3) & ~3,
                                          kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rm =
        __builtin_amdgcn_make_buffer_rsrc((void *)(mask + (size_t)r * wpr), (short)0, wpr * 8, kRsrcWord3);
    uint32_t *om = (uint32_t *)(out_mask + (size_t)r * wpr);
    uint4 d[kInFlight][kPieces];
    uint32_t mw[kInFlight];
    // chunk K (past the row) reads zeros without touching memory
    auto load = [&](int b, int c) {
        c = min(c, K);
#pragma unroll
        for (int p = 0; p < kPieces; p++)
            d[b][p] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, c * kChunk * ES + p * 1024 + lane * 16, 0, NT ? 2 : 0));
        mw[b] = __builtin_amdgcn_raw_buffer_load_b32(rm, c * 256 + lane * 4, 0, NT ? 2 : 0);
        __builtin_amdgcn_sched_barrier(0);
    };
    uint32_t acc = 0;
    int c = wave;
#pragma unroll
    for (int b = 0; b < kInFlight; b++) load(b, c + b * kWaves);
    for (; c < K; c += kInFlight * kWaves) {
#pragma unroll
        for (int b = 0; b < kInFlight; b++) {
            const int cc = c + b * kWaves;
            if (cc < K) {
#pragma unroll
                for (int p = 0; p < kPieces; p++) acc ^= fold(d[b][p]);
                const int wi = cc * 64 + lane;  // the dword's index in the mask row
                if (wi < 2 * wpr) om[wi] = mw[b];
            }
            load(b, cc + kInFlight * kWaves);
        }
    }
    // keeps the loads live; a row whose words fold to this constant writes
    // it into its own output row's first word
    if (acc == 0x9E3779B9u) om[0] = acc;
}

}  // namespace

// Reads B rows of V logits (es = 2: bf16, 4: float32; rows `stride`
// elements apart, 16-byte aligned) and their mask rows (wpr words each),
// writing a mask row's worth of words per row to out_mask (B x wpr words,
// device memory).  Returns 0, or 1 for arguments it does not take.
extern "C" int cg_floor_read_rows(const void *logits, int es, int B, int V, int64_t stride, const uint64_t *mask,
                                  int wpr, uint64_t *out_mask, void *stream) {
    if (B <= 0 || V <= 0 || (es != 2 && es != 4) || wpr * 64 < V || ((uintptr_t)logits % 16) != 0 ||
        ((stride * es) % 16) != 0)
        return 1;
    hipStream_t st = (hipStream_t)stream;
    const bool nt = (size_t)B * (size_t)V * (size_t)es > kStreamBytes;
#define CG_FLOOR(E, N)                                                                                        \
    hipLaunchKernelGGL((k_read_floor<E, N>), dim3(B), dim3(1024), 0, st, (const char *)logits, V, stride, mask, \
                       wpr, out_mask)
    if (es == 2) {
        if (nt) CG_FLOOR(2, true);
        else CG_FLOOR(2, false);
    } else {
        if (nt) CG_FLOOR(4, true);
        else CG_FLOOR(4, false);
    }
#undef CG_FLOOR
    return hipGetLastError() == hipSuccess ? 0 : 1;
}
