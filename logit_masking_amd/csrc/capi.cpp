// capi.cpp -- the C ABI (include/cg.h): argument checks, device upload, and
// the host walker behind cg_try_input.
#include <string.h>

#include <algorithm>
#include <vector>

#include "cg_internal.hpp"

namespace cg {
const char *last_error();
int launch_init(const cg_grammar *g, cg_state *states, int B, hipStream_t st);
int launch_advance(const cg_grammar *g, cg_state *states, int B, const int32_t *ids, int32_t *steps,
                   int32_t *status, hipStream_t st);
int launch_fill(const cg_grammar *g, const cg_state *states, int B, uint64_t *mask, int wpr, hipStream_t st);
size_t sample_workspace_bytes(int B, int V);
int launch_sample(const void *logits, int dt, int B, int V, int64_t stride, const uint64_t *mask, int wpr,
                  const float *temp, const uint64_t *seed, const int32_t *step, void *ws, int32_t *out_id,
                  float *out_lp, hipStream_t st);
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

}  // namespace

extern "C" {

int cg_compile_grammar(const char *spec_json, size_t spec_len, const uint8_t *tok_bytes, const uint32_t *tok_offsets,
                       int32_t vocab_size, const cg_options *opts, cg_grammar **out) {
    if (!out) return arg_error("out is NULL");
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
        if (upload(&g->dev.comb, g->host_comb, g->comb_len) || upload(&g->dev.tokw, tokw.data(), tokw.size()) ||
            upload(&g->dev.tokinfo, tokinfo.data(), V)) {
            set_error("device upload failed: %s", hipGetErrorString(hipGetLastError()));
            release(g);
            return CG_E_DEVICE;
        }
    }
    *out = g;
    return CG_OK;
}

void cg_free_grammar(cg_grammar *g) { release(g); }

int cg_grammar_info(const cg_grammar *g, cg_info *info) {
    if (!g || !info) return arg_error("NULL argument");
    info->vocab_size = g->V;
    info->words_per_row = (g->V + 63) / 64;
    info->max_token_len = g->max_len;
    info->n_states = g->n_states;
    info->table_entries = (int32_t)g->comb_len;
    info->table_bytes = (int32_t)(g->comb_len * sizeof(uint64_t));
    info->compile_ms = g->compile_ms;
    return CG_OK;
}

int cg_init_state(const cg_grammar *g, cg_state *d_states, int32_t batch, void *stream) {
    if (!on_device(g)) return arg_error("grammar has no device tables");
    if (batch < 0 || (batch > 0 && !d_states)) return arg_error("bad states / batch");
    return launch_init(g, d_states, batch, (hipStream_t)stream);
}

int cg_fill_bitmask(const cg_grammar *g, const cg_state *d_states, int32_t batch, uint64_t *d_mask,
                    int32_t words_per_row, void *stream) {
    if (!on_device(g)) return arg_error("grammar has no device tables");
    if (batch < 0 || (batch > 0 && (!d_states || !d_mask))) return arg_error("bad states / mask / batch");
    if (words_per_row < (g->V + 63) / 64) return arg_error("words_per_row < ceil(vocab_size / 64)");
    return launch_fill(g, d_states, batch, d_mask, words_per_row, (hipStream_t)stream);
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
                         d_step, d_workspace, d_out_ids, d_out_logprob, (hipStream_t)stream);
}

int cg_advance(const cg_grammar *g, cg_state *d_states, int32_t batch, const int32_t *d_token_ids, int32_t *d_step,
               int32_t *d_status, void *stream) {
    if (!on_device(g)) return arg_error("grammar has no device tables");
    if (batch < 0 || (batch > 0 && (!d_states || !d_token_ids || !d_step || !d_status)))
        return arg_error("bad arguments");
    return launch_advance(g, d_states, batch, d_token_ids, d_step, d_status, (hipStream_t)stream);
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
        if (!step_byte(w, bytes[i], g->host_comb, g->k)) break;
    *refused_at = i;
    *complete = (i == len && w.q == g->k.accept) ? 1 : 0;
    return CG_OK;
}

const char *cg_last_error(void) { return last_error(); }

}  // extern "C"
