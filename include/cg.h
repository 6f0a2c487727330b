/*
 * cg.h -- C ABI of the constrained-decoding hot path on MI355X (gfx950).
 *
 * At every decode step a byte-level pushdown automaton masks the logits so
 * that only continuations legal under the grammar can be generated, and
 * sampling runs after masking ("Constrained decoding", section "The
 * guarantee").  The contract is a handful of calls over plain pointers and
 * sizes that name no model, tokenizer, device type or file ("Constrained
 * decoding", section "The guarantee is not tied to this engine").
 *
 *   cg_compile_grammar   spec + vocabulary -> automaton tables (host, once)
 *   cg_init_state        every row at the start of the grammar (device)
 *   cg_fill_bitmask      packed token bitmask per row (device)
 *   cg_apply_mask_sample masked softmax + greedy / Gumbel-max pick (device)
 *   cg_advance           walk the chosen tokens, update rows (device)
 *   cg_sample_advance    the last two in one launch (device)
 *   cg_sample_advance_fill  the same, then the next step's bitmask (device)
 *   cg_sample_advance_plan, cg_fill_walk  its two launches, one call each
 *   cg_fill_draft        masks along each row's k-token draft (device)
 *   cg_force_bytes       engine-written bytes (an evaluated result) (device)
 *   cg_eval_calc         evaluate a calc span (host)
 *   cg_eval_strop        evaluate a string-operation span (host)
 *   cg_contract_model_spec  integer-string contract: the model-facing spec (host)
 *   cg_contract_reverse  the exact inverse, then validation (host)
 *   cg_try_input         where a candidate string is refused (host)
 *
 * Conventions
 *   - Device pointers ("d_") are HIP device memory owned by the caller.
 *     `stream` is a hipStream_t passed as void* (NULL = default stream).
 *   - Per-step calls are asynchronous on `stream`: they never synchronise,
 *     never allocate, never print.  Their return code reports argument and
 *     launch errors only; outcomes that depend on data (a refused forced
 *     token, a finished row) come back in device arrays.
 *   - Errors: a negative CG_E_* code; cg_last_error() then holds a message
 *     (thread-local), for compile errors with the JSON path of the offending
 *     part of the spec.
 *   - A compiled grammar is immutable and may be used from several streams
 *     at once; free it only after every stream using it has drained.
 */
#ifndef CG_H
#define CG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- error codes ---------------------------------------------------------- */
#define CG_OK 0
#define CG_E_ARG (-1)         /* bad argument (null pointer, size, dtype, handle) */
#define CG_E_PARSE (-2)       /* spec is not valid JSON / not a grammar spec */
#define CG_E_UNSUPPORTED (-3) /* construct outside the supported subset (fail closed) */
#define CG_E_LIMIT (-4)       /* automaton or vocabulary beyond a size limit */
#define CG_E_VOCAB (-5)       /* malformed vocabulary (offsets) */
#define CG_E_DEVICE (-6)      /* HIP runtime error (allocation, copy, launch) */
#define CG_E_EVAL (-7)        /* calc span: division by zero, or a value outside int64 */
#define CG_E_INVALID (-8)     /* contract: the generated text does not map onto the original schema */

/* ---- per-row status written by cg_advance --------------------------------- */
#define CG_ROW_OK 0       /* token accepted, row continues */
#define CG_ROW_DONE 1     /* token accepted, the row's bytes are now a complete member */
#define CG_ROW_CAPPED 2   /* token accepted, row reached the generation cap */
#define CG_ROW_REJECTED 3 /* token refused (illegal, out of range, or row finished); row unchanged */
#define CG_ROW_NOOP 4     /* token id -1 (or an empty forced string): nothing to do */
#define CG_ROW_INJECT 5   /* token accepted; the row now sits in a region the engine writes
                             (cg_force_bytes): its mask is empty until then */

/* ---- row state flags (cg_state.flags) ------------------------------------- */
#define CG_FLAG_DONE 1u
#define CG_FLAG_CAPPED 2u

/* options of cg_compile_grammar */
#define CG_HOST_ONLY 1u /* compile for cg_try_input only: nothing is uploaded */

typedef struct cg_grammar cg_grammar; /* opaque, library-owned */

typedef struct {
    uint32_t gen_cap; /* tokens per constrained generation; 0 means 2048
                         ("A valid call also has to end": the engine caps a
                         constrained generation at 2048 tokens) */
    uint32_t flags;   /* CG_HOST_ONLY or 0 */
} cg_options;

/*
 * One row's automaton configuration (24 bytes, plain data: a snapshot is a
 * copy).  Caller-allocated device memory, written only by cg_init_state and
 * cg_advance; the fields are the library's business.
 */
typedef struct {
    uint16_t q;     /* control state */
    uint16_t ret;   /* state to resume after the open string */
    uint32_t cnt;   /* code points still allowed in the open string */
    uint64_t stk;   /* container kinds of open any-JSON containers, bit 0 innermost */
    uint8_t depth;  /* containers on that stack */
    uint8_t ws;     /* length of the current whitespace run */
    uint8_t flags;  /* CG_FLAG_DONE | CG_FLAG_CAPPED */
    uint8_t pad0;
    uint32_t pad1;
} cg_state;

typedef struct {
    int32_t vocab_size;
    int32_t words_per_row;  /* ceil(vocab_size / 64) */
    int32_t max_token_len;  /* longest token, bytes (<= 32) */
    int32_t n_states;       /* control states after trimming */
    int32_t table_entries;  /* packed transition slots (8 bytes each) */
    int32_t table_bytes;    /* bytes of the transition table staged per workgroup */
    double compile_ms;      /* host time of parse + build + pack */
    int32_t state_masks;    /* states whose plain-configuration mask was computed once at
                               compile time (0: none, or the table would exceed 64 MiB) */
    int32_t pad;
    double total_ms;        /* the whole cg_compile_grammar call that built the handle: the
                               automaton, the vocabulary tables, the precomputed masks and
                               the upload (a cached handle keeps its first compile's time) */
    int64_t max_bytes;      /* longest member of the language in bytes when it is finite
                               (every string at its cap, every whitespace run at ws_max,
                               every optional key present), -1 when it is infinite (an
                               uncapped string, an array without maxItems, any-JSON values,
                               calc expressions, text): how long a constrained output can
                               get ("Constrained decoding", "A valid call also has to end") */
} cg_info;

/*
 * Compile a grammar spec against a vocabulary and upload the tables to the
 * current HIP device.
 *
 * spec_json/spec_len: UTF-8 JSON, one of
 *   {"kind":"calc", "int_min":0, "int_max":999, "ws_max":2, "depth_cap":16}
 *       the span "<calc>" W E W "</calc>", E := T (W op W T)*,
 *       T := INT | "(" W E W ")", op one of + - * /, INT canonical decimal in
 *       [int_min, int_max] ("Evaluator aware decoding", "This is a grammar
 *       problem");
 *   {"kind":"calc_text", "int_min":0, "int_max":999, "ws_max":2, "depth_cap":16}
 *       text with evaluated spans: TEXT* (CALC RESULT TEXT*)* "<end>", TEXT =
 *       LF or printable ASCII other than '<', CALC the span above, RESULT =
 *       "<result>" "-"? digit{1,20} "</result>" or "<result_error>" MSG
 *       "</result_error>" (MSG: printable ASCII other than '<') -- written by
 *       the engine (cg_force_bytes), never sampled: rows inside it have an
 *       empty mask ("Evaluator aware decoding", "A concrete prototype on
 *       llama.cpp");
 *       With "evaluators":["calc","strop"] (default ["calc"]) the text may
 *       also hold string-operation spans, "<strop>" NAME "(" ARGS ")"
 *       "</strop>" (see cg_eval_strop; string arguments are '"' printable
 *       ASCII other than '"', '\\' and '<' '"', integers "-"? 1-6 digits,
 *       W "," W between arguments), followed by "<result>" TEXT'
 *       "</result>" (TEXT': printable ASCII other than '<') or the error
 *       block ("Evaluator aware decoding", "Not just arithmetic: string
 *       operations");
 *   {"kind":"json_schema", "schema":{...}, settings...}
 *       a JSON value of the schema ("Guided Decoding & Structured-Output
 *       Reliability", "Design 1 -- base schema, validators-first ordering");
 *   {"kind":"tool_call", "tools":[{"name":N, "parameters":{object schema}}...]}
 *       N "(" args-object ")" -- the grammar arms at "name(" ("Constrained
 *       decoding", "Where it arms, and therefore where it stops").
 *   Settings (defaults in brackets): ws_max [4] longest whitespace run;
 *   open_string_cap [256] code points of a string without maxLength (null:
 *   uncapped); open_int_digits [20] digits of an integer without both
 *   bounds; depth_cap [16] open containers ({, [, or calc parentheses).
 *   ("A valid call also has to end": bounded whitespace and open fields.)
 *   Supported schema subset: type object/array/string/integer/number/
 *   boolean/null; properties (declared order is emitted order), required,
 *   additionalProperties:false (required whenever properties is given);
 *   string enum; maxLength; integer minimum/maximum; items; maxItems;
 *   anyOf whose alternatives start with different bytes; {} = any JSON
 *   value; the string pattern "^-?(0|[1-9][0-9]*)$" (a canonical signed
 *   integer, see cg_contract_model_spec).  Anything else -- $ref, any other
 *   pattern, format, oneOf, allOf, minItems,
 *   minLength, multipleOf, ... -- is refused with CG_E_UNSUPPORTED and its
 *   JSON path ("Constrained Decoding Under Matched Conditions", "What exists
 *   beyond the experiment": typed fail-closed refusals).
 * tok_bytes/tok_offsets/vocab_size: token t is tok_bytes[tok_offsets[t] ..
 *   tok_offsets[t+1]); offsets has vocab_size+1 non-decreasing entries
 *   starting at 0 (host memory, copied).  Empty tokens are never allowed.
 *   At most 32 bytes per token.
 * opts: may be NULL (gen_cap 2048, upload).
 * out: receives the handle.  Returns CG_OK or a CG_E_* code.
 * Compiled grammars are cached: a compile with the same spec text,
 * vocabulary, options and device returns the same read-only handle with one
 * more reference (cg_free_grammar drops one); up to 8 handles no one holds
 * are kept for later identical compiles ("Evaluator aware decoding", "Where
 * XGrammar-2 could take this": cross-grammar caching keeps repeated grammars
 * from costing compilation).  Thread-safe.
 */
int cg_compile_grammar(const char *spec_json, size_t spec_len, const uint8_t *tok_bytes,
                       const uint32_t *tok_offsets, int32_t vocab_size, const cg_options *opts, cg_grammar **out);

/* Drop one reference to a grammar; its memory is released when none is left
 * and it falls out of the cache.  NULL is ignored. */
void cg_free_grammar(cg_grammar *g);

/* Sizes of a compiled grammar. */
int cg_grammar_info(const cg_grammar *g, cg_info *info);

/* The grammar cache: live entries (held or idle), compiles answered from it,
 * compiles that built new tables.  cg_cache_clear releases every idle entry. */
int cg_cache_stats(int32_t *entries, int64_t *hits, int64_t *misses);
int cg_cache_clear(void);

/* Set d_states[0..batch) to the start of the grammar (flags cleared). */
int cg_init_state(const cg_grammar *g, cg_state *d_states, int32_t batch, void *stream);

/* Bytes of the workspace cg_fill_bitmask needs for `batch` rows of this
 * grammar (0 if batch < 1; 0 on a bad handle). */
size_t cg_fill_workspace_bytes(const cg_grammar *g, int32_t batch);

/*
 * Packed token bitmask: bit (t & 63) of d_mask[r * words_per_row + (t >> 6)]
 * is 1 iff row r is not finished and the bytes of token t are a legal
 * continuation of the row's bytes (the row's bytes followed by token t can
 * still be completed to a member) without taking a byte the engine writes
 * (a token may end where an engine-written region begins, not go into it;
 * a row inside one gets an all-zero row).  Pad bits past vocab_size are 0.
 * words_per_row must be >= ceil(vocab_size / 64); words beyond that are
 * left untouched.  Depends only on the states, so it may run before the
 * logits exist ("Evaluator aware decoding", "Why isn't this in production
 * APIs yet?": masks come from pure automaton state ahead of the step).
 * d_workspace: cg_fill_workspace_bytes(g, batch) bytes of device memory,
 *   16-byte aligned, owned by the caller (the per-row list of token tiles
 *   to walk); its contents need no initialisation and are scratch after the
 *   call.  Calls that share a workspace must not overlap.
 */
int cg_fill_bitmask(const cg_grammar *g, const cg_state *d_states, int32_t batch, uint64_t *d_mask,
                    int32_t words_per_row, void *d_workspace, void *stream);

/*
 * cg_fill_bitmask for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops that forbid allocation): the same
 * arguments without the workspace, the same masks.  The per-row tile lists
 * live in a device array inside the library, one per device, of
 * CG_FILL_NOALLOC_SCRATCH_BYTES; its address is taken when a grammar is
 * first compiled on that device.  Every call on a device shares that array,
 * so calls on one device must not overlap in time (two streams running
 * them at once race); the array needs no initialisation.
 * CG_E_LIMIT (nothing launched) when cg_fill_workspace_bytes(g, batch)
 * exceeds the array; CG_E_DEVICE if its address could not be taken.
 */
#define CG_FILL_NOALLOC_SCRATCH_BYTES (16u << 20)
int cg_fill_bitmask_noalloc(const cg_grammar *g, const cg_state *d_states, int32_t batch, uint64_t *d_mask,
                            int32_t words_per_row, void *stream);

/* Longest draft cg_fill_draft takes. */
#define CG_MAX_DRAFT 64

/* Bytes of the workspace cg_fill_draft needs (0 if batch < 1 or k out of range). */
size_t cg_draft_workspace_bytes(const cg_grammar *g, int32_t batch, int32_t k);

/*
 * Masks along a draft, for speculative decoding: row r has k draft tokens
 * d_draft[r * k + j] (-1 pads a shorter draft).  The draft is walked from
 * the row (cg_advance's rules, with d_step for the cap; d_step may be NULL
 * for steps of 0) and position j = 0..k gets the row's configuration after
 * the first j draft tokens, in d_path_states[r * (k + 1) + j], and its mask,
 * in d_masks[(r * (k + 1) + j) * words_per_row ...] (cg_fill_bitmask's
 * layout).  d_accept_len[r] = how many draft tokens in a row are legal; the
 * positions after them get empty masks (the configuration is marked
 * finished).  The target model's logits at position j are masked with mask j
 * and a verifier keeps a prefix of at most d_accept_len[r] tokens; the row
 * then takes d_path_states at the kept length (and d_step += that length).
 * The rows themselves are not changed.  "Evaluator aware decoding", "Where
 * XGrammar-2 could take this": speculative pipelines verify drafts along
 * forced-token paths; every position is masked by the automaton's state
 * there.
 * k <= CG_MAX_DRAFT; d_workspace: cg_draft_workspace_bytes(g, batch, k)
 * bytes, 16-byte aligned, scratch.
 */
int cg_fill_draft(const cg_grammar *g, const cg_state *d_states, const int32_t *d_step, int32_t batch,
                  const int32_t *d_draft, int32_t k, cg_state *d_path_states, uint64_t *d_masks,
                  int32_t words_per_row, int32_t *d_accept_len, void *d_workspace, void *stream);

/* Bytes of the workspace cg_apply_mask_sample needs for (batch, vocab) (0 if batch or vocab < 1). */
size_t cg_sample_workspace_bytes(int32_t batch, int32_t vocab);

/*
 * Masked softmax and pick, per row r:
 *   logits x = d_logits[r * row_stride + t], t < vocab (dtype 0: float32,
 *   1: bfloat16); allowed = mask bit; T = d_temperature[r].
 *   T == 0: greedy, the allowed token of largest x (lowest id on ties),
 *     logprob = x_id - logsumexp_allowed(x).
 *   T > 0: a draw from softmax(x / T) restricted to the allowed tokens, by
 *     two-level Gumbel-max over chunks of 2048 ids: chunk c has log-mass
 *     L_c = logsumexp_{i in c, allowed}(x_i / T); the chunk is
 *     argmax_c L_c + G(1, c), then the token argmax_{i in chunk} x_i/T +
 *     G(0, i) (lowest index on ties), where G(l, i) = -ln(-ln u),
 *     u = (w + 1/2) 2^-32, and w is word (i & 3) of Philox4x32-10 (Salmon et
 *     al., SC'11) at counter (i >> 2, d_step[r], l, 0) with key d_seed[r]
 *     (low word first).  logprob = x_id / T - logsumexp_allowed(x / T).
 *   An allowed token whose logit is -inf carries no probability.  No allowed
 *   token of finite logit: id = -1, logprob = 0.
 * ("Constrained decoding", "The guarantee": sampling runs after masking.)
 * row_stride >= vocab elements; vocab <= 4,194,304 (2048 chunks).
 * d_workspace: cg_sample_workspace_bytes(batch, vocab) bytes, 16-byte
 *   aligned; may be NULL when that size is 0 (the sampler keeps every
 *   intermediate on chip, so it always is).
 * Outputs: d_out_ids[batch] int32, d_out_logprob[batch] float32.
 */
int cg_apply_mask_sample(const void *d_logits, int32_t dtype, int32_t batch, int32_t vocab, int64_t row_stride,
                         const uint64_t *d_mask, int32_t words_per_row, const float *d_temperature,
                         const uint64_t *d_seed, const int32_t *d_step, void *d_workspace, int32_t *d_out_ids,
                         float *d_out_logprob, void *stream);

/*
 * cg_apply_mask_sample followed by cg_advance on the picked ids, in one launch:
 * the same picks, log-probabilities, states, steps and statuses as the two
 * calls in sequence (vocab = the grammar's vocabulary).  d_step is read by
 * the sampler (Philox counter) and then incremented for accepted tokens.
 * The workgroup that picks a row's token also walks it, so the chosen id
 * never round-trips through memory between the two steps ("Constrained
 * decoding", "The guarantee": sampling runs after masking, and the sampled
 * token is the automaton's next transition).
 */
int cg_sample_advance(const cg_grammar *g, const void *d_logits, int32_t dtype, int32_t batch, int64_t row_stride,
                      const uint64_t *d_mask, int32_t words_per_row, const float *d_temperature,
                      const uint64_t *d_seed, int32_t *d_step, void *d_workspace, int32_t *d_out_ids,
                      float *d_out_logprob, cg_state *d_states, int32_t *d_status, void *stream);

/*
 * One decode step and the next step's bitmask: cg_sample_advance (same
 * arguments, same results), whose workgroups then plan each row's next mask
 * from the state they have just committed -- the base words and the token
 * tiles worth walking, the first part of cg_fill_bitmask -- followed by the
 * walk that completes it (two launches on `stream`).  The mask depends on
 * the automaton's state alone, so it is begun the moment the state is known
 * ("Evaluator aware decoding", "Why isn't this in production APIs yet?").
 * d_mask is read as this step's mask and rewritten in place: afterwards (in
 * stream order) it holds exactly what cg_fill_bitmask writes for the updated
 * states (words beyond ceil(vocab_size / 64) untouched).  d_fill_workspace:
 * as for cg_fill_bitmask (cg_fill_workspace_bytes(g, batch) bytes, 16-byte
 * aligned, no initialisation, scratch after the call).  The first step of a
 * batch takes its mask from cg_fill_bitmask.
 */
int cg_sample_advance_fill(const cg_grammar *g, const void *d_logits, int32_t dtype, int32_t batch,
                           int64_t row_stride, uint64_t *d_mask, int32_t words_per_row, const float *d_temperature,
                           const uint64_t *d_seed, int32_t *d_step, void *d_workspace, int32_t *d_out_ids,
                           float *d_out_logprob, cg_state *d_states, int32_t *d_status, void *d_fill_workspace,
                           void *stream);

/*
 * The two launches of cg_sample_advance_fill as calls of their own (so that
 * a caller may time them apart, or put other work between them): the first
 * (same arguments) samples, commits and plans, leaving d_mask holding the
 * next masks' base words and d_fill_workspace the token tiles to walk; the
 * second completes d_mask from those (the arguments of cg_fill_bitmask, with
 * the updated d_states and the same workspace).  Nothing may use d_mask or
 * the workspace between the two.
 */
int cg_sample_advance_plan(const cg_grammar *g, const void *d_logits, int32_t dtype, int32_t batch,
                           int64_t row_stride, uint64_t *d_mask, int32_t words_per_row, const float *d_temperature,
                           const uint64_t *d_seed, int32_t *d_step, void *d_workspace, int32_t *d_out_ids,
                           float *d_out_logprob, cg_state *d_states, int32_t *d_status, void *d_fill_workspace,
                           void *stream);
int cg_fill_walk(const cg_grammar *g, const cg_state *d_states, int32_t batch, uint64_t *d_mask,
                 int32_t words_per_row, void *d_workspace, void *stream);

/*
 * Walk d_token_ids[r] for every row: -1 is a no-op (CG_ROW_NOOP).  A token
 * whose bytes continue the row legally is committed: d_step[r] += 1, then
 * the row is DONE if its bytes form a complete member, CAPPED if
 * d_step[r] >= gen_cap, INJECT if it now sits where the engine writes (see
 * cg_force_bytes).  Otherwise (illegal, a byte the engine writes, id out of
 * range, or the row is already finished) the row is left unchanged and
 * d_status[r] is CG_ROW_REJECTED.  Ids may come from cg_apply_mask_sample or be forced by
 * the caller: a forced token is a transition the model did not choose
 * ("Evaluator aware decoding", "A concrete prototype on llama.cpp").
 * d_step: in/out, tokens accepted so far (the caller zeroes it at start).
 */
int cg_advance(const cg_grammar *g, cg_state *d_states, int32_t batch, const int32_t *d_token_ids, int32_t *d_step,
               int32_t *d_status, void *stream);

/*
 * Walk each row's forced byte string: row r takes
 * d_bytes[d_offsets[r] .. d_offsets[r+1]) (device memory, caller-owned;
 * d_bytes holds n_bytes bytes, d_offsets batch+1 entries).  An empty string
 * is a no-op (CG_ROW_NOOP); offsets out of order or past n_bytes give
 * CG_ROW_REJECTED with nothing read.  The engine
 * writes text the model did not choose -- an evaluated result -- and the
 * automaton follows: injection is a grammar transition the model did not
 * choose ("Evaluator aware decoding", "A concrete prototype on llama.cpp").
 * Engine-written bytes are legal here; text the model may write is too.
 * All bytes legal: the row takes the walked configuration and d_status[r]
 * is OK, DONE (a complete member), or INJECT (still inside a region the
 * engine writes).  A refused byte, or a finished row: CG_ROW_REJECTED, row
 * unchanged.  Forced bytes are not generation steps: the step counter and
 * the cap are untouched.  Tokenizing the forced text for the model's own
 * forward pass is the engine's business; the automaton walks bytes.
 */
int cg_force_bytes(const cg_grammar *g, cg_state *d_states, int32_t batch, const uint8_t *d_bytes, size_t n_bytes,
                   const uint32_t *d_offsets, int32_t *d_status, void *stream);

/*
 * Host-side evaluator of a calc span ("Evaluator aware decoding", "The core
 * idea": the engine evaluates the span and writes the result back).  `span`
 * is "<calc>...</calc>" or the bare expression: integers, + - * /,
 * parentheses, whitespace; * and / before + and -, left to right, / truncating
 * toward zero.  CG_OK with *value; CG_E_PARSE for a malformed span;
 * CG_E_EVAL for division by zero or any literal or intermediate value
 * outside int64, with cg_last_error() exactly "division by zero" or "out of
 * range" (text an engine can inject as <result_error>).
 */
int cg_eval_calc(const uint8_t *span, size_t len, int64_t *value);

/*
 * The integer-string contract ("Constrained Decoding Under Matched
 * Conditions", "The system boundary I am testing"): the caller's schema asks
 * for canonical signed-integer strings ({"type": "string", "pattern":
 * "^-?(0|[1-9][0-9]*)$"}), the model writes native JSON integers, and an
 * exact inverse maps them back before the result is checked against the
 * caller's schema.  Host only; off the per-step path.
 *
 * cg_contract_model_spec: ext_spec is a json_schema spec (cg_compile_grammar's
 * format); writes the model-facing spec -- every such string replaced by
 * {"type": "integer"} -- as compact JSON with a terminating zero into
 * out[cap] (*out_len = its length; CG_E_LIMIT and the needed length if cap is
 * too small) and the number of replaced fields into *n_fields.  The
 * model-facing spec is compiled once as a check (CG_E_UNSUPPORTED with the
 * path when it does not compile, e.g. an integer string beside another
 * numeric alternative of an anyOf).
 *
 * cg_contract_reverse: text is one generation under the model-facing spec.
 * Each integer where the original schema has an integer string becomes a
 * string holding the integer's text, digit for digit (no parsing: any
 * length); everything else is kept.  The object is written compactly to
 * out[cap] and validated against ext_spec: CG_OK, or CG_E_INVALID when a
 * field is not an integer, the text is not JSON, or the original schema
 * refuses the result (the output is still written when it fits).
 */
int cg_contract_model_spec(const char *ext_spec, size_t len, char *out, size_t cap, size_t *out_len,
                           int32_t *n_fields);
int cg_contract_reverse(const char *ext_spec, size_t len, const uint8_t *text, size_t text_len, char *out,
                        size_t cap, size_t *out_len);

/*
 * Host-side evaluator of a string-operation span ("Evaluator aware
 * decoding", "Not just arithmetic: string operations"):
 * "<strop>" NAME "(" ARGS ")" "</strop>" as the calc_text grammar with the
 * "strop" evaluator spells it.  count(s, t): non-overlapping occurrences of
 * t in s, left to right (an empty t occurs len + 1 times); len(s);
 * reverse(s); upper(s): ASCII letters upper-cased; substr(s, i, j): the
 * characters from i up to j, negative positions counted from the end, both
 * clamped to the string.  Writes the result text (count and len as decimal
 * text) with a terminating zero to out[cap]; *out_len = its length.
 * CG_E_PARSE for a malformed span, CG_E_LIMIT when cap is too small.
 */
int cg_eval_strop(const uint8_t *span, size_t len, char *out, size_t cap, size_t *out_len);

/*
 * Host-side diagnostic: run `bytes` against the automaton from its start.
 * *refused_at = index of the first refused byte (len if none); *complete =
 * 1 iff all bytes were accepted and form a complete member ("Constrained
 * decoding", "Reading the grammar for a tool": try-input says where a
 * candidate would have been refused).  The whole language is walked,
 * engine-written regions included.
 */
int cg_try_input(const cg_grammar *g, const uint8_t *bytes, size_t len, size_t *refused_at, int *complete);

/* Message of the last error on this thread ("" if none). */
const char *cg_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* CG_H */
