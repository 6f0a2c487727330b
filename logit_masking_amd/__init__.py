"""logit_masking_amd -- Python binding of libcg.so, the MI355X constrained-decoding
hot path (grammar -> pushdown automaton tables, token bitmask, masked
sampling, state advance).  Argument marshalling only: every step runs in the
library's HIP kernels.  Device buffers are torch tensors; torch supplies
memory and the current HIP stream, nothing else.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcg.so")

CG_OK, CG_E_ARG, CG_E_PARSE, CG_E_UNSUPPORTED, CG_E_LIMIT, CG_E_VOCAB, CG_E_DEVICE, CG_E_EVAL, CG_E_INVALID = \
    0, -1, -2, -3, -4, -5, -6, -7, -8
ROW_OK, ROW_DONE, ROW_CAPPED, ROW_REJECTED, ROW_NOOP, ROW_INJECT = 0, 1, 2, 3, 4, 5
FLAG_DONE, FLAG_CAPPED = 1, 2
HOST_ONLY = 1
STATE_BYTES = 24
DTYPE_F32, DTYPE_BF16 = 0, 1
FILL_NOALLOC_SCRATCH_BYTES = 16 << 20  # CG_FILL_NOALLOC_SCRATCH_BYTES

# Symbols the C ABI (include/cg.h) exports.
EXPORTS = ["cg_compile_grammar", "cg_free_grammar", "cg_grammar_info", "cg_init_state", "cg_fill_workspace_bytes",
           "cg_fill_bitmask", "cg_sample_advance", "cg_sample_advance_fill",
           "cg_sample_advance_plan", "cg_fill_walk", "cg_force_bytes", "cg_eval_calc", "cg_draft_workspace_bytes",
           "cg_fill_draft", "cg_contract_model_spec", "cg_contract_reverse", "cg_cache_stats", "cg_cache_clear",
           "cg_eval_strop", "cg_fill_bitmask_noalloc",
           "cg_sample_workspace_bytes", "cg_apply_mask_sample", "cg_advance", "cg_try_input", "cg_last_error"]


class CgError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class Options(ctypes.Structure):
    _fields_ = [("gen_cap", ctypes.c_uint32), ("flags", ctypes.c_uint32)]


class Info(ctypes.Structure):
    _fields_ = [("vocab_size", ctypes.c_int32), ("words_per_row", ctypes.c_int32),
                ("max_token_len", ctypes.c_int32), ("n_states", ctypes.c_int32),
                ("table_entries", ctypes.c_int32), ("table_bytes", ctypes.c_int32),
                ("compile_ms", ctypes.c_double), ("state_masks", ctypes.c_int32), ("pad", ctypes.c_int32),
                ("total_ms", ctypes.c_double), ("max_bytes", ctypes.c_int64)]


_lib = None


def lib():
    """Load libcg.so; fails loudly when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with logit_masking_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.cg_compile_grammar.argtypes = [ctypes.c_char_p, sz, vp, vp, i32, ctypes.POINTER(Options),
                                         ctypes.POINTER(vp)]
        L.cg_free_grammar.argtypes = [vp]
        L.cg_free_grammar.restype = None
        L.cg_grammar_info.argtypes = [vp, ctypes.POINTER(Info)]
        L.cg_init_state.argtypes = [vp, vp, i32, vp]
        L.cg_fill_workspace_bytes.argtypes = [vp, i32]
        L.cg_fill_workspace_bytes.restype = sz
        L.cg_fill_bitmask.argtypes = [vp, vp, i32, vp, i32, vp, vp]
        L.cg_fill_bitmask_noalloc.argtypes = [vp, vp, i32, vp, i32, vp]
        L.cg_sample_workspace_bytes.argtypes = [i32, i32]
        L.cg_sample_workspace_bytes.restype = sz
        L.cg_apply_mask_sample.argtypes = [vp, i32, i32, i32, i64, vp, i32, vp, vp, vp, vp, vp, vp, vp]
        L.cg_advance.argtypes = [vp, vp, i32, vp, vp, vp, vp]
        L.cg_force_bytes.argtypes = [vp, vp, i32, vp, sz, vp, vp, vp]
        L.cg_contract_model_spec.argtypes = [ctypes.c_char_p, sz, vp, sz, ctypes.POINTER(sz),
                                             ctypes.POINTER(ctypes.c_int32)]
        L.cg_contract_reverse.argtypes = [ctypes.c_char_p, sz, vp, sz, vp, sz, ctypes.POINTER(sz)]
        L.cg_draft_workspace_bytes.argtypes = [vp, i32, i32]
        L.cg_eval_strop.argtypes = [vp, sz, vp, sz, ctypes.POINTER(sz)]
        L.cg_eval_strop.restype = ctypes.c_int
        L.cg_cache_stats.argtypes = [ctypes.POINTER(i32), ctypes.POINTER(i64), ctypes.POINTER(i64)]
        L.cg_cache_stats.restype = ctypes.c_int
        L.cg_cache_clear.argtypes = []
        L.cg_cache_clear.restype = ctypes.c_int
        L.cg_draft_workspace_bytes.restype = sz
        L.cg_fill_draft.argtypes = [vp, vp, vp, i32, vp, i32, vp, vp, i32, vp, vp, vp]
        L.cg_eval_calc.argtypes = [vp, sz, ctypes.POINTER(ctypes.c_int64)]
        L.cg_sample_advance.argtypes = [vp, vp, i32, i32, i64, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.cg_sample_advance_fill.argtypes = [vp, vp, i32, i32, i64, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.cg_sample_advance_plan.argtypes = [vp, vp, i32, i32, i64, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.cg_fill_walk.argtypes = [vp, vp, i32, vp, i32, vp, vp]
        L.cg_try_input.argtypes = [vp, vp, sz, ctypes.POINTER(sz), ctypes.POINTER(ctypes.c_int)]
        L.cg_last_error.restype = ctypes.c_char_p
        for name in ("cg_compile_grammar", "cg_grammar_info", "cg_init_state", "cg_fill_bitmask",
                     "cg_fill_bitmask_noalloc", "cg_sample_advance",
                     "cg_sample_advance_fill", "cg_sample_advance_plan", "cg_fill_walk",
                     "cg_force_bytes", "cg_eval_calc", "cg_fill_draft", "cg_contract_model_spec",
                     "cg_contract_reverse",
                     "cg_apply_mask_sample", "cg_advance", "cg_try_input"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc):
    if rc != CG_OK:
        raise CgError(rc, lib().cg_last_error().decode(errors="replace"))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(getattr(stream, "cuda_stream", stream) or 0)


def _dev(t, dtype, name, ndim=None):
    import torch
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")
    return t


def _states(t, name="states"):
    """Rows of cg_state: a contiguous [B, 24] uint8 device tensor."""
    import torch
    _dev(t, torch.uint8, name, 2)
    if t.shape[1] != STATE_BYTES:
        raise ValueError(f"{name} must be [B, {STATE_BYTES}] (cg_state rows)")
    return t


class Grammar:
    """A compiled grammar (cg_compile_grammar) bound to a vocabulary."""

    def __init__(self, spec_json: bytes, blob: bytes, offsets, gen_cap: int = 2048, host_only: bool = False):
        import numpy as np
        L = lib()
        if isinstance(spec_json, str):
            spec_json = spec_json.encode()
        off = np.ascontiguousarray(np.asarray(offsets, dtype=np.uint32))
        bl = np.frombuffer(blob if blob else b"\0", dtype=np.uint8)
        self._keep = (off, bl)
        h = ctypes.c_void_p()
        opts = Options(gen_cap, HOST_ONLY if host_only else 0)
        _check(L.cg_compile_grammar(spec_json, len(spec_json), bl.ctypes.data, off.ctypes.data, len(off) - 1,
                                    ctypes.byref(opts), ctypes.byref(h)))
        self._h = h
        self.V = len(off) - 1
        self.W = (self.V + 63) // 64
        self.gen_cap = gen_cap

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:
            _lib.cg_free_grammar(h)
            self._h = None

    def info(self) -> dict:
        i = Info()
        _check(lib().cg_grammar_info(self._h, ctypes.byref(i)))
        return {k: getattr(i, k) for k, _ in Info._fields_}

    def try_input(self, data: bytes):
        """(refused_at, complete) of the host walker over the packed table."""
        buf = ctypes.create_string_buffer(data, len(data)) if data else None
        ra, cp = ctypes.c_size_t(), ctypes.c_int()
        _check(lib().cg_try_input(self._h, buf, len(data), ctypes.byref(ra), ctypes.byref(cp)))
        return ra.value, bool(cp.value)

    # ---- device calls (async on the current stream) --------------------
    def new_states(self, B: int, device="cuda"):
        import torch
        return torch.empty((B, STATE_BYTES), dtype=torch.uint8, device=device)

    def init_state(self, states, stream=None):
        import torch
        _states(states)
        _check(lib().cg_init_state(self._h, _ptr(states), states.shape[0], _stream(stream)))

    def fill_workspace_bytes(self, B: int) -> int:
        return int(lib().cg_fill_workspace_bytes(self._h, B))

    def new_fill_workspace(self, B: int, device="cuda"):
        """Device buffer for fill_bitmask over B rows (no initialisation needed)."""
        import torch
        return torch.empty(max(2, (self.fill_workspace_bytes(B) + 15) // 16 * 2), dtype=torch.int64, device=device)

    def fill_bitmask(self, states, mask, workspace=None, stream=None):
        """workspace: from new_fill_workspace(B); None allocates one for this call."""
        import torch
        _states(states)
        _dev(mask, torch.int64, "mask", 2)
        if mask.shape[0] < states.shape[0]:
            raise ValueError("mask has fewer rows than states")
        B = states.shape[0]
        if workspace is None:
            workspace = self.new_fill_workspace(B, states.device)
        if workspace.numel() * workspace.element_size() < self.fill_workspace_bytes(B):
            raise ValueError("fill workspace too small")
        _check(lib().cg_fill_bitmask(self._h, _ptr(states), B, _ptr(mask), mask.shape[1], _ptr(workspace),
                                     _stream(stream)))

    def fill_bitmask_noalloc(self, states, mask, stream=None):
        """cg_fill_bitmask_noalloc: fill_bitmask with the library's own
        per-device scratch (no workspace; calls on one device must not
        overlap)."""
        import torch
        _states(states)
        _dev(mask, torch.int64, "mask", 2)
        if mask.shape[0] < states.shape[0]:
            raise ValueError("mask has fewer rows than states")
        _check(lib().cg_fill_bitmask_noalloc(self._h, _ptr(states), states.shape[0], _ptr(mask), mask.shape[1],
                                             _stream(stream)))

    def sample_advance(self, logits, mask, temperature, seed, steps, workspace, out_ids, out_logprob, states,
                       status, stream=None):
        """cg_sample_advance: apply_mask_sample + advance in one launch (same
        tensors and meanings as those two calls; steps is read, then bumped)."""
        import torch
        if logits.dtype == torch.float32:
            dt = DTYPE_F32
        elif logits.dtype == torch.bfloat16:
            dt = DTYPE_BF16
        else:
            raise ValueError("logits must be float32 or bfloat16")
        if not logits.is_cuda or logits.dim() != 2 or logits.stride(1) != 1 or logits.shape[1] < self.V:
            raise ValueError("logits must be a 2-D device tensor [B, >= vocab] with unit column stride")
        B = logits.shape[0]
        _dev(mask, torch.int64, "mask", 2)
        _dev(temperature, torch.float32, "temperature", 1)
        _dev(seed, torch.int64, "seed", 1)
        _states(states)
        for t, n in ((steps, "steps"), (out_ids, "out_ids"), (status, "status")):
            _dev(t, torch.int32, n, 1)
        _dev(out_logprob, torch.float32, "out_logprob", 1)
        if workspace.numel() * workspace.element_size() < sample_workspace_bytes(B, self.V):
            raise ValueError("workspace too small")
        for t, n in ((mask, "mask"), (temperature, "temperature"), (seed, "seed"), (steps, "steps"),
                     (out_ids, "out_ids"), (out_logprob, "out_logprob"), (states, "states"), (status, "status")):
            if t.shape[0] < B:
                raise ValueError(f"{n} has fewer rows than logits")
        _check(lib().cg_sample_advance(self._h, _ptr(logits), dt, B, logits.stride(0), _ptr(mask), mask.shape[1],
                                       _ptr(temperature), _ptr(seed), _ptr(steps), _ptr(workspace), _ptr(out_ids),
                                       _ptr(out_logprob), _ptr(states), _ptr(status), _stream(stream)))

    def sample_advance_fill(self, logits, mask, temperature, seed, steps, workspace, out_ids, out_logprob, states,
                            status, fill_workspace=None, stream=None, split=False):
        """cg_sample_advance_fill: sample_advance, then the next step's mask
        written over `mask` (fill_workspace: from new_fill_workspace(B); None
        allocates one for this call).  split=True makes the first of its two
        launches only (cg_sample_advance_plan); fill_walk completes the mask."""
        import torch
        if logits.dtype == torch.float32:
            dt = DTYPE_F32
        elif logits.dtype == torch.bfloat16:
            dt = DTYPE_BF16
        else:
            raise ValueError("logits must be float32 or bfloat16")
        if not logits.is_cuda or logits.dim() != 2 or logits.stride(1) != 1 or logits.shape[1] < self.V:
            raise ValueError("logits must be a 2-D device tensor [B, >= vocab] with unit column stride")
        B = logits.shape[0]
        _dev(mask, torch.int64, "mask", 2)
        _dev(temperature, torch.float32, "temperature", 1)
        _dev(seed, torch.int64, "seed", 1)
        _states(states)
        for t, n in ((steps, "steps"), (out_ids, "out_ids"), (status, "status")):
            _dev(t, torch.int32, n, 1)
        _dev(out_logprob, torch.float32, "out_logprob", 1)
        if workspace.numel() * workspace.element_size() < sample_workspace_bytes(B, self.V):
            raise ValueError("workspace too small")
        for t, n in ((mask, "mask"), (temperature, "temperature"), (seed, "seed"), (steps, "steps"),
                     (out_ids, "out_ids"), (out_logprob, "out_logprob"), (states, "states"), (status, "status")):
            if t.shape[0] < B:
                raise ValueError(f"{n} has fewer rows than logits")
        if fill_workspace is None:
            fill_workspace = self.new_fill_workspace(B)
        elif fill_workspace.numel() * fill_workspace.element_size() < self.fill_workspace_bytes(B):
            raise ValueError("fill workspace too small")
        fn = lib().cg_sample_advance_plan if split else lib().cg_sample_advance_fill
        _check(fn(self._h, _ptr(logits), dt, B, logits.stride(0), _ptr(mask), mask.shape[1], _ptr(temperature),
                  _ptr(seed), _ptr(steps), _ptr(workspace), _ptr(out_ids), _ptr(out_logprob), _ptr(states),
                  _ptr(status), _ptr(fill_workspace), _stream(stream)))

    def fill_walk(self, states, mask, workspace, stream=None):
        """cg_fill_walk: the second launch of sample_advance_fill (after
        split=True, with the same mask and fill workspace)."""
        import torch
        _states(states)
        _dev(mask, torch.int64, "mask", 2)
        B = states.shape[0]
        if mask.shape[0] < B:
            raise ValueError("mask has fewer rows than states")
        _dev(workspace, None, "workspace")
        if workspace.numel() * workspace.element_size() < self.fill_workspace_bytes(B):
            raise ValueError("fill workspace too small")
        _check(lib().cg_fill_walk(self._h, _ptr(states), B, _ptr(mask), mask.shape[1], _ptr(workspace),
                                  _stream(stream)))

    def advance(self, states, ids, steps, status, stream=None):
        import torch
        _states(states)
        for t, n in ((ids, "ids"), (steps, "steps"), (status, "status")):
            _dev(t, torch.int32, n, 1)
            if t.shape[0] < states.shape[0]:
                raise ValueError(f"{n} has fewer rows than states")
        _check(lib().cg_advance(self._h, _ptr(states), states.shape[0], _ptr(ids), _ptr(steps), _ptr(status),
                                _stream(stream)))

    def draft_workspace_bytes(self, B: int, k: int) -> int:
        return int(lib().cg_draft_workspace_bytes(self._h, B, k))

    def fill_draft(self, states, steps, draft, path_states, masks, accept_len, workspace=None, stream=None):
        """cg_fill_draft: draft [B, k] int32 (-1 pads); path_states [B, k+1, 24]
        uint8; masks [B, k+1, W] int64; accept_len [B] int32; steps [B] int32
        or None."""
        import torch
        _states(states)
        B = states.shape[0]
        _dev(draft, torch.int32, "draft", 2)
        k = draft.shape[1]
        if draft.shape[0] < B:
            raise ValueError("draft has fewer rows than states")
        _dev(path_states, torch.uint8, "path_states", 3)
        if path_states.shape[2] != STATE_BYTES:
            raise ValueError(f"path_states must be [B, k+1, {STATE_BYTES}]")
        _dev(masks, torch.int64, "masks", 3)
        _dev(accept_len, torch.int32, "accept_len", 1)
        if steps is not None:
            _dev(steps, torch.int32, "steps", 1)
        if path_states.shape[0] < B or path_states.shape[1] != k + 1 or masks.shape[0] < B or masks.shape[1] != k + 1:
            raise ValueError("path_states / masks must be [B, k+1, ...]")
        if workspace is None:
            n = self.draft_workspace_bytes(B, k)
            workspace = torch.empty(max(2, (n + 15) // 16 * 2), dtype=torch.int64, device=states.device)
        if workspace.numel() * workspace.element_size() < self.draft_workspace_bytes(B, k):
            raise ValueError("draft workspace too small")
        _check(lib().cg_fill_draft(self._h, _ptr(states), _ptr(steps), B, _ptr(draft), k, _ptr(path_states),
                                   _ptr(masks), masks.shape[2], _ptr(accept_len), _ptr(workspace), _stream(stream)))

    def force_bytes(self, states, data, offsets, status, stream=None):
        """cg_force_bytes: row r walks data[offsets[r]:offsets[r+1]] (uint8 /
        int32 device tensors, offsets has B+1 entries)."""
        import torch
        _states(states)
        B = states.shape[0]
        _dev(data, torch.uint8, "data", 1)
        _dev(offsets, torch.int32, "offsets", 1)
        if offsets.shape[0] < B + 1:
            raise ValueError("offsets needs B+1 entries")
        _dev(status, torch.int32, "status", 1)
        if status.shape[0] < B:
            raise ValueError("status has fewer rows than states")
        _check(lib().cg_force_bytes(self._h, _ptr(states), B, _ptr(data), data.numel(), _ptr(offsets),
                                    _ptr(status), _stream(stream)))


def eval_calc(span: bytes):
    """cg_eval_calc: (CG_OK, value) or (error code, message)."""
    if isinstance(span, str):
        span = span.encode()
    buf = ctypes.create_string_buffer(span, len(span)) if span else None
    v = ctypes.c_int64()
    rc = lib().cg_eval_calc(buf, len(span), ctypes.byref(v))
    if rc != CG_OK:
        return rc, lib().cg_last_error().decode(errors="replace")
    return CG_OK, v.value


def eval_strop(span: bytes):
    """cg_eval_strop: (CG_OK, result bytes) or (error code, message)."""
    if isinstance(span, str):
        span = span.encode()
    buf = ctypes.create_string_buffer(span, len(span)) if span else None
    rc, out = _sized_call(lambda b, c, n: lib().cg_eval_strop(buf, len(span), b, c, n))
    if rc != CG_OK:
        return rc, lib().cg_last_error().decode(errors="replace")
    return CG_OK, out


def cache_stats():
    """(entries, hits, misses) of the library's grammar cache."""
    e, h, m = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int64()
    _check(lib().cg_cache_stats(ctypes.byref(e), ctypes.byref(h), ctypes.byref(m)))
    return e.value, h.value, m.value


def cache_clear():
    _check(lib().cg_cache_clear())


def _sized_call(fn, *args):
    """Call an output-buffer function, growing the buffer once if needed."""
    cap = 1 << 16
    for _ in range(2):
        buf = ctypes.create_string_buffer(cap)
        n = ctypes.c_size_t()
        rc = fn(*args, buf, cap, ctypes.byref(n))
        if rc != CG_E_LIMIT:
            return rc, buf.raw[:n.value]
        cap = n.value + 1
    return rc, b""


def contract_model_spec(ext_spec):
    """cg_contract_model_spec: (model-facing spec bytes, replaced fields)."""
    if isinstance(ext_spec, str):
        ext_spec = ext_spec.encode()
    nf = ctypes.c_int32()
    rc, out = _sized_call(lambda b, c, n: lib().cg_contract_model_spec(ext_spec, len(ext_spec), b, c, n,
                                                                       ctypes.byref(nf)))
    _check(rc)
    return out, nf.value


def contract_reverse(ext_spec, text: bytes):
    """cg_contract_reverse: (rc, output bytes, message); rc is CG_OK or
    CG_E_INVALID (other codes raise)."""
    if isinstance(ext_spec, str):
        ext_spec = ext_spec.encode()
    tb = ctypes.create_string_buffer(text, len(text)) if text else None
    rc, out = _sized_call(lambda b, c, n: lib().cg_contract_reverse(ext_spec, len(ext_spec), tb, len(text), b, c, n))
    if rc not in (CG_OK, CG_E_INVALID):
        _check(rc)
    msg = "" if rc == CG_OK else lib().cg_last_error().decode(errors="replace")
    return rc, out, msg


def sample_workspace_bytes(B: int, V: int) -> int:
    return int(lib().cg_sample_workspace_bytes(B, V))


def new_workspace(B: int, V: int, device="cuda"):
    """A workspace for apply_mask_sample (possibly empty)."""
    import torch
    n = sample_workspace_bytes(B, V)
    return torch.zeros(max(1, (n + 15) // 16 * 2), dtype=torch.float64, device=device)


def apply_mask_sample(logits, mask, temperature, seed, step, workspace, out_ids, out_logprob, vocab=None,
                      stream=None):
    """cg_apply_mask_sample on torch tensors: logits [B, stride] float32 or
    bfloat16, mask [B, W] int64, temperature [B] float32, seed [B] int64
    (the u64 bits), step [B] int32, outputs ids [B] int32, logprob [B] float32."""
    import torch
    if logits.dtype == torch.float32:
        dt = DTYPE_F32
    elif logits.dtype == torch.bfloat16:
        dt = DTYPE_BF16
    else:
        raise ValueError("logits must be float32 or bfloat16")
    if not logits.is_cuda or logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be a 2-D device tensor with unit column stride")
    B = logits.shape[0]
    V = logits.shape[1] if vocab is None else vocab
    _dev(mask, torch.int64, "mask", 2)
    _dev(temperature, torch.float32, "temperature", 1)
    _dev(seed, torch.int64, "seed", 1)
    _dev(step, torch.int32, "step", 1)
    _dev(out_ids, torch.int32, "out_ids", 1)
    _dev(out_logprob, torch.float32, "out_logprob", 1)
    if workspace.numel() * workspace.element_size() < sample_workspace_bytes(B, V):
        raise ValueError("workspace too small")
    for t, n in ((mask, "mask"), (temperature, "temperature"), (seed, "seed"), (step, "step"),
                 (out_ids, "out_ids"), (out_logprob, "out_logprob")):
        if t.shape[0] < B:
            raise ValueError(f"{n} has fewer rows than logits")
    _check(lib().cg_apply_mask_sample(_ptr(logits), dt, B, V, logits.stride(0), _ptr(mask), mask.shape[1],
                                      _ptr(temperature), _ptr(seed), _ptr(step), _ptr(workspace), _ptr(out_ids),
                                      _ptr(out_logprob), _stream(stream)))
