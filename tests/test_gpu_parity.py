"""GPU parity: the HIP path (through the C ABI) against the oracle.

Masks must match bit for bit; greedy picks index for index; sampled picks
index for index under the shared Philox stream, with log-probabilities
within 1e-5 and near-ties (oracle top-2 margin < 1e-6) reported apart.
"""
import numpy as np
import pytest

import logit_masking_amd as cg
from logit_masking_amd import workloads as W
from oracle import oracle as O
from tests.gpu_util import NTHREADS, device_rows, gpu_masks, oracle_masks, random_walk, say

pytestmark = pytest.mark.gpu

LOGPROB_TOL = 1e-5
NEAR_TIE = 1e-6


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available()
    return torch


def _setup(cfg, V=None, gen_cap=W.GEN_CAP):
    blob, off = W.make_vocab(cfg, V)
    toks = [blob[off[i]:off[i + 1]] for i in range(len(off) - 1)]
    g = cg.Grammar(W.spec_json(cfg), blob, off, gen_cap=gen_cap)
    og = O.load_spec(W.spec_json(cfg))
    return g, og, blob, off, toks


def _walks(og, toks, B, seed, max_len, gen_cap=W.GEN_CAP):
    rng = W.SplitMix(seed)
    seqs, rows = [], []
    for r in range(B):
        s, row = random_walk(og, toks, rng.below(max_len + 1), rng, gen_cap=gen_cap)
        seqs.append(s)
        rows.append(row)
    return seqs, rows


def _compare_masks(got, want, V, what):
    Wv = (V + 63) // 64
    diff = np.nonzero(got[:, :Wv] != want[:, :Wv])
    if len(diff[0]):
        r, w = diff[0][0], diff[1][0]
        x = int(got[r, w]) ^ int(want[r, w])
        bit = (x & -x).bit_length() - 1
        raise AssertionError(f"{what}: {len(diff[0])} mask words differ; first row {r} token {w * 64 + bit}")


# ---------------------------------------------------------------------------
# masks
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg,B,V,max_len", [
    (1, 64, None, 40),
    (2, 24, None, 60),
    (3, 16, None, 60),
    (4, 12, None, 80),
    (5, 12, None, 80),
    (3, 40, 5000, 40),     # several tiles and a ragged tail (5000 = 78 words + 8)
    (5, 33, 777, 50),      # odd batch, ragged vocab
])
def test_mask_parity(torch_dev, cfg, B, V, max_len):
    say("mask", cfg, B, V)
    g, og, blob, off, toks = _setup(cfg, V)
    seqs, rows = _walks(og, toks, B, seed=cfg * 7919 + B, max_len=max_len)
    st, steps, status = device_rows(g, seqs)
    torch_dev.cuda.synchronize()
    assert [int(x) for x in steps.cpu()] == [r.step for r in rows]
    got = gpu_masks(g, st)
    want, _ = oracle_masks(og, rows, blob, off)
    _compare_masks(got, want, len(toks), f"config {cfg}")
    # pad bits of the last word are zero; done rows are all zero
    V = len(toks)
    if V % 64:
        assert np.all(got[:, V // 64] >> np.uint64(V % 64) == 0)
    for r, row in enumerate(rows):
        if row.done:
            assert not got[r].any()
        else:
            assert got[r].any()


def _plain(states_np, g_start_is_string=False):
    """Rows in a plain configuration: no whitespace run, no open container
    (the fill copies such a row's precomputed state mask)."""
    ws = states_np[:, 17]
    depth = states_np[:, 16]
    stk = states_np[:, 8:16].copy().view(np.uint64)[:, 0]
    return (ws == 0) & (depth == 0) & (stk == 0) & (states_np[:, 18] == 0)


@pytest.mark.parametrize("cfg,V", [(2, None), (3, 20000), (4, 20000), (6, 20000), (5, 5000)])
def test_state_mask_table(torch_dev, cfg, V):
    """Masks of rows in plain configurations come from the table computed at
    compile time; they must equal the oracle's like every other row, and
    the table must be there (and be used by a fair share of the rows)."""
    say("state masks", cfg, V)
    g, og, blob, off, toks = _setup(cfg, V)
    info = g.info()
    assert info["state_masks"] > 0
    seqs, rows = _walks(og, toks, 96, seed=cfg * 31 + 5, max_len=60)
    st, steps, status = device_rows(g, seqs)
    got = gpu_masks(g, st)
    want, _ = oracle_masks(og, rows, blob, off)
    _compare_masks(got, want, len(toks), f"config {cfg} state masks")
    plain = _plain(st.cpu().numpy())
    say("state masks", cfg, "plain rows", int(plain.sum()), "of", len(rows), "table rows", info["state_masks"])
    if cfg != 5:
        assert plain.sum() >= 5


STRING_PREFIXES = {
    2: [b'{"eligibility":{"criteria_met":true,"reason_code":"eligible"},"action":"decline","appointment":{"date":"',
        b'{"eligibility":{"criteria_met":true,"reason_code":"eligible"},"action":"decline","appointment":null,'
        b'"response_text":"'],
    3: [b'calculate({"expression":"', b'store_record({"key":"k","value":{"', b'store_record({"key":"k","value":["',
        b'calendar({"action":"list","date":"', b'set_timer({"seconds":5,"label":"'],
    4: [b'{"reasoning":"'],
    5: [b'{"', b'["', b'{"a":"', b'[[{"k":[1,"'],
}
STRING_TAILS = [b"", b"a", b"ab c", b"\\", b"\\u", b"\\u00", b"\\uD7", b"\xc3", b"\xe2\x82", b"\xf0\x9f",
                b"\xf0\x9f\x98", b'\\"', b"\\n", b"x" * 9, b"x" * 10, b"x" * 19, b"x" * 20, b"y" * 40,
                b"z" * 255, b"z" * 256, b"w" * 699, b"w" * 700, b"v" * 1999, b"v" * 2000]


@pytest.mark.parametrize("cfg", sorted(STRING_PREFIXES))
def test_mask_parity_inside_strings(torch_dev, cfg):
    """Rows parked inside open strings: at a code-point boundary (the
    per-token summary path), mid UTF-8 sequence, after a backslash, inside a
    \\u escape, at and below every cap."""
    say("strings", cfg)
    g, og, blob, off, toks = _setup(cfg)
    seqs, rows = [], []
    for pre in STRING_PREFIXES[cfg]:
        for tail in STRING_TAILS:
            row = O.Row(og, W.GEN_CAP)
            data = pre + tail
            if og.feed(og.clone(row.conf), data) != len(data):
                continue
            for b in data:
                row.advance(bytes([b]))
            seqs.append(list(data))
            rows.append(row)
    assert len(rows) >= 20
    st, steps, status = device_rows(g, seqs)
    got = gpu_masks(g, st)
    want, _ = oracle_masks(og, rows, blob, off)
    _compare_masks(got, want, len(toks), f"config {cfg} in strings")


# Tokens for the walk's string paths: after a closing quote a second string
# opened and closed (or left open) inside the token, escapes, multi-byte code
# points and brackets in it; quotes escaped, first or not; code points around
# the cap.
WALK_TOKENS = [
    b'":"abc', b'":"a', b'":"', b'":"ab",', b'":"ab"', b'":"a\\"b', b'":"a\\\\"', b'":"\xc3\xa9x"',
    b'":"\xe2\x82\xac"}', b'","x"', b'","x":"y"', b'"],"a"', b'"}', b'"},{"k":"v"', b'":["a","b"]',
    b'":{"x":"y"}', b'" : "z"', b'":""', b'":"\\u00e9"', b'":"\\u00', b'":"' + b"a" * 20,
    b'":"' + b"a" * 25 + b'"', b'":"abcde"', b'":"abcdef"', b'":"abcdefg"', b'x":"y', b'ab","c',
    b'\xc3\xa9":"x', b'\\\\":"q"', b'"abc"', b'"ab"c', b'"x"y"z"', b'"a":"b"', b'{"a":"b","c":"d"}',
    b'["x","y"]', b'"\\"q"', b'"\\u0041"', b'"a\\nb"', b' "a"', b'"' + b"q" * 28 + b'"', b'"abc',
    b'"', b'"":"', b'\xa9"', b'\xa9":"x"', b'\x82\xac', b'\x82\xac"}', b'abcdef"', b'abcdefg"',
    b'[{"a":["b",{"c":"d"}]}]', b'"]]]', b'"}}', b'":[[["x"', b'":1,"b":"c"',
]
WALK_PREFIXES = [b"", b"{", b"[", b'{"', b'{"ab', b'{"abcde', b'{"a":"', b'{"a":"xy', b'["', b'["a\\',
                 b'["\xc3', b'["\xe2\x82', b'{"a":["b","', b'[[{"k":"', b'{"a":"\\u00', b'{"a":1,"',
                 b'[[["', b'{"a":{"b":[', b'["\\', b'{"a\\']


@pytest.mark.parametrize("cap", [None, 6])
def test_walk_string_paths(torch_dev, cap):
    """The walk's string paths against the oracle, word for word: tokens whose
    bytes after a closing quote open a second string (jumped with that
    string's summary, closed or left open, escapes and multi-byte code points
    inside), escaped quotes (walked byte by byte), code points before and at
    a cap of 6; rows inside strings (at a code-point boundary, after a
    backslash, mid UTF-8) and outside them, in objects and arrays up to the
    depth cap ("Constrained decoding", "The guarantee")."""
    import json
    say("walk string paths", cap)
    spec = json.dumps({"kind": "json_schema", "ws_max": 2, "open_string_cap": cap, "depth_cap": 4,
                       "schema": {"anyOf": [{"type": "object"}, {"type": "array"}]}}).encode()
    og = O.load_spec(spec)
    toks = [bytes([i]) for i in range(256)] + WALK_TOKENS
    blob = b"".join(toks)
    off = np.cumsum([0] + [len(t) for t in toks]).tolist()
    g = cg.Grammar(spec, blob, off)
    seqs, rows = [], []
    for pre in WALK_PREFIXES:
        row = O.Row(og, W.GEN_CAP)
        if og.feed(og.clone(row.conf), pre) != len(pre):
            continue
        for b in pre:
            row.advance(bytes([b]))
        seqs.append(list(pre))
        rows.append(row)
    assert len(rows) >= 15, len(rows)
    st, steps, status = device_rows(g, seqs)
    got = gpu_masks(g, st)
    want, _ = oracle_masks(og, rows, blob, off)
    _compare_masks(got, want, len(toks), f"walk string paths, cap {cap}")
    # the crafted tokens must take part: some allowed, some refused
    allowed = np.unpackbits(want.view(np.uint8), axis=1, bitorder="little")[:, 256:len(toks)]
    assert allowed.any() and not allowed.all()


def test_calc_prefix_sweep(torch_dev):
    """Config 1 over 2048 random valid prefixes (byte ids through cg_advance)."""
    say("calc sweep")
    g, og, blob, off, toks = _setup(1)
    rng = W.SplitMix(77)
    seqs, rows = [], []
    for r in range(2048):
        row = O.Row(og, W.GEN_CAP)
        seq = []
        for _ in range(rng.below(41)):
            nb = sorted(og.next_bytes(row.conf))
            if not nb:
                break
            b = nb[rng.below(len(nb))]
            row.advance(bytes([b]))
            seq.append(b)
        seqs.append(seq)
        rows.append(row)
    st, _, _ = device_rows(g, seqs)
    got = gpu_masks(g, st)
    want, _ = oracle_masks(og, rows, blob, off)
    _compare_masks(got, want, len(toks), "calc sweep")


def test_mask_extra_words_untouched(torch_dev):
    g, og, blob, off, toks = _setup(2, 1000)
    st = g.new_states(3)
    g.init_state(st)
    mask = torch_dev.full((3, g.W + 5), 7, dtype=torch_dev.int64, device="cuda")
    g.fill_bitmask(st, mask)
    m = mask.cpu().numpy()
    assert np.all(m[:, g.W:] == 7)


def test_gen_cap_and_statuses(torch_dev):
    torch = torch_dev
    say("advance statuses")
    g, og, blob, off, toks = _setup(5, 2000, gen_cap=3)
    B = 6
    st = g.new_states(B)
    g.init_state(st)
    steps = torch.zeros(B, dtype=torch.int32, device="cuda")
    status = torch.zeros(B, dtype=torch.int32, device="cuda")
    lb, rb, one = ord("["), ord("]"), ord("1")
    # row 0: "[" "1" "," -> capped at 3; row 1: "[" "]" -> done; row 2: illegal "x";
    # row 3: -1 no-op; row 4: id out of range; row 5: "[" then forced "]" then more
    plan = [[lb, one, ord(",")], [lb, rb, -1], [ord("x"), -1, -1], [-1, -1, -1], [len(toks) + 5, -1, -1],
            [lb, rb, lb]]
    want_status = [[0, 0, 2], [0, 1, 4], [3, 4, 4], [4, 4, 4], [3, 4, 4], [0, 1, 3]]
    for k in range(3):
        ids = torch.tensor([p[k] for p in plan], dtype=torch.int32, device="cuda")
        g.advance(st, ids, steps, status)
        assert status.cpu().tolist() == [w[k] for w in want_status], k
    assert steps.cpu().tolist() == [3, 2, 0, 0, 0, 2]
    flags = st.cpu().numpy()[:, 18]
    assert flags.tolist() == [cg.FLAG_CAPPED, cg.FLAG_DONE, 0, 0, 0, cg.FLAG_DONE]
    mask = gpu_masks(g, st)
    assert not mask[0].any() and not mask[1].any() and not mask[5].any()
    assert mask[2].any() and mask[3].any()


def test_empty_batch_and_empty_tokens(torch_dev):
    torch = torch_dev
    blob = b"[]1"
    off = [0, 1, 2, 2, 3]  # token 2 is empty: never allowed
    g = cg.Grammar(W.spec_json(5), blob, off)
    st = g.new_states(0)
    g.init_state(st)
    g.fill_bitmask(st, torch.zeros((0, 1), dtype=torch.int64, device="cuda"))
    st = g.new_states(1)
    g.init_state(st)
    m = gpu_masks(g, st)
    assert int(m[0, 0]) == 0b0001  # only "["
    ids = torch.tensor([0], dtype=torch.int32, device="cuda")
    steps = torch.zeros(1, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    g.advance(st, ids, steps, status)
    m = gpu_masks(g, st)
    assert int(m[0, 0]) == 0b1011  # "[", "]", "1" but not the empty token
    ids[0] = 2
    g.advance(st, ids, steps, status)
    assert status.item() == cg.ROW_REJECTED


def test_longest_tokens(torch_dev):
    """32-byte tokens (the maximum) walk every byte."""
    og = O.load_spec(W.spec_json(5))
    toks = [bytes([i]) for i in range(256)] + [b'["' + b"a" * 30, b'[' + b"1" * 31, b'{"' + b"\xc3\xa9" * 15,
                                               b"[" * 32, b"[" * 31 + b"x"]
    blob = b"".join(toks)
    off = np.cumsum([0] + [len(t) for t in toks]).tolist()
    g = cg.Grammar(W.spec_json(5), blob, off)
    st = g.new_states(1)
    g.init_state(st)
    got = gpu_masks(g, st)
    want = og.mask(og.start(), blob, off)
    assert np.array_equal(got[0], want)


# ---------------------------------------------------------------------------
# sampling
# ---------------------------------------------------------------------------
def _sample_case(torch, cfg, B, V, T, step, row_stride=None, mask_words=None, seed=5):
    """Random masks (some rows empty) and seeded logits; GPU pick vs oracle."""
    import torch as _t
    rng = np.random.default_rng(seed)
    c = W.CONFIGS[cfg]
    logits = W.make_logits(cfg, step, B, V, "cuda", row_stride=row_stride)
    Wn = (V + 63) // 64 if mask_words is None else mask_words
    bits = rng.random((B, V)) < rng.choice([0.002, 0.05, 0.5, 0.95], size=(B, 1))
    bits[0, :] = False  # a finished row
    if B > 2:
        bits[2, :] = False
        bits[2, V - 1] = True  # only the last id
    words = np.zeros((B, Wn), dtype=np.uint64)
    packed = np.packbits(bits, axis=1, bitorder="little")
    pw = np.zeros((B, Wn * 8), dtype=np.uint8)
    pw[:, :packed.shape[1]] = packed
    words[:] = pw.view(np.uint64)
    mask = _t.from_numpy(words.view(np.int64)).cuda()
    temp = _t.full((B,), float(T), dtype=_t.float32, device="cuda")
    seeds = np.array(W.row_seeds(cfg, B), dtype=np.uint64)
    seed_t = _t.from_numpy(seeds.view(np.int64)).cuda()
    steps = _t.full((B,), step, dtype=_t.int32, device="cuda")
    ws = cg.new_workspace(B, V)
    ids = _t.empty(B, dtype=_t.int32, device="cuda")
    lp = _t.empty(B, dtype=_t.float32, device="cuda")
    cg.apply_mask_sample(logits, mask, temp, seed_t, steps, ws, ids, lp, vocab=V)
    _t.cuda.synchronize()
    x = logits[:, :V].float().cpu().numpy().astype(np.float64)
    return x, bits, seeds, ids.cpu().numpy(), lp.cpu().numpy()


@pytest.mark.parametrize("cfg,B,V,T", [
    (1, 4, 512, 0.0),
    (2, 64, 32000, 0.7),
    (2, 16, 32000, 0.0),
    (3, 32, 128256, 0.7),
    (4, 16, 151936, 0.0),
    (5, 16, 256000, 1.0),
    (5, 16, 256000, 0.0),
    (3, 9, 5001, 0.7),     # ragged: 3 chunks, last one partial, V % 8 != 0
])
def test_sample_parity(torch_dev, cfg, B, V, T):
    say("sample", cfg, B, V, T)
    x, bits, seeds, ids, lp = _sample_case(torch_dev, cfg, B, V, T, step=11)
    ties = 0
    for r in range(B):
        i, l, info = O.sample_row(x[r], bits[r], T, int(seeds[r]), 11)
        if i < 0:
            assert ids[r] == -1 and lp[r] == 0.0
            continue
        if T > 0 and min(info["margin_chunk"], info["margin_token"]) < NEAR_TIE:
            # greedy compares stored values exactly (ties -> lowest id): never exempt
            ties += 1
            assert bits[r, ids[r]]
            continue
        assert ids[r] == i, (r, ids[r], i, info)
        assert abs(lp[r] - l) < LOGPROB_TOL, (r, lp[r], l)
    say("near-ties", cfg, B, V, T, ties)
    assert ties <= max(1, B // 10)


@pytest.mark.parametrize("cfg,V,T,strides,mask_words", [
    (3, 128256, 0.7, (128256 + 64, 128256 + 3), 2010),   # bf16
    (3, 128256, 0.0, (128256 + 3,), 2004),
    (2, 32000, 0.7, (32000 + 4, 32000 + 1), 505),       # float32
])
def test_sample_strided_and_wide_mask(torch_dev, cfg, V, T, strides, mask_words):
    """row_stride > vocab, misaligned stride (rows not 16-byte aligned: the
    bounds-checked loads), extra mask words."""
    say("strided", cfg, T, strides)
    for stride in strides:
        x, bits, seeds, ids, lp = _sample_case(torch_dev, cfg, 8, V, T, step=3, row_stride=stride,
                                               mask_words=mask_words)
        for r in range(8):
            i, l, info = O.sample_row(x[r], bits[r], T, int(seeds[r]), 3)
            if i < 0:
                assert ids[r] == -1
                continue
            if T == 0 or min(info["margin_chunk"], info["margin_token"]) >= NEAR_TIE:
                assert ids[r] == i and abs(lp[r] - l) < LOGPROB_TOL, (stride, r, ids[r], i)


def test_sample_fp32_greedy_ties(torch_dev):
    import torch
    B, V = 3, 3000
    logits = torch.zeros((B, V), dtype=torch.float32, device="cuda")
    logits[0, 100] = 2.0
    logits[0, 2500] = 2.0   # tie across chunks -> lowest id
    logits[1, 10] = 1.0
    logits[1, 11] = 1.0     # tie inside a lane group
    mask = torch.full((B, (V + 63) // 64), -1, dtype=torch.int64, device="cuda")
    temp = torch.zeros(B, dtype=torch.float32, device="cuda")
    seed = torch.zeros(B, dtype=torch.int64, device="cuda")
    step = torch.zeros(B, dtype=torch.int32, device="cuda")
    ids = torch.empty(B, dtype=torch.int32, device="cuda")
    lp = torch.empty(B, dtype=torch.float32, device="cuda")
    cg.apply_mask_sample(logits, mask, temp, seed, step, cg.new_workspace(B, V), ids, lp)
    assert ids.cpu().tolist() == [100, 10, 0]


def test_fill_workspace_reuse_and_size(torch_dev):
    """The fill workspace needs no initialisation and may be reused by later
    calls with fewer rows; a workspace that is too small is refused."""
    torch = torch_dev
    say("fill workspace")
    g, og, blob, off, toks = _setup(3, 20000)
    seqs, rows = _walks(og, toks, 24, 0xF111, 40)
    st, _, _ = device_rows(g, seqs)
    ws = g.new_fill_workspace(24)
    ws.fill_(-1)  # stale contents must not matter
    want, _ = oracle_masks(og, rows, blob, off)
    for B in (24, 7):
        mask = torch.full((B, g.W), 0x5A5A5A5A5A5A5A5A, dtype=torch.int64, device="cuda")
        g.fill_bitmask(st[:B].contiguous(), mask, ws)
        torch.cuda.synchronize()
        _compare_masks(mask.cpu().numpy().view(np.uint64), want[:B], len(toks), f"workspace reuse B={B}")
    assert g.fill_workspace_bytes(24) > g.fill_workspace_bytes(7) > 0 == g.fill_workspace_bytes(0)
    small = torch.empty(max(1, g.fill_workspace_bytes(7) // 8 - 1), dtype=torch.int64, device="cuda")
    with pytest.raises(ValueError):
        g.fill_bitmask(st[:8].contiguous(), torch.empty((8, g.W), dtype=torch.int64, device="cuda"), small)


@pytest.mark.parametrize("design", sorted(W.DESIGN_SCHEMAS))
def test_design_mask_parity(torch_dev, design):
    """Decision designs 2-5 (vocab of config 2): masks of rows at random
    legal prefixes, bit-exact, and a sampled lock-step trajectory."""
    say("design", design)
    blob, off = W.make_vocab(2)
    toks = [blob[off[i]:off[i + 1]] for i in range(len(off) - 1)]
    spec = W.design_spec_json(design)
    g = cg.Grammar(spec, blob, off)
    og = O.load_spec(spec)
    seqs, rows = _walks(og, toks, 32, seed=0xD0 + design, max_len=120)
    st, steps, status = device_rows(g, seqs)
    got = gpu_masks(g, st)
    want, _ = oracle_masks(og, rows, blob, off)
    _compare_masks(got, want, len(toks), f"design {design}")
    # a few sampled steps from these rows
    import torch
    B, V = len(rows), len(toks)
    mask = torch.empty((B, g.W), dtype=torch.int64, device="cuda")
    temp = torch.full((B,), 0.7, dtype=torch.float32, device="cuda")
    seeds = np.array(W.row_seeds(2, B), dtype=np.uint64)
    seed_t = torch.from_numpy(seeds.view(np.int64)).cuda()
    ws = cg.new_workspace(B, V)
    ids = torch.empty(B, dtype=torch.int32, device="cuda")
    lp = torch.empty(B, dtype=torch.float32, device="cuda")
    ties = 0
    for s in range(12):
        logits = W.make_logits(2, 100 + s, B, V, "cuda")
        g.fill_bitmask(st, mask)
        g.sample_advance(logits, mask, temp, seed_t, steps, ws, ids, lp, st, status)
        m_dev = mask.cpu().numpy().view(np.uint64)
        ids_dev, lp_dev, stat = ids.cpu().numpy(), lp.cpu().numpy(), status.cpu().numpy()
        x = logits.float().cpu().numpy().astype(np.float64)
        words, _ = oracle_masks(og, rows, blob, off)
        for r in range(B):
            assert np.array_equal(m_dev[r], words[r]), (design, s, r)
            bits = O.unpack_mask(words[r], V)
            i, l, info = O.sample_row(x[r], bits, 0.7, int(seeds[r]), rows[r].step)
            if i >= 0 and min(info["margin_chunk"], info["margin_token"]) < NEAR_TIE:
                ties += 1
                assert bits[ids_dev[r]]
            else:
                assert ids_dev[r] == i and (i < 0 or abs(lp_dev[r] - l) < LOGPROB_TOL)
            assert stat[r] == rows[r].advance(None if ids_dev[r] < 0 else toks[ids_dev[r]])
    say("near-ties (trajectory)", ties)
    assert ties <= 2
