"""Edge cases of the device path against the oracle: the largest vocabulary
the sampler takes, one past it, -inf logits, extreme temperatures, a large
batch, and the fill at a vocabulary of a million tokens."""
import numpy as np
import pytest

import logit_masking_amd as cg
from logit_masking_amd import workloads as W
from oracle import oracle as O
from tests.gpu_util import NTHREADS, device_rows, gpu_masks, oracle_masks, random_walk, say

pytestmark = pytest.mark.gpu

V_MAX = 4_194_304  # 2048 chunk summaries of 24 bytes fill the 48 KiB the sampler gives them
NEAR_TIE = 1e-6


def _run_sample(x, bits, T, seeds, step, dtype, stray_rows=()):
    """x: float64 [B, V] (values representable in dtype), bits: bool [B, V];
    stray_rows: rows whose mask words also set every bit past V (a caller's
    mask may carry such bits; they allow nothing)."""
    import torch
    B, V = x.shape
    logits = torch.from_numpy(x).to(dtype).cuda()
    W_ = (V + 63) // 64
    pad = np.zeros((B, W_ * 64), dtype=bool)
    pad[:, :V] = bits
    for r in stray_rows:
        pad[r, V:] = True
    words = np.packbits(pad.reshape(B, W_, 64)[:, :, ::-1], axis=2, bitorder="big").view(">u8").astype(np.uint64)
    mask = torch.from_numpy(words.reshape(B, W_).view(np.int64)).cuda()
    temp = torch.full((B,), float(T), dtype=torch.float32, device="cuda")
    seed_t = torch.from_numpy(np.asarray(seeds, dtype=np.uint64).view(np.int64)).cuda()
    steps = torch.full((B,), step, dtype=torch.int32, device="cuda")
    ws = cg.new_workspace(B, V)
    ids = torch.empty(B, dtype=torch.int32, device="cuda")
    lp = torch.empty(B, dtype=torch.float32, device="cuda")
    cg.apply_mask_sample(logits, mask, temp, seed_t, steps, ws, ids, lp)
    torch.cuda.synchronize()
    return logits.double().cpu().numpy(), ids.cpu().numpy(), lp.cpu().numpy()


def _check(x, bits, T, seeds, step, ids, lp):
    ties = 0
    for r in range(x.shape[0]):
        i, l, info = O.sample_row(x[r], bits[r], T, int(seeds[r]), step)
        if i < 0:
            assert ids[r] == -1 and lp[r] == 0.0, r
            continue
        if T > 0 and min(info["margin_chunk"], info["margin_token"]) < NEAR_TIE:
            ties += 1
            assert bits[r, ids[r]]
            continue
        assert ids[r] == i, (r, ids[r], i)
        assert abs(lp[r] - l) < 1e-5, (r, lp[r], l)
    say("near-ties", ties, "of", x.shape[0], "rows")
    return ties


@pytest.mark.parametrize("dtype_name,T", [("bfloat16", 0.7), ("bfloat16", 0.0), ("float32", 0.7)])
def test_sample_max_vocab(dtype_name, T):
    import torch
    say("max vocab", dtype_name, T)
    rng = np.random.default_rng(11)
    B = 2
    x = rng.normal(scale=3.0, size=(B, V_MAX))
    bits = rng.random((B, V_MAX)) < 0.3
    dt = getattr(torch, dtype_name)
    xs, ids, lp = _run_sample(x, bits, T, [12345, 67890], 4, dt)
    assert _check(xs, bits, T, [12345, 67890], 4, ids, lp) <= 1


@pytest.mark.parametrize("dtype_name,T", [("bfloat16", 0.7), ("bfloat16", 0.0), ("float32", 0.7), ("float32", 0.0)])
def test_sample_sparse_rows(dtype_name, T):
    """Aligned rows of more than 16 chunks take the sparse stream: the mask is
    staged in LDS and, after each wave's first chunk, a lane reads a 16-byte
    piece of logits only when one of its ids is allowed.  Vocabulary 100,000
    (49 chunks, the last one ragged): a single allowed id in a middle chunk;
    a single one at the last id, with every mask bit past V set; one allowed
    id per 4096; ids allowed only in the first 16 chunks (the ones read
    whole); every id; none."""
    import torch
    say("sparse rows", dtype_name, T)
    rng = np.random.default_rng(21)
    B, V = 6, 100_000
    x = rng.normal(scale=3.0, size=(B, V))
    bits = np.zeros((B, V), dtype=bool)
    bits[0, 40_000] = True
    bits[1, V - 1] = True
    bits[2, rng.choice(V, V // 4096, replace=False)] = True
    bits[3, :16 * 2048] = rng.random(16 * 2048) < 0.5
    bits[4, :] = True
    seeds = [int(s) for s in rng.integers(0, 2**63, size=B)]
    dt = getattr(torch, dtype_name)
    xs, ids, lp = _run_sample(x, bits, T, seeds, 3, dt, stray_rows=(1,))
    assert ids[0] == 40_000 and ids[1] == V - 1 and ids[5] == -1
    assert _check(xs, bits, T, seeds, 3, ids, lp) <= 1


def test_sample_vocab_over_limit():
    import torch
    say("over limit")
    V = V_MAX + 1
    logits = torch.zeros((1, V), dtype=torch.bfloat16, device="cuda")
    mask = torch.zeros((1, (V + 63) // 64), dtype=torch.int64, device="cuda")
    one = lambda dt, v: torch.full((1,), v, dtype=dt, device="cuda")
    ws = cg.new_workspace(1, V)
    with pytest.raises(cg.CgError) as e:
        cg.apply_mask_sample(logits, mask, one(torch.float32, 0.7), one(torch.int64, 1), one(torch.int32, 0), ws,
                             one(torch.int32, 0), one(torch.float32, 0))
    assert e.value.code == cg.CG_E_ARG


@pytest.mark.parametrize("T", [0.0, 0.7])
def test_minus_infinity_logits(T):
    """-inf logits carry no probability; a row whose allowed logits are all
    -inf has nothing to draw (-1)."""
    import torch
    say("-inf", T)
    rng = np.random.default_rng(12)
    B, V = 6, 40000
    x = rng.normal(scale=2.0, size=(B, V))
    bits = rng.random((B, V)) < 0.4
    x[rng.random((B, V)) < 0.3] = -np.inf
    x[1, :] = np.where(bits[1], -np.inf, x[1, :])      # every allowed logit -inf
    x[2, 2048:4096] = -np.inf                         # a whole chunk
    seeds = list(range(100, 100 + B))
    for dt in (torch.bfloat16, torch.float32):
        xs, ids, lp = _run_sample(x, bits, T, seeds, 9, dt)
        _check(xs, bits, T, seeds, 9, ids, lp)
        assert ids[1] == -1


@pytest.mark.parametrize("T", [1e-3, 50.0])
def test_extreme_temperatures(T):
    import torch
    say("temperature", T)
    rng = np.random.default_rng(13)
    B, V = 8, 128256
    x = rng.normal(scale=3.0, size=(B, V))
    bits = rng.random((B, V)) < 0.5
    seeds = [int(s) for s in rng.integers(0, 2**63, size=B)]
    xs, ids, lp = _run_sample(x, bits, T, seeds, 2, torch.bfloat16)
    assert _check(xs, bits, T, seeds, 2, ids, lp) <= 1


def test_large_batch():
    """4096 rows at once; 64 of them checked against the oracle."""
    import torch
    say("large batch")
    rng = np.random.default_rng(14)
    B, V = 4096, 32000
    x = rng.normal(scale=2.0, size=(B, V)).astype(np.float32).astype(np.float64)
    bits = rng.random((B, V)) < 0.6
    seeds = [int(s) for s in rng.integers(0, 2**63, size=B)]
    xs, ids, lp = _run_sample(x, bits, 0.7, seeds, 5, torch.float32)
    chk = list(range(0, B, 64))
    assert _check(xs[chk], bits[chk], 0.7, [seeds[r] for r in chk], 5, ids[chk], lp[chk]) <= 2


def test_fill_million_token_vocab():
    """The tool-call grammar over a vocabulary of 1,000,000 tokens: masks of
    rows at random prefixes, bit-exact."""
    say("million vocab")
    blob, off = W.make_vocab(3, 1_000_000)
    toks = [blob[off[i]:off[i + 1]] for i in range(len(off) - 1)]
    g = cg.Grammar(W.spec_json(3), blob, off)
    og = O.load_spec(W.spec_json(3))
    rng = W.SplitMix(15)
    seqs, rows = [], []
    for r in range(8):
        s, row = random_walk(og, toks, rng.below(40), rng)
        seqs.append(s)
        rows.append(row)
    st, steps, _ = device_rows(g, seqs)
    got = gpu_masks(g, st)
    want, _ = oracle_masks(og, rows, blob, off)
    assert np.array_equal(got[:, :want.shape[1]], want)


def _stored(x, dt):
    """float64 values rounded to dtype as the device stores them."""
    import torch
    return torch.from_numpy(np.asarray(x, dtype=np.float64)).to(dt).double().numpy()


def _lse64(v):
    m = np.max(v)
    return float(m + np.log(np.sum(np.exp(v - m))))


def _token_contended_row(rng, dt, Tf, seed, step, V, x, bits, r):
    """Only chunk 3 has allowed ids (64 of them); two of them get token scores
    x/T + G(0, i) between 2e-6 and 4e-5 apart, the rest score 6 lower.  The
    ids are drawn again on every attempt: on a bf16 grid the rounding of the
    second value is what lands the gap, and it depends on the noise."""
    for attempt in range(4000):
        ids = 3 * 2048 + np.sort(rng.choice(2048, 64, replace=False))
        G = O.gumbel(O.philox_words(seed, step, 0, ids))
        xi = _stored([Tf * (4.0 - G[0])], dt)[0]
        S = xi / Tf + G[0]
        for k in range(1, len(ids)):
            xj = _stored([Tf * (S + 1e-5 - G[k])], dt)[0]
            d = xj / Tf + G[k] - S
            if 2e-6 < abs(d) < 4e-5:
                xs = _stored(Tf * (S - 6.0 - G - rng.random(len(ids))), dt)
                xs[0], xs[k] = xi, xj
                x[r, ids] = xs
                bits[r, ids] = True
                return
    raise AssertionError("no contended token pair found")


def _chunk_contended_row(rng, dt, Tf, seed, step, V, x, bits, r, same_wave=False):
    """Two chunks hold one dominant allowed id and three companions 2-6
    lower (in x / T) each; their chunk scores L_c + G(1, c) are between 2e-6
    and 2e-5 apart (inside the screening window), every other chunk is
    masked.  The companions are drawn again on every attempt (they move the
    chunk's log-mass, and with it where the rounding lands the gap).
    same_wave: the second chunk is 16 or 32, reduced by the same wave as
    chunk 0, whose copy of its best chunk then holds only one of the two."""
    K = V // 2048
    G1 = O.gumbel(O.philox_words(seed, step, 1, np.arange(K)))
    def chunk_vals(c, score):
        # dominant + companions whose log-sum-exp of x / T is close to score
        o = 2.0 + 4.0 * rng.random(3)
        top_z = score - np.log1p(np.exp(-o).sum())
        top = _stored([Tf * top_z], dt)[0]
        v = _stored(np.concatenate([[top], top - Tf * o]), dt)
        pos = c * 2048 + np.sort(rng.choice(2048, 4, replace=False))
        return pos, v
    for attempt in range(4000):
        pa, va = chunk_vals(0, 4.0 - G1[0])
        S = _lse64(va / Tf) + G1[0]
        for c in (range(16, K, 16) if same_wave else range(1, K)):
            pb, vb = chunk_vals(c, S + 1e-5 - G1[c])
            d = _lse64(vb / Tf) + G1[c] - S
            if 2e-6 < abs(d) < 2e-5:
                x[r, pa], x[r, pb] = va, vb
                bits[r, pa] = bits[r, pb] = True
                return
    raise AssertionError("no contended chunk pair found")


@pytest.mark.parametrize("dtype_name", ["float32", "bfloat16"])
def test_sample_contended_picks(dtype_name):
    """Rows whose two best candidates are closer than the float screening
    can order, so the sampler must decide in double: two tokens of one chunk
    (the pick inside the chunk, from the stash for bf16 and from memory for
    float32), or two chunks (their log-masses recomputed exactly; half of
    these pairs are reduced by the same wave, so for bf16 the winner may be
    the one its stash does not hold, and is read from memory).  Each
    row's oracle margin at that level is checked to lie between the near-tie
    bound (1e-6) and the screening window, so every row takes the exact
    path, and every pick must equal the oracle's."""
    import torch
    say("contended", dtype_name)
    dt = getattr(torch, dtype_name)
    T, step = 0.7, 7
    Tf = float(np.float32(T))
    rng = np.random.default_rng(21)
    B, V = 16, 48 * 2048
    x = np.full((B, V), -30.0)
    bits = np.zeros((B, V), dtype=bool)
    seeds = [int(s) for s in rng.integers(0, 2**63, size=B)]
    for r in range(B):
        if r % 2 == 0:
            _token_contended_row(rng, dt, Tf, seeds[r], step, V, x, bits, r)
        else:
            _chunk_contended_row(rng, dt, Tf, seeds[r], step, V, x, bits, r, same_wave=r % 4 == 1)
    xs, ids, lp = _run_sample(x, bits, T, seeds, step, dt)
    for r in range(B):
        i, l, info = O.sample_row(xs[r], bits[r], T, seeds[r], step)
        margin = info["margin_token"] if r % 2 == 0 else info["margin_chunk"]
        assert NEAR_TIE < margin < 5e-5, (r, info)
        assert ids[r] == i, (r, ids[r], i, info)
        assert abs(lp[r] - l) < 1e-5, (r, lp[r], l)


def test_fill_many_row_blocks():
    """A batch of 16,421 rows (the walk scans its rows' tile counts in blocks
    of 8192 rows: two full blocks and a ragged third), made of 48 rows at
    random legal prefixes repeated in a seeded order: every row's mask
    equals its prototype's oracle mask, bit-exact.  One fused step over the
    whole batch (sample, advance, next mask) then equals the separate calls."""
    import torch
    say("row blocks")
    cfg = 3
    blob, off = W.make_vocab(cfg, 20000)
    V = len(off) - 1
    toks = [blob[off[i]:off[i + 1]] for i in range(V)]
    g = cg.Grammar(W.spec_json(cfg), blob, off)
    og = O.load_spec(W.spec_json(cfg))
    rng = W.SplitMix(0xB10C)
    seqs, orows = [], []
    for _ in range(48):
        s, row = random_walk(og, toks, rng.below(40), rng)
        seqs.append(s)
        orows.append(row)
    st_p, steps_p, _ = device_rows(g, seqs)
    want, _ = oracle_masks(og, orows, blob, off)
    B = 2 * 8192 + 37
    pick = np.random.default_rng(3).integers(0, 48, size=B)
    pick_t = torch.from_numpy(pick).cuda()
    st = st_p.index_select(0, pick_t).contiguous()
    got = gpu_masks(g, st)
    assert np.array_equal(got[:, :want.shape[1]], want[pick])
    # one fused step over the whole batch against the separate calls
    steps = steps_p.index_select(0, pick_t).contiguous()
    temp = torch.full((B,), 0.7, dtype=torch.float32, device="cuda")
    seed = torch.from_numpy(np.array(W.row_seeds(cfg, B), dtype=np.uint64).view(np.int64)).cuda()
    ws = cg.new_workspace(B, V)
    fws = g.new_fill_workspace(B)
    logits = W.make_logits(cfg, 0, B, V, "cuda")
    out = []
    for fused in (False, True):
        s_st, s_steps = st.clone(), steps.clone()
        status = torch.zeros(B, dtype=torch.int32, device="cuda")
        ids = torch.empty(B, dtype=torch.int32, device="cuda")
        lp = torch.empty(B, dtype=torch.float32, device="cuda")
        mask = torch.empty((B, g.W), dtype=torch.int64, device="cuda")
        g.fill_bitmask(s_st, mask, fws)
        if fused:
            g.sample_advance_fill(logits, mask, temp, seed, s_steps, ws, ids, lp, s_st, status, fws)
        else:
            g.sample_advance(logits, mask, temp, seed, s_steps, ws, ids, lp, s_st, status)
            g.fill_bitmask(s_st, mask, fws)
        torch.cuda.synchronize()
        out.append((ids, lp.view(torch.int32), s_st, s_steps, status, mask))
    for a, b in zip(*out):
        assert torch.equal(a, b)
    assert int((out[0][4] == cg.ROW_OK).sum()) + int((out[0][4] == cg.ROW_DONE).sum()) > B // 2


@pytest.mark.parametrize("max_len", [4, 12, 28])
def test_fill_token_length_classes(max_len):
    """The walk is specialised by the longest token's length in 4-byte words;
    vocabularies whose longest token is 4, 12 or 28 bytes (the tool-call
    vocabulary cut to that length, duplicates dropped, one token padded to
    the full length) reach the word counts the workloads do not: masks of
    rows at random legal prefixes against the oracle, bit-exact."""
    say("token length", max_len)
    cfg = 3
    blob0, off0 = W.make_vocab(cfg, 6000)
    toks, seen = [], set()
    for i in range(len(off0) - 1):
        t = blob0[off0[i]:off0[i + 1]][:max_len]
        if t not in seen:
            seen.add(t)
            toks.append(t)
    longest = b'"' + b"a" * (max_len - 1)
    if longest not in seen:
        toks.append(longest)
    assert max(len(t) for t in toks) == max_len
    blob = b"".join(toks)
    off = np.concatenate([[0], np.cumsum([len(t) for t in toks])]).tolist()
    g = cg.Grammar(W.spec_json(cfg), blob, off)
    og = O.load_spec(W.spec_json(cfg))
    rng = W.SplitMix(0x1E7 + max_len)
    seqs, rows = [], []
    for _ in range(32):
        s, row = random_walk(og, toks, rng.below(40), rng)
        seqs.append(s)
        rows.append(row)
    st, _, _ = device_rows(g, seqs)
    want, _ = oracle_masks(og, rows, blob, off)
    got = gpu_masks(g, st)
    assert np.array_equal(got[:, :want.shape[1]], want)


def test_binding_rejects_bad_shapes():
    """The binding refuses buffers the kernels would read or write past:
    rows of the wrong width, a mask or a fill workspace too small for the
    batch (fill_walk included)."""
    import torch
    say("binding shapes")
    blob, off = W.make_vocab(3, 4096)
    g = cg.Grammar(W.spec_json(3), blob, off, gen_cap=W.GEN_CAP)
    B = 8
    st = g.new_states(B)
    g.init_state(st)
    mask = torch.zeros((B, g.W), dtype=torch.int64, device="cuda")
    fws = g.new_fill_workspace(B)
    g.fill_bitmask(st, mask, fws)
    bad = torch.zeros((B, cg.STATE_BYTES + 8), dtype=torch.uint8, device="cuda")
    for call in (lambda: g.fill_bitmask(bad, mask, fws), lambda: g.init_state(bad),
                 lambda: g.fill_walk(bad, mask, fws), lambda: g.fill_bitmask_noalloc(bad, mask)):
        with pytest.raises(ValueError):
            call()
    with pytest.raises(ValueError):
        g.fill_walk(st, mask[:B - 1], fws)
    with pytest.raises(ValueError):
        g.fill_walk(st, mask, g.new_fill_workspace(1)[:1])
    with pytest.raises(ValueError):
        g.fill_bitmask(st, mask, g.new_fill_workspace(1)[:1])
    torch.cuda.synchronize()
