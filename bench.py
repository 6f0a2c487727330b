"""Benchmark of the constrained-decoding hot path on one MI355X.

A step is one pass of the whole path over the batch: mask_softmax_sample +
advance + the next step's fill_bitmask, as cg_sample_advance_fill (one
launch samples, commits and plans each row's next mask; a second walks the
listed token tiles).  --plain-fill runs cg_fill_bitmask then
cg_sample_advance; --separate runs cg_fill_bitmask, cg_apply_mask_sample and
cg_advance as three calls.  Workload: the tool-call grammar (8 tools),
vocabulary 128,256, batch 256, bf16 N(0, 3^2) logits, T = 0.7 Philox
Gumbel sampling, a 256-step trajectory from the start state (the 256-token
bench cap of "Constrained decoding", "What it is worth"), engine cap 2048.
Logits for every step are generated before the timed region and stay in HBM.

Prints one JSON line.  --gpus above 1 is refused: the path shards by rows
with no exchange, and bench.py measures one GPU.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E
CONFIG = 3
WORKLOADS = {
    1: "calc span grammar, vocab 512, batch 4, fp32 N(0,1) logits, greedy",
    2: "decision schema, vocab 32000, batch 64, fp32 N(0,4) logits, T=0.7 Philox two-level Gumbel",
    3: "tool-call grammar (8 tools), vocab 128256, batch 256, bf16 N(0,9) logits, T=0.7 Philox two-level Gumbel",
    4: "integer-answer contract, vocab 151936, batch 1024, bf16 N(0,1) logits, greedy",
    5: "recursive JSON, vocab 256000, batch 512, bf16 Student-t(3) logits, T=1.0 Philox two-level Gumbel",
    6: "text with calc spans, vocab 128256, batch 256, bf16 N(0,9) logits, T=0.7 Philox two-level Gumbel",
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_sample_hbm_traffic_toolcall_v128k_b256.md")
# the sources of the measured launch: the sampler and the plan it runs
KERNEL_SRCS = [os.path.join(ROOT, "logit_masking_amd", "csrc", f) for f in ("sample.hip", "fill_plan.hpp")]


def kernel_source_sha():
    import hashlib
    h = hashlib.sha256()
    for p in KERNEL_SRCS:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per k_sample launch from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by a device copy of known size),
    or None when the kernels have changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE):
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].split(": ", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("sample.hip + fill_plan.hpp sha256") != kernel_source_sha():
        return None
    try:
        return float(vals["hbm bytes per launch"])
    except (KeyError, ValueError):
        return None


def read_floor(pool, mask, B, V, es, W, stream, reps=72):
    """The memory floor of the masked-sample launch: libcg_floor.so's
    read-only kernel (the sampler's grid, chunk walk and bytes, no
    arithmetic) over the same logits pool, an event pair around each launch
    as for the sampler.  None when that library is not built."""
    import ctypes

    import torch
    path = os.path.join(ROOT, "logit_masking_amd", "libcg_floor.so")
    if not os.path.exists(path):
        return None
    f = ctypes.CDLL(path).cg_floor_read_rows
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p,
                  ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    out_mask = torch.empty_like(mask)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for i, (e0, e1) in enumerate(evs):
        x = pool[i % len(pool)]
        e0.record(stream)
        assert f(x.data_ptr(), es, B, V, x.stride(0), mask.data_ptr(), W, out_mask.data_ptr(), stream.cuda_stream) == 0
        e1.record(stream)
    torch.cuda.synchronize()
    ms = np.array([e0.elapsed_time(e1) for e0, e1 in evs[8:]])
    nbytes = B * V * es + 2 * B * W * 8
    return {"kernel": "k_read_floor (the sampler's grid, chunk walk and bytes: logits and mask read, a mask "
                      "written; no arithmetic)",
            "bytes": nbytes, "us": round(1e3 * ms.mean(), 2), "p50_us": round(1e3 * pct(ms, 50), 2),
            "GBps": round(nbytes / (ms.mean() * 1e-3) / 1e9, 1),
            "frac_of_peak": round(nbytes / (ms.mean() * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}


def pct(a, q):
    return float(np.percentile(np.asarray(a), q))


def cpu_baseline(rec, B, V, blob, off, budget_s, cfg=CONFIG):
    """The oracle as it stands, on a bounded sample of the same workload, and
    the run's own parity check: the checked rows of the measured trajectory
    (rec["rows"]) are replayed on the host from the GPU's own logits.  At
    every step each row still generating gets a full-vocabulary oracle mask
    (compared word by word with the mask the device used) and a float64
    two-level sample (compared with the device's pick and log-probability;
    a pick whose oracle margin at either level is below 1e-6 is a near-tie,
    counted apart); the row then takes the device's pick, whose status must
    equal the oracle's.  Finished rows must have an empty mask and id -1.
    Only the oracle's mask and sample work is timed, until the budget is
    spent ("Constrained Decoding Under Matched Conditions", "The artifact
    validator does not trust the remote summary": the run recounts its own
    results)."""
    import logit_masking_amd.workloads as W
    from oracle import oracle as O
    og = O.load_spec(W.spec_json(cfg))
    toks = [blob[off[i]:off[i + 1]] for i in range(V)]
    threads = min(16, os.cpu_count() or 1)
    chk = rec["rows"]
    rows = [O.Row(og, W.GEN_CAP) for _ in chk]
    seeds = W.row_seeds(cfg, B)
    T = W.CONFIGS[cfg]["T"]
    Wv = (V + 63) // 64
    par = {"rows_checked": len(chk), "row_steps": 0, "steps_checked": 0, "mask_word_mismatches": 0,
           "pick_mismatches": 0, "near_ties": 0, "max_logprob_err": 0.0, "status_mismatches": 0,
           "finished_row_violations": 0, "blank_live_rows": 0}
    checks = walked = 0
    t_cpu = t_mask = 0.0
    t1 = None
    # the warmup steps before the measured trajectory: the rows follow the
    # device's picks unchecked
    for s in range(rec["pre_ids"].shape[0]):
        for k in range(len(chk)):
            i = int(rec["pre_ids"][s, chk[k]])
            rows[k].advance(None if i < 0 else toks[i])
    for s in range(rec["ids"].shape[0]):
        live = [k for k in range(len(chk)) if not rows[k].done]
        for k in range(len(chk)):
            if rows[k].done and (rec["masks"][s, k, :Wv].any() or rec["ids"][s, chk[k]] != -1):
                par["finished_row_violations"] += 1
        if not live or t_cpu >= budget_s:
            break
        x = rec["x"][s]  # the checked rows' logits at this step (bf16 bits or float32)
        if x.dtype == np.uint16:
            x = (x.astype(np.uint32) << np.uint32(16)).view(np.float32)
        t0 = time.perf_counter()
        words, w = og.mask_rows([rows[k].conf for k in live], [False] * len(live), blob, off, threads)
        tm = time.perf_counter()
        res = [O.sample_row(x[k].astype(np.float64), O.unpack_mask(words[j], V), T, seeds[chk[k]], rows[k].step)
               for j, k in enumerate(live)]
        t_cpu += time.perf_counter() - t0
        t_mask += tm - t0
        if s == 20:  # the same masks again on one thread (rows in mixed states by now)
            u0 = time.perf_counter()
            og.mask_rows([rows[k].conf for k in live], [False] * len(live), blob, off, 1)
            t1 = (len(live) * V, time.perf_counter() - u0, tm - t0)
        checks += len(live) * V
        walked += w
        par["row_steps"] += len(live)
        par["steps_checked"] = s + 1
        for j, k in enumerate(live):
            r = chk[k]
            par["mask_word_mismatches"] += int(np.count_nonzero(rec["masks"][s, k, :Wv] != words[j][:Wv]))
            if not words[j].any():
                par["blank_live_rows"] += 1
            i, lp, info = res[j]
            gi, glp = int(rec["ids"][s, r]), float(rec["lp"][s, r])
            near = T > 0 and min(info["margin_chunk"], info["margin_token"]) < 1e-6
            par["near_ties"] += int(near)
            if gi != i:
                par["pick_mismatches"] += int(not near)
            else:
                par["max_logprob_err"] = max(par["max_logprob_err"], abs(glp - lp))
            # the oracle row follows the device's pick
            st = rows[k].advance(None if gi < 0 else toks[gi])
            par["status_mismatches"] += int(st != int(rec["status"][s, r]))
    par["rows_done"] = sum(int(r.complete) for r in rows)
    par["rows_capped"] = sum(int(r.done and not r.complete) for r in rows)
    par["max_logprob_err"] = float(f"{par['max_logprob_err']:.3g}")
    base = {
        "value": checks / t_cpu if t_cpu > 0 else None,
        "unit": "token-checks/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"rows {chk[0]}-{chk[-1]} of the measured trajectory on the device's own logits, steps "
                  f"0-{par['steps_checked'] - 1}, every row still generating: full-vocabulary mask + float64 "
                  f"two-level sample per row-step; {par['row_steps']} row-steps, {checks} token checks, "
                  f"{walked / max(1, checks):.2f} bytes walked per check, {t_cpu:.1f} s",
        "us_per_row_step": 1e6 * t_cpu / max(1, par["row_steps"]),
        "mask_token_checks_per_s": checks / t_mask if t_mask > 0 else None,
        "sample_GBps": (par["row_steps"] * (2 * V + 8 * ((V + 63) // 64) + 8) / (t_cpu - t_mask) / 1e9
                        if t_cpu > t_mask else None),
        "mask_step20_token_checks_per_s": ({"threads": threads, "value": t1[0] / t1[2], "1_thread": t1[0] / t1[1]}
                                          if t1 and t1[1] > 0 and t1[2] > 0 else None),
        "bytes_walked_per_check": walked / max(1, checks),
        "nproc": os.cpu_count(),
        "cpu_model": cpu_model(),
    }
    return base, par


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def state_classes(g, cg, st0, pool, temp, seed, steps, ws, fws, B, V, stream, reps=30):
    """The fill and the sample timed on two batches of one state class
    each: every row in the state of the densest live row at the start of
    the timed region (inside a string, where most tokens may follow) and
    every row in the sparsest one's (a structural state).  Events on the
    launch stream around each of `reps` calls; the states are not changed."""
    import torch
    mask = torch.empty((B, g.W), dtype=torch.int64, device=st0.device)
    g.fill_bitmask(st0, mask, fws, stream)
    torch.cuda.synchronize()
    bits = np.unpackbits(mask.cpu().numpy().view(np.uint8), axis=1).sum(axis=1)
    live = np.nonzero(bits > 0)[0]
    if len(live) == 0:
        return None
    picks = {"string_interior": int(live[np.argmax(bits[live])]),
             "structural": int(live[np.argmin(bits[live])])}
    ids = torch.empty(B, dtype=torch.int32, device=st0.device)
    lp = torch.empty(B, dtype=torch.float32, device=st0.device)
    out = {}
    for name, r in picks.items():
        st = st0[r:r + 1].repeat(B, 1).contiguous()
        g.fill_bitmask(st, mask, fws, stream)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
        torch.cuda.synchronize()
        for i in range(reps):
            ev[i][0].record(stream)
            g.fill_bitmask(st, mask, fws, stream)
            ev[i][1].record(stream)
            cg.apply_mask_sample(pool[i % len(pool)], mask, temp, seed, steps, ws, ids, lp, stream=stream)
            ev[i][2].record(stream)
        torch.cuda.synchronize()
        f = np.array([e[0].elapsed_time(e[1]) for e in ev]) * 1e3
        sm = np.array([e[1].elapsed_time(e[2]) for e in ev]) * 1e3
        out[name] = {"row": r, "allowed_frac": round(float(bits[r]) / V, 4),
                     "us_fill": round(float(f.mean()), 2), "us_sample": round(float(sm.mean()), 2)}
    return out


def inject_bench(args):
    """--inject: the decode loop of text with calc spans (vocab 128,256, batch
    256, bf16, T = 0.7), the logits leaning toward each row's script so that
    rows write spans.  After every step the host reads the statuses; rows at
    CG_ROW_INJECT get their span evaluated (cg_eval_calc) and the result
    forced (cg_force_bytes) before the next step ("Evaluator aware decoding",
    "A concrete prototype on llama.cpp": injected-token counts and the
    latency of each injection).  Prints one JSON line."""
    import torch
    import logit_masking_amd as cg
    from logit_masking_amd import workloads as W
    cfg = 6
    c = W.CONFIGS[cfg]
    B, T = c["B"], c["T"]
    blob, off = W.make_vocab(cfg)
    V = len(off) - 1
    toks = [blob[off[i]:off[i + 1]] for i in range(V)]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    g = cg.Grammar(W.spec_json(cfg), blob, off, gen_cap=W.GEN_CAP)
    pre = W.ScriptTokens(toks)
    rng = W.SplitMix(c["seed"])
    scripts = [W.calc_text_script(rng, W.SPECS[cfg], 2 + rng.below(4)) for _ in range(B)]
    npool = max(1, min(args.pool, args.steps))
    pool = [W.make_logits(cfg, s, B, V, dev) for s in range(npool)]
    st = g.new_states(B, dev)
    g.init_state(st)
    steps = torch.zeros(B, dtype=torch.int32, device=dev)
    status = torch.zeros(B, dtype=torch.int32, device=dev)
    fstatus = torch.zeros(B, dtype=torch.int32, device=dev)
    mask = torch.empty((B, g.W), dtype=torch.int64, device=dev)
    temp = torch.full((B,), T, dtype=torch.float32, device=dev)
    seed = torch.from_numpy(np.array(W.row_seeds(cfg, B), dtype=np.uint64).view(np.int64)).to(dev)
    ws = cg.new_workspace(B, V, dev)
    fws = g.new_fill_workspace(B, dev)
    ids = torch.empty(B, dtype=torch.int32, device=dev)
    lp = torch.empty(B, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    texts = [bytearray() for _ in range(B)]
    seg_i, seg_start = [0] * B, [0] * B
    done = [False] * B
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    dev_step_ms, inj_wall, inj_eval, inj_kernel, inj_rows, inj_bytes, inj_toks = [], [], [], [], [], [], []
    # load every kernel and the evaluator once before anything is timed
    g.force_bytes(st, torch.zeros(1, dtype=torch.uint8, device=dev), torch.zeros(B + 1, dtype=torch.int32, device=dev),
                  fstatus, stream)
    cg.eval_calc(b"<calc>1</calc>")
    torch.cuda.synchronize()
    n_err = 0
    for s in range(args.warmup + args.steps):
        # untimed: lean each row's logits toward the next token of its script
        ri, ti = [], []
        for r in range(B):
            if done[r]:
                continue
            seg = scripts[r][min(seg_i[r], len(scripts[r]) - 1)]
            written = bytes(texts[r][seg_start[r]:])
            if seg.startswith(written) and len(written) < len(seg):
                ri.append(r)
                ti.append(pre.longest(seg[len(written):]))
        x = pool[s % npool].clone()
        if ri:
            ri_t, ti_t = torch.tensor(ri, device=dev), torch.tensor(ti, device=dev)
            x[ri_t, ti_t] = x[ri_t, ti_t] + 40.0
        torch.cuda.synchronize()
        ev[0].record(stream)
        g.fill_bitmask(st, mask, fws, stream)
        g.sample_advance(x, mask, temp, seed, steps, ws, ids, lp, st, status, stream)
        ev[1].record(stream)
        ids_h = ids.cpu().numpy()          # the engine reads the picks back anyway
        stat_h = status.cpu().numpy()
        dev_step_ms.append(ev[0].elapsed_time(ev[1]))
        for r in range(B):
            if ids_h[r] >= 0 and stat_h[r] not in (cg.ROW_REJECTED, cg.ROW_NOOP):
                texts[r] += toks[ids_h[r]]
            if stat_h[r] in (cg.ROW_DONE, cg.ROW_CAPPED):
                done[r] = True
        inj = [r for r in range(B) if stat_h[r] == cg.ROW_INJECT]
        if not inj:
            if all(done):
                break
            continue
        # the injection: evaluate the closed spans on the host, force the results
        t0 = time.perf_counter()
        data, offs = bytearray(), [0]
        k = 0
        for r in range(B):
            if k < len(inj) and inj[k] == r:
                rc, v = cg.eval_calc(bytes(texts[r][texts[r].rindex(b"<calc>"):]))
                if rc == cg.CG_OK:
                    res = b"<result>%d</result>" % v
                else:
                    res = b"<result_error>" + v.encode() + b"</result_error>"
                    n_err += 1
                data += res
                texts[r] += res
                k += 1
            offs.append(len(data))
        t1 = time.perf_counter()
        h_data = torch.frombuffer(data, dtype=torch.uint8).pin_memory()
        h_offs = torch.tensor(offs, dtype=torch.int32).pin_memory()
        d_data = h_data.to(dev, non_blocking=True)
        d_offs = h_offs.to(dev, non_blocking=True)
        ev[2].record(stream)
        g.force_bytes(st, d_data, d_offs, fstatus, stream)
        ev[3].record(stream)
        fst = fstatus.cpu().numpy()
        t2 = time.perf_counter()
        for r in inj:
            if fst[r] != cg.ROW_OK:
                raise RuntimeError(f"forced result refused on row {r}: status {fst[r]}")
            seg_i[r] += 1
            seg_start[r] = len(texts[r])
        if s >= args.warmup:
            inj_wall.append(t2 - t0)
            inj_eval.append(t1 - t0)
            inj_kernel.append(ev[2].elapsed_time(ev[3]))
            inj_rows.append(len(inj))
            for r in inj:
                res = bytes(data[offs[r]:offs[r + 1]])
                inj_bytes.append(len(res))
                inj_toks.append(pre.count(res))
    n_inj = int(sum(inj_rows))
    wall = np.array(inj_wall) * 1e6
    ev_us = np.array(inj_eval) * 1e6 / np.maximum(1, np.array(inj_rows))
    out = {
        "metric": "injection latency per decode step with injections (host evaluation + forced-byte walk), "
                  "median us",
        "value": round(pct(wall, 50), 2) if len(wall) else None,
        "unit": "us",
        "n_gpus": 1,
        "steps": len(dev_step_ms) - args.warmup,
        "warmup": args.warmup,
        "higher_is_better": False,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "text with calc spans, vocab 128256, batch 256, bf16 N(0,9) logits leaning +40 "
                               "toward each row's script, T=0.7, engine cap 2048", "batch": B, "vocab": V},
        "injection_steps": len(wall),
        "injected_rows": n_inj,
        "error_results": n_err,
        "us_per_injection_step": {"mean": round(float(wall.mean()), 2), "p50": round(pct(wall, 50), 2),
                                  "p99": round(pct(wall, 99), 2)} if len(wall) else None,
        "injected_rows_per_step": round(float(np.mean(inj_rows)), 2) if inj_rows else None,
        "us_host_eval_per_span": {"p50": round(pct(ev_us, 50), 2), "p99": round(pct(ev_us, 99), 2)} if len(ev_us) else None,
        "us_force_kernel": {"p50": round(1e3 * pct(inj_kernel, 50), 2), "p99": round(1e3 * pct(inj_kernel, 99), 2)}
        if inj_kernel else None,
        "injected_bytes_mean": round(float(np.mean(inj_bytes)), 2) if inj_bytes else None,
        "injected_tokens_mean": round(float(np.mean(inj_toks)), 2) if inj_toks else None,
        "us_device_step": {"p50": round(1e3 * pct(dev_step_ms[args.warmup:], 50), 2),
                           "mean": round(1e3 * float(np.mean(dev_step_ms[args.warmup:])), 2)},
        "note": "latency = from the step's statuses on the host to the forced statuses back on the host: "
                "span evaluation for every row at CG_ROW_INJECT, the results' bytes to the device, "
                "cg_force_bytes, and the statuses read back",
        "rows_done": int(sum(done)),
    }
    print(json.dumps(out))


def draft_bench(args):
    """--draft K: masks along K-token drafts at the tool-call workload (vocab
    128,256, batch 256).  The drafts are the trajectory's own next K tokens
    (all legal), taken from the states of a recorded 256-step run.  One
    cg_fill_draft call (the path walk + one fill over B (K+1) configurations)
    is timed against the same masks made one position at a time (K + 1
    fills and K advances).  Prints one JSON line."""
    import torch
    import logit_masking_amd as cg
    from logit_masking_amd import workloads as W
    c = W.CONFIGS[CONFIG]
    B, T, K = c["B"], c["T"], args.draft
    blob, off = W.make_vocab(CONFIG)
    V = len(off) - 1
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    g = cg.Grammar(W.spec_json(CONFIG), blob, off, gen_cap=W.GEN_CAP)
    n = 96
    st = g.new_states(B, dev)
    g.init_state(st)
    steps = torch.zeros(B, dtype=torch.int32, device=dev)
    status = torch.zeros(B, dtype=torch.int32, device=dev)
    mask = torch.empty((B, g.W), dtype=torch.int64, device=dev)
    temp = torch.full((B,), T, dtype=torch.float32, device=dev)
    seed = torch.from_numpy(np.array(W.row_seeds(CONFIG, B), dtype=np.uint64).view(np.int64)).to(dev)
    ws = cg.new_workspace(B, V, dev)
    fws = g.new_fill_workspace(B, dev)
    ids_hist = torch.full((n + K, B), -1, dtype=torch.int32, device=dev)
    lp = torch.empty(B, dtype=torch.float32, device=dev)
    hist_st, hist_steps = [], []
    for s in range(n + K):
        hist_st.append(st.clone())
        hist_steps.append(steps.clone())
        logits = W.make_logits(CONFIG, s % 64, B, V, dev)
        g.fill_bitmask(st, mask, fws)
        g.sample_advance(logits, mask, temp, seed, steps, ws, ids_hist[s], lp, st, status)
    torch.cuda.synchronize()
    path = torch.empty((B, K + 1, cg.STATE_BYTES), dtype=torch.uint8, device=dev)
    masks = torch.empty((B, K + 1, g.W), dtype=torch.int64, device=dev)
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    dws = torch.empty(max(2, (g.draft_workspace_bytes(B, K) + 15) // 16 * 2), dtype=torch.int64, device=dev)
    drafts = [ids_hist[s:s + K].t().contiguous() for s in range(n)]
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    acc_sum = 0
    st2 = g.new_states(B, dev)
    steps2 = torch.zeros(B, dtype=torch.int32, device=dev)
    for rep in range(2):  # the first pass loads the kernels
        for s in range(n):
            ev[s][0].record(stream)
            g.fill_draft(hist_st[s], hist_steps[s], drafts[s], path, masks, acc, dws, stream)
            ev[s][1].record(stream)
            if rep == 1:
                acc_sum += int(acc.sum().item())
            # the same positions one at a time
            st2.copy_(hist_st[s])
            steps2.copy_(hist_steps[s])
            evs[s][0].record(stream)
            for j in range(K + 1):
                g.fill_bitmask(st2, mask, fws, stream)
                if j < K:
                    g.advance(st2, drafts[s][:, j].contiguous(), steps2, status, stream)
            evs[s][1].record(stream)
        torch.cuda.synchronize()
    t_draft = np.array([a.elapsed_time(b) for a, b in ev]) * 1e3
    t_seq = np.array([a.elapsed_time(b) for a, b in evs]) * 1e3
    out = {
        "metric": f"masks along {K}-token drafts: us per cg_fill_draft call (batch {B})",
        "value": round(pct(t_draft, 50), 2),
        "unit": "us",
        "n_gpus": 1,
        "higher_is_better": False,
        "dtype": "int (automaton)",
        "data": "synthetic",
        "config": {"workload": f"tool-call grammar (8 tools), vocab {V}, batch {B}, drafts = the next {K} tokens "
                               f"of a recorded T=0.7 trajectory, {n} draft positions", "batch": B, "vocab": V, "k": K},
        "us_fill_draft": {"p50": round(pct(t_draft, 50), 2), "mean": round(float(t_draft.mean()), 2)},
        "us_one_position_at_a_time": {"p50": round(pct(t_seq, 50), 2), "mean": round(float(t_seq.mean()), 2)},
        "token_checks_per_s": round(B * (K + 1) * V / (pct(t_draft, 50) * 1e-6), 1),
        "draft_tokens_legal_mean": round(acc_sum / (n * B), 3),
    }
    print(json.dumps(out))


def overlap_bench(args):
    """--overlap: the mask is a function of the rows' states alone, so it can
    be computed while the model's forward pass runs ("Evaluator aware
    decoding", "Why isn't this in production APIs yet?").  A stand-in for the
    end of the forward pass -- the lm_head product of a batch of hidden
    states (4096 wide, bf16) with a [4096, 128256] weight, which makes the
    step's logits -- runs on the main stream while cg_fill_bitmask runs on a
    second stream; cg_sample_advance waits for both.  Timed against the same
    three calls on one stream.  Tool-call workload, batch 256.  Prints one
    JSON line."""
    import torch
    import logit_masking_amd as cg
    from logit_masking_amd import workloads as W
    c = W.CONFIGS[CONFIG]
    B, T = c["B"], c["T"]
    blob, off = W.make_vocab(CONFIG)
    V = len(off) - 1
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    g = cg.Grammar(W.spec_json(CONFIG), blob, off, gen_cap=W.GEN_CAP)
    hidden = 4096
    gen = torch.Generator(device=dev)
    gen.manual_seed(12345)
    w_head = (torch.randn((hidden, V), generator=gen, device=dev) * (3.0 / hidden ** 0.5)).to(torch.bfloat16)
    hs = [torch.randn((B, hidden), generator=gen, device=dev).to(torch.bfloat16) for _ in range(8)]
    mask = torch.empty((B, g.W), dtype=torch.int64, device=dev)
    temp = torch.full((B,), T, dtype=torch.float32, device=dev)
    seed = torch.from_numpy(np.array(W.row_seeds(CONFIG, B), dtype=np.uint64).view(np.int64)).to(dev)
    ws = cg.new_workspace(B, V, dev)
    fws = g.new_fill_workspace(B, dev)
    ids = torch.empty(B, dtype=torch.int32, device=dev)
    lp = torch.empty(B, dtype=torch.float32, device=dev)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream(device=dev)  # default priority
    n = args.steps

    def run(overlap, st, steps, status):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ready = torch.cuda.Event()
        torch.cuda.synchronize()
        e0.record(main)
        for s in range(n):
            if overlap:
                side.wait_stream(main)                 # the previous step's advance
                g.fill_bitmask(st, mask, fws, side)
                ready.record(side)
                logits = torch.matmul(hs[s % len(hs)], w_head)
                main.wait_event(ready)
            else:
                g.fill_bitmask(st, mask, fws, main)
                logits = torch.matmul(hs[s % len(hs)], w_head)
            g.sample_advance(logits, mask, temp, seed, steps, ws, ids, lp, st, status, main)
        e1.record(main)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    def fresh():
        st = g.new_states(B, dev)
        g.init_state(st)
        return st, torch.zeros(B, dtype=torch.int32, device=dev), torch.zeros(B, dtype=torch.int32, device=dev)

    for _ in range(2):  # load kernels and the GEMM plan
        run(False, *fresh())
        run(True, *fresh())
    st_a, steps_a, status_a = fresh()
    us_serial = run(False, st_a, steps_a, status_a)
    st_b, steps_b, status_b = fresh()
    us_overlap = run(True, st_b, steps_b, status_b)
    same = bool(torch.equal(st_a, st_b) and torch.equal(steps_a, steps_b))
    # the product alone
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(main)
    for s in range(n):
        torch.matmul(hs[s % len(hs)], w_head)
    e1.record(main)
    torch.cuda.synchronize()
    us_gemm = e0.elapsed_time(e1) * 1e3 / n
    out = {
        "metric": "us per decode step with the fill on a second stream, behind a stand-in lm_head product",
        "value": round(us_overlap, 2),
        "unit": "us",
        "n_gpus": 1,
        "steps": n,
        "higher_is_better": False,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"tool-call grammar (8 tools), vocab {V}, batch {B}; lm_head stand-in "
                               f"[{B}, {hidden}] x [{hidden}, {V}] bf16 (hipBLASLt via torch.matmul)",
                   "batch": B, "vocab": V},
        "us_step_one_stream": round(us_serial, 2),
        "us_step_fill_on_second_stream": round(us_overlap, 2),
        "us_lm_head_alone": round(us_gemm, 2),
        "same_trajectory": same,
    }
    print(json.dumps(out))


def compile_times(args):
    """--compile-times: cg_compile_grammar for every workload, the grammar
    cache cleared first: the spec-to-automaton part and the whole call
    (vocabulary tables, precomputed masks, upload), host wall-clock.  The
    pages keep compilation out of latency with warm-up and ask that caching
    keep it from blowing up ("Constrained Decoding Under Matched Conditions";
    "Evaluator aware decoding", "Where XGrammar-2 could take this").  Prints
    one JSON line."""
    import torch
    import logit_masking_amd as cg
    from logit_masking_amd import workloads as W
    torch.cuda.set_device(0)
    res = {}
    for cfg in sorted(W.SPECS):
        blob, off = W.make_vocab(cfg)
        cg.cache_clear()
        t0 = time.perf_counter()
        g = cg.Grammar(W.spec_json(cfg), blob, off, gen_cap=W.GEN_CAP)
        wall = 1e3 * (time.perf_counter() - t0)
        info = g.info()
        t1 = time.perf_counter()
        g2 = cg.Grammar(W.spec_json(cfg), blob, off, gen_cap=W.GEN_CAP)  # answered from the cache
        cached = 1e3 * (time.perf_counter() - t1)
        res[str(cfg)] = {"vocab": len(off) - 1, "automaton_ms": round(info["compile_ms"], 2),
                         "total_ms": round(info["total_ms"], 2), "binding_wall_ms": round(wall, 2),
                         "cached_ms": round(cached, 3), "table_bytes": info["table_bytes"],
                         "state_masks": info["state_masks"],
                         "max_bytes": info["max_bytes"] if info["max_bytes"] >= 0 else None}
        del g, g2
    print(json.dumps({"metric": "cg_compile_grammar time per workload (ms)", "unit": "ms", "n_gpus": 1,
                      "higher_is_better": False, "data": "synthetic", "configs": res}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--pool", type=int, default=64, help="distinct logits buffers cycled over the steps")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--separate", action="store_true",
                    help="cg_apply_mask_sample and cg_advance as two launches instead of cg_sample_advance")
    ap.add_argument("--plain-fill", action="store_true",
                    help="cg_fill_bitmask + cg_sample_advance per step, instead of cg_sample_advance_fill (the next "
                         "step's mask planned in the sampler's launch, then walked)")
    ap.add_argument("--no-classes", action="store_true",
                    help="skip the per-state-class timings (a kernel trace then holds the trajectory's launches only)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a 64 MiB device-to-device copy (reference for HBM byte counters)")
    ap.add_argument("--config", type=int, default=CONFIG,
                    help="workload (1-6); the headline line is config 3, the others are for reference")
    ap.add_argument("--draft", type=int, default=0,
                    help="measure masks along K-token drafts instead (its own JSON line)")
    ap.add_argument("--overlap", action="store_true",
                    help="measure the fill on a second stream behind a stand-in lm_head product (its own JSON line)")
    ap.add_argument("--inject", action="store_true",
                    help="measure result injection on text with calc spans instead (its own JSON line)")
    ap.add_argument("--compile-times", action="store_true",
                    help="time cg_compile_grammar for every workload instead (its own JSON line)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: rows shard across GPUs with no exchange, and runs on more than one "
              "GPU are not supported", file=sys.stderr)
        sys.exit(2)

    if args.inject:
        inject_bench(args)
        return
    if args.compile_times:
        compile_times(args)
        return
    if args.draft:
        draft_bench(args)
        return
    if args.overlap:
        overlap_bench(args)
        return

    import torch
    import logit_masking_amd as cg
    from logit_masking_amd import workloads as W

    cfg = args.config
    c = W.CONFIGS[cfg]
    B, T = c["B"], c["T"]
    blob, off = W.make_vocab(cfg)
    V = len(off) - 1
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    g = cg.Grammar(W.spec_json(cfg), blob, off, gen_cap=W.GEN_CAP)
    info = g.info()
    total = args.warmup + args.steps
    es = 2 if c["dtype"] == "bf16" else 4
    # the pool of logits buffers stays within 16 GB of HBM
    npool = max(1, min(args.pool, total, (16 << 30) // (B * V * es)))
    pool = [W.make_logits(cfg, s, B, V, dev) for s in range(npool)]
    st = g.new_states(B, dev)
    g.init_state(st)
    steps = torch.zeros(B, dtype=torch.int32, device=dev)
    status = torch.zeros(B, dtype=torch.int32, device=dev)
    mask = torch.empty((B, g.W), dtype=torch.int64, device=dev)
    temp = torch.full((B,), T, dtype=torch.float32, device=dev)
    seed = torch.from_numpy(np.array(W.row_seeds(cfg, B), dtype=np.uint64).view(np.int64)).to(dev)
    ws = cg.new_workspace(B, V, dev)
    fws = g.new_fill_workspace(B, dev)
    ids_hist = torch.full((total, B), -1, dtype=torch.int32, device=dev)
    lp = torch.empty(B, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(s, ev=None):
        ids = ids_hist[s]
        if fused_fill:
            # this step's mask was left by the previous call (the first by
            # cg_fill_bitmask); timed apart, the call's two launches are made
            # as two calls with events between them
            if ev is None:
                g.sample_advance_fill(pool[s % npool], mask, temp, seed, steps, ws, ids, lp, st, status, fws, stream)
                return
            ev[0].record(stream)
            g.sample_advance_fill(pool[s % npool], mask, temp, seed, steps, ws, ids, lp, st, status, fws, stream,
                                  split=True)
            ev[1].record(stream)
            g.fill_walk(st, mask, fws, stream)
            ev[2].record(stream)
            ev[3].record(stream)
            return
        if ev is not None:
            ev[0].record(stream)
        g.fill_bitmask(st, mask, fws, stream)
        if ev is not None:
            ev[1].record(stream)
        if args.separate:
            cg.apply_mask_sample(pool[s % npool], mask, temp, seed, steps, ws, ids, lp, stream=stream)
            if ev is not None:
                ev[2].record(stream)
            g.advance(st, ids, steps, status, stream)
        else:
            # mask_softmax_sample + advance in one launch
            g.sample_advance(pool[s % npool], mask, temp, seed, steps, ws, ids, lp, st, status, stream)
            if ev is not None:
                ev[2].record(stream)
        if ev is not None:
            ev[3].record(stream)

    fused_fill = not (args.plain_fill or args.separate)
    if fused_fill:
        g.fill_bitmask(st, mask, fws, stream)
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    # the timed region: K steps between two events, nothing else on the stream
    st0, steps0, mask0 = st.clone(), steps.clone(), mask.clone()
    start_ev = torch.cuda.Event(enable_timing=True)
    end_ev = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start_ev.record(stream)
    for k in range(args.steps):
        step(args.warmup + k)
    end_ev.record(stream)
    t_enq = time.perf_counter() - t0  # host time to enqueue the K steps (no synchronisation inside)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region_ms = start_ev.elapsed_time(end_ev)
    ms_per_step = region_ms / args.steps
    st_h = steps.cpu().numpy()
    flags = st.cpu().numpy()[:, 18]
    # the same K steps replayed from the same configurations with an event
    # pair around every launch: per-kernel durations on the launch stream
    st.copy_(st0)
    steps.copy_(steps0)
    mask.copy_(mask0)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        step(args.warmup + k, evs[k])
    torch.cuda.synchronize()
    if fused_fill:  # [0, 1): sample + advance + next plan; [1, 2): the walk
        samp_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
        fill_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    else:
        fill_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
        samp_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    adv_ms = np.array([e[2].elapsed_time(e[3]) for e in evs])
    assert np.array_equal(steps.cpu().numpy(), st_h), "replay diverged from the timed trajectory"
    # and once more with one event at each step boundary only (an event
    # between two launches stretches the step): the step's percentiles
    st.copy_(st0)
    steps.copy_(steps0)
    mask.copy_(mask0)
    evb = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    evb[0].record(stream)
    for k in range(args.steps):
        step(args.warmup + k)
        evb[k + 1].record(stream)
    torch.cuda.synchronize()
    step_ms = np.array([evb[k].elapsed_time(evb[k + 1]) for k in range(args.steps)])
    assert np.array_equal(steps.cpu().numpy(), st_h), "replay diverged from the timed trajectory"

    # and once more, recording for the parity check (the masks of rows 0-127
    # as the sampler reads them; every row's pick, log-probability and
    # status), with cg_fill_bitmask timed on the same states before each
    # step (the fill's own rate; in the fused step its plan runs inside the
    # sampler's launch)
    st.copy_(st0)
    steps.copy_(steps0)
    mask.copy_(mask0)
    chk = list(range(min(128, B)))
    chk_t = torch.tensor(chk, dtype=torch.long, device=dev)
    rec_mask = torch.empty((args.steps, len(chk), g.W), dtype=torch.int64, device=dev)
    rec_lp = torch.empty((args.steps, B), dtype=torch.float32, device=dev)
    rec_status = torch.empty((args.steps, B), dtype=torch.int32, device=dev)
    fmask = torch.empty_like(mask)
    fused_mask_diff = torch.zeros((), dtype=torch.int64, device=dev)
    evf = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        evf[k][0].record(stream)
        g.fill_bitmask(st, fmask, fws, stream)
        evf[k][1].record(stream)
        if fused_fill:
            rec_mask[k].copy_(mask.index_select(0, chk_t))
            fused_mask_diff += (fmask[:, :g.W] != mask[:, :g.W]).sum()
        else:
            rec_mask[k].copy_(fmask.index_select(0, chk_t))
        step(args.warmup + k)
        rec_lp[k].copy_(lp)
        rec_status[k].copy_(status)
    torch.cuda.synchronize()
    assert np.array_equal(steps.cpu().numpy(), st_h), "replay diverged from the timed trajectory"
    fillb_ms = np.array([e[0].elapsed_time(e[1]) for e in evf])

    # masked sample: every logit (bf16) and mask word read once, id + logprob
    # written; fused, also each row's state, step and status
    sample_bytes = B * V * es + B * g.W * 8 + B * 8
    if not args.separate:
        sample_bytes += B * (2 * 24 + 2 * 4 + 4)
    if fused_fill:
        sample_bytes += B * g.W * 8  # the next mask's words, written once by the plan
    sample_gbps = sample_bytes / (samp_ms.mean() * 1e-3) / 1e9
    fill_checks = B * V / (fillb_ms.mean() * 1e-3)
    dominant = "fill_bitmask" if fill_ms.mean() >= samp_ms.mean() else "mask_softmax_sample"
    kernel_name = ("k_sample (mask_softmax_sample)" if args.separate
                   else "k_sample (mask_softmax_sample + advance, one launch)" if not fused_fill
                   else "k_sample (mask_softmax_sample + advance + the next mask's plan, one launch)")
    roofline = {
        "kernel": kernel_name,
        "bound": "hbm",
        "achieved": round(sample_gbps, 1),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(sample_gbps / HBM_PEAK_GBPS, 4),
        "traffic": recorded_traffic() if cfg == CONFIG else None,
    }
    out = {
        "metric": "token-checks/s (fill_bitmask) + masked-sample GB/s vs HBM peak; µs/step",
        "value": round(B * V / (ms_per_step * 1e-3), 1),
        "unit": "token-checks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": c["dtype"],
        "data": "synthetic",
        "config": {"workload": WORKLOADS[cfg] + f", {args.steps}-step trajectory, engine cap 2048",
                   "batch": B, "vocab": V, "logits_pool": npool},
        "step": ("cg_sample_advance_fill (sample + advance + next plan; walk)" if fused_fill
                 else "cg_fill_bitmask; cg_apply_mask_sample; cg_advance" if args.separate
                 else "cg_fill_bitmask; cg_sample_advance"),
        "fill_token_checks_per_s": round(fill_checks, 1),
        "us_fill_bitmask": {"mean": round(1e3 * fillb_ms.mean(), 2), "p50": round(1e3 * pct(fillb_ms, 50), 2),
                            "p99": round(1e3 * pct(fillb_ms, 99), 2),
                            "note": "cg_fill_bitmask (plan + walk launches) on the trajectory's states before each "
                                    "step, events around the call"},
        "masked_sample_GBps": round(sample_gbps, 1),
        "masked_sample_frac_hbm": round(sample_gbps / HBM_PEAK_GBPS, 4),
        "us_per_step": {"mean": round(1e3 * ms_per_step, 2), "p50": round(1e3 * pct(step_ms, 50), 2),
                        "p99": round(1e3 * pct(step_ms, 99), 2)},
        "us_fill": {"mean": round(1e3 * fill_ms.mean(), 2), "p50": round(1e3 * pct(fill_ms, 50), 2),
                    "p99": round(1e3 * pct(fill_ms, 99), 2)},
        "us_sample": {"mean": round(1e3 * samp_ms.mean(), 2), "p50": round(1e3 * pct(samp_ms, 50), 2),
                      "p99": round(1e3 * pct(samp_ms, 99), 2)},
        "us_advance": {"mean": round(1e3 * adv_ms.mean(), 2)} if args.separate else "fused into us_sample",
        "wall_us_per_step": round(1e6 * wall / args.steps, 2),
        "host_enqueue_us_per_step": round(1e6 * t_enq / args.steps, 2),
        "dominant_kernel": dominant,
        "rows_done": int((flags & 1).sum()),
        "rows_capped": int(((flags & 2) > 0).sum()),
        "tokens_accepted_mean": float(st_h.mean()),
        "compile_ms": round(info["compile_ms"], 2),
        "compile_total_ms": round(info["total_ms"], 2),
        "table_bytes": info["table_bytes"],
        "max_bytes": info["max_bytes"] if info["max_bytes"] >= 0 else None,
        "roofline": roofline,
    }
    # a plain device-to-device copy of 256 MiB: what the memory system gives
    # a stream here, beside the published peak
    src = torch.empty(128 << 20, dtype=torch.int16, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    c0.record(stream)
    for _ in range(10):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 10 * 2 * src.numel() * 2 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst
    out["copy_GBps"] = round(copy_gbps, 1)
    out["masked_sample_frac_copy"] = round(sample_gbps / copy_gbps, 4)
    floor = read_floor(pool, mask, B, V, es, g.W, stream)
    out["read_floor"] = floor
    if floor is not None:
        # the sampler's time against the floor's, both event pairs around one launch
        out["masked_sample_frac_floor"] = round(floor["us"] / (1e3 * samp_ms.mean()), 4)
    if not (args.separate or args.no_classes):
        out["state_classes"] = state_classes(g, cg, st0, pool, temp, seed, steps0, ws, fws, B, V, stream)
    if args.calib_copy:
        src = torch.empty(32 << 20, dtype=torch.int16, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(20):
            torch.neg(src, out=dst)  # an elementwise kernel: reads and writes 64 MiB
        torch.cuda.synchronize()
        out["calib_copy_bytes"] = src.numel() * 2
    if fused_fill:
        out["fused_mask_equals_fill_bitmask"] = int(fused_mask_diff.item()) == 0
    if not args.no_cpu:
        xs = {}
        for k in range(args.steps):  # the checked rows' logits of every pool buffer the trajectory used
            i = (args.warmup + k) % npool
            if i not in xs:  # bf16 as its bits (uint16), float32 as is
                x = pool[i].index_select(0, chk_t)
                xs[i] = (x.view(torch.int16).cpu().numpy().view(np.uint16) if x.dtype == torch.bfloat16
                         else x.cpu().numpy())
        rec = {"rows": chk, "masks": rec_mask.cpu().numpy().view(np.uint64),
               "pre_ids": ids_hist[:args.warmup].cpu().numpy(), "ids": ids_hist[args.warmup:].cpu().numpy(),
               "lp": rec_lp.cpu().numpy(), "status": rec_status.cpu().numpy(),
               "x": [xs[(args.warmup + k) % npool] for k in range(args.steps)]}
        base, par = cpu_baseline(rec, B, V, blob, off, args.cpu_budget, cfg)
        out["cpu_baseline"] = base
        out["parity"] = par
        # the fill's byte-steps: the oracle's mean bytes walked per token check
        # on the checked rows times the fill's token-checks/s
        out["fill_byte_steps_per_s"] = round(base["bytes_walked_per_check"] * fill_checks, 1)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
