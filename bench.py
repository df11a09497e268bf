#!/usr/bin/env python3
"""Decode benchmark of the indexer -> Top-K -> sparse-MLA path on one MI355X.

One step = index_score_topk + sparse_mla_attn over one batch of the decode32k workload
(32 requests x 32768 context x 1 new token; 64 indexer heads x 128 on e4m3 keys; Top-K 2048;
128 heads over a bf16 576-wide latent cache).  Inputs sit in HBM before timing; the timed
steps rotate over several independent replicas of every input so that the 256 MB last-level
cache cannot serve a step from the previous one.  Prints one JSON line.

--workload tiny|prefill64k|decode1m|ragged measures another workload the same way (one
input replica: their inputs dwarf the last-level cache) and prints its own line; the default
line is decode32k.  --k-fmt mxfp8 runs the indexer on MXFP8 keys and queries (one scale byte
per 32 dims) instead of e4m3 keys with one fp32 scale per token, and labels its line so.
--select block runs block-granular selection instead: the scorer keeps one score per 64-key
page (its largest), the K/64 best pages are kept and expanded to their causal positions, and
the attention reads those K positions.  Step times are the median of --repeats timed loops of
--steps steps.  By default the untimed warmup runs steps until at least 100 ms of device time
have passed (at least 5 steps; the count is reported): the GPU's clock takes ~15 ms of steady
work to settle, and a serving loop runs at the settled clock.  --warmup W runs exactly W.  The
oracle baseline times the fp64 CPU oracle on every query token of batches of at most
--cpu-tokens tokens, and on a bounded sample of that many tokens otherwise.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP8_PEAK = 5.0e15              # dense FP8 matrix FLOP/s, published
BF16_PEAK = 2.5e15             # dense bf16 matrix FLOP/s, published


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic(inp, block=False):
    """Compulsory bytes / flops per step, stage by stage (inputs read once, outputs written
    once, only the selected rows gathered), and per launch of each entry point.  block: the
    scorer writes one score per 64-key page, the selection reads those and writes K/64 pages
    plus K expanded positions, and the attention reads the causal rows of the kept pages
    (at most K: counted as min(K, n))."""
    import numpy as np
    sh = inp.wl.shape
    n = inp.positions.astype(np.int64) + 1
    k = np.minimum(sh.K, n)
    kb = (sh.D_I + 4) if not sh.fp32 else 4 * sh.D_I            # key code + scale per position
    qb = sh.H_I * sh.D_I * (2 if not sh.fp32 else 4) + 4 * sh.H_I  # q_I + w per token
    # each request's keys are read once however many of its tokens query them
    idx_bytes = int(sum(int(L) * kb for L in inp.seq_lens)) + inp.T * qb
    idx_flops = int((2 * sh.H_I * sh.D_I * n).sum())
    topk_bytes = 4 * sh.K * inp.T
    row = sh.D_qk * (1 if sh.kv_fp8 else 2) + (4 if sh.kv_fp8 else 0)
    # selected rows + indices + q + O (bf16) + lse
    attn_bytes = int((k * row).sum()) + inp.T * (4 * sh.K + sh.H * (sh.D_qk * 2 + sh.D_v * 2 + 4))
    attn_flops = int((2 * sh.H * k * (sh.D_qk + sh.D_v)).sum())
    if block:
        nb = (n + 63) // 64
        topk_bytes = 4 * (sh.K // 64) * inp.T + 4 * sh.K * inp.T
        return dict(idx_bytes=idx_bytes, idx_flops=idx_flops, topk_bytes=topk_bytes,
                    attn_bytes=attn_bytes, attn_flops=attn_flops,
                    idx_kernel_bytes=idx_bytes + int(4 * nb.sum()),
                    topk_kernel_bytes=int(4 * nb.sum()) + topk_bytes)
    return dict(idx_bytes=idx_bytes, idx_flops=idx_flops, topk_bytes=topk_bytes,
                attn_bytes=attn_bytes, attn_flops=attn_flops,
                # unfused entry points: the scorer also writes one fp32 score per candidate,
                # the selection reads them back
                idx_kernel_bytes=idx_bytes + int(4 * n.sum()),
                topk_kernel_bytes=int(4 * n.sum()) + topk_bytes)


def t_roof(a):
    hb = HBM_PEAK_GBS * 1e9
    return (max(a["idx_bytes"] / hb, a["idx_flops"] / FP8_PEAK) + a["topk_bytes"] / hb
            + max(a["attn_bytes"] / hb, a["attn_flops"] / BF16_PEAK))


def measured_traffic(entry_point: str):
    """HBM bytes per launch of an entry point from the committed FETCH_SIZE / WRITE_SIZE counter
    record (scaled by the copy calibration), or None when any kernel source it covers has
    changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "decode32k_traffic.json")
    try:
        rec = json.load(open(path))["entry_points"][entry_point]
    except (OSError, KeyError, ValueError):
        return None
    pkg = os.path.join(ROOT, "top_indexed_sparse_amd")
    for rel, digest in rec["sources"].items():
        try:
            with open(os.path.join(pkg, rel), "rb") as f:
                if hashlib.sha256(f.read()).hexdigest() != digest:
                    return None
        except OSError:
            return None
    return rec["bytes_per_launch"]


def host_info():
    """CPU model, usable cores and the BLAS numpy runs on (for the baseline record)."""
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = "unknown"
    try:
        import threadpoolctl
        infos = [i for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
        if infos:
            i = infos[0]
            blas = (f"{i.get('internal_api')} {i.get('version')} "
                    f"({i.get('threading_layer')}, {i.get('num_threads')} threads)")
    except Exception:  # pragma: no cover - informational only
        pass
    return cores, model, blas


def baseline_tokens(inp, n_sample: int):
    """The tokens the oracle is timed on: every token of a batch of at most n_sample tokens;
    otherwise the first and last token, the tokens at positions 2046..2049, each request's
    first and last query token, and a seeded random fill up to n_sample."""
    import numpy as np
    T = inp.T
    if T <= n_sample:
        return list(range(T))
    pick = {0, T - 1}
    for p in (2046, 2047, 2048, 2049):
        pick |= set(np.nonzero(inp.positions == p)[0].tolist())
    for b in range(inp.B):
        a, e = int(inp.cu_q[b]), int(inp.cu_q[b + 1])
        if e > a:
            pick |= {a, e - 1}
    rng = np.random.default_rng(12345)
    rest = np.setdiff1d(np.arange(T), np.array(sorted(pick)))
    need = max(0, n_sample - len(pick))
    pick |= set(rng.choice(rest, size=min(need, rest.size), replace=False).tolist())
    return sorted(pick)


def cpu_baseline(inp, r_idx, r_out, out_bf16, tokens, unit, block=False):
    """The fp64 oracle timed on this host on a bounded sample of the same inputs; also a
    parity gate against the GPU results for those tokens (recall, and attention on the GPU's
    own selection within the gate: 1e-2 bf16 cache / 2e-2 e4m3 cache, plus half a bf16 ulp
    of the value when the output is stored in bf16)."""
    import numpy as np
    from oracle import Oracle
    cores, model, blas = host_info()
    orc = Oracle(inp)
    t0 = time.perf_counter()
    chosen = []
    for t in tokens:                       # the oracle's own chain, timed
        if block:
            idx = orc.block_topk(t, inp.wl.shape.K // 64)[3]
        else:
            idx, S, kth = orc.topk(t)
        orc.attention(t, idx)
        chosen.append(idx)
    dt = time.perf_counter() - t0
    sh = inp.wl.shape
    tol = 2e-2 if sh.kv_fp8 else 1e-2
    recall_hits = recall_tot = 0
    worst = -np.inf
    for t, idx in zip(tokens, chosen):     # parity of the GPU results (not timed)
        g = r_idx[t]
        recall_hits += len(set(g[g >= 0].tolist()) & set(idx[idx >= 0].tolist()))
        recall_tot += int((idx >= 0).sum())
        og, _ = orc.attention(t, g)        # attention on the GPU's own selected set
        gate = tol
        if out_bf16:
            _, E = np.frexp(np.abs(og) + tol)
            gate = tol + np.ldexp(1.0, E - 9)
        worst = max(worst, float(np.max(np.abs(r_out[t] - og) - gate)))
    whole = len(tokens) == inp.T
    sample = (f"{len(tokens)} of {inp.T} query tokens" + ("" if whole else
              " (first/last, positions 2046-2049, request edges, seeded random fill)")
              + ": the full per-token chain (e4m3/bf16 decode, fp64 scores, full-sort "
              + ("block selection" if block else "Top-K") + ", fp64 attention)")
    rec = dict(value=len(tokens) / dt, unit=unit, cores=cores, kind="oracle", sample=sample,
               cpu_model=model, blas=blas)
    if not whole:
        rec["extrapolated_s_per_step"] = dt / len(tokens) * inp.T
    return rec, dt, recall_hits / max(1, recall_tot), worst


def dense_ab(args):
    """Gather form (sparse_mla_attn) against dense-masked form (sparse_mla_attn_dense) of the
    attention over the same selections, on the prefill workload's shapes (e4m3 latent cache,
    K = 2048): one batch per band of causal lengths (lo, hi], i.e. the query tokens at
    positions lo .. hi-1 of a hi-token sequence.  The dense form reads and multiplies every
    causal row; the gather form only the K selected ones."""
    import numpy as np
    import torch
    import synth
    import top_indexed_sparse_amd as tis
    from synth.device import to_device
    base = synth.workload(synth.PREFILL64K)
    sh = base.shape
    bands = [(0, 2048), (2048, 4096), (4096, 8192), (8192, 16384)]
    rows = []
    stream = torch.cuda.current_stream()
    for lo, hi in bands:
        wl = synth.reduced(base, [hi], [hi - lo], name=f"prefill-band-{lo}-{hi}")
        inp = synth.make(wl, "continuous")
        d = to_device(inp)
        bt = tis.Batch(inp.seq_lens, inp.cu_q, inp.page_table, inp.n_pages)
        T, K = inp.T, sh.K
        idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
        tis.index_score_topk(bt, d.q_idx, d.w, d.k_pool, d.k_scale, K, idx)
        out = torch.empty((T, sh.H, sh.D_v), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((T, sh.H), dtype=torch.float32, device="cuda")
        kvd = tis.TIS_E4M3
        wsg = torch.empty(max(1, tis.sparse_mla_attn_workspace_size(bt, K, sh.H, sh.D_qk, sh.D_v,
                                                                    kvd)),
                          dtype=torch.uint8, device="cuda")
        wsd = torch.empty(max(1, tis.sparse_mla_attn_dense_workspace_size(bt, K, sh.H, sh.D_qk,
                                                                          sh.D_v, kvd)),
                          dtype=torch.uint8, device="cuda")
        res = {}
        for form, fn, ws in (("gather", tis.sparse_mla_attn, wsg),
                             ("dense", tis.sparse_mla_attn_dense, wsd)):
            for _ in range(2):
                fn(bt, d.q, d.kv_pool, d.kv_scale, idx, sh.softmax_scale, out, lse, ws=ws)
            runs = []
            for _ in range(max(1, args.repeats)):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                e0.record(stream)
                for _ in range(args.steps):
                    fn(bt, d.q, d.kv_pool, d.kv_scale, idx, sh.softmax_scale, out, lse, ws=ws)
                e1.record(stream)
                torch.cuda.synchronize()
                runs.append(e0.elapsed_time(e1) / args.steps)
            res[form] = float(np.median(runs))
        n = inp.positions.astype(np.int64) + 1
        row = {"band": [lo, hi], "tokens": T, "mean_causal": float(n.mean()),
               "selected_fraction": float((np.minimum(K, n) / n).mean()),
               "gather_ms": round(res["gather"], 3), "dense_ms": round(res["dense"], 3),
               "dense_over_gather": round(res["dense"] / res["gather"], 3)}
        log(f"band ({lo}, {hi}]: {T} tokens, selected {row['selected_fraction']:.2f} of the "
            f"causal rows; gather {res['gather']:.2f} ms, dense {res['dense']:.2f} ms")
        rows.append(row)
        del d, idx, out, lse, wsg, wsd
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "prefill attention: dense-masked form / gather form time",
                      "unit": "ratio", "higher_is_better": False, "n_gpus": 1,
                      "steps": args.steps, "repeats": args.repeats, "data": "synthetic",
                      "config": {"workload": "prefill64k bands", "topk": base.shape.K,
                                 "heads": sh.H, "qk_dim": sh.D_qk, "v_dim": sh.D_v,
                                 "kv_cache": "fp8"},
                      "bands": rows}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=-1,
                    help="untimed warmup steps (default: until 100 ms of device time, >= 5)")
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--repeats", type=int, default=5,
                    help="timed loops of --steps steps each; the median is reported")
    ap.add_argument("--cpu-tokens", type=int, default=256,
                    help="oracle baseline sample size (tokens) for batches larger than this")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="decode32k",
                    choices=["tiny", "decode32k", "prefill64k", "decode1m", "ragged"])
    ap.add_argument("--k-fmt", default="e4m3", choices=["e4m3", "mxfp8"],
                    help="indexer key format: e4m3 + fp32 scale per token, or MXFP8")
    ap.add_argument("--select", default="token", choices=["token", "block"],
                    help="Top-K positions, or the K/64 best 64-position pages")
    ap.add_argument("--dense-ab", action="store_true",
                    help="only run the A/B of the attention's gather form against its "
                         "dense-masked form on bands of causal length of the prefill "
                         "workload's shapes, and print one JSON line")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (8 times) and exit: the "
                         "reference for scaling FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the multi-GPU "
              "sharding of this path is a design note, not built.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        nbytes = args.copy_calibration << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(8):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": nbytes, "launches": 8}), flush=True)
        return

    import synth
    import top_indexed_sparse_amd as tis
    from synth.device import to_device

    torch.cuda.set_device(0)
    if args.dense_ab:
        dense_ab(args)
        return
    mx = args.k_fmt == "mxfp8"
    block = args.select == "block"
    main_line = args.workload == "decode32k" and not mx and not block
    wl = synth.workload(synth.NAMES.index(args.workload))
    sh = wl.shape
    if args.workload != "decode32k":
        args.replicas = 1
    t0 = time.perf_counter()
    inp = synth.make(wl, "continuous", k_fmt=None if sh.fp32 else args.k_fmt)
    log(f"generated {wl.name} in {time.perf_counter() - t0:.1f}s")
    base = to_device(inp)
    reps = [base] + [type(base)(**{k: (v.clone() if v is not None else None)
                                   for k, v in vars(base).items()})
                     for _ in range(args.replicas - 1)]
    bt = tis.Batch(inp.seq_lens, inp.cu_q, inp.page_table, inp.n_pages)
    T, K = inp.T, sh.K
    idx = [torch.empty((T, K), dtype=torch.int32, device="cuda") for _ in reps]
    out_dt = torch.float32 if sh.fp32 else torch.bfloat16
    out = [torch.empty((T, sh.H, sh.D_v), dtype=out_dt, device="cuda") for _ in reps]
    lse = [torch.empty((T, sh.H), dtype=torch.float32, device="cuda") for _ in reps]
    Kb = K // 64
    ws_i = torch.empty(max(1, (tis.index_score_topk_block_workspace_size(bt, sh.H_I, sh.D_I, Kb)
                               if block else
                               tis.index_score_topk_workspace_size(bt, sh.H_I, sh.D_I, K))),
                       dtype=torch.uint8, device="cuda")
    bidx = [torch.empty((T, Kb), dtype=torch.int32, device="cuda") for _ in reps]
    kv_code = tis.TIS_F32 if sh.fp32 else (tis.TIS_E4M3 if sh.kv_fp8 else tis.TIS_BF16)
    ws_a_bytes = tis.sparse_mla_attn_workspace_size(bt, K, sh.H, sh.D_qk, sh.D_v, kv_code)
    ws_a = torch.empty(max(1, ws_a_bytes),
                       dtype=torch.uint8, device="cuda")

    def step(i):
        r = i % len(reps)
        d = reps[r]
        if block:
            tis.index_score_topk_block(bt, d.q_idx, d.w, d.k_pool, d.k_scale, Kb, bidx[r],
                                       topk_idx=idx[r], ws=ws_i)
        else:
            tis.index_score_topk(bt, d.q_idx, d.w, d.k_pool, d.k_scale, K, idx[r], ws=ws_i)
        tis.sparse_mla_attn(bt, d.q, d.kv_pool, d.kv_scale, idx[r], sh.softmax_scale, out[r],
                            lse[r], ws=ws_a)

    stream = torch.cuda.current_stream()

    def timed_once(fn, n):
        """Average ms per call of fn(i), i = 0..n-1, between HIP events on the stream the
        library launches on (torch's current stream), synchronised on both sides."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    def timed(fn, n, runs=None):
        """Median over `repeats` timed loops of exactly n calls each (and the loops' values)."""
        runs = runs if runs is not None else []
        for _ in range(max(1, args.repeats)):
            runs.append(timed_once(fn, n))
        return float(np.median(runs))

    def warm(fn, w):
        """Untimed calls of fn: exactly w, or (w < 0) until 100 ms of device time have passed
        and at least 5 calls; returns the count."""
        if w >= 0:
            for i in range(w):
                fn(i)
            torch.cuda.synchronize()
            return w
        n, t0 = 0, time.perf_counter()
        while n < 5 or time.perf_counter() - t0 < 0.1:
            for _ in range(5):
                fn(n)
                n += 1
            torch.cuda.synchronize()
        return n

    n_warm = warm(step, args.warmup)
    step_runs = []
    step_ms = timed(step, args.steps, step_runs)

    # each entry point alone, over the same replicas: the scorer (unfused, writes scores),
    # the selection over those scores, the attention call
    ld = ((tis.blocks_of(bt.max_n) if block else bt.max_n) + 3) // 4 * 4
    scores = [torch.empty((T, ld), dtype=torch.float32, device="cuda") for _ in reps]

    def score(i):
        d = reps[i % len(reps)]
        if block:
            tis.index_score_block(bt, d.q_idx, d.w, d.k_pool, d.k_scale, scores[i % len(reps)])
        else:
            tis.index_score(bt, d.q_idx, d.w, d.k_pool, d.k_scale, scores[i % len(reps)])

    def select(i):
        r = i % len(reps)
        if block:
            tis.topk_block_select(bt, scores[r], Kb, bidx[r], topk_idx=idx[r])
        else:
            tis.topk_select(bt, scores[r], K, idx[r])

    def attend(i):
        r = i % len(reps)
        d = reps[r]
        tis.sparse_mla_attn(bt, d.q, d.kv_pool, d.kv_scale, idx[r], sh.softmax_scale, out[r],
                            lse[r], ws=ws_a)

    for fn in (score, select, attend):
        warm(fn, max(args.warmup, len(reps)) if args.warmup >= 0 else -1)
    a = algorithmic(inp, block)
    kv = "f32" if sh.fp32 else ("fp8" if sh.kv_fp8 else "bf16")
    calls = {
        ("index_score_block" if block else "index_score"): dict(
                            ms=timed(score, args.steps), bytes=a["idx_kernel_bytes"],
                            flops=a["idx_flops"], peak=FP8_PEAK,
                            kernels=["idx_score_f32_kernel" if sh.fp32 else
                                     "idx_score_group_kernel" if inp.T >= 4 * inp.B else
                                     "idx_score_fp8_kernel"]),
        ("topk_block_select" if block else "topk_select"): dict(
            ms=timed(select, args.steps), bytes=a["topk_kernel_bytes"], flops=0, peak=FP8_PEAK,
            kernels=["topk_select_kernel"] + (["expand_blocks_kernel"] if block else [])),
        "sparse_mla_attn": dict(ms=timed(attend, args.steps), bytes=a["attn_bytes"],
                                flops=a["attn_flops"], peak=BF16_PEAK,
                                kernels=[f"mla_attn_{kv}_kernel"] + (
                                    ["mla_combine_kernel"] if ws_a_bytes > 0 and not sh.fp32
                                    else [])),
    }
    for c in calls.values():
        c["gbs"] = c["bytes"] / (c["ms"] * 1e-3) / 1e9
        c["tflops"] = c["flops"] / (c["ms"] * 1e-3) / 1e12
        # the roofline that binds: matrix throughput above the ridge point, HBM below it
        c["mfma"] = c["flops"] / c["bytes"] > c["peak"] / (HBM_PEAK_GBS * 1e9)
    dom_name = max(calls, key=lambda k: calls[k]["ms"])
    dom = calls[dom_name]
    roof_s = t_roof(a)
    decode = all(int(x) <= 1 for x in inp.q_lens)
    if dom["mfma"]:
        roofline = {"bound": "mfma", "entry_point": dom_name, "kernels": dom["kernels"],
                    "achieved": dom["tflops"], "peak": dom["peak"] / 1e12, "unit": "TFLOP/s",
                    "frac": dom["tflops"] * 1e12 / dom["peak"], "traffic": None,
                    "launch_us": dom["ms"] * 1e3, "flops_per_launch": dom["flops"]}
    else:
        roofline = {"bound": "hbm", "entry_point": dom_name, "kernels": dom["kernels"],
                    "achieved": dom["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": dom["gbs"] / HBM_PEAK_GBS,
                    "traffic": measured_traffic(dom_name) if main_line else None,
                    "traffic_unit": "bytes/launch", "launch_us": dom["ms"] * 1e3,
                    "bytes_per_launch": dom["bytes"]}
    res = {
        "metric": ("sparse-attn decode queries/s @32K ctx (index+topk+attn)" if main_line else
                   f"{wl.name} {'queries' if decode else 'tokens'}/s (index+topk+attn)"
                   + (", MXFP8 indexer" if mx else "")
                   + (", block-granular selection" if block else "")),
        "value": T * 1000.0 / step_ms,
        "unit": "queries/s" if decode else "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": n_warm,
        "ms_per_step": step_ms,
        "repeats": len(step_runs),
        "ms_per_step_runs": [round(x, 5) for x in step_runs],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp32" if sh.fp32 else
                  f"{'mxfp8' if mx else 'fp8'} indexer / bf16 attention over a {kv} cache, "
                  "fp32 accumulate"),
        "data": "synthetic",
        "config": ({"workload": "decode32k", "batch": T, "context": int(inp.seq_lens[0]),
                    "new_tokens_per_request": 1, "indexer_heads": sh.H_I, "indexer_dim": sh.D_I,
                    "topk": K, "heads": sh.H, "qk_dim": sh.D_qk, "v_dim": sh.D_v,
                    "kv_cache": "bf16", "index_keys": "e4m3+fp32 scale/token",
                    "input_replicas": len(reps)} if main_line else
                   {"workload": wl.name, "requests": inp.B, "query_tokens": T,
                    "index_keys": ("fp32" if sh.fp32 else "mxfp8 (e8m0 byte/32 dims)" if mx
                                   else "e4m3+fp32 scale/token"),
                    "selection": ("K/64 pages of 64 positions (max score per page)" if block
                                  else "K positions"),
                    "max_context": int(inp.seq_lens.max()),
                    "cached_tokens": int(inp.seq_lens.sum()), "indexer_heads": sh.H_I,
                    "indexer_dim": sh.D_I, "topk": K, "heads": sh.H, "qk_dim": sh.D_qk,
                    "v_dim": sh.D_v, "kv_cache": kv, "input_replicas": len(reps)}),
        "roofline": roofline,
        "chain_roofline": {"t_roof_us": roof_s * 1e6, "t_step_us": step_ms * 1e3,
                           "frac": roof_s / (step_ms * 1e-3),
                           "attn_tflops": a["attn_flops"] / (calls["sparse_mla_attn"]["ms"] * 1e-3) / 1e12,
                           "calls": {k: {"us": round(v["ms"] * 1e3, 2), "GB/s": round(v["gbs"], 1),
                                         "TFLOP/s": round(v["tflops"], 1)}
                                     for k, v in calls.items()}},
    }
    if not args.no_cpu_baseline:
        torch.cuda.synchronize()
        toks = baseline_tokens(inp, args.cpu_tokens)
        ix = torch.as_tensor(toks, dtype=torch.long, device="cuda")
        ri = dict(zip(toks, idx[0].index_select(0, ix).cpu().numpy()))
        ro = dict(zip(toks, out[0].index_select(0, ix).float().cpu().numpy().astype(np.float64)))
        cb, secs, rec, excess = cpu_baseline(inp, ri, ro, out_dt == torch.bfloat16, toks,
                                             res["unit"], block)
        log(f"cpu oracle: {secs:.1f}s for {len(toks)} tokens on {cb['cores']} cores "
            f"({cb['cpu_model']}, {cb['blas']}); GPU recall {rec:.5f}, attention error "
            f"{excess:+.2e} relative to its gate")
        if rec < 0.999 or excess > 0.0:
            log("PARITY GATE FAILED")
            sys.exit(1)
        res["cpu_baseline"] = cb
    log(f"step {step_ms * 1e3:.1f} us; alone: " + ", ".join(
        f"{k} {v['ms'] * 1e3:.1f} us ({v['gbs']:.0f} GB/s)" for k, v in calls.items())
        + f"; chain roofline {roof_s * 1e6:.1f} us")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
