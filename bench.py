#!/usr/bin/env python3
"""Decode benchmark of the indexer -> Top-K -> sparse-MLA path on one MI355X.

One step = index_score_topk + sparse_mla_attn over one batch of the decode32k workload
(32 requests x 32768 context x 1 new token; 64 indexer heads x 128 on e4m3 keys; Top-K 2048;
128 heads over a bf16 576-wide latent cache).  Inputs sit in HBM before timing; the timed
steps rotate over several independent replicas of every input so that the 256 MB last-level
cache cannot serve a step from the previous one.  Prints one JSON line.
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


def algorithmic(inp):
    """Compulsory bytes / flops per step, stage by stage (inputs read once, outputs written
    once, only the selected rows gathered)."""
    import numpy as np
    sh = inp.wl.shape
    n = inp.positions.astype(np.int64) + 1
    k = np.minimum(sh.K, n)
    kbytes = 1 if not sh.fp32 else 4 * 1
    kb = (sh.D_I + 4) if not sh.fp32 else 4 * sh.D_I
    qb = sh.H_I * sh.D_I * (2 if not sh.fp32 else 4) + 4 * sh.H_I
    # each request's keys are read once however many of its tokens query them
    idx_bytes = int(sum(int(L) * kb for L in inp.seq_lens)) + inp.T * qb
    idx_flops = int((2 * sh.H_I * sh.D_I * n).sum())
    topk_bytes = 4 * sh.K * inp.T
    row = sh.D_qk * (1 if sh.kv_fp8 else 2) + (4 if sh.kv_fp8 else 0)
    attn_bytes = int((k * row).sum()) + inp.T * sh.H * (sh.D_qk * 2 + sh.D_v * 2 + 4)
    attn_flops = int((2 * sh.H * k * (sh.D_qk + sh.D_v)).sum())
    del kbytes
    return dict(idx_bytes=idx_bytes, idx_flops=idx_flops, topk_bytes=topk_bytes,
                attn_bytes=attn_bytes, attn_flops=attn_flops,
                # the unfused scorer also writes one fp32 score per candidate
                idx_kernel_bytes=idx_bytes + int(4 * n.sum()))


def t_roof(a):
    hb = HBM_PEAK_GBS * 1e9
    return (max(a["idx_bytes"] / hb, a["idx_flops"] / FP8_PEAK) + a["topk_bytes"] / hb
            + max(a["attn_bytes"] / hb, a["attn_flops"] / BF16_PEAK))


def cpu_baseline(inp, r_idx, r_out, tokens):
    """The fp64 oracle timed on this host on a bounded sample of the same inputs; also a
    parity gate against the GPU results for those tokens."""
    import numpy as np
    from oracle import Oracle
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    orc = Oracle(inp)
    t0 = time.perf_counter()
    recall_hits = recall_tot = 0
    worst = 0.0
    for t in tokens:
        idx, S, kth = orc.topk(t)
        o, _ = orc.attention(t, idx)
        g = r_idx[t]
        recall_hits += len(set(g[g >= 0].tolist()) & set(idx[idx >= 0].tolist()))
        recall_tot += int((idx >= 0).sum())
        # attention on the GPU's own set for the output comparison
        og, _ = orc.attention(t, g)
        worst = max(worst, float(np.abs(r_out[t] - og).max()))
    dt = time.perf_counter() - t0
    return dict(value=len(tokens) / dt, unit="queries/s", cores=cores, kind="oracle",
                sample=f"{len(tokens)} of {inp.T} decode tokens (full per-token chain: e4m3 "
                       f"decode, fp64 scores, full-sort Top-K, fp64 attention)",
                seconds=dt), recall_hits / max(1, recall_tot), worst


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--cpu-tokens", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the multi-GPU "
              "sharding of this path is a design note, not built.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import top_indexed_sparse_amd as tis
    from synth.device import to_device

    torch.cuda.set_device(0)
    wl = synth.workload(synth.DECODE32K)
    sh = wl.shape
    t0 = time.perf_counter()
    inp = synth.make(wl, "continuous")
    log(f"generated {wl.name} in {time.perf_counter() - t0:.1f}s")
    base = to_device(inp)
    reps = [base] + [type(base)(**{k: (v.clone() if v is not None else None)
                                   for k, v in vars(base).items()})
                     for _ in range(args.replicas - 1)]
    bt = tis.Batch(inp.seq_lens, inp.cu_q, inp.page_table, inp.n_pages)
    T, K = inp.T, sh.K
    idx = [torch.empty((T, K), dtype=torch.int32, device="cuda") for _ in reps]
    out = [torch.empty((T, sh.H, sh.D_v), dtype=torch.bfloat16, device="cuda") for _ in reps]
    lse = [torch.empty((T, sh.H), dtype=torch.float32, device="cuda") for _ in reps]
    ws_i = torch.empty(tis.index_score_topk_workspace_size(bt, sh.H_I, sh.D_I, K),
                       dtype=torch.uint8, device="cuda")
    ws_a = torch.empty(max(1, tis.sparse_mla_attn_workspace_size(bt, K, sh.H, sh.D_qk, sh.D_v,
                                                                 tis.TIS_BF16)),
                       dtype=torch.uint8, device="cuda")

    def step(i):
        r = i % len(reps)
        d = reps[r]
        tis.index_score_topk(bt, d.q_idx, d.w, d.k_pool, d.k_scale, K, idx[r], ws=ws_i)
        tis.sparse_mla_attn(bt, d.q, d.kv_pool, d.kv_scale, idx[r], sh.softmax_scale, out[r],
                            lse[r], ws=ws_a)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    step_ms = e0.elapsed_time(e1) / args.steps

    # dominant kernel: the FP8 scorer, timed alone over the same replicas
    ld = (bt.max_n + 3) // 4 * 4
    scores = torch.empty((T, ld), dtype=torch.float32, device="cuda")
    for i in range(args.warmup):
        d = reps[i % len(reps)]
        tis.index_score(bt, d.q_idx, d.w, d.k_pool, d.k_scale, scores)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        d = reps[i % len(reps)]
        tis.index_score(bt, d.q_idx, d.w, d.k_pool, d.k_scale, scores)
    e1.record(stream)
    torch.cuda.synchronize()
    idx_ms = e0.elapsed_time(e1) / args.steps

    # attention kernel alone (its share of the step)
    e0.record(stream)
    for i in range(args.steps):
        r = i % len(reps)
        d = reps[r]
        tis.sparse_mla_attn(bt, d.q, d.kv_pool, d.kv_scale, idx[r], sh.softmax_scale, out[r],
                            lse[r], ws=ws_a)
    e1.record(stream)
    torch.cuda.synchronize()
    attn_ms = e0.elapsed_time(e1) / args.steps

    a = algorithmic(inp)
    roof_s = t_roof(a)
    ach = a["idx_kernel_bytes"] / (idx_ms * 1e-3) / 1e9
    res = {
        "metric": "sparse-attn decode queries/s @32K ctx (index+topk+attn)",
        "value": T * 1000.0 / step_ms,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 indexer / bf16 attention, fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": "decode32k", "batch": T, "context": int(inp.seq_lens[0]),
                   "new_tokens_per_request": 1, "indexer_heads": sh.H_I, "indexer_dim": sh.D_I,
                   "topk": K, "heads": sh.H, "qk_dim": sh.D_qk, "v_dim": sh.D_v,
                   "kv_cache": "bf16", "index_keys": "e4m3+fp32 scale/token",
                   "input_replicas": len(reps)},
        "roofline": {"bound": "hbm", "kernel": "idx_score_fp8_kernel",
                     "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": ach / HBM_PEAK_GBS, "traffic": None,
                     "launch_us": idx_ms * 1e3, "bytes_per_launch": a["idx_kernel_bytes"]},
        "chain_roofline": {"t_roof_us": roof_s * 1e6, "t_step_us": step_ms * 1e3,
                           "frac": roof_s / (step_ms * 1e-3),
                           "attn_us": attn_ms * 1e3,
                           "attn_gbs": a["attn_bytes"] / (attn_ms * 1e-3) / 1e9,
                           "attn_tflops": a["attn_flops"] / (attn_ms * 1e-3) / 1e12},
    }
    if not args.no_cpu_baseline:
        torch.cuda.synchronize()
        ri = idx[0].cpu().numpy()
        ro = out[0].float().cpu().numpy().astype(np.float64)
        ntok = max(1, min(args.cpu_tokens, T))
        cb, rec, err = cpu_baseline(inp, ri, ro, list(range(ntok)))
        log(f"cpu oracle: {cb['seconds']:.1f}s for {ntok} tokens; GPU recall {rec:.5f}, "
            f"attention max-abs {err:.2e}")
        if rec < 0.999 or err > 1e-2:
            log("PARITY GATE FAILED")
            sys.exit(1)
        cb.pop("seconds")
        res["cpu_baseline"] = cb
    log(f"step {step_ms * 1e3:.1f} us (scorer alone {idx_ms * 1e3:.1f} us, attention alone "
        f"{attn_ms * 1e3:.1f} us); chain roofline {roof_s * 1e6:.1f} us")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
