"""Shared GPU-test helpers: run the HIP path on a generated batch through the C ABI, and the
parity gates against the oracle.  (Not a test module.)"""
from __future__ import annotations

import math
import sys
from types import SimpleNamespace

import numpy as np
import torch

import top_indexed_sparse_amd as tis
from synth.device import to_device


def note(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def make_batch(inp) -> tis.Batch:
    return tis.Batch(inp.seq_lens, inp.cu_q, inp.page_table, inp.n_pages)


def _out_dtype(sh, out):
    """Attention output dtype: 'f32', 'bf16', or None for the default (fp32 with the tiny
    workload's fp32 kernels and with e4m3 caches, bf16 with a bf16 cache)."""
    if sh.fp32:
        return torch.float32
    if out is None:
        out = "f32" if sh.kv_fp8 else "bf16"
    return {"f32": torch.float32, "bf16": torch.bfloat16}[out]


def run_path(inp, unfused: bool = True, K: int | None = None, out: str | None = None,
             out_f32: bool = False, qmode: int | None = None) -> SimpleNamespace:
    """Fused index_score_topk + sparse_mla_attn (and optionally the unfused chain); qmode is
    the indexer's query mode (default: FP8 for bf16 queries, as stored for fp32 ones)."""
    sh = inp.wl.shape
    K = sh.K if K is None else K
    d = to_device(inp)
    bt = make_batch(inp)
    T = inp.T
    r = SimpleNamespace()
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    val = torch.empty((T, K), dtype=torch.float32, device="cuda")
    tis.index_score_topk(bt, d.q_idx, d.w, d.k_pool, d.k_scale, K, idx, val, qmode=qmode)
    if unfused:
        ld = (bt.max_n + 3) // 4 * 4
        scores = torch.full((T, ld), float("nan"), dtype=torch.float32, device="cuda")
        tis.index_score(bt, d.q_idx, d.w, d.k_pool, d.k_scale, scores, qmode=qmode)
        idx2 = torch.empty_like(idx)
        val2 = torch.empty_like(val)
        tis.topk_select(bt, scores, K, idx2, val2)
    out_dt = _out_dtype(sh, "f32" if out_f32 else out)
    o = torch.empty((T, sh.H, sh.D_v), dtype=out_dt, device="cuda")
    lse = torch.empty((T, sh.H), dtype=torch.float32, device="cuda")
    tis.sparse_mla_attn(bt, d.q, d.kv_pool, d.kv_scale, idx, sh.softmax_scale, o, lse)
    torch.cuda.synchronize()
    r.idx = idx.cpu().numpy()
    r.val = val.cpu().numpy()
    if unfused:
        r.scores = scores.cpu().numpy()
        r.idx2 = idx2.cpu().numpy()
        r.val2 = val2.cpu().numpy()
    r.out = o.float().cpu().numpy().astype(np.float64)
    r.out_bf16 = out_dt == torch.bfloat16
    r.lse = lse.cpu().numpy().astype(np.float64)
    r.dev, r.batch = d, bt
    return r


def attend(inp, r, out: str):
    """The attention call again on the selection of a run_path result, with another output
    dtype; returns a result to check with check_attention."""
    sh = inp.wl.shape
    out_dt = _out_dtype(sh, out)
    idx = torch.from_numpy(r.idx).cuda()
    o = torch.empty((inp.T, sh.H, sh.D_v), dtype=out_dt, device="cuda")
    lse = torch.empty((inp.T, sh.H), dtype=torch.float32, device="cuda")
    tis.sparse_mla_attn(r.batch, r.dev.q, r.dev.kv_pool, r.dev.kv_scale, idx, sh.softmax_scale,
                        o, lse)
    torch.cuda.synchronize()
    return SimpleNamespace(idx=r.idx, out=o.float().cpu().numpy().astype(np.float64),
                           out_bf16=out_dt == torch.bfloat16,
                           lse=lse.cpu().numpy().astype(np.float64))


class SampledRows:
    """Rows of a [T, ...] device tensor copied to the host for a set of tokens only, indexed
    by token like the full array (``rows[t]`` or ``rows[t, sl]``)."""

    def __init__(self, dev: torch.Tensor, tokens, as_f64: bool = False):
        self.pos = {int(t): i for i, t in enumerate(tokens)}
        ix = torch.as_tensor(list(tokens), dtype=torch.long, device=dev.device)
        rows = dev.index_select(0, ix)
        self.rows = rows.float().cpu().numpy().astype(np.float64) if as_f64 else rows.cpu().numpy()

    def __getitem__(self, key):
        if isinstance(key, tuple):
            return self.rows[(self.pos[int(key[0])],) + key[1:]]
        return self.rows[self.pos[int(key)]]


def run_path_sampled(inp, tokens, outs=None) -> SimpleNamespace:
    """The same launches as run_path over the whole batch, for batches whose outputs do not fit
    the host: fused and unfused Top-K are compared on the device for every token, outputs are
    checked finite on the device, and only the rows of ``tokens`` come back to the host.
    ``outs`` lists the attention output dtypes to run ('bf16', 'f32'; default: the default
    dtype only); ``r.att[dtype]`` holds each run's sampled rows."""
    sh = inp.wl.shape
    K = sh.K
    d = to_device(inp)
    bt = make_batch(inp)
    T = inp.T
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    val = torch.empty((T, K), dtype=torch.float32, device="cuda")
    tis.index_score_topk(bt, d.q_idx, d.w, d.k_pool, d.k_scale, K, idx, val)
    ld = (bt.max_n + 3) // 4 * 4
    scores = torch.full((T, ld), float("nan"), dtype=torch.float32, device="cuda")
    tis.index_score(bt, d.q_idx, d.w, d.k_pool, d.k_scale, scores)
    idx2 = torch.empty_like(idx)
    val2 = torch.empty_like(val)
    tis.topk_select(bt, scores, K, idx2, val2)
    torch.cuda.synchronize()
    r = SimpleNamespace()
    r.fused_equal = bool(torch.equal(idx, idx2)) and bool(torch.equal(val, val2))
    r.scores = SampledRows(scores, tokens)
    del scores, idx2, val2
    r.idx = SampledRows(idx, tokens)
    r.val = SampledRows(val, tokens)
    r.att = {}
    for name in (outs or [None]):
        out_dt = _out_dtype(sh, name)
        o = torch.empty((T, sh.H, sh.D_v), dtype=out_dt, device="cuda")
        lse = torch.empty((T, sh.H), dtype=torch.float32, device="cuda")
        tis.sparse_mla_attn(bt, d.q, d.kv_pool, d.kv_scale, idx, sh.softmax_scale, o, lse)
        torch.cuda.synchronize()
        a = SimpleNamespace(idx=r.idx, out_bf16=out_dt == torch.bfloat16)
        a.out_finite = bool(torch.isfinite(o).all())
        a.lse_finite = bool(torch.isfinite(lse).all())
        a.out = SampledRows(o, tokens, as_f64=True)
        a.lse = SampledRows(lse, tokens, as_f64=True)
        r.att["bf16" if a.out_bf16 else "f32"] = a
        del o, lse
    return r


def check_topk(inp, orc, idx, tokens, exact: bool, K: int | None = None):
    """Top-K gate.  Exact mode: identical ints.  Continuous: recall >= 0.999 overall, every
    index in the symmetric difference within 1e-3 relative of the k-th score, full sets when
    k_t = n_t, ascending order and -1 padding always."""
    K = inp.wl.shape.K if K is None else K
    inter = total = 0
    worst = 1.0
    for t in tokens:
        o_idx, S, kth = orc.topk(t, K)
        g = idx[t]
        n = S.shape[0]
        k = min(K, n)
        gs = g[:k]
        assert np.all(g[k:] == -1), (t, "padding")
        assert np.all(np.diff(gs) > 0) and gs.min() >= 0 and gs.max() < n, (t, "order/range")
        if exact:
            assert np.array_equal(g, o_idx), (t, "exact-mode Top-K differs")
            continue
        a, b = set(gs.tolist()), set(o_idx[:k].tolist())
        if k == n:
            assert a == b, (t, "k_t = n_t must select everything")
        common = len(a & b)
        inter += common
        total += k
        worst = min(worst, common / k)
        for s in a ^ b:
            assert abs(S[s] - kth) <= 1e-3 * abs(kth), (t, s, S[s], kth)
    if not exact and total:
        rec = inter / total
        assert rec >= 0.999, f"recall {rec:.5f} (worst token {worst:.4f})"
        return rec, worst
    return 1.0, 1.0


def bf16_half_ulp(x):
    """Half the bf16 spacing at |x| (8 significant bits): 2^(e - 8) for |x| in [2^e, 2^(e+1))."""
    _, E = np.frexp(np.abs(np.asarray(x, np.float64)))
    return np.ldexp(1.0, E - 9)


def check_attention(inp, orc, r, tokens, tol: float | None = None, lse_tol: float = 1e-3):
    """Attention gate on the GPU's own selected set: |O_gpu - O_oracle| <= tol elementwise,
    plus, for an output stored in bf16, the half-ulp of that storage rounding at the value
    (tol + bf16_half_ulp(|O_oracle| + tol)): the gate bounds the computation, and a bf16
    output of magnitude above 4 cannot be closer than its own spacing allows."""
    sh = inp.wl.shape
    if tol is None:
        tol = 2e-2 if sh.kv_fp8 else 1e-2
    out_bf16 = getattr(r, "out_bf16", False)
    worst = worst_lse = worst_excess = 0.0
    for t in tokens:
        o, lse = orc.attention(t, r.idx[t])
        err = np.abs(r.out[t] - o)
        gate = tol + (bf16_half_ulp(np.abs(o) + tol) if out_bf16 else 0.0)
        worst_excess = max(worst_excess, float(np.max(err - gate)))
        fin = np.isfinite(lse)
        lerr = np.abs(r.lse[t][fin] - lse[fin]).max() if fin.any() else 0.0
        assert np.array_equal(np.isfinite(r.lse[t]), fin), (t, "lse -inf pattern")
        worst = max(worst, float(err.max()))
        worst_lse = max(worst_lse, lerr)
    assert worst_excess <= 0.0, (f"attention error above its gate by {worst_excess:.3e} "
                                 f"(max-abs {worst:.3e}, tol {tol}, bf16 output {out_bf16})")
    assert worst_lse <= lse_tol, f"lse max-abs error {worst_lse:.3e} > {lse_tol}"
    return worst, worst_lse


def check_scores(inp, orc, scores, tokens):
    """Unfused scores against the oracle: relative error (diagnostic bound 1e-4)."""
    worst = 0.0
    for t in tokens:
        S = orc.scores(t)
        g = scores[t, : S.shape[0]].astype(np.float64)
        den = np.maximum(np.abs(S), 1e-6 * max(1e-30, np.abs(S).max()))
        worst = max(worst, float(np.max(np.abs(g - S) / den)))
    return worst


def sample_tokens(inp, n: int, seed: int = 0):
    """First and last tokens, tokens around position 2047/2048, each request's chunk edges,
    and a seeded random sample."""
    T = inp.T
    pick = {0, T - 1}
    for b in range(inp.B):
        a, e = int(inp.cu_q[b]), int(inp.cu_q[b + 1])
        if e > a:
            pick |= {a, e - 1}
    pos = inp.positions
    for p in (2046, 2047, 2048, 2049):
        pick |= set(np.nonzero(pos == p)[0].tolist())
    rng = np.random.default_rng(seed)
    extra = rng.choice(T, size=min(T, n), replace=False)
    pick |= set(extra.tolist())
    return sorted(pick)


def math_ok(x):
    return x is not None and math.isfinite(x)
