"""GPU parity of the MXFP8 indexer (keys with one scale byte per 32 dims, the query quantised
per 32 dims in the kernel's prologue) against the oracle on seeded inputs, through the C ABI.

Gates as for the per-token e4m3 indexer: in the exact input mode (integers in [-3, 3], which
MXFP8 holds exactly) scores and Top-K are bit-exact; otherwise recall >= 0.999 with every
mismatch within 1e-3 relative of the k-th score and a score error bound of 1e-4 relative;
fused == unfused bit for bit; attention is gated as everywhere else."""
import numpy as np
import pytest
import torch

import synth
import top_indexed_sparse_amd as tis
from oracle import Oracle, cache_append as oracle_append
from synth.device import to_device
from tests.gpu_path import (check_attention, check_scores, check_topk, make_batch, note,
                            run_path, run_path_sampled, sample_tokens)

pytestmark = pytest.mark.gpu


def _check(inp, r, tokens, exact):
    orc = Oracle(inp)
    assert orc.qmode == "mxfp8" and orc.k_fmt == "mxfp8"
    assert np.array_equal(r.idx, r.idx2), "fused vs unfused Top-K"
    assert np.array_equal(r.val, r.val2), "fused vs unfused Top-K values"
    for t in tokens[:8]:
        sel = r.idx[t][r.idx[t] >= 0]
        assert np.array_equal(r.val[t][: sel.size], r.scores[t, sel]), t
    serr = check_scores(inp, orc, r.scores, tokens)
    rec = check_topk(inp, orc, r.idx, tokens, exact)
    aerr = check_attention(inp, orc, r, tokens)
    note(f"  {inp.wl.name}/{inp.mode}/mxfp8: score rel err {serr:.2e}, recall {rec}, "
         f"attn err {aerr[0]:.2e}")
    if exact:
        assert serr == 0.0
    else:
        assert serr < 1e-4
    return serr


@pytest.mark.parametrize("mode", ["continuous", "exact"])
def test_mx_decode_shapes_small(mode):
    # decode32k shapes (the decode scorer); a request shorter than K, a ragged tail page
    wl = synth.reduced(synth.workload(synth.DECODE32K), [4096, 1500, 5000, 2049], [1, 1, 2, 1])
    inp = synth.make(wl, mode, k_fmt="mxfp8")
    note(f"case mx decode-small mode={mode} T={inp.T}")
    r = run_path(inp)
    _check(inp, r, list(range(inp.T)), mode == "exact")


@pytest.mark.parametrize("mode", ["continuous", "exact"])
def test_mx_prefill_shapes_small(mode):
    # prefill shapes (the shared-page prefill scorer): every token queries its prefix
    wl = synth.reduced(synth.workload(synth.PREFILL64K), [2600], [2600])
    inp = synth.make(wl, mode, k_fmt="mxfp8")
    note(f"case mx prefill-small mode={mode} T={inp.T}")
    r = run_path(inp)
    _check(inp, r, sample_tokens(inp, 120), mode == "exact")


@pytest.mark.parametrize("mode", ["continuous", "exact"])
def test_mx_ragged_small(mode):
    # random page table with poisoned slack pages (scale byte 2^20), mixed decode and prefill
    L = [1024, 3000, 700, 5000, 64, 2100]
    q = [1, 300, 1, 1, 64, 1]
    wl = synth.reduced(synth.workload(synth.RAGGED), L, q)
    inp = synth.make(wl, mode, k_fmt="mxfp8")
    note(f"case mx ragged-small mode={mode} T={inp.T}")
    r = run_path(inp)
    _check(inp, r, sample_tokens(inp, 80), mode == "exact")


def test_mx_decode32k_full():
    """The 32 x 32K decode workload with MXFP8 keys, every token against the oracle."""
    inp = synth.make(synth.workload(synth.DECODE32K), "continuous", k_fmt="mxfp8")
    note(f"case mx decode32k full T={inp.T}")
    r = run_path(inp)
    _check(inp, r, list(range(inp.T)), False)


def test_mx_planted_block_dominates():
    """decode1m shapes (16 key splits per token in the attention) with MXFP8 keys: the planted
    block of high-relevance keys still dominates the selection."""
    wl = synth.reduced(synth.workload(synth.DECODE1M), [70000, 40000], [1, 1])
    inp = synth.make(wl, "continuous", k_fmt="mxfp8")
    note("case mx decode1m-small")
    r = run_path(inp)
    _check(inp, r, list(range(inp.T)), False)
    for b in range(inp.B):
        off = inp.info["planted"][b]
        sel = r.idx[b][r.idx[b] >= 0]
        assert np.mean((sel >= off) & (sel < off + 4096)) > 0.5


def test_mx_keys_appended_on_the_gpu_score_like_the_oracles():
    """cache_append writes MXFP8 keys bit for bit as the oracle's append does; scores computed
    over the GPU-written cache then match the oracle over the oracle-written one."""
    wl = synth.reduced(synth.workload(synth.DECODE32K), [3000, 700, 4100], [1, 1, 1])
    inp = synth.make(wl, "continuous", k_fmt="mxfp8")
    note("case mx append then score")
    rng = np.random.default_rng(77)
    rows = (rng.standard_normal((inp.T, 128)) * 2.0 ** rng.integers(-6, 6, (inp.T, 1))).astype(
        np.float32)
    pool, scl = inp.k_pool.copy(), inp.k_scale.copy()
    for b in range(inp.B):
        a, e = int(inp.cu_q[b]), int(inp.cu_q[b + 1])
        pool, scl = oracle_append(pool, scl, inp.page_table[b], inp.positions[a:e], rows[a:e],
                                  "mxfp8")
    d = to_device(inp)
    bt = make_batch(inp)
    tis.cache_append(bt, torch.from_numpy(rows).cuda(), d.k_pool, d.k_scale)
    torch.cuda.synchronize()
    assert np.array_equal(d.k_pool.cpu().numpy(), pool)
    assert np.array_equal(d.k_scale.cpu().numpy(), scl)
    ld = (bt.max_n + 3) // 4 * 4
    scores = torch.full((inp.T, ld), float("nan"), dtype=torch.float32, device="cuda")
    tis.index_score(bt, d.q_idx, d.w, d.k_pool, d.k_scale, scores)
    torch.cuda.synchronize()
    inp.k_pool, inp.k_scale = pool, scl
    err = check_scores(inp, Oracle(inp), scores.cpu().numpy(), list(range(inp.T)))
    note(f"  score rel err {err:.2e}")
    assert err < 1e-4
