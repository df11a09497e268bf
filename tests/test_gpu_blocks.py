"""GPU parity of block-granular selection (through the C ABI) against the oracle.

For each case: the block scores equal the largest GPU token score of each page's causal
positions (bit for bit: the same fp32 values); the selection over the GPU's block scores equals
the oracle's selection over the same scores (bit for bit); the expansion equals the oracle's;
fused == unfused; against the oracle's own fp64 block scores the selection is bit-exact in the
exact input mode and otherwise has recall >= 0.999 with every mismatched page within 1e-3
relative of the kb-th block score; attention over the expanded positions passes the usual gate."""
import numpy as np
import pytest
import torch

import synth
import top_indexed_sparse_amd as tis
from oracle import Oracle, block_scores, expand_blocks, topk_blocks
from synth.device import to_device
from tests.gpu_path import (check_attention, make_batch, note, sample_tokens)

pytestmark = pytest.mark.gpu


def run_blocks(inp, K_blocks):
    sh = inp.wl.shape
    d = to_device(inp)
    bt = make_batch(inp)
    T = inp.T
    nb = tis.blocks_of(bt.max_n)
    ld = (nb + 3) // 4 * 4
    ldt = (bt.max_n + 3) // 4 * 4
    tok = torch.full((T, ldt), float("nan"), dtype=torch.float32, device="cuda")
    tis.index_score(bt, d.q_idx, d.w, d.k_pool, d.k_scale, tok)
    bsc = torch.full((T, ld), float("nan"), dtype=torch.float32, device="cuda")
    tis.index_score_block(bt, d.q_idx, d.w, d.k_pool, d.k_scale, bsc)
    bi = torch.empty((T, K_blocks), dtype=torch.int32, device="cuda")
    bv = torch.empty((T, K_blocks), dtype=torch.float32, device="cuda")
    ti = torch.empty((T, 64 * K_blocks), dtype=torch.int32, device="cuda")
    tis.topk_block_select(bt, bsc, K_blocks, bi, bv, ti)
    fbi = torch.empty_like(bi)
    fbv = torch.empty_like(bv)
    fti = torch.empty_like(ti)
    tis.index_score_topk_block(bt, d.q_idx, d.w, d.k_pool, d.k_scale, K_blocks, fbi, fbv, fti)
    out_dt = torch.float32 if sh.kv_fp8 else torch.bfloat16
    o = torch.empty((T, sh.H, sh.D_v), dtype=out_dt, device="cuda")
    lse = torch.empty((T, sh.H), dtype=torch.float32, device="cuda")
    tis.sparse_mla_attn(bt, d.q, d.kv_pool, d.kv_scale, ti, sh.softmax_scale, o, lse)
    torch.cuda.synchronize()
    r = type("R", (), {})()
    r.tok, r.bsc = tok.cpu().numpy(), bsc.cpu().numpy()
    r.bi, r.bv, r.ti = bi.cpu().numpy(), bv.cpu().numpy(), ti.cpu().numpy()
    r.fused_equal = (torch.equal(bi, fbi) and torch.equal(bv, fbv) and torch.equal(ti, fti))
    r.fbi, r.fbv, r.fti = fbi.cpu().numpy(), fbv.cpu().numpy(), fti.cpu().numpy()
    r.idx = r.ti
    r.out = o.float().cpu().numpy().astype(np.float64)
    r.out_bf16 = out_dt == torch.bfloat16
    r.lse = lse.cpu().numpy().astype(np.float64)
    return r


def check_blocks(inp, r, tokens, K_blocks, exact):
    orc = Oracle(inp)
    if not r.fused_equal:
        for name, u, f in (("block_idx", r.bi, r.fbi), ("block_val", r.bv, r.fbv),
                           ("topk_idx", r.ti, r.fti)):
            bad = np.argwhere(~((u == f) | (np.isnan(u) & np.isnan(f))) if u.dtype.kind == "f"
                              else u != f)
            if bad.size:
                t0 = int(bad[0][0])
                note(f"  {name}: {len(bad)} entries differ, first token {t0}: "
                     f"unfused {u[t0][:12].tolist()} fused {f[t0][:12].tolist()}")
    hits = total = 0
    for t in tokens:
        n = int(inp.positions[t]) + 1
        nb = -(-n // 64)
        # block scores are the GPU token scores' page maxima, bit for bit
        gb = block_scores(r.tok[t, :n].astype(np.float64))
        assert np.array_equal(r.bsc[t, :nb].astype(np.float64), gb), (t, "block max")
        # the selection over the GPU's block scores is the oracle's, bit for bit
        sel, _ = topk_blocks(r.bsc[t, :nb].astype(np.float64), K_blocks)
        assert np.array_equal(r.bi[t], sel), (t, "block selection")
        kb = min(K_blocks, nb)
        assert np.array_equal(r.bv[t, :kb], r.bsc[t, sel[:kb]]), (t, "block values")
        assert np.array_equal(r.ti[t], expand_blocks(r.bi[t], n)), (t, "expansion")
        # against the oracle's fp64 scores
        oblk, obs, kth, _ = orc.block_topk(t, K_blocks)
        if exact:
            assert np.array_equal(r.bi[t], oblk), (t, "exact-mode block selection")
            continue
        a, b = set(r.bi[t][:kb].tolist()), set(oblk[:kb].tolist())
        hits += len(a & b)
        total += kb
        for j in a ^ b:
            assert abs(obs[j] - kth) <= 1e-3 * abs(kth), (t, j, obs[j], kth)
    rec = hits / total if total else 1.0
    assert r.fused_equal, "fused vs unfused block selection"
    if not exact:
        assert rec >= 0.999, f"block recall {rec:.5f}"
    err = check_attention(inp, orc, r, tokens)
    note(f"  {inp.wl.name}/{inp.mode}: block recall {rec:.5f}, attn err {err[0]:.2e}")
    return rec


@pytest.mark.parametrize("mode", ["continuous", "exact"])
def test_blocks_decode_shapes_small(mode):
    wl = synth.reduced(synth.workload(synth.DECODE32K), [4096, 1500, 5000, 2049, 70], [1, 1, 2, 1, 1])
    inp = synth.make(wl, mode)
    note(f"case blocks decode-small mode={mode} T={inp.T}")
    r = run_blocks(inp, 32)
    check_blocks(inp, r, list(range(inp.T)), 32, mode == "exact")


@pytest.mark.parametrize("mode", ["continuous", "exact"])
def test_blocks_prefill_shapes_small(mode):
    wl = synth.reduced(synth.workload(synth.PREFILL64K), [2600], [2600])
    inp = synth.make(wl, mode)
    note(f"case blocks prefill-small mode={mode} T={inp.T}")
    r = run_blocks(inp, 8)
    check_blocks(inp, r, sample_tokens(inp, 100), 8, mode == "exact")


@pytest.mark.parametrize("mode", ["continuous", "exact"])
def test_blocks_ragged_small(mode):
    L = [1024, 3000, 700, 5000, 64, 2100]
    q = [1, 300, 1, 1, 64, 1]
    wl = synth.reduced(synth.workload(synth.RAGGED), L, q)
    inp = synth.make(wl, mode)
    note(f"case blocks ragged-small mode={mode} T={inp.T}")
    r = run_blocks(inp, 16)
    check_blocks(inp, r, sample_tokens(inp, 80), 16, mode == "exact")


def test_blocks_mxfp8_keys():
    wl = synth.reduced(synth.workload(synth.DECODE32K), [4096, 3000, 5000], [1, 1, 1])
    inp = synth.make(wl, "exact", k_fmt="mxfp8")
    note("case blocks mxfp8 exact")
    r = run_blocks(inp, 32)
    check_blocks(inp, r, list(range(inp.T)), 32, True)


def test_blocks_out_of_range_pages():
    """A page-table entry outside the pool gives its block the score -inf (never selected while
    other blocks remain) and no attended position."""
    wl = synth.reduced(synth.workload(synth.DECODE32K), [3000, 5000], [1, 1])
    inp = synth.make(wl, "continuous")
    inp.page_table = inp.page_table.copy()
    inp.page_table[0, 5] = inp.n_pages + 7
    inp.page_table[1, 0] = -3
    note("case blocks out-of-range pages")
    r = run_blocks(inp, 32)
    assert r.bsc[0, 5] == -np.inf and r.bsc[1, 0] == -np.inf
    assert 5 not in r.bi[0].tolist() and 0 not in r.bi[1].tolist()
    assert not np.any((r.ti[0] >= 320) & (r.ti[0] < 384))


def test_blocks_planted_block():
    """decode1m shapes: the 4096-position planted block spans 64 pages, so the 32 kept pages
    lie (almost) all inside it."""
    wl = synth.reduced(synth.workload(synth.DECODE1M), [70000, 40000], [1, 1])
    inp = synth.make(wl, "continuous")
    note("case blocks planted block")
    r = run_blocks(inp, 32)
    check_blocks(inp, r, list(range(inp.T)), 32, False)
    for b in range(inp.B):
        off = inp.info["planted"][b]
        sel = r.bi[b][r.bi[b] >= 0]
        frac = np.mean((64 * sel + 63 >= off) & (64 * sel < off + 4096))
        note(f"  request {b}: {frac:.3f} of the kept pages overlap the planted block")
        assert frac > 0.9


def test_blocks_decode32k_full():
    inp = synth.make(synth.workload(synth.DECODE32K), "continuous")
    note(f"case blocks decode32k full T={inp.T}")
    r = run_blocks(inp, 32)
    check_blocks(inp, r, list(range(inp.T)), 32, False)
