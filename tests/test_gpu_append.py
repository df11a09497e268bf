"""GPU parity of cache_append (through the C ABI) against the oracle's cache append: every byte
of the pool and every scale bit-exact, for e4m3, MXFP8 and bf16 caches, fp32 and bf16 rows, the
indexer-key and latent row widths; then one decode step over the appended caches (index,
Top-K, attention) against the oracle."""
import dataclasses

import numpy as np
import pytest
import torch

import synth
import top_indexed_sparse_amd as tis
from oracle import cache_append
from tests.gpu_path import note, run_path
from tests.test_gpu_parity import _common

pytestmark = pytest.mark.gpu


def _awkward_rows(rng, n, D):
    """Gaussian rows of the generator's scale plus rows that stress the quantiser."""
    rows = rng.standard_normal((n, D)).astype(np.float32)
    if n > 1:
        rows[1] = 0.0                                 # all zeros: scale 1, codes 0
        rows[1, 3] = -0.0
    if n > 2:
        rows[2] *= 1e-3
        rows[2, 7] = 50.0                             # one spike: most codes subnormal
    if n > 3:
        rows[3] = (rng.standard_normal(D) * 1e-30).astype(np.float32)
    if n > 4:
        rows[4, :2] = [1.0, np.array([0x3cf6db6e], np.uint32).view(np.float32)[0]]
        rows[4, 2:] = 0.0                             # an fp32 quotient that decides a tie
    if n > 5:
        rows[5] = (rng.standard_t(2, D) * 3).astype(np.float32)
    return rows


def _batch(rng, D):
    """Requests of mixed lengths and query counts (one with none, one whose last page entry is
    outside the pool), pages in a shuffled order, pool bytes random."""
    seq_lens = np.array([200, 70, 1000, 64, 300, 129], np.int32)
    q_lens = np.array([1, 3, 2, 1, 0, 1], np.int32)
    cu_q = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    stride = 16
    n_pages = 40
    perm = rng.permutation(n_pages).astype(np.int32)
    pt = np.full((len(seq_lens), stride), -1, np.int32)
    k = 0
    for b, L in enumerate(seq_lens):
        for j in range(-(-int(L) // 64)):
            pt[b, j] = perm[k % n_pages]
            k += 1
    pt[5, 2] = n_pages + 3                      # request 5's new token (position 128) is dropped
    return seq_lens, q_lens, cu_q, pt, n_pages


@pytest.mark.parametrize("D", [128, 576])
@pytest.mark.parametrize("rows_dt", ["f32", "bf16"])
@pytest.mark.parametrize("pool_dt", ["e4m3", "mxfp8", "bf16"])
def test_append_bit_exact(D, rows_dt, pool_dt):
    rng = np.random.default_rng(1000 * D + (rows_dt == "bf16") * 10 +
                                {"e4m3": 0, "bf16": 1, "mxfp8": 2}[pool_dt])
    seq_lens, q_lens, cu_q, pt, n_pages = _batch(rng, D)
    T = int(cu_q[-1])
    note(f"case cache_append D={D} rows={rows_dt} pool={pool_dt} T={T}")
    rows = _awkward_rows(rng, T, D)
    if rows_dt == "bf16":  # the rows as the bf16 values the call receives
        rows_dev = torch.from_numpy(rows).to(torch.bfloat16)
        rows = rows_dev.float().numpy()
    else:
        rows_dev = torch.from_numpy(rows)
    if pool_dt == "e4m3":
        pool = rng.integers(0, 0x7F, (n_pages, 64, D), dtype=np.uint8)
        scale = (rng.random((n_pages, 64)) + 0.5).astype(np.float32)
    elif pool_dt == "mxfp8":
        pool = rng.integers(0, 0x7F, (n_pages, 64, D), dtype=np.uint8)
        scale = rng.integers(0, 255, (n_pages, 64, D // 32), dtype=np.uint8)
    else:
        pool = rng.integers(0, 1 << 14, (n_pages, 64, D), dtype=np.uint16)
        scale = None
    # oracle: request by request, the query tokens' positions
    ref_pool, ref_scale = pool, scale
    for b in range(len(seq_lens)):
        a, e = int(cu_q[b]), int(cu_q[b + 1])
        if e > a:
            pos = np.arange(int(seq_lens[b]) - (e - a), int(seq_lens[b]))
            ref_pool, ref_scale = cache_append(ref_pool, ref_scale, pt[b], pos, rows[a:e],
                                               pool_dt)
    bt = tis.Batch(seq_lens, cu_q, pt, n_pages)
    if pool_dt in ("e4m3", "mxfp8"):
        dpool = torch.from_numpy(pool).cuda()
        dscale = torch.from_numpy(scale).cuda()
    else:
        dpool = torch.from_numpy(pool.view(np.int16)).view(torch.bfloat16).cuda()
        dscale = None
    tis.cache_append(bt, rows_dev.cuda(), dpool, dscale)
    torch.cuda.synchronize()
    if pool_dt == "e4m3":
        got = dpool.cpu().numpy()
        assert np.array_equal(dscale.cpu().numpy().view(np.uint32), ref_scale.view(np.uint32))
    elif pool_dt == "mxfp8":
        got = dpool.cpu().numpy()
        assert np.array_equal(dscale.cpu().numpy(), ref_scale)
    else:
        got = dpool.cpu().view(torch.int16).numpy().view(np.uint16)
    bad = np.argwhere(got != ref_pool)
    assert bad.size == 0, f"{len(bad)} bytes differ, first at {bad[:4].tolist()}"
    # something was written (and the dropped token's page stayed as it was)
    assert not np.array_equal(got, pool)


@pytest.mark.parametrize("kv_fp8", [False, True])
def test_decode_step_on_appended_cache(kv_fp8):
    """One decode step: the new tokens' indexer keys and latent rows are appended (e4m3 keys;
    bf16 or e4m3 latent rows), the device caches equal the oracle's appended caches byte for
    byte, and the chain over them passes the parity gates against the oracle."""
    base = synth.workload(synth.DECODE32K)
    wl = synth.reduced(base, [3000, 4096, 1500, 5000], [1, 1, 2, 1],
                       shape=dataclasses.replace(base.shape, kv_fp8=kv_fp8))
    inp = synth.make(wl, "continuous")
    sh = wl.shape
    rng = np.random.default_rng(20261208 + kv_fp8)
    T = inp.T
    k_rows = rng.standard_normal((T, sh.D_I)).astype(np.float32)
    c_rows = rng.standard_normal((T, sh.D_qk)).astype(np.float32)
    note(f"case decode step after append kv_fp8={kv_fp8} T={T}")
    # oracle side
    kp, ks = inp.k_pool, inp.k_scale
    cp, cs = inp.kv_pool, inp.kv_scale
    fmt = "e4m3" if kv_fp8 else "bf16"
    for t in range(T):
        b, p = int(inp.req[t]), int(inp.positions[t])
        kp, ks = cache_append(kp, ks, inp.page_table[b], [p], k_rows[t:t + 1], "e4m3")
        cp, cs = cache_append(cp, cs, inp.page_table[b], [p], c_rows[t:t + 1], fmt)
    # device side: append to the original caches
    bt = tis.Batch(inp.seq_lens, inp.cu_q, inp.page_table, inp.n_pages)
    dk = torch.from_numpy(inp.k_pool).cuda()
    dks = torch.from_numpy(inp.k_scale).cuda()
    if kv_fp8:
        dc = torch.from_numpy(inp.kv_pool).cuda()
        dcs = torch.from_numpy(inp.kv_scale).cuda()
    else:
        dc = torch.from_numpy(inp.kv_pool.view(np.int16)).view(torch.bfloat16).cuda()
        dcs = None
    tis.cache_append(bt, torch.from_numpy(k_rows).cuda(), dk, dks)
    tis.cache_append(bt, torch.from_numpy(c_rows).cuda(), dc, dcs)
    torch.cuda.synchronize()
    assert np.array_equal(dk.cpu().numpy(), kp)
    assert np.array_equal(dks.cpu().numpy().view(np.uint32), ks.view(np.uint32))
    if kv_fp8:
        assert np.array_equal(dc.cpu().numpy(), cp)
        assert np.array_equal(dcs.cpu().numpy().view(np.uint32), cs.view(np.uint32))
    else:
        assert np.array_equal(dc.cpu().view(torch.int16).numpy().view(np.uint16), cp)
    # the step over the appended caches (the same bytes) against the oracle
    inp2 = dataclasses.replace(inp, k_pool=kp, k_scale=ks, kv_pool=cp, kv_scale=cs)
    r = run_path(inp2)
    _common(inp2, r, list(range(T)), False)
