"""GPU parity of the decode scorer at its larger key chunks (through the C ABI).

A decode workgroup scores a chunk of 512 * np keys of one token; the library takes np = 8
(4,096 keys) unless few long rows would leave it running several rounds of workgroups, when
it takes 16 or 32 pages per wave.  These batches are sized so that its rule picks 16 (two
rows of about 1M keys) and 32 (four such rows), with row ends that leave the last chunk
partial: waves whose pages in range are not a multiple of the four-page ring step, waves
with none, and a last page with fewer than 64 keys; at 32 pages also with MXFP8 keys and with
the bf16 query used as stored.  Exact-mode inputs (integer queries, keys and weights) make
every score exact, so sampled scores are compared bit for bit with the oracle; entries past a
row's range must stay as they were."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import synth
import top_indexed_sparse_amd as tis
from oracle import Oracle
from oracle.method import decode_rows, token_scores
from synth.device import to_device
from tests.gpu_path import make_batch, note

pytestmark = pytest.mark.gpu

M = 1 << 20
SENTINEL = -12345.5


def _inputs(lens, random_pages, k_fmt="e4m3"):
    base = synth.workload(synth.DECODE1M, "exact")
    # a narrow latent cache: the scorer does not read it, and the inputs stay small
    sh = replace(base.shape, H=16, D_qk=64, D_v=32)
    wl = synth.reduced(base, lens, [1] * len(lens), name="decode-long-chunks", shape=sh,
                       paged_random=random_pages)
    return synth.make(wl, "exact", k_fmt=k_fmt)


def _positions(n, rng):
    """Chunk and page edges of every chunk size, the row's ends and a seeded random fill."""
    pick = set(range(min(n, 64))) | set(range(max(0, n - 200), n))
    for step in (4096, 8192, 16384):
        for c in range(step, n, step):
            pick |= {c - 1, c, c + 63, c + 64}
    pick |= set(rng.integers(0, n, size=3000).tolist())
    return np.array(sorted(p for p in pick if 0 <= p < n), dtype=np.int64)


LONG4 = [M - 1, M - 777, M - 5005, M - 25391]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("lens,random_pages,k_fmt,bf16_query", [
    ([M - 777, M - 9000], False, "e4m3", False),        # 16 pages per wave
    (LONG4, True, "e4m3", False),                       # 32 pages per wave
    (LONG4, True, "mxfp8", False),                      # MXFP8 keys and query
    (LONG4, False, "e4m3", True),                       # the bf16 query as stored
    # long rows among short ones: the launches are planned per run of tokens, each with its
    # own chunk size
    ([M - 777] + [3000 + 97 * i for i in range(20)] + [M - 9000], True, "e4m3", False),
])
def test_decode_scorer_long_chunks(lens, random_pages, k_fmt, bf16_query):
    inp = _inputs(lens, random_pages, k_fmt)
    note(f"case decode scorer chunks: lens {lens}, random pages {random_pages}, keys {k_fmt}, "
         f"bf16 query {bf16_query}")
    d = to_device(inp)
    bt = make_batch(inp)
    qmode = tis.TIS_QMODE_BF16 if bf16_query else None
    T = inp.T
    ld = (bt.max_n + 3) // 4 * 4 + 8
    scores = torch.full((T, ld), SENTINEL, dtype=torch.float32, device="cuda")
    tis.index_score(bt, d.q_idx, d.w, d.k_pool, d.k_scale, scores, qmode=qmode)
    nb = -(-bt.max_n // 64)
    ldb = (nb + 3) // 4 * 4 + 8
    blocks = torch.full((T, ldb), SENTINEL, dtype=torch.float32, device="cuda")
    tis.index_score_block(bt, d.q_idx, d.w, d.k_pool, d.k_scale, blocks, qmode=qmode)
    torch.cuda.synchronize()
    S = scores.cpu().numpy()
    Bk = blocks.cpu().numpy()
    orc = Oracle(inp, qmode="none" if bf16_query else None)
    rng = np.random.default_rng(7)
    for t in range(T):
        b = int(inp.req[t])
        n = int(inp.positions[t]) + 1
        assert np.all(S[t, n:] == SENTINEL), f"token {t}: a score past its range was written"
        pos = _positions(n, rng)
        k = decode_rows(inp.k_pool, inp.k_scale, inp.page_table[b], pos, k_fmt)
        want = token_scores(orc.q_hat(t), inp.w[t].astype(np.float64), k)
        got = S[t, pos].astype(np.float64)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (t, pos[bad[:5]], got[bad[:5]], want[bad[:5]])
        # block scores: the largest causal score of each sampled page
        nbt = -(-n // 64)
        assert np.all(Bk[t, nbt:] == SENTINEL), f"token {t}: a page score past its range"
        # pages at the chunk edges of every chunk size, the last ones and a seeded fill
        edge = [c // 64 + o for step in (4096, 8192, 16384) for c in range(step, n, step)
                for o in (-1, 0)]
        pages = np.unique(np.concatenate([np.asarray(edge, dtype=np.int64),
                                          np.arange(max(0, nbt - 8), nbt),
                                          rng.integers(0, nbt, size=200)]))
        for j in pages:
            pp = np.arange(64 * j, min(64 * j + 64, n))
            kp = decode_rows(inp.k_pool, inp.k_scale, inp.page_table[b], pp, k_fmt)
            wj = token_scores(orc.q_hat(t), inp.w[t].astype(np.float64), kp).max()
            assert Bk[t, j] == wj, (t, j, Bk[t, j], wj)
        note(f"  token {t}: n={n}, {pos.size} scores and {pages.size} page scores exact")
