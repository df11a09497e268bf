"""The seeded generator: determinism, page independence, poison and structure."""
import numpy as np

import synth
from oracle import decode_rows


def _small(cfg, **kw):
    wl = synth.workload(cfg)
    return synth.reduced(wl, [200, 64, 130], [3, 1, 2], **kw)


def test_deterministic_bytes():
    for cfg in range(5):
        wl = synth.workload(cfg) if cfg == 0 else _small(cfg)
        a = synth.make(wl, "continuous")
        b = synth.make(wl, "continuous")
        for f in ("q_idx", "w", "k_pool", "k_scale", "q", "kv_pool", "kv_scale", "page_table"):
            x, y = getattr(a, f), getattr(b, f)
            assert (x is None and y is None) or np.array_equal(x, y), (cfg, f)
        c = synth.make(wl, "exact")
        assert not np.array_equal(a.q_idx, c.q_idx)


def test_layout_and_poison():
    wl = _small(synth.DECODE1M, structure="none")
    inp = synth.make(wl, "continuous", random_pages=True)
    assert inp.T == 6 and inp.cu_q.tolist() == [0, 3, 4, 6]
    assert inp.positions.tolist() == [197, 198, 199, 63, 128, 129]
    P = inp.n_pages
    used = set()
    for b, L in enumerate(inp.seq_lens):
        npg = -(-int(L) // 64)
        used |= set(inp.page_table[b, :npg].tolist())
        # tail slots of the last page are poisoned
        last = inp.page_table[b, npg - 1]
        tail = int(L) - (npg - 1) * 64
        assert np.all(inp.kv_scale[last, tail:] == 1e4) and np.all(inp.k_scale[last, tail:] == 1e4)
        assert np.all(inp.kv_scale[last, :tail] < 1e3)
    for p in set(range(P)) - used:
        assert np.all(inp.k_pool[p] == 0x7E) and np.all(inp.kv_scale[p] == 1e4)


def test_pages_are_independent_of_placement():
    wl = _small(synth.DECODE32K)
    a = synth.make(wl, "continuous", random_pages=False)
    b = synth.make(wl, "continuous", random_pages=True)
    for r in range(wl.B):
        pos = np.arange(int(a.seq_lens[r]))
        for pool, sc, fmt in (("k_pool", "k_scale", "e4m3"), ("kv_pool", "kv_scale", "bf16")):
            x = decode_rows(getattr(a, pool), getattr(a, sc), a.page_table[r], pos, fmt)
            y = decode_rows(getattr(b, pool), getattr(b, sc), b.page_table[r], pos, fmt)
            assert np.array_equal(x, y)


def test_quantisation_recipe():
    wl = _small(synth.PREFILL64K, structure="none")
    inp = synth.make(wl, "continuous")
    # per-token e4m3: the largest code magnitude of a row is 448 (scale = amax/448)
    codes = inp.kv_pool[inp.page_table[0, 0]]
    mags = codes & 0x7F
    assert np.all(mags.max(axis=1) == 0x7E)
    # w in [0, 1/8)
    assert inp.w.min() >= 0 and inp.w.max() < 1 / 8


def test_structures():
    wl = synth.reduced(synth.workload(synth.PREFILL64K), [6400], [6400])
    inp = synth.make(wl, "continuous")
    hp = inp.info["heavy_positions"][0]
    assert len(hp) == 64
    sc = inp.kv_scale.reshape(-1)[:6400]
    assert np.median(sc[hp]) > 6 * np.median(np.delete(sc, hp))
    wl = synth.reduced(synth.workload(synth.DECODE1M), [20000], [1])
    inp = synth.make(wl, "continuous")
    off = inp.info["planted"][0]
    assert 0 <= off <= 20000 - 4097
    L = synth.workload(synth.RAGGED).seq_lens
    assert len(L) == 64 and min(L) >= 1024 and max(L) <= 262144
    q = synth.workload(synth.RAGGED).q_lens
    assert sum(1 for x in q if x > 1) == 16
