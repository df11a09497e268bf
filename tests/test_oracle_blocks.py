"""Pins of the oracle's block-granular selection: hand-worked rows, a brute-force block scan, the
equivalence of max-score block selection with walking the token ranking until K/64 distinct
blocks are met, the expansion against a loop, and planted mistakes that the pins must catch."""
import json
import os

import numpy as np
import pytest

from oracle import block_scores, expand_blocks, topk_blocks, topk_token

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _val(x):
    return -np.inf if x == "-inf" else float(x)


def _golden():
    g = json.load(open(os.path.join(GOLD, "block_select_handworked.json")))
    out = []
    for r in g["rows"]:
        if "S" in r:
            S = np.array([_val(x) for x in r["S"]])
        else:
            sp = r["S_sparse"]
            S = np.full(sp["n"], float(sp["fill"]))
            for k, v in sp["at"].items():
                S[int(k)] = v
        out.append((S, r))
    return out


def _brute_block_scores(S, page):
    """Position by position: each score raises its block's running maximum."""
    n = len(S)
    bs = [-np.inf] * (-(-n // page))
    for s in range(n):
        b = s // page
        if S[s] > bs[b]:
            bs[b] = S[s]
    return np.array(bs)


def _walk_token_ranking(S, K_blocks, page):
    """Blocks met, in order, when walking the positions by (score desc, position asc), until
    K_blocks distinct ones (an independent statement of max-score block selection)."""
    order = sorted(range(len(S)), key=lambda s: (-S[s], s))
    seen = []
    for s in order:
        b = s // page
        if b not in seen:
            seen.append(b)
        if len(seen) == K_blocks:
            break
    out = np.full(K_blocks, -1, np.int32)
    out[:len(seen)] = sorted(seen)
    return out


def _rows(rng):
    rows = []
    for n in (1, 63, 64, 65, 200, 1000, 4097):
        rows.append(rng.standard_normal(n))
        rows.append(rng.integers(-3, 4, n).astype(np.float64))        # many ties
    r = rng.standard_normal(700)
    r[rng.random(700) < 0.2] = -np.inf                                # out-of-range pages
    rows.append(r)
    return rows


def test_handworked_rows():
    for S, r in _golden():
        p = r["page"]
        bs = block_scores(S, page=p)
        assert np.array_equal(bs, np.array([_val(x) for x in r["block_scores"]])), r["work"]
        blk, kth = topk_blocks(bs, r["K"])
        assert blk.tolist() == r["blocks"], r["work"]
        assert kth == _val(r["kth"]), r["work"]
        ex = expand_blocks(blk, len(S), page=p)
        if "expanded" in r:
            assert ex.tolist() == r["expanded"], r["work"]
        else:
            assert ex[:4].tolist() == r["expanded_first"][:3] + [ex[3]] and ex[63] == 63
            for k, v in r["expanded_at"].items():
                assert ex[int(k)] == v, (k, r["work"])


def test_default_block_is_the_cache_page():
    S = np.zeros(130)
    S[64] = 1.0
    assert block_scores(S).tolist() == [0.0, 1.0, 0.0]
    assert expand_blocks(np.array([2]), 130)[:3].tolist() == [128, 129, -1]


def test_brute_force_block_scan():
    rng = np.random.default_rng(31)
    for S in _rows(rng):
        assert np.array_equal(block_scores(S), _brute_block_scores(S, 64))


def test_equals_walking_the_token_ranking():
    rng = np.random.default_rng(32)
    for S in _rows(rng):
        for K_blocks in (1, 2, 5, 32, 100):
            blk, _ = topk_blocks(block_scores(S), K_blocks)
            assert np.array_equal(blk, _walk_token_ranking(S, K_blocks, 64)), (len(S), K_blocks)


def test_invariants():
    rng = np.random.default_rng(33)
    for S in _rows(rng):
        n = len(S)
        nb = -(-n // 64)
        blk, _ = topk_blocks(block_scores(S), 4096)
        assert blk[:nb].tolist() == list(range(nb)) and np.all(blk[nb:] == -1)
        top, _ = topk_token(S, 1)
        b1, _ = topk_blocks(block_scores(S), 1)
        assert b1[0] == top[0] // 64               # the best token's block is the best block


def test_expansion_against_a_loop():
    rng = np.random.default_rng(34)
    for n in (1, 64, 65, 1000):
        nb = -(-n // 64)
        blocks = np.sort(rng.choice(nb, size=min(nb, 5), replace=False)).astype(np.int32)
        blocks = np.concatenate([blocks, [-1, -1]]).astype(np.int32)
        ex = expand_blocks(blocks, n)
        for i, b in enumerate(blocks):
            for r in range(64):
                want = 64 * b + r if (b >= 0 and 64 * b + r < n) else -1
                assert ex[64 * i + r] == want


def test_pins_catch_planted_mistakes(monkeypatch):
    import oracle.method as M
    real_bs, real_tb, real_ex = M.block_scores, M.topk_blocks, M.expand_blocks

    def sum_scores(S, page=64):
        S = np.asarray(S, np.float64)
        return np.array([S[page * j:page * (j + 1)].sum() for j in range(-(-len(S) // page))])

    def drop_partial_block(S, page=64):
        return real_bs(S, page)[:len(S) // page]

    def ties_to_higher(bs, K):
        bs = np.asarray(bs, np.float64)
        order = np.lexsort((-np.arange(bs.size), -bs))
        k = min(K, bs.size)
        out = np.full(K, -1, np.int32)
        out[:k] = np.sort(order[:k])
        return out, (float(bs[order[k - 1]]) if k else None)

    def expand_inclusive(blocks, n, page=64):
        return real_ex(blocks, n + 1, page)

    bads = {"sum": ("block_scores", sum_scores), "partial": ("block_scores", drop_partial_block),
            "ties": ("topk_blocks", ties_to_higher), "clip": ("expand_blocks", expand_inclusive)}
    import sys
    T = sys.modules[__name__]      # the module these checks run in, as pytest imported it
    for name, (fn, bad) in bads.items():
        monkeypatch.setattr(T, fn, bad)
        failed = False
        for chk in (test_handworked_rows, test_brute_force_block_scan,
                    test_equals_walking_the_token_ranking, test_expansion_against_a_loop,
                    test_default_block_is_the_cache_page):
            try:
                chk()
            except (AssertionError, IndexError, ValueError):
                failed = True
        assert failed, name
        monkeypatch.setattr(T, fn, {"block_scores": real_bs, "topk_blocks": real_tb,
                                    "expand_blocks": real_ex}[fn])
