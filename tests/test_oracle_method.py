"""Pins of the oracle's method functions against hand-worked values, brute force, closed
forms and invariants.  Each pin is chosen so that a plausible slip (a dropped ReLU or weight,
a transposed operand, a wrong tie rule, an off-by-one in the causal range, a missing max
subtraction) fails at least one of them; ``test_pins_catch_planted_mistakes`` checks that."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import synth
from oracle import (Oracle, a0_quantize, a0_scale, brute, decode_rows, sparse_mla_token,
                    token_scores, topk_token)
from oracle.codecs import E4M3_TABLE

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- A0
def _a0_brute(amax):
    if amax == 0:
        return 1.0
    for e in range(-160, 160):
        if amax <= 448.0 * 2.0 ** e:
            return 2.0 ** e
    raise AssertionError


def test_a0_scale_is_smallest_power_of_two():
    rng = np.random.default_rng(3)
    vals = [0.0, 448.0, 449.0, 447.0, 1.0, 3.0, 2.0, 0.875, 0.8750001, 224.0, 1e-30, 1e30,
            448.0 * 2 ** -20, 448.0 * 2 ** -20 * (1 + 2 ** -40), 1.75, 3.5, 3.50001]
    vals += list(np.abs(rng.normal(0, 1, 2000))) + list(np.exp(rng.uniform(-60, 60, 2000)))
    got = a0_scale(np.array(vals))
    for a, s in zip(vals, got):
        assert s == _a0_brute(a), a


def test_a0_quantize_bounds_and_exact_ints():
    rng = np.random.default_rng(4)
    q = rng.normal(0, 1, (50, 8, 128))
    qh, s = a0_quantize(q)
    assert np.all(np.abs(q / s[..., None]) <= 448.0)
    # each scaled value lands on the e4m3 grid
    grid = set(E4M3_TABLE[~np.isnan(E4M3_TABLE)].tolist())
    assert set(np.unique(qh / s[..., None]).tolist()) <= grid
    # relative error of a 3-bit mantissa RNE: at most 2^-4 in the normal range
    big = np.abs(q / s[..., None]) >= 2.0 ** -6
    assert np.all(np.abs(qh - q)[big] <= 2.0 ** -4 * np.abs(q)[big] * (1 + 1e-12))
    # small integers are reproduced exactly (scale 2^-7 or 2^-8)
    qi = rng.integers(-3, 4, (20, 4, 32)).astype(np.float64)
    qh, s = a0_quantize(qi)
    assert np.array_equal(qh, qi)


# ----------------------------------------------------------------------------- cache rows
def _e4m3_page_case():
    """The hand-worked e4m3 pages of tests/golden/e4m3_rows_handworked.json as raw arrays."""
    g = json.load(open(os.path.join(GOLD, "e4m3_rows_handworked.json")))
    P, page, D = g["n_pages"], g["page_size"], g["dim"]
    pool = np.full((P, page, D), g["fill"]["code"], dtype=np.uint8)
    scale = np.full((P, page), g["fill"]["scale"], dtype=np.float32)
    for e in g["slots"]:
        pool.reshape(-1, D)[e["slot"]] = e["codes"]
        if "scale_bits" in e:
            sc = np.array([int(e["scale_bits"], 16)], np.uint32).view(np.float32)[0]
        else:
            sc = np.float32(e["scale"])
        scale.reshape(-1)[e["slot"]] = sc
    exp = np.array([[float(Fraction(v)) for v in row] for row in g["expected_exact"]])
    assert np.array_equal(exp, np.array(g["expected"]))
    return pool, scale, np.array(g["page_table"]), np.array(g["positions"]), exp


def test_e4m3_rows_handworked():
    """decode_rows on e4m3 pages: code times the slot's own scale (non-unit, non-dyadic),
    through a page table that is not the identity."""
    pool, scale, pt, pos, exp = _e4m3_page_case()
    got = decode_rows(pool, scale, pt, pos, "e4m3")
    assert np.array_equal(got, exp)


# ----------------------------------------------------------------------------- scores / topk
def test_handworked_scores_and_topk():
    gold = json.load(open(os.path.join(GOLD, "score_handworked.json")))
    for c in gold["cases"]:
        S = token_scores(np.array(c["q"]), np.array(c["w"]), np.array(c["k"]))
        assert np.array_equal(S, np.array(c["scores"])), c["name"]
        for key in ("topk2", "topk3"):
            if key in c:
                K = int(key[-1])
                idx, _ = topk_token(S, K)
                assert idx.tolist() == c[key], c["name"]


@settings(max_examples=60, deadline=None)
@given(st.integers(1, 4), st.integers(1, 6), st.integers(1, 24), st.integers(0, 10 ** 6))
def test_scores_match_loops(H, D, n, seed):
    rng = np.random.default_rng(seed)
    q = rng.normal(0, 1, (H, D))
    w = rng.uniform(0, 1, H)
    k = rng.normal(0, 1, (n, D))
    ours = token_scores(q, w, k)
    ref = np.array(brute.score_loops(q.tolist(), w.tolist(), k.tolist()))
    assert np.allclose(ours, ref, rtol=1e-12, atol=1e-12)


@settings(max_examples=80, deadline=None)
@given(st.integers(1, 40), st.integers(1, 45), st.integers(0, 10 ** 6), st.booleans())
def test_topk_matches_rank_definition(n, K, seed, ties):
    rng = np.random.default_rng(seed)
    S = rng.integers(0, 4, n).astype(np.float64) if ties else rng.normal(0, 1, n)
    if ties:
        S[rng.random(n) < 0.3] = -0.0           # signed zeros tie with +0.0
    idx, kth = topk_token(S, K)
    assert idx.tolist() == brute.topk_by_rank(S.tolist(), K)
    k = min(K, n)
    sel = idx[:k]
    assert kth == np.sort(S)[::-1][k - 1]
    assert np.all(np.diff(sel) > 0) and np.all(idx[k:] == -1)


def test_topk_invariants():
    rng = np.random.default_rng(5)
    S = rng.normal(0, 1, 1000)
    a, _ = topk_token(S, 100)
    b, _ = topk_token(2.0 * S, 100)          # positive rescaling keeps the set
    assert np.array_equal(a, b)
    c, _ = topk_token(S, 5000)               # K >= n keeps everything
    assert np.array_equal(c[:1000], np.arange(1000)) and np.all(c[1000:] == -1)
    d, _ = topk_token(np.zeros(10), 3)       # all tied: lowest positions
    assert d.tolist() == [0, 1, 2]


# ----------------------------------------------------------------------------- attention
@settings(max_examples=40, deadline=None)
@given(st.integers(1, 3), st.integers(2, 6), st.integers(1, 5), st.integers(1, 12),
       st.integers(0, 10 ** 6))
def test_attention_full_selection_equals_dense_loops(H, Dqk, Dv, n, seed):
    Dv = min(Dv, Dqk)
    rng = np.random.default_rng(seed)
    q = rng.normal(0, 1, (H, Dqk))
    rows = rng.normal(0, 1, (n, Dqk))
    o, lse = sparse_mla_token(q, rows, 0.37, Dv)
    o2, lse2 = brute.attention_loops(q.tolist(), rows.tolist(), 0.37, Dv)
    assert np.allclose(o, np.array(o2), rtol=1e-12, atol=1e-12)
    assert np.allclose(lse, np.array(lse2), rtol=1e-12, atol=1e-12)


def test_attention_closed_forms():
    rng = np.random.default_rng(6)
    H, Dqk, Dv, n = 4, 12, 8, 30
    q = rng.normal(0, 1, (H, Dqk))
    rows = rng.normal(0, 1, (n, Dqk))
    # softmax weights: with one-hot value rows the output *is* the weight vector
    onehot = np.concatenate([np.eye(n), rng.normal(0, 1, (n, 3))], axis=1)
    qq = rng.normal(0, 1, (H, n + 3))
    p, lse = sparse_mla_token(qq, onehot, 0.5, n)
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-12) and np.all(p > 0)
    z = 0.5 * qq @ onehot.T
    assert np.allclose(p, np.exp(z - lse[:, None]), atol=1e-14)
    # one selected row: output is that row's value part; lse is its logit
    o, lse = sparse_mla_token(q, rows[3:4], 0.7, Dv)
    assert np.array_equal(o, np.repeat(rows[3:4, :Dv], H, axis=0))
    assert np.allclose(lse, 0.7 * q @ rows[3])
    # all rows equal: output equals the row, lse = z + ln n
    same = np.repeat(rows[5:6], n, axis=0)
    o, lse = sparse_mla_token(q, same, 0.7, Dv)
    assert np.allclose(o, rows[5, :Dv][None, :], atol=1e-14)
    assert np.allclose(lse, 0.7 * q @ rows[5] + math.log(n), atol=1e-12)
    # zero query: equal logits, output is the mean row, lse = ln n
    o, lse = sparse_mla_token(np.zeros((H, Dqk)), rows, 0.7, Dv)
    assert np.allclose(o, rows[:, :Dv].mean(axis=0)[None, :], atol=1e-14)
    assert np.allclose(lse, math.log(n), atol=1e-14)
    # no rows
    o, lse = sparse_mla_token(q, rows[:0], 0.7, Dv)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


# ----------------------------------------------------------------------------- end to end
def test_tiny_end_to_end_against_loops():
    inp = synth.make(synth.workload(synth.TINY), "continuous")
    orc = Oracle(inp)
    sh = inp.wl.shape
    for t in (0, 7):
        b, p = int(inp.req[t]), int(inp.positions[t])
        k = inp.k_pool.reshape(-1, sh.D_I)[: p + 1]           # identity page table
        S = brute.score_loops(inp.q_idx[t].tolist(), inp.w[t].tolist(), k.tolist())
        idx, S2, _ = orc.topk(t)
        assert np.allclose(S2, S, rtol=1e-12)
        assert idx.tolist() == brute.topk_by_rank(S, sh.K)
        rows = inp.kv_pool.reshape(-1, sh.D_qk)[idx]
        o2, lse2 = brute.attention_loops(inp.q[t].tolist(), rows.tolist(), sh.softmax_scale,
                                         sh.D_v)
        o, lse = orc.attention(t, idx)
        assert np.allclose(o, o2, atol=1e-12) and np.allclose(lse, lse2, atol=1e-12)
        # K >= n: the sparse result is dense causal attention over positions 0..p
        allidx = np.arange(p + 1)
        o3, _ = orc.attention(t, allidx)
        o4, _ = brute.attention_loops(inp.q[t].tolist(),
                                      inp.kv_pool.reshape(-1, sh.D_qk)[: p + 1].tolist(),
                                      sh.softmax_scale, sh.D_v)
        assert np.allclose(o3, o4, atol=1e-12)


def test_exact_mode_scores_are_exact_dyadics():
    wl = synth.reduced(synth.workload(synth.DECODE32K), [512, 700], [1, 3])
    inp = synth.make(wl, "exact")
    orc = Oracle(inp)
    for t in range(inp.T):
        S = orc.scores(t)
        # integer arithmetic: w in quarters, q/k small integers
        b, p = int(inp.req[t]), int(inp.positions[t])
        qi = (inp.q_idx[t].astype(np.uint32) << 16).view(np.float32).astype(np.int64)
        k = decode_rows(inp.k_pool, inp.k_scale, inp.page_table[b], np.arange(p + 1), "e4m3")
        dots = k.astype(np.int64) @ qi.T
        w4 = (inp.w[t] * 4).astype(np.int64)
        S4 = np.maximum(dots, 0) @ w4
        assert np.array_equal(S * 4, S4.astype(np.float64))


def test_page_permutation_invariance():
    wl = synth.reduced(synth.workload(synth.RAGGED), [300, 129, 64], [5, 1, 64],
                       structure="none")
    a = synth.make(wl, "continuous", random_pages=False)
    b = synth.make(wl, "continuous", random_pages=True)
    assert not np.array_equal(a.page_table, b.page_table)
    oa, ob = Oracle(a), Oracle(b)
    for t in range(a.T):
        ia, Sa, _ = oa.topk(t, K=48)
        ib, Sb, _ = ob.topk(t, K=48)
        assert np.array_equal(Sa, Sb) and np.array_equal(ia, ib)
        xa, la = oa.attention(t, ia)
        xb, lb = ob.attention(t, ib)
        assert np.array_equal(xa, xb) and np.array_equal(la, lb)


def test_pins_catch_planted_mistakes():
    """Plant plausible slips in copies of the oracle's functions; some pin must fail."""
    gold = json.load(open(os.path.join(GOLD, "score_handworked.json")))
    rng = np.random.default_rng(9)
    q, w, k = rng.normal(0, 1, (3, 5)), rng.uniform(0, 1, 3), rng.normal(0, 1, (9, 5))
    ref = np.array(brute.score_loops(q.tolist(), w.tolist(), k.tolist()))
    wrong_scores = [
        lambda q, w, k: (k @ q.T) @ w,                               # ReLU dropped
        lambda q, w, k: np.maximum(k @ q.T, 0).sum(axis=1),         # weights dropped
        lambda q, w, k: np.maximum(k @ q.T, 0) @ w[::-1],           # heads misaligned
        lambda q, w, k: np.maximum(k @ -q.T, 0) @ w,                # sign flip
    ]
    for f in wrong_scores:
        bad = not np.allclose(f(q, w, k), ref)
        for c in gold["cases"]:
            bad |= not np.array_equal(f(np.array(c["q"]), np.array(c["w"]), np.array(c["k"])),
                                      np.array(c["scores"]))
        assert bad
    S = rng.integers(0, 3, 30).astype(np.float64)
    K = int((S == 2).sum()) + 2            # the boundary splits the tie group of 1s
    good = brute.topk_by_rank(S.tolist(), K)
    wrong_topk = [
        lambda S, K: np.sort(np.argsort(-S, kind="stable")[::-1][:K]),   # smallest instead
        lambda S, K: np.sort(np.lexsort((-np.arange(len(S)), -S))[:K]),  # higher index wins
        lambda S, K: np.argsort(-S, kind="stable")[:K],                  # not ascending
    ]
    for f in wrong_topk:
        assert list(f(S, K)) != good
    q2, rows = rng.normal(0, 1, (2, 6)), rng.normal(0, 1, (7, 6))
    o_ref, _ = brute.attention_loops(q2.tolist(), rows.tolist(), 0.4, 4)

    def no_scale(q, r, s, dv):
        return sparse_mla_token(q, r, 1.0, dv)

    def v_from_tail(q, r, s, dv):
        return sparse_mla_token(q, r[:, ::-1], s, dv)

    for f in (no_scale, v_from_tail):
        o, _ = f(q2, rows, 0.4, 4)
        assert not np.allclose(o, o_ref)
    # e4m3 rows: the scale dropped, applied twice, taken from the position instead of the
    # slot, or the page table ignored
    from oracle.codecs import e4m3_decode
    pool, scale, pt, pos, exp = _e4m3_page_case()
    flat, sflat = pool.reshape(-1, pool.shape[-1]), scale.reshape(-1).astype(np.float64)
    slot = pt[pos // 64] * 64 + pos % 64
    wrong_rows = [
        e4m3_decode(flat[slot]),
        e4m3_decode(flat[slot]) * (sflat[slot] ** 2)[:, None],
        e4m3_decode(flat[slot]) * sflat[pos][:, None],
        e4m3_decode(flat[pos]) * sflat[pos][:, None],
    ]
    for rows_bad in wrong_rows:
        assert not np.array_equal(rows_bad, exp)
