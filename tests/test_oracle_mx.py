"""Pins of the oracle's MXFP8 quantiser (the indexer's Q/K format with one power-of-two scale per
32 elements) and of the scores and cache rows built on it: hand-worked groups, a brute-force
search for the shared exponent, torch's float8 cast on the same quotients, the quantiser's
error bound, integer rows it must hold exactly, page placement, and planted mistakes that the
pins must catch."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import (cache_append, decode_rows, mx_decode, mx_quantize, mx_quantize_query,
                    mx_scale_exponent, token_scores)
from oracle.codecs import e4m3_decode

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden_groups():
    g = json.load(open(os.path.join(GOLD, "mxfp8_groups_handworked.json")))
    out = []
    for gr in g["groups"]:
        x = np.zeros(32, np.float32)
        for k, v in gr["x"].items():
            x[int(k)] = np.float32(v)
        codes = np.zeros(32, np.uint8)
        for k, v in gr["codes"].items():
            codes[int(k)] = v
        out.append((x, gr["byte"], codes, gr["work"]))
    return out


def _brute_exponent(a: float) -> int:
    """The largest integer E with 2^E <= a, by stepping through the integers; minus 8, clamped
    to [-127, 127]; -127 for a = 0."""
    if a == 0.0:
        return -127
    E = -160
    while 2.0 ** (E + 1) <= a:
        E += 1
    return int(min(127, max(-127, E - 8)))


def _magnitudes(rng):
    """fp32 magnitudes over the whole range: random, exact powers of two and their fp32
    neighbours, subnormals, the largest finite value."""
    a = list(np.exp2(rng.uniform(-149, 128, 400)).astype(np.float32))
    for e in range(-149, 128, 3):
        p = np.float32(2.0 ** e)
        a += [p, np.nextafter(p, np.float32(0)), np.nextafter(p, np.float32(np.inf))]
    a += [np.float32(0), np.finfo(np.float32).max, np.finfo(np.float32).tiny]
    return [float(x) for x in a if np.isfinite(x)]


def _rows(rng):
    """Rows of the indexer's shapes and distributions, plus awkward ones (groups of 32)."""
    out = [rng.standard_normal(128).astype(np.float32) for _ in range(40)]
    out += [(rng.standard_normal(128) * 2.0 ** rng.integers(-40, 40)).astype(np.float32)
            for _ in range(20)]
    out += [(rng.standard_t(2, 128) * 3).astype(np.float32) for _ in range(20)]
    spiky = (rng.standard_normal(128) * 1e-4).astype(np.float32)
    spiky[3] = 100.0                     # one large value: the rest of its group underflows
    out.append(spiky)
    out.append((rng.standard_normal(128) * 1e-41).astype(np.float32))   # fp32 subnormals
    z = np.zeros(128, np.float32)
    z[40:72] = rng.standard_normal(32).astype(np.float32)                # zero groups around
    out.append(z)
    return out


def _torch_quantize(x):
    """Codes through the brute-force exponent and torch's e4m3 cast of the clamped quotient."""
    x = np.asarray(x, np.float64)
    g = x.reshape(-1, 32)
    X = np.array([_brute_exponent(float(np.abs(r).max())) for r in g])
    v = np.clip(g * np.exp2(-X.astype(np.float64))[:, None], -448.0, 448.0)
    c = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return c.reshape(x.shape), (X + 127).astype(np.uint8)


# ------------------------------------------------------------------------------------ pins
def test_handworked_groups():
    for x, byte, codes, work in _golden_groups():
        c, b = mx_quantize(x.astype(np.float64))
        assert int(b[0]) == byte, work
        assert np.array_equal(c, codes), work


def test_exponent_brute_force():
    rng = np.random.default_rng(20261210)
    a = _magnitudes(rng)
    got = mx_scale_exponent(np.array(a))
    want = np.array([_brute_exponent(v) for v in a])
    assert np.array_equal(got, want)


def test_matches_torch_cast():
    rng = np.random.default_rng(20261211)
    for x in _rows(rng):
        c, b = mx_quantize(x.astype(np.float64))
        tc, tb = _torch_quantize(x)
        assert np.array_equal(b, tb)
        assert np.array_equal(c, tc)


def test_error_bound():
    """Per element with v = x / 2^X: |decoded - x| <= 2^X (2^-4 |v| + 2^-10) when |v| <= 448
    (half an e4m3 quantum), and decoded = sign(x) 448 2^X with |x| < 512 2^X when it saturates.
    The group's largest magnitude lands in [256, 512) 2^X unless X was clamped."""
    rng = np.random.default_rng(20261212)
    for x in _rows(rng):
        c, b = mx_quantize(x.astype(np.float64))
        dec = mx_decode(c, b)
        X = b.astype(np.int64) - 127
        xg = x.astype(np.float64).reshape(-1, 32)
        dg = dec.reshape(-1, 32)
        for g in range(xg.shape[0]):
            s = 2.0 ** X[g]
            v = xg[g] / s
            ok = np.abs(v) <= 448.0
            assert np.all(np.abs(dg[g][ok] - xg[g][ok]) <= s * (2.0 ** -4 * np.abs(v[ok]) + 2.0 ** -10))
            assert np.all(np.abs(dg[g][~ok]) == 448.0 * s)
            assert np.all(np.sign(dg[g][~ok]) == np.sign(xg[g][~ok]))
            amax = np.abs(xg[g]).max()
            if amax > 0 and -127 < X[g] < 127:
                assert 256.0 * s <= amax < 512.0 * s
        assert np.all((c & 0x7F) <= 0x7E)     # never the NaN code


def test_integer_rows_exact_and_scores():
    """Integers in [-3, 3] (the exact-mode inputs) survive MXFP8 unchanged (amax 1, 2 or 3 puts
    every value on an e4m3 grid point), so MXFP8 scores equal the integer scores exactly."""
    rng = np.random.default_rng(20261213)
    q = rng.integers(-3, 4, (64, 128)).astype(np.float64)
    k = rng.integers(-3, 4, (300, 128)).astype(np.float64)
    k[7] = 0.0                               # an all-zero row
    w = rng.choice([0.25, 0.5, 1.0], 64)
    qh = mx_quantize_query(q)
    kc, kb = mx_quantize(k)
    kh = mx_decode(kc, kb)
    assert np.array_equal(qh, q) and np.array_equal(kh, k)
    S = token_scores(qh, w, kh)
    ref = np.array([sum(w[h] * max(0.0, float(np.dot(q[h], k[s]))) for h in range(64))
                    for s in range(300)])
    assert np.array_equal(S, ref)


def test_page_placement_mxfp8():
    """Rows land in page_table[p // 64] * 64 + p % 64 with their D/32 scale bytes and read back
    through decode_rows; other slots keep their bytes; out-of-pool pages are skipped."""
    rng = np.random.default_rng(20261214)
    P, D = 5, 128
    pool = rng.integers(0, 0x7E, (P, 64, D), dtype=np.uint8)
    scl = rng.integers(100, 140, (P, 64, D // 32), dtype=np.uint8)
    pt = np.array([3, 0, 7], np.int32)                 # page 2 lies outside
    pos = np.array([0, 5, 64, 129], np.int64)          # 129: page 2 -> skipped
    rows = rng.standard_normal((4, D)).astype(np.float32)
    newp, news = cache_append(pool, scl, pt, pos, rows, "mxfp8")
    keep = [0, 1, 2]
    got = decode_rows(newp, news, pt, pos[keep], "mxfp8")
    for j, i in enumerate(keep):
        c, b = mx_quantize(rows[i].astype(np.float64))
        assert np.array_equal(got[j], mx_decode(c, b))
    written = {3 * 64 + 0, 3 * 64 + 5, 0 * 64 + 0}
    for slot in range(P * 64):
        if slot not in written:
            assert np.array_equal(newp.reshape(-1, D)[slot], pool.reshape(-1, D)[slot])
            assert np.array_equal(news.reshape(-1, D // 32)[slot], scl.reshape(-1, D // 32)[slot])


# --------------------------------------------------------------------- planted mistakes
def _pin_checks(M):
    def handworked():
        for x, byte, codes, _ in _golden_groups():
            c, b = M.mx_quantize(x.astype(np.float64))
            assert int(b[0]) == byte and np.array_equal(c, codes)

    def torch_cast():
        rng = np.random.default_rng(20261211)
        for x in _rows(rng):
            c, b = M.mx_quantize(x.astype(np.float64))
            tc, tb = _torch_quantize(x)
            assert np.array_equal(b, tb) and np.array_equal(c, tc)

    def brute():
        rng = np.random.default_rng(20261210)
        a = _magnitudes(rng)
        assert np.array_equal(M.mx_scale_exponent(np.array(a)),
                              np.array([_brute_exponent(v) for v in a]))
    return (handworked, torch_cast, brute)


def test_pins_catch_planted_mistakes(monkeypatch):
    """Each plausible slip in the MXFP8 quantiser fails one of the pins above."""
    import oracle.method as M
    from oracle.codecs import e4m3_encode
    real_q, real_x = M.mx_quantize, M.mx_scale_exponent

    def quantize_with(expo=None, rnd=None, group=32, saturate=True):
        def q(x, group_=32):
            x = np.asarray(x, np.float64)
            xg = x.reshape(x.shape[:-1] + (x.shape[-1] // group, group))
            X = (expo or real_x)(np.abs(xg).max(axis=-1))
            v = np.ldexp(xg, -X[..., None])
            if saturate:
                v = np.clip(v, -448.0, 448.0)
            if rnd is not None:
                v = rnd(v)
            c = e4m3_encode(v).reshape(x.shape)
            b = (X + 127).astype(np.uint8)
            if group != 32:   # report one byte per 32 (the first of each pair of groups)
                b = b.reshape(b.shape[:-1] + (-1, 32 // group))[..., 0]
            return c, b
        return q

    def ceil_exponent(amax):
        amax = np.asarray(amax, np.float64)
        X = np.where(amax > 0, np.ceil(np.log2(np.where(amax > 0, amax, 1.0))) - 8, -127)
        return np.clip(X, -127, 127).astype(np.int64)

    def emax7(amax):
        return np.clip(real_x(amax) + 1, -127, 127)

    def unclamped(amax):
        amax = np.asarray(amax, np.float64)
        _, E = np.frexp(amax)
        return np.where(amax > 0, E - 9, -127).astype(np.int64)

    def truncate(v):
        a = np.abs(v)
        e = np.where(a >= 2.0 ** -6, np.floor(np.log2(np.maximum(a, 2.0 ** -6))), -6)
        qn = np.ldexp(1.0, (e - 3).astype(int))
        return np.copysign(np.floor(a / qn) * qn, v)

    bads = {
        "ceil exponent": quantize_with(expo=ceil_exponent),
        "emax 7": quantize_with(expo=emax7),
        "no clamp of X": quantize_with(expo=unclamped),
        "truncation": quantize_with(rnd=truncate),
        "group 16": quantize_with(group=16),
        "no saturation": quantize_with(saturate=False),
    }
    for name, bad in bads.items():
        monkeypatch.setattr(M, "mx_quantize", bad)
        if name in ("ceil exponent", "emax 7", "no clamp of X"):
            monkeypatch.setattr(M, "mx_scale_exponent",
                                {"ceil exponent": ceil_exponent, "emax 7": emax7,
                                 "no clamp of X": unclamped}[name])
        failed = False
        for chk in _pin_checks(M):
            try:
                chk()
            except (AssertionError, ValueError):
                failed = True
        assert failed, name
        monkeypatch.setattr(M, "mx_quantize", real_q)
        monkeypatch.setattr(M, "mx_scale_exponent", real_x)
