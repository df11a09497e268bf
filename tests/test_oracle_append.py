"""Pins of the oracle's cache append (per-token e4m3 quantiser and page placement): hand-worked
rows, torch's float8 cast on the same fp32 quotients, the quantiser's error bound, the page
placement through the table, and planted mistakes that the pins must catch."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import cache_append, decode_rows, quantize_row_e4m3
from oracle.codecs import e4m3_decode

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _torch_quantize(x):
    """The same quantiser through numpy's fp32 division and torch's e4m3 cast (an independent
    implementation of the two roundings)."""
    x = np.asarray(x, dtype=np.float32)
    s = np.float32(np.abs(x).max()) / np.float32(448.0)
    s = np.float32(1.0) if s == 0 else s
    y = np.clip(x / s, np.float32(-448.0), np.float32(448.0)).astype(np.float32)
    return torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy(), s


def _rows(rng):
    """Rows of the shapes and distributions of the cached rows, plus awkward ones."""
    out = [rng.standard_normal(576).astype(np.float32) for _ in range(40)]
    out += [rng.standard_normal(128).astype(np.float32) * 8 for _ in range(40)]
    out += [(rng.standard_t(2, 576) * 3).astype(np.float32) for _ in range(20)]  # heavy tails
    spiky = rng.standard_normal(576).astype(np.float32) * 1e-3
    spiky[17] = 50.0                        # one large value: most codes land on subnormals
    out.append(spiky)
    tiny = (rng.standard_normal(128) * 1e-30).astype(np.float32)
    out.append(tiny)
    out.append(np.zeros(128, np.float32))
    lone = np.zeros(128, np.float32)
    lone[5] = -3.0
    out.append(lone)
    return out


def test_handworked_rows():
    g = json.load(open(os.path.join(GOLD, "e4m3_append_handworked.json")))
    for r in g["rows"]:
        codes, scale = quantize_row_e4m3(np.array(r["x"], np.float32))
        if "scale_bits" in r:
            assert hex(int(np.float32(scale).view(np.uint32))) == r["scale_bits"], r["work"]
        else:
            assert float(scale) == r["scale"], r["work"]
        assert codes.tolist() == r["codes"], r["work"]


def test_matches_torch_cast():
    rng = np.random.default_rng(20261205)
    for x in _rows(rng):
        c, s = quantize_row_e4m3(x)
        tc, ts = _torch_quantize(x)
        assert np.float32(s) == ts
        assert np.array_equal(c, tc)


def test_error_bound():
    """|decoded - x| <= scale*(2^-4 |y| + 2^-10) + 2^-24 |x| with y = fp32(x/scale): half an
    e4m3 quantum (normal binades: 2^(e-4) <= 2^-4 |y|; subnormals: 2^-10) plus the fp32
    rounding of the quotient.  The largest magnitude decodes to within that bound of amax."""
    rng = np.random.default_rng(20261206)
    for x in _rows(rng):
        c, s = quantize_row_e4m3(x)
        s = float(s)
        x64 = x.astype(np.float64)
        y = (x64 / s).astype(np.float32).astype(np.float64)
        dec = e4m3_decode(c) * s
        bound = s * (2.0 ** -4 * np.abs(y) + 2.0 ** -10) + 2.0 ** -24 * np.abs(x64)
        assert np.all(np.abs(dec - x64) <= bound + 1e-300)
        assert np.max(np.abs(c & 0x7F)) <= 0x7E          # never the NaN code


def test_page_placement():
    """Rows land in page_table[p // 64] * 64 + p % 64 and read back through decode_rows; other
    slots keep their bytes; a position whose page entry lies outside the pool is skipped."""
    rng = np.random.default_rng(20261207)
    P, D = 6, 128
    pool = rng.integers(0, 256, (P, 64, D), dtype=np.uint8)
    pool[pool == 0x7F] = 0
    pool[pool == 0xFF] = 0
    scl = rng.random((P, 64)).astype(np.float32) + 0.5
    pt = np.array([4, 1, 9, 0], np.int32)            # page 2 of the request lies outside
    pos = np.array([0, 63, 64, 130, 200], np.int64)  # 130: page 2 -> skipped
    rows = rng.standard_normal((5, D)).astype(np.float32)
    newp, news = cache_append(pool, scl, pt, pos, rows, "e4m3")
    keep = [0, 1, 2, 4]
    got = decode_rows(newp, news, pt, pos[keep], "e4m3")
    for j, i in enumerate(keep):
        c, s = quantize_row_e4m3(rows[i])
        assert np.array_equal(got[j], e4m3_decode(c) * float(s))
    written = {4 * 64 + 0, 4 * 64 + 63, 1 * 64 + 0, 0 * 64 + 8}
    for slot in range(P * 64):
        if slot not in written:
            assert np.array_equal(newp.reshape(-1, D)[slot], pool.reshape(-1, D)[slot]), slot
            assert news.reshape(-1)[slot] == scl.reshape(-1)[slot]
    # the arguments are left as they were
    assert not np.shares_memory(newp, pool)
    # bf16 pools: round to nearest even, scales untouched
    bpool = rng.integers(0, 1 << 15, (P, 64, D), dtype=np.uint16)
    b2, s2 = cache_append(bpool, None, pt, pos, rows, "bf16")
    assert s2 is None
    back = decode_rows(b2, None, pt, pos[keep], "bf16")
    assert np.all(np.abs(back - rows[keep]) <= 2.0 ** -8 * np.abs(rows[keep]))  # half a bf16 ulp
    untouched = [sl for sl in range(P * 64) if sl not in written]
    assert np.array_equal(b2.reshape(-1, D)[untouched], bpool.reshape(-1, D)[untouched])


def test_pins_catch_planted_mistakes(monkeypatch):
    """Each plausible slip in the quantiser fails one of the pins above."""
    import oracle.method as M
    real = M.quantize_row_e4m3

    def truncating(x):  # codes by truncation instead of round-to-nearest-even
        x = np.asarray(x, np.float32).astype(np.float64)
        s = float(np.float32(np.abs(x).max() / 448.0)) or 1.0
        y = (x / s).astype(np.float32).astype(np.float64)
        a = np.abs(y)
        e = np.where(a >= 2.0 ** -6, np.floor(np.log2(np.maximum(a, 2.0 ** -6))), -6)
        q = np.ldexp(1.0, (e - 3).astype(int))
        r = np.copysign(np.floor(a / q) * q, y)
        from oracle.codecs import e4m3_encode
        return e4m3_encode(r), np.float32(s)

    def scale_by_max_code(x):  # scale = amax/480 (a wrong top value)
        x = np.asarray(x, np.float32).astype(np.float64)
        s = float(np.float32(np.abs(x).max() / 480.0)) or 1.0
        from oracle.codecs import e4m3_encode
        return e4m3_encode(np.clip((x / s).astype(np.float32), -448, 448)), np.float32(s)

    def no_fp32_quotient(x):  # the quotient kept in fp64 (one rounding fewer than the data's)
        x = np.asarray(x, np.float32).astype(np.float64)
        s = float(np.float32(np.abs(x).max() / 448.0)) or 1.0
        from oracle.codecs import e4m3_encode
        return e4m3_encode(np.clip(x / s, -448, 448)), np.float32(s)

    for bad in (truncating, scale_by_max_code, no_fp32_quotient):
        monkeypatch.setattr(M, "quantize_row_e4m3", bad)
        failed = False
        for t in (_handworked_check(M), _torch_check(M)):
            try:
                t()
            except AssertionError:
                failed = True
        assert failed, bad.__name__
    monkeypatch.setattr(M, "quantize_row_e4m3", real)


def _handworked_check(M):
    def run():
        g = json.load(open(os.path.join(GOLD, "e4m3_append_handworked.json")))
        for r in g["rows"]:
            codes, scale = M.quantize_row_e4m3(np.array(r["x"], np.float32))
            assert codes.tolist() == r["codes"]
            if "scale" in r:
                assert float(scale) == r["scale"]
    return run


def _torch_check(M):
    def run():
        rng = np.random.default_rng(20261205)
        for x in _rows(rng):
            c, s = M.quantize_row_e4m3(x)
            tc, ts = _torch_quantize(x)
            assert np.float32(s) == ts and np.array_equal(c, tc)
    return run
