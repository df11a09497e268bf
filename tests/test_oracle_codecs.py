"""Pins of the oracle's storage codecs: OCP E4M3FN fixed points, torch's casts as a second
opinion, exhaustive bf16 patterns."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import E4M3_TABLE, bf16_decode, bf16_round, e4m3_decode, e4m3_encode, e4m3_round

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_e4m3_spec_points():
    spec = json.load(open(os.path.join(GOLD, "e4m3_spec_points.json")))
    for p in spec["points"]:
        v = e4m3_decode(np.array([int(p["code"], 16)]))[0]
        assert v == p["value"] and np.signbit(v) == np.signbit(p["value"]), p
    for c in spec["nan_codes"]:
        assert np.isnan(E4M3_TABLE[int(c, 16)])
    assert np.sum(np.isnan(E4M3_TABLE)) == 2


def test_e4m3_table_structure():
    pos = E4M3_TABLE[:0x7F]
    assert np.all(np.diff(pos) > 0)                    # strictly increasing magnitudes
    assert np.array_equal(E4M3_TABLE[0x80:0xFF], -pos)  # sign bit mirrors
    # every binade holds 8 equally spaced values with quantum 2^(e-3)
    for e in range(-6, 9):
        vals = pos[(pos >= 2.0 ** e) & (pos < 2.0 ** (e + 1))]
        assert len(vals) == (8 if e < 8 else 7)
        assert np.allclose(np.diff(vals), 2.0 ** (e - 3))


def test_e4m3_decode_matches_torch_cast():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    t = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(e4m3_decode(codes), t)


def _midpoints():
    pos = E4M3_TABLE[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    return pos, mids


def test_e4m3_round_ties_to_even():
    pos, mids = _midpoints()
    r = e4m3_round(mids)
    codes = e4m3_encode(mids)
    for i, m in enumerate(mids):
        lo, hi = i, i + 1                       # neighbouring codes
        want = lo if lo % 2 == 0 else hi        # even mantissa = even code within a binade
        assert codes[i] == want and r[i] == pos[want], (m, codes[i], want)
    # just below / above a midpoint go to the nearer neighbour
    below = np.nextafter(mids, 0)
    above = np.nextafter(mids, np.inf)
    assert np.array_equal(e4m3_encode(below), np.arange(0, 0x7E))
    assert np.array_equal(e4m3_encode(above), np.arange(1, 0x7F))
    assert e4m3_round(np.array([464.0]))[0] == 448.0     # tie at the top goes to even (448)
    with pytest.raises(ValueError):
        e4m3_round(np.array([464.5]))


def test_e4m3_round_matches_torch_cast():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.uniform(-448, 448, 200000), rng.normal(0, 1, 100000),
                        rng.normal(0, 0.01, 50000), _midpoints()[1], -_midpoints()[1]])
    x = x.astype(np.float32)
    t = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(x.astype(np.float64)), t)


def test_bf16_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = bf16_decode(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.normal(0, 1, 300000), rng.normal(0, 1e-3, 1000)]).astype(np.float32)
    # exact midpoints between neighbouring bf16 values, both parities
    b = rng.integers(0x0080, 0x7F00, 20000).astype(np.uint32)
    mids = ((b << 16) | 0x8000).view(np.float32)
    x = np.concatenate([x, mids, -mids])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_round(x), ref)
