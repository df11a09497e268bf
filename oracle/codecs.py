"""Exact storage-format codecs (oracle side).

E4M3FN is the OCP 8-bit floating point format "E4M3" (the variant without infinities):
1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes
subnormals m/8 * 2^-6; the all-ones pattern S.1111.111 is NaN and there is no infinity, so
the largest finite magnitude is 1.75 * 2^8 = 448.  bf16 is the top half of an IEEE binary32.
"""
from __future__ import annotations

import numpy as np


def _build_e4m3_table() -> np.ndarray:
    tab = np.empty(256, dtype=np.float64)
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 0xF, c & 0x7
        if e == 0xF and m == 0x7:
            v = np.nan
        elif e == 0:
            v = (m / 8.0) * 2.0 ** -6
        else:
            v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
        tab[c] = -v if s else v
    return tab


E4M3_TABLE = _build_e4m3_table()
_POS_VALUES = E4M3_TABLE[:0x7F]          # codes 0x00..0x7E, strictly increasing


def e4m3_decode(codes) -> np.ndarray:
    """uint8 codes -> fp64 values (table lookup)."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_round(x) -> np.ndarray:
    """Round fp64 values to the nearest e4m3 value, ties to even mantissa.

    |x| must not exceed 464 (values above round to no finite code).  The quantum of the
    binade [2^e, 2^(e+1)) is 2^(e-3); below 2^-6 the subnormal quantum 2^-9 applies."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(a > 464.0) or np.any(~np.isfinite(a)):
        raise ValueError("value outside the finite e4m3 range")
    _, E = np.frexp(a)                      # a = f * 2^E, f in [0.5, 1)  ->  e = E - 1
    e = np.where(a >= 2.0 ** -6, E - 1, -6)
    quantum = np.ldexp(1.0, e - 3)
    r = np.rint(a / quantum) * quantum      # a/quantum is exact (power-of-two scaling)
    return np.copysign(r, x)


def e4m3_encode(x) -> np.ndarray:
    """fp64 -> e4m3 codes by round-to-nearest-even (sign kept, also for zero)."""
    r = e4m3_round(x)
    a = np.abs(r)
    idx = np.searchsorted(_POS_VALUES, a)
    assert np.all(_POS_VALUES[idx] == a)
    return (idx | (np.signbit(r).astype(np.int64) << 7)).astype(np.uint8)


def bf16_decode(bits) -> np.ndarray:
    """uint16 bf16 bit patterns -> fp64 by placing them in the top half of a binary32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def bf16_round(x) -> np.ndarray:
    """fp32 values -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
