"""The method, written out as its plain definition in fp64 (oracle side; test infrastructure).

Source: "Day 0 Support for New LLM Architectures" (Step 1, sparse attention modules): a
light indexer scores every earlier position for each query, the Top-K positions are kept,
and exact attention then reads only those rows of the low-rank (latent + RoPE) KV cache;
Key Optimization 1 orders the chain as relevance scoring, head-weight application, Top-K.
Key Optimization 2 quantises the indexer's query dynamically; here that is one power-of-two
scale per (token, head) so that the scaled query fits e4m3 (the reading used throughout).
The score formula, the shapes and the tie rule (lower position wins) are the build's
contract; the pages give them only in prose.
"""
from __future__ import annotations

import numpy as np

from .codecs import bf16_decode, bf16_round, e4m3_decode, e4m3_encode, e4m3_round

PAGE = 64


# ----------------------------------------------------------------------------- A0
def a0_scale(amax) -> np.ndarray:
    """Smallest power of two s with amax <= 448*s (s = 1 when amax = 0).

    Written with the binary exponent: amax = m*2^E with m in [0.5, 1); since 448 = 0.875*2^9,
    s = 2^(E-9) when m <= 0.875 and 2^(E-8) otherwise."""
    amax = np.asarray(amax, dtype=np.float64)
    m, E = np.frexp(amax)
    s = np.where(m <= 0.875, np.ldexp(1.0, E - 9), np.ldexp(1.0, E - 8))
    return np.where(amax == 0.0, 1.0, s)


def a0_quantize(q) -> tuple[np.ndarray, np.ndarray]:
    """Dynamic e4m3 quantisation of an indexer query [..., H, D]: per (token, head) power-of-
    two scale s; returns (q_hat, s) with q_hat = RNE_e4m3(q/s)*s, the value the scorer uses."""
    q = np.asarray(q, dtype=np.float64)
    s = a0_scale(np.abs(q).max(axis=-1))
    return e4m3_round(q / s[..., None]) * s[..., None], s


# ----------------------------------------------------------------------------- cache rows
def decode_rows(pool, scale, pt_row, positions, fmt: str) -> np.ndarray:
    """Logical positions of one request -> fp64 rows, through its page table.

    Physical slot of position s: page_table[s // 64] * 64 + s % 64.  ``fmt`` is 'f32',
    'bf16' (uint16 bits), 'e4m3' (uint8 codes times the slot's fp32 scale, exact in fp64) or
    'mxfp8' (uint8 codes, scale bytes [n_pages][64][D/32]: mx_decode)."""
    positions = np.asarray(positions, dtype=np.int64)
    D = pool.shape[-1]
    flat = pool.reshape(-1, D)
    slot = np.asarray(pt_row, dtype=np.int64)[positions // PAGE] * PAGE + positions % PAGE
    raw = flat[slot]
    if fmt == "f32":
        return raw.astype(np.float64)
    if fmt == "bf16":
        return bf16_decode(raw)
    if fmt == "e4m3":
        return e4m3_decode(raw) * scale.reshape(-1)[slot].astype(np.float64)[:, None]
    if fmt == "mxfp8":
        return mx_decode(raw, scale.reshape(-1, D // MX_GROUP)[slot])
    raise ValueError(fmt)


# ----------------------------------------------------------------------------- N1
def quantize_row_e4m3(x) -> tuple[np.ndarray, np.float32]:
    """One cached row's per-token e4m3 quantisation, for the FP8 cache of "Day 0 Support for
    New LLM Architectures", Key Optimization 2 (FP8 cache whose scale factors are computed
    online; here one fp32 scale per token over the whole row).

    scale = amax/448 rounded to fp32, so that the largest magnitude maps to the largest finite
    e4m3 value (448); a scale of 0 (an all-zero row, or amax/448 below the fp32 range) is
    replaced by 1.  Each element's code is the e4m3 round-to-nearest-even of the fp32 quotient
    x/scale, clamped to +-448 first.  Both quotients are formed in fp64 from fp32 operands and
    rounded once to fp32, which equals the correctly rounded fp32 division (53 >= 2*24 + 2
    bits).  x: fp32 values (one row).  Returns (uint8 codes, fp32 scale)."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    amax = float(np.abs(x).max()) if x.size else 0.0
    scale = float(np.float32(amax / 448.0))
    if scale == 0.0:
        scale = 1.0
    y = (x / scale).astype(np.float32).astype(np.float64)
    return e4m3_encode(np.clip(y, -448.0, 448.0)), np.float32(scale)


# ----------------------------------------------------------------------------- N2 (MXFP8)
MX_GROUP = 32          # elements that share one scale ("Day 0 Support for New LLM
                       # Architectures", Key Optimization 2: the indexer's Q and K, group 32)
MX_E4M3_EMAX = 8       # exponent of e4m3's largest binade: 448 = 1.75 * 2^8


def mx_scale_exponent(amax) -> np.ndarray:
    """Shared exponent X of one MXFP8 group, the microscaling format named by Key Optimization 2
    of "Day 0 Support for New LLM Architectures" (8-bit elements, one power-of-two scale per
    32 of them).  The pages give only the name and the group size; the reading here is the
    usual microscaling rule: X = floor(log2 amax) - 8 (8 = the element format's largest
    exponent), so the largest magnitude of the group lands in e4m3's top binade [256, 512)
    after division by 2^X.  X is clamped to the scale byte's range [-127, 127]; an all-zero
    group (amax = 0) takes X = -127."""
    amax = np.asarray(amax, dtype=np.float64)
    _, E = np.frexp(amax)                   # amax = m * 2^E, m in [0.5, 1): floor(log2) = E - 1
    X = np.where(amax > 0, E - 1 - MX_E4M3_EMAX, -127)
    return np.clip(X, -127, 127).astype(np.int64)


def mx_quantize(x, group: int = MX_GROUP) -> tuple[np.ndarray, np.ndarray]:
    """Quantise rows [..., D] to MXFP8: for each run of ``group`` consecutive elements, the
    shared exponent X of mx_scale_exponent, the scale byte X + 127 (an E8M0 power of two), and
    each element's e4m3 code by round-to-nearest-even of x / 2^X clamped to +-448 (the
    division by a power of two is exact; values in (448, 512) saturate).  The sign of zero is
    kept.  Returns (codes uint8 [..., D], scale bytes uint8 [..., D/group])."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    if D % group:
        raise ValueError("row width must be a multiple of the group size")
    xg = x.reshape(x.shape[:-1] + (D // group, group))
    X = mx_scale_exponent(np.abs(xg).max(axis=-1))
    v = np.ldexp(xg, -X[..., None])
    codes = e4m3_encode(np.clip(v, -448.0, 448.0))
    return codes.reshape(x.shape), (X + 127).astype(np.uint8)


def mx_decode(codes, sbytes, group: int = MX_GROUP) -> np.ndarray:
    """MXFP8 rows -> fp64: each code's e4m3 value times 2^(byte - 127) of its group (exact)."""
    codes = np.asarray(codes, dtype=np.uint8)
    sb = np.asarray(sbytes, dtype=np.uint8).astype(np.int64)
    D = codes.shape[-1]
    v = e4m3_decode(codes).reshape(codes.shape[:-1] + (D // group, group))
    return np.ldexp(v, (sb - 127)[..., None]).reshape(codes.shape)


def mx_quantize_query(q) -> np.ndarray:
    """The indexer query as the MXFP8 scorer uses it: q_I [..., H, D] quantised per (token,
    head, 32 consecutive dims) and decoded again (fp64)."""
    codes, sb = mx_quantize(q)
    return mx_decode(codes, sb)


def cache_append(pool, scale, pt_row, positions, rows, fmt: str):
    """Append new rows of one request to a paged cache ("Day-0 Support for Large Model
    Inference", Core Operator Optimization 1: the selection index is kept on the device and
    updated incrementally; "Achieving Day-0 Readiness ... Million-Token Context", section 2.2:
    fixed-size blocks located through a block index table).

    Row i goes to logical position positions[i], i.e. physical slot
    page_table[p // 64] * 64 + p % 64, and is stored in the cache's format: 'e4m3' codes with
    the slot's fp32 scale (quantize_row_e4m3), 'mxfp8' codes with the slot's D/32 scale bytes
    (mx_quantize of the fp32 row; scale is then uint8 [n_pages][64][D/32]), or 'bf16' (round
    to nearest even, scale untouched).  A position whose page-table entry lies outside the
    pool is not written.  Returns updated copies (pool, scale); the arguments are not
    modified."""
    pool = np.array(pool, copy=True)
    scale = None if scale is None else np.array(scale, copy=True)
    D = pool.shape[-1]
    flat = pool.reshape(-1, D)
    sflat = None if scale is None else (
        scale.reshape(-1, D // MX_GROUP) if fmt == "mxfp8" else scale.reshape(-1))
    n_slots = flat.shape[0]
    rows = np.asarray(rows, dtype=np.float32)
    for i, p in enumerate(np.asarray(positions, dtype=np.int64)):
        page = int(np.asarray(pt_row)[p // PAGE])
        slot = page * PAGE + int(p % PAGE)
        if page < 0 or slot >= n_slots:
            continue
        if fmt == "e4m3":
            flat[slot], sflat[slot] = quantize_row_e4m3(rows[i])
        elif fmt == "mxfp8":
            flat[slot], sflat[slot] = mx_quantize(rows[i])
        elif fmt == "bf16":
            flat[slot] = bf16_round(rows[i])
        else:
            raise ValueError(fmt)
    return pool, scale


# ----------------------------------------------------------------------------- A1
def token_scores(q_hat, w, k_hat) -> np.ndarray:
    """S[s] = sum_h w[h] * max(0, q_hat[h] . k_hat[s]) for every row s of k_hat (fp64)."""
    dots = np.asarray(k_hat, np.float64) @ np.asarray(q_hat, np.float64).T     # [n, H]
    return np.maximum(dots, 0.0) @ np.asarray(w, np.float64)


# ----------------------------------------------------------------------------- A2
def topk_token(S, K: int):
    """Top-K of one query: the k = min(K, n) largest S under (score desc, position asc).

    Returns (idx[K] int32 ascending, -1 padded; the k-th largest score, or None if k = 0).
    A full stable sort; -0.0 and +0.0 compare equal, so they tie and the position decides."""
    S = np.asarray(S, dtype=np.float64)
    n = S.shape[0]
    k = min(int(K), n)
    order = np.lexsort((np.arange(n), -S))   # primary: -S ascending; secondary: position
    sel = np.sort(order[:k])
    out = np.full(int(K), -1, dtype=np.int32)
    out[:k] = sel
    return out, (float(S[order[k - 1]]) if k > 0 else None)


# ----------------------------------------------------------------------------- A3/A4
def sparse_mla_token(q, rows, scale: float, D_v: int):
    """Exact attention of one token over its selected latent rows (fp64).

    z[h,s] = scale * q[h] . rows[s] (all D_qk dims); p = softmax_s(z); o[h] = sum_s p[h,s] *
    rows[s, :D_v]; lse[h] = max_s z + ln sum_s exp(z - max).  No rows: o = 0, lse = -inf."""
    q = np.asarray(q, np.float64)
    rows = np.asarray(rows, np.float64)
    H = q.shape[0]
    if rows.shape[0] == 0:
        return np.zeros((H, D_v)), np.full(H, -np.inf)
    z = float(scale) * (q @ rows.T)
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    l = e.sum(axis=1, keepdims=True)
    o = (e @ rows[:, :D_v]) / l
    return o, (m + np.log(l))[:, 0]


# ----------------------------------------------------------------------------- driver
class Oracle:
    """The oracle over one batch of raw inputs.

    ``inp`` carries the boundary's raw arrays: seq_lens, cu_q, positions, req, page_table,
    q_idx, w, k_pool, k_scale, q, kv_pool, kv_scale, ``wl.shape`` (H_I, D_I, K, H, D_qk,
    D_v, fp32, kv_fp8, softmax_scale) and ``k_fmt``, the indexer key cache's format ('f32',
    'e4m3' with one fp32 scale per token, or 'mxfp8' with one scale byte per 32 dims).
    ``qmode`` is 'fp8' (A0 applied to q_I, as the e4m3 scorer does), 'mxfp8' (q_I quantised
    per 32 dims, as the MXFP8 scorer does) or 'none' (q_I used as stored); the default
    follows the key format."""

    def __init__(self, inp, qmode: str | None = None):
        self.inp = inp
        self.sh = inp.wl.shape
        self.k_fmt = getattr(inp, "k_fmt", None) or ("f32" if self.sh.fp32 else "e4m3")
        self.qmode = qmode or {"f32": "none", "e4m3": "fp8", "mxfp8": "mxfp8"}[self.k_fmt]
        self._kcache = (None, None)

    # -- indexer keys of one request, decoded once
    def k_rows(self, b: int, n: int) -> np.ndarray:
        cb, rows = self._kcache
        if cb != b or rows.shape[0] < n:
            inp = self.inp
            L = int(inp.seq_lens[b])
            rows = decode_rows(inp.k_pool, inp.k_scale, inp.page_table[b], np.arange(L),
                               self.k_fmt)
            self._kcache = (b, rows)
        return rows[:n]

    def q_hat(self, t: int) -> np.ndarray:
        qi = self.inp.q_idx[t]
        qi = qi.astype(np.float64) if self.sh.fp32 else bf16_decode(qi)
        if self.qmode == "fp8":
            qi, _ = a0_quantize(qi)
        elif self.qmode == "mxfp8":
            qi = mx_quantize_query(qi)
        return qi

    def scores(self, t: int) -> np.ndarray:
        """S[t, 0..p_t] (fp64)."""
        b, p = int(self.inp.req[t]), int(self.inp.positions[t])
        return token_scores(self.q_hat(t), self.inp.w[t].astype(np.float64),
                            self.k_rows(b, p + 1))

    def topk(self, t: int, K: int | None = None):
        S = self.scores(t)
        idx, kth = topk_token(S, self.sh.K if K is None else K)
        return idx, S, kth

    def block_topk(self, t: int, K_blocks: int):
        """Block-granular selection of token t: (block ids, block scores, kb-th block score,
        expanded positions)."""
        S = self.scores(t)
        bs = block_scores(S)
        blk, kth = topk_blocks(bs, K_blocks)
        return blk, bs, kth, expand_blocks(blk, S.shape[0])

    def attention(self, t: int, idx):
        """Attention of token t over the positions in ``idx`` (entries <0 or >=L_b skipped)."""
        inp, sh = self.inp, self.sh
        b = int(inp.req[t])
        L = int(inp.seq_lens[b])
        idx = np.asarray(idx, dtype=np.int64)
        idx = idx[(idx >= 0) & (idx < L)]
        fmt = "f32" if sh.fp32 else ("e4m3" if sh.kv_fp8 else "bf16")
        rows = decode_rows(inp.kv_pool, inp.kv_scale, inp.page_table[b], idx, fmt)
        q = inp.q[t].astype(np.float64) if sh.fp32 else bf16_decode(inp.q[t])
        return sparse_mla_token(q, rows, sh.softmax_scale, sh.D_v)


# ----------------------------------------------------------------------------- N4
def block_scores(S, page: int = PAGE) -> np.ndarray:
    """Block (page) scores of one query for block-granular selection ("Day-0 Adaptation for
    Trillion-Parameter Models": the index selection returns blocks of the cache layout, fetched
    whole; "Achieving Day-0 Readiness ... Million-Token Context", section 2.2: fixed-size
    blocks located through a block index table).  The pages do not say how a block is scored;
    the reading here: a block's score is the largest token score among its causal positions,
    so a block is kept whenever it holds a token the token-level selection would rank high.

    S: the n = p_t + 1 token scores of positions 0..p_t.  Returns ceil(n / page) block scores,
    block j covering positions [page*j, min(page*(j+1), n))."""
    S = np.asarray(S, dtype=np.float64)
    n = S.shape[0]
    nb = -(-n // page)
    return np.array([S[page * j:min(page * (j + 1), n)].max() for j in range(nb)],
                    dtype=np.float64)


def topk_blocks(bs, K_blocks: int):
    """Top blocks of one query: the kb = min(K_blocks, nb) largest block scores under (score
    desc, block asc), as topk_token orders positions.  Returns (block ids [K_blocks] int32
    ascending, -1 padded; the kb-th largest block score, or None if kb = 0)."""
    return topk_token(bs, K_blocks)


def expand_blocks(blocks, n: int, page: int = PAGE) -> np.ndarray:
    """Positions attended for selected blocks: entry page*i + r is page*blocks[i] + r when that
    position is causal (< n) and the block is not padding, else -1 ([len(blocks) * page])."""
    blocks = np.asarray(blocks, dtype=np.int64)
    pos = blocks[:, None] * page + np.arange(page)[None, :]
    ok = (blocks[:, None] >= 0) & (pos < n)
    return np.where(ok, pos, -1).reshape(-1).astype(np.int32)
