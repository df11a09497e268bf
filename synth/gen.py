"""Seeded, page-regenerable synthetic inputs for the five workloads, as raw storage bytes.

Recipe (the same bytes go to the GPU path and to the oracle):
  * every random draw comes from ``numpy.random.Philox`` keyed by (seed, tensor, request,
    block), one block per logical 64-token page (cache tensors) or per 64 query tokens
    (query-side tensors), so any page can be regenerated on its own;
  * continuous mode: q_I, k_I, q and latent rows ~ N(0,1) in fp32, indexer weights
    w ~ U(0,1)/w_div; exact mode: q_I, k_I integers in [-3,3] with k scale 1 and w drawn from
    {1/4, 1/2, 1} (attention inputs stay continuous);
  * bf16 storage: fp32 -> bf16 with torch's round-to-nearest-even cast;
  * e4m3 storage with one fp32 scale per cached token: scale = amax/448, codes = torch's
    float8_e4m3fn cast of clamp(x/scale, +-448);
  * MXFP8 indexer keys (``k_fmt='mxfp8'``): per 32 consecutive dims a scale byte 127 + X with
    X = floor(log2 amax) - 8 (clamped to [-127, 127]), codes = torch's float8_e4m3fn cast of
    clamp(x / 2^X, +-448);
  * structure: 'heavy' scales a seeded 1% of positions x8 in both caches before quantisation;
    'planted' adds sqrt(D_I)*u_b to a block of 4096 k_I rows at a seeded offset, u_b the unit
    vector along sum_h w[h] q_I[h] of the request's query token; 'ragged' uses a seeded random
    page table over a pool with 25% slack;
  * every cache slot that holds no token (slack pages, the tail of a request's last page, the
    spare page that unused page-table entries point at) holds poison: code 0x7E (448) with
    scale 1e4 (MXFP8: scale byte 147, i.e. 2^20), bf16 0x7F00, or fp32 1e30, so a read of a
    wrong slot shows in the results.

Nothing here computes a score, a selection or an attention output.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

from .workloads import PAGE, Workload, seed_of

T_QIDX, T_W, T_KIDX, T_Q, T_KV, T_STRUCT, T_PAGES = 1, 2, 3, 4, 5, 6, 7
POISON_E4M3 = 0x7E
POISON_SCALE = 1.0e4
POISON_BF16 = 0x7F00
POISON_F32 = 1.0e30
POISON_MX_BYTE = 147
MX_GROUP = 32


def _rng(seed: int, tensor: int, b: int, block: int) -> np.random.Generator:
    key = (((seed * 16 + tensor) << 24 | b) << 32) | block
    return np.random.Generator(np.random.Philox(key=key))


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even (torch cast)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_e4m3_per_token(rows: np.ndarray):
    """Per-row fp32 scale amax/448 and e4m3fn codes of clamp(x/scale, +-448) (torch cast)."""
    rows = np.ascontiguousarray(rows, dtype=np.float32)
    amax = np.abs(rows).max(axis=1)
    scale = (amax / np.float32(448.0)).astype(np.float32)
    scale[scale == 0] = np.float32(1.0)
    y = np.clip(rows / scale[:, None], -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def to_mxfp8(rows: np.ndarray):
    """Per 32-dim group: scale byte 127 + X, X = floor(log2 amax) - 8 clamped to [-127, 127]
    (-127 for an all-zero group), and e4m3fn codes of clamp(x / 2^X, +-448) (torch cast)."""
    rows = np.ascontiguousarray(rows, dtype=np.float32)
    n, D = rows.shape
    g = rows.astype(np.float64).reshape(n, D // MX_GROUP, MX_GROUP)
    amax = np.abs(g).max(axis=2)
    _, E = np.frexp(amax)
    X = np.clip(np.where(amax > 0, E - 9, -127), -127, 127)
    y = np.clip(np.ldexp(g, -X[..., None]), -448.0, 448.0).reshape(n, D)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, (X + 127).astype(np.uint8)


def ints_to_e4m3(rows: np.ndarray) -> np.ndarray:
    """Exact e4m3 codes of small integers (|x| <= 3 are all representable)."""
    t = torch.from_numpy(np.ascontiguousarray(rows, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@dataclass
class Inputs:
    wl: Workload
    mode: str
    seed: int
    seq_lens: np.ndarray      # int32 [B]
    q_lens: np.ndarray        # int32 [B]
    cu_q: np.ndarray          # int32 [B+1]
    positions: np.ndarray     # int32 [T]  absolute position of each query token
    req: np.ndarray           # int32 [T]  request of each query token
    page_table: np.ndarray    # int32 [B, pt_stride]
    n_pages: int
    q_idx: np.ndarray         # [T,H_I,D_I] f32 (tiny) or uint16 bf16 bits
    w: np.ndarray             # [T,H_I] f32
    k_pool: np.ndarray        # [P,64,D_I] f32 (tiny) or uint8 e4m3 codes
    k_scale: np.ndarray | None  # [P,64] f32, [P,64,D_I/32] uint8 (MXFP8) or None (tiny)
    q: np.ndarray             # [T,H,D_qk] f32 (tiny) or uint16 bf16 bits
    kv_pool: np.ndarray       # [P,64,D_qk] f32 / uint16 bf16 / uint8 e4m3
    kv_scale: np.ndarray | None  # [P,64] f32 or None
    info: dict = field(default_factory=dict)
    k_fmt: str = "e4m3"       # indexer key cache: 'f32' | 'e4m3' | 'mxfp8'

    @property
    def T(self) -> int:
        return int(self.cu_q[-1])

    @property
    def B(self) -> int:
        return int(self.seq_lens.shape[0])


def _page_table(wl: Workload, seed: int, random_pages: bool):
    npg = [-(-L // PAGE) for L in wl.seq_lens]
    need = int(sum(npg))
    stride = max(npg)
    if random_pages:
        P = int(np.ceil(need * 1.25)) + 1
        perm = _rng(seed, T_PAGES, 0, 0).permutation(P).astype(np.int32)
    else:
        P = need + 1
        perm = np.arange(P, dtype=np.int32)
    spare = int(perm[need])  # a poisoned page that every unused table entry points at
    pt = np.full((wl.B, stride), spare, dtype=np.int32)
    o = 0
    for b, n in enumerate(npg):
        pt[b, :n] = perm[o:o + n]
        o += n
    used = np.zeros(P, dtype=bool)
    used[perm[:need]] = True
    return pt, P, used


def make(wl: Workload, mode: str = "continuous", seed: int | None = None,
         random_pages: bool | None = None, k_fmt: str | None = None) -> Inputs:
    """Generate every input of workload ``wl`` in ``mode`` ('continuous' | 'exact').  ``k_fmt``
    is the indexer key cache's format: 'e4m3' (one fp32 scale per token, the default) or
    'mxfp8' (one scale byte per 32 dims); fp32 workloads keep fp32 keys."""
    assert mode in ("continuous", "exact")
    sh = wl.shape
    k_fmt = "f32" if sh.fp32 else (k_fmt or "e4m3")
    assert k_fmt in (("f32",) if sh.fp32 else ("e4m3", "mxfp8"))
    mx = k_fmt == "mxfp8"
    seed = seed_of(wl.cfg, mode) if seed is None else int(seed)
    rp = wl.paged_random if random_pages is None else bool(random_pages)
    exact = mode == "exact"

    seq_lens = np.asarray(wl.seq_lens, dtype=np.int32)
    q_lens = np.asarray(wl.q_lens, dtype=np.int32)
    assert np.all(q_lens >= 0) and np.all(q_lens <= seq_lens) and q_lens.sum() >= 1
    cu_q = np.zeros(wl.B + 1, dtype=np.int32)
    cu_q[1:] = np.cumsum(q_lens)
    T = int(cu_q[-1])
    req = np.repeat(np.arange(wl.B, dtype=np.int32), q_lens)
    positions = np.concatenate([np.arange(L - q, L, dtype=np.int32)
                                for L, q in zip(seq_lens, q_lens)])
    pt, P, used = _page_table(wl, seed, rp)

    f32 = sh.fp32
    q_idx = np.empty((T, sh.H_I, sh.D_I), dtype=np.float32 if f32 else np.uint16)
    w = np.empty((T, sh.H_I), dtype=np.float32)
    q = np.empty((T, sh.H, sh.D_qk), dtype=np.float32 if f32 else np.uint16)
    k_pool = np.empty((P, PAGE, sh.D_I), dtype=np.float32 if f32 else np.uint8)
    k_scale = None if f32 else (np.empty((P, PAGE, sh.D_I // MX_GROUP), dtype=np.uint8) if mx
                                else np.empty((P, PAGE), dtype=np.float32))
    kv_dt = np.float32 if f32 else (np.uint8 if sh.kv_fp8 else np.uint16)
    kv_pool = np.empty((P, PAGE, sh.D_qk), dtype=kv_dt)
    kv_scale = np.empty((P, PAGE), dtype=np.float32) if (sh.kv_fp8 and not f32) else None
    info: dict = {}

    ex = ThreadPoolExecutor(_workers())

    # ---- query-side tensors, per 64-token block of each request
    def q_task(b, blk):
        t0 = int(cu_q[b]) + blk * 64
        n = min(64, int(cu_q[b + 1]) - t0)
        g1, g2, g4 = _rng(seed, T_QIDX, b, blk), _rng(seed, T_W, b, blk), _rng(seed, T_Q, b, blk)
        if exact:
            qi = g1.integers(-3, 4, size=(n, sh.H_I, sh.D_I)).astype(np.float32)
            ww = g2.choice(np.array([0.25, 0.5, 1.0], dtype=np.float32), size=(n, sh.H_I))
        else:
            qi = g1.standard_normal((n, sh.H_I, sh.D_I), dtype=np.float32)
            ww = (g2.random((n, sh.H_I), dtype=np.float32) / np.float32(sh.w_div)).astype(np.float32)
        qq = g4.standard_normal((n, sh.H, sh.D_qk), dtype=np.float32)
        q_idx[t0:t0 + n] = qi if f32 else to_bf16_bits(qi)
        w[t0:t0 + n] = ww
        q[t0:t0 + n] = qq if f32 else to_bf16_bits(qq)

    list(ex.map(lambda a: q_task(*a),
                [(b, blk) for b in range(wl.B) for blk in range(-(-int(q_lens[b]) // 64))]))

    # ---- structure that depends on the query side
    heavy = {}
    planted = {}
    if wl.structure == "heavy":
        for b in range(wl.B):
            L = int(seq_lens[b])
            heavy[b] = np.sort(_rng(seed, T_STRUCT, b, 0).permutation(L)[: int(0.01 * L)])
        info["heavy_positions"] = heavy
    if wl.structure == "planted":
        for b in range(wl.B):
            L = int(seq_lens[b])
            off = int(_rng(seed, T_STRUCT, b, 1).integers(0, max(1, L - 4096)))
            t = int(cu_q[b + 1]) - 1
            qi = q_idx[t].astype(np.float32) if f32 else \
                (q_idx[t].astype(np.uint32) << 16).view(np.float32)
            u = (w[t][:, None] * qi).sum(axis=0, dtype=np.float64)
            u = (u / np.linalg.norm(u)).astype(np.float32)
            planted[b] = (off, u)
        info["planted"] = {b: off for b, (off, _) in planted.items()}

    # ---- cache tensors, per logical page, written to their physical pages
    def cache_task(b, j0, j1):
        L = int(seq_lens[b])
        n = (j1 - j0) * PAGE
        s0 = j0 * PAGE
        pos = np.arange(s0, s0 + n)
        valid = pos < L
        # indexer keys
        kr = np.empty((n, sh.D_I), dtype=np.float32)
        for j in range(j0, j1):
            g = _rng(seed, T_KIDX, b, j)
            sl = slice((j - j0) * PAGE, (j - j0 + 1) * PAGE)
            kr[sl] = g.integers(-3, 4, size=(PAGE, sh.D_I)).astype(np.float32) if exact else \
                g.standard_normal((PAGE, sh.D_I), dtype=np.float32)
        # latent rows
        cr = np.empty((n, sh.D_qk), dtype=np.float32)
        for j in range(j0, j1):
            g = _rng(seed, T_KV, b, j)
            cr[(j - j0) * PAGE:(j - j0 + 1) * PAGE] = g.standard_normal((PAGE, sh.D_qk),
                                                                        dtype=np.float32)
        if b in heavy:
            h = heavy[b]
            h = h[(h >= s0) & (h < s0 + n)] - s0
            kr[h] *= np.float32(8.0)
            cr[h] *= np.float32(8.0)
        if b in planted and not exact:
            off, u = planted[b]
            lo, hi = max(off, s0), min(off + 4096, s0 + n)
            if lo < hi:
                kr[lo - s0:hi - s0] += np.float32(np.sqrt(sh.D_I)) * u[None, :]
        if f32:
            kc, ks = np.where(valid[:, None], kr, np.float32(POISON_F32)), None
            cc, cs = np.where(valid[:, None], cr, np.float32(POISON_F32)), None
        else:
            if mx:
                kc, ks = to_mxfp8(kr)
            elif exact:
                kc, ks = ints_to_e4m3(kr), np.ones(n, dtype=np.float32)
            else:
                kc, ks = to_e4m3_per_token(kr)
            kc[~valid] = POISON_E4M3
            ks[~valid] = POISON_MX_BYTE if mx else POISON_SCALE
            if sh.kv_fp8:
                cc, cs = to_e4m3_per_token(cr)
                cc[~valid] = POISON_E4M3
                cs[~valid] = POISON_SCALE
            else:
                cc, cs = to_bf16_bits(cr), None
                cc[~valid] = POISON_BF16
        for j in range(j0, j1):
            p = int(pt[b, j])
            sl = slice((j - j0) * PAGE, (j - j0 + 1) * PAGE)
            k_pool[p] = kc[sl].reshape(PAGE, sh.D_I)
            kv_pool[p] = cc[sl].reshape(PAGE, sh.D_qk)
            if k_scale is not None:
                k_scale[p] = ks[sl]
            if kv_scale is not None:
                kv_scale[p] = cs[sl]

    tasks = []
    for b in range(wl.B):
        npg = -(-int(seq_lens[b]) // PAGE)
        for j0 in range(0, npg, 64):
            tasks.append((b, j0, min(npg, j0 + 64)))
    list(ex.map(lambda a: cache_task(*a), tasks))
    ex.shutdown()

    # ---- poison every page that holds no token
    unused = np.nonzero(~used)[0]
    if f32:
        k_pool[unused] = POISON_F32
        kv_pool[unused] = POISON_F32
    else:
        k_pool[unused] = POISON_E4M3
        k_scale[unused] = POISON_MX_BYTE if mx else POISON_SCALE
        if sh.kv_fp8:
            kv_pool[unused] = POISON_E4M3
            kv_scale[unused] = POISON_SCALE
        else:
            kv_pool[unused] = POISON_BF16

    return Inputs(wl=wl, mode=mode, seed=seed, seq_lens=seq_lens, q_lens=q_lens, cu_q=cu_q,
                  positions=positions, req=req, page_table=pt, n_pages=P, q_idx=q_idx, w=w,
                  k_pool=k_pool, k_scale=k_scale, q=q, kv_pool=kv_pool, kv_scale=kv_scale,
                  info=info, k_fmt=k_fmt)
