"""The five synthetic workloads of the indexer -> Top-K -> sparse-MLA path, as plain data.

Each workload names its shapes, storage formats and structure.  Nothing here computes any
part of the method; ``synth.gen`` turns a workload plus a seed into raw input bytes.

Workloads (numbered 0..4):
  0 tiny      - fp32 everywhere; 1 request, context 512, 8 query tokens at 504..511; indexer
                4 heads x 32; Top-K 64; attention 8 heads, latent 64 + RoPE 16 (QK 80, V 64).
  1 decode32k - 32 requests x context 32768 x 1 new token; indexer 64 heads x 128, q_I bf16,
                k_I e4m3 + per-token fp32 scale; Top-K 2048; attention 128 heads, QK 576
                (512 latent + 64 RoPE), V 512; latent cache bf16; softmax scale 1/sqrt(192).
  2 prefill64k- 1 sequence of 65536 tokens, every token a query over its causal prefix;
                workload-1 shapes; latent cache e4m3 + per-token scale; 1% heavy-hitter rows.
  3 decode1m  - 4 requests x context 1,048,576 x 1 new token; e4m3 caches; a planted block of
                4096 contiguous high-relevance key positions per request.
  4 ragged    - 64 requests, lengths log-uniform in [1K, 256K]; 48 decode one token, 16 run a
                4096-token chunked-prefill slice; random page table with poisoned slack pages.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np

PAGE = 64  # tokens per KV page (both caches)

TINY, DECODE32K, PREFILL64K, DECODE1M, RAGGED = range(5)
NAMES = ("tiny", "decode32k", "prefill64k", "decode1m", "ragged")


@dataclass(frozen=True)
class Shape:
    H_I: int            # indexer heads
    D_I: int            # indexer head dim
    K: int              # Top-K
    H: int              # attention query heads
    D_qk: int           # latent + RoPE width of each cached row
    D_v: int            # value width (leading D_v dims of the same row)
    fp32: bool          # every tensor stored as fp32 (tiny workload)
    kv_fp8: bool        # latent cache e4m3 + per-token scale (else bf16)
    softmax_scale: float
    w_div: float        # indexer weights drawn U(0,1)/w_div in continuous mode


SHAPE_TINY = Shape(H_I=4, D_I=32, K=64, H=8, D_qk=80, D_v=64, fp32=True, kv_fp8=False,
                   softmax_scale=1.0 / math.sqrt(80.0), w_div=1.0)
SHAPE_BF16KV = Shape(H_I=64, D_I=128, K=2048, H=128, D_qk=576, D_v=512, fp32=False,
                     kv_fp8=False, softmax_scale=1.0 / math.sqrt(192.0), w_div=8.0)
SHAPE_FP8KV = replace(SHAPE_BF16KV, kv_fp8=True)


@dataclass(frozen=True)
class Workload:
    name: str
    cfg: int
    shape: Shape
    seq_lens: tuple          # context length L_b of each request (query tokens included)
    q_lens: tuple            # query tokens of each request: the last q_len positions
    structure: str = "none"  # none | heavy | planted | ragged
    paged_random: bool = False  # seeded page permutation with poisoned slack pages

    @property
    def B(self) -> int:
        return len(self.seq_lens)

    @property
    def T(self) -> int:
        return int(sum(self.q_lens))


def seed_of(cfg: int, mode: str) -> int:
    """Seed rule: 20260000 + 10*cfg + mode (0 continuous, 1 exact)."""
    return 20260000 + 10 * cfg + (1 if mode == "exact" else 0)


def ragged_lengths(seed: int, B: int = 64, lo: int = 1024, hi: int = 262144,
                   n_prefill: int = 16, chunk: int = 4096):
    """Seeded lengths for the ragged workload: L_b = floor(exp(U(ln lo, ln hi))); a seeded
    choice of ``n_prefill`` requests run a chunk of min(chunk, L_b) query tokens, the rest 1."""
    rng = np.random.Generator(np.random.Philox(key=(seed << 40) | (0xA11 << 8)))
    L = np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), size=B))).astype(np.int64)
    L = np.clip(L, lo, hi)
    pre = rng.permutation(B)[:n_prefill]
    q = np.ones(B, dtype=np.int64)
    q[pre] = np.minimum(chunk, L[pre])
    return tuple(int(x) for x in L), tuple(int(x) for x in q)


def workload(cfg: int, mode: str = "continuous") -> Workload:
    """The full-size workload ``cfg`` (0..4)."""
    if cfg == TINY:
        return Workload("tiny", cfg, SHAPE_TINY, (512,), (8,))
    if cfg == DECODE32K:
        return Workload("decode32k", cfg, SHAPE_BF16KV, (32768,) * 32, (1,) * 32)
    if cfg == PREFILL64K:
        return Workload("prefill64k", cfg, SHAPE_FP8KV, (65536,), (65536,), structure="heavy")
    if cfg == DECODE1M:
        return Workload("decode1m", cfg, SHAPE_FP8KV, (1048576,) * 4, (1,) * 4,
                        structure="planted")
    if cfg == RAGGED:
        L, q = ragged_lengths(seed_of(cfg, mode))
        return Workload("ragged", cfg, SHAPE_FP8KV, L, q, structure="ragged", paged_random=True)
    raise ValueError(cfg)


def reduced(wl: Workload, seq_lens, q_lens, name: str | None = None, **kw) -> Workload:
    """Same shapes, formats and structure at smaller lengths (for oracle-sized parity cases)."""
    return replace(wl, name=name or wl.name + "-reduced", seq_lens=tuple(int(x) for x in seq_lens),
                   q_lens=tuple(int(x) for x in q_lens), **kw)
