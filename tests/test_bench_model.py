"""Host logic of bench.py: the one-GPU guard and the algorithmic byte / flop model behind every
roofline figure it prints (no GPU needed)."""
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _stand_in(cfg, seq_lens, q_lens):
    """The fields of a generated batch that the model reads, without generating tensors."""
    wl = synth.workload(cfg)
    seq_lens = np.asarray(seq_lens, np.int64)
    positions = np.concatenate([np.arange(L - q, L) for L, q in zip(seq_lens, q_lens)])
    return SimpleNamespace(wl=wl, seq_lens=seq_lens, positions=positions, T=int(sum(q_lens)),
                           q_lens=np.asarray(q_lens))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_decode32k_model():
    """32 requests x 32768 positions, one query each at position 32767 (so k_t = K = 2048)."""
    inp = _stand_in(synth.DECODE32K, [32768] * 32, [1] * 32)
    a = bench.algorithmic(inp)
    keys = 32 * 32768
    # indexer: an e4m3 key (128 B) and its fp32 scale per cached position, read once; bf16 q_I
    # (64 x 128) and fp32 w (64) per token
    assert a["idx_bytes"] == keys * (128 + 4) + 32 * (64 * 128 * 2 + 64 * 4)
    assert a["idx_flops"] == 2 * 64 * 128 * keys
    # selection output: 2048 int32 per token
    assert a["topk_bytes"] == 32 * 2048 * 4
    # attention: 2048 bf16 rows of 576 per token, plus indices, q (128 x 576 bf16), O (128 x
    # 512 bf16) and lse (128 fp32)
    per_token = 2048 * 1152 + 2048 * 4 + 128 * 576 * 2 + 128 * 512 * 2 + 128 * 4
    assert a["attn_bytes"] == 32 * per_token
    assert a["attn_flops"] == 32 * 2 * 128 * 2048 * (576 + 512)
    # unfused calls: the scorer also writes, and the selection reads back, one fp32 per position
    assert a["idx_kernel_bytes"] == a["idx_bytes"] + 4 * keys
    assert a["topk_kernel_bytes"] == 4 * keys + a["topk_bytes"]
    # every stage is HBM-bound here: 17.41 us + 0.03 us + 10.59 us at 8 TB/s
    assert bench.t_roof(a) * 1e6 == pytest.approx(28.0, rel=5e-3)


def test_causal_prefill_model():
    """One 4096-token prefill: token at position p has p + 1 candidates and min(K, p + 1)
    selected keys; the attention stage is matrix-bound (flops per byte above the bf16 ridge)."""
    L = 4096
    inp = _stand_in(synth.PREFILL64K, [L], [L])
    a = bench.algorithmic(inp)
    n = np.arange(1, L + 1)
    k = np.minimum(2048, n)
    assert a["idx_flops"] == 2 * 64 * 128 * int(n.sum())
    assert a["attn_flops"] == 2 * 128 * (576 + 512) * int(k.sum())
    # e4m3 latent rows: 576 code bytes + a 4-byte scale each
    assert a["attn_bytes"] == int(k.sum()) * 580 + L * (2048 * 4 + 128 * (576 * 2 + 512 * 2 + 4))
    assert a["attn_flops"] / a["attn_bytes"] > bench.BF16_PEAK / (bench.HBM_PEAK_GBS * 1e9)
