"""Upload a generated batch to the GPU as torch tensors (plain copies of the raw bytes)."""
from __future__ import annotations

from types import SimpleNamespace

import numpy as np
import torch


def _t(a, device, kind):
    if a is None:
        return None
    if kind == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_device(inp, device="cuda") -> SimpleNamespace:
    """q_idx/q as bf16 (or fp32), caches as uint8 e4m3 codes / bf16 / fp32, scales fp32."""
    f32 = inp.wl.shape.fp32
    kv_kind = "f32" if f32 else ("raw" if inp.wl.shape.kv_fp8 else "bf16")
    return SimpleNamespace(
        q_idx=_t(inp.q_idx, device, "f32" if f32 else "bf16"),
        w=_t(inp.w, device, "f32"),
        k_pool=_t(inp.k_pool, device, "raw"),
        k_scale=_t(inp.k_scale, device, "f32"),
        q=_t(inp.q, device, "f32" if f32 else "bf16"),
        kv_pool=_t(inp.kv_pool, device, kv_kind),
        kv_scale=_t(inp.kv_scale, device, "f32"),
    )
