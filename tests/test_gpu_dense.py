"""GPU parity of the dense-masked attention (sparse_mla_attn_dense: every causal row read and
multiplied, the selection as a row mask) against the oracle, through the C ABI.  The selection
comes from index_score_topk; both the gather form and the dense form are gated against the
oracle's attention over that selection (the same gates as everywhere: 1e-2 bf16 cache, 2e-2
e4m3 cache, plus half a bf16 ulp of the value for a bf16 output)."""
import dataclasses

import numpy as np
import pytest
import torch

import synth
import top_indexed_sparse_amd as tis
from oracle import Oracle
from synth.device import to_device
from tests.gpu_path import check_attention, make_batch, note, sample_tokens

pytestmark = pytest.mark.gpu


def _run(inp, out_name):
    sh = inp.wl.shape
    d = to_device(inp)
    bt = make_batch(inp)
    T, K = inp.T, sh.K
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    tis.index_score_topk(bt, d.q_idx, d.w, d.k_pool, d.k_scale, K, idx)
    out_dt = {"f32": torch.float32, "bf16": torch.bfloat16}[out_name]
    res = {}
    for form, fn in (("gather", tis.sparse_mla_attn), ("dense", tis.sparse_mla_attn_dense)):
        o = torch.empty((T, sh.H, sh.D_v), dtype=out_dt, device="cuda")
        lse = torch.empty((T, sh.H), dtype=torch.float32, device="cuda")
        fn(bt, d.q, d.kv_pool, d.kv_scale, idx, sh.softmax_scale, o, lse)
        torch.cuda.synchronize()
        r = type("R", (), {})()
        r.idx = idx.cpu().numpy()
        r.out = o.float().cpu().numpy().astype(np.float64)
        r.out_bf16 = out_dt == torch.bfloat16
        r.lse = lse.cpu().numpy().astype(np.float64)
        res[form] = r
    return res


def _check(inp, res, tokens):
    orc = Oracle(inp)
    errs = {}
    for form, r in res.items():
        errs[form] = check_attention(inp, orc, r, tokens)
    diff = float(np.max(np.abs(res["dense"].out[tokens] - res["gather"].out[tokens])))
    note(f"  {inp.wl.name}/{inp.mode}: gather err {errs['gather'][0]:.2e}, dense err "
         f"{errs['dense'][0]:.2e}, |dense - gather| {diff:.2e}")


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["continuous", "exact"])
def test_dense_prefill_shapes_small(mode, out):
    # e4m3 latent cache with heavy rows; causal ranges up to 2600 (two 2048-position splits)
    wl = synth.reduced(synth.workload(synth.PREFILL64K), [2600], [2600])
    inp = synth.make(wl, mode)
    note(f"case dense prefill-small mode={mode} out={out} T={inp.T}")
    res = _run(inp, out)
    _check(inp, res, sample_tokens(inp, 100))


def test_dense_decode_shapes_bf16_cache():
    # bf16 cache, decode tokens over ranges up to 9000 (five splits), one shorter than K
    wl = synth.reduced(synth.workload(synth.DECODE32K), [9000, 1500, 4100, 6000], [1, 1, 2, 1])
    inp = synth.make(wl, "continuous")
    note(f"case dense decode-small T={inp.T}")
    res = _run(inp, "bf16")
    _check(inp, res, list(range(inp.T)))


def test_dense_ragged_small():
    L = [1024, 3000, 700, 5000, 64, 2100]
    q = [1, 300, 1, 1, 64, 1]
    wl = synth.reduced(synth.workload(synth.RAGGED), L, q)
    inp = synth.make(wl, "continuous")
    note(f"case dense ragged-small T={inp.T}")
    res = _run(inp, "f32")
    _check(inp, res, sample_tokens(inp, 80))
