"""The allocation-free fused selection (index_score_topk_noalloc) against index_score_topk
with a caller workspace, through the C ABI: two calls in a row on the library's per-device
scratch, the second over a smaller batch (so it runs over what the first left there)."""
import numpy as np
import pytest
import torch

import synth
import top_indexed_sparse_amd as tis
from synth.device import to_device
from tests.gpu_path import make_batch, note

pytestmark = pytest.mark.gpu


def _both(inp, K):
    d, bt = to_device(inp), make_batch(inp)
    T = inp.T
    ref_i = torch.full((T, K), -7, dtype=torch.int32, device="cuda")
    ref_v = torch.full((T, K), 7.0, dtype=torch.float32, device="cuda")
    tis.index_score_topk(bt, d.q_idx, d.w, d.k_pool, d.k_scale, K, ref_i, ref_v)
    got_i = torch.full((T, K), -9, dtype=torch.int32, device="cuda")
    got_v = torch.full((T, K), 9.0, dtype=torch.float32, device="cuda")
    tis.index_score_topk_noalloc(bt, d.q_idx, d.w, d.k_pool, d.k_scale, K, got_i, got_v)
    torch.cuda.synchronize()
    return ref_i.cpu().numpy(), ref_v.cpu().numpy(), got_i.cpu().numpy(), got_v.cpu().numpy()


@pytest.mark.parametrize("mode", ["continuous", "exact"])
def test_noalloc_matches_workspace_call(mode):
    base = synth.workload(synth.DECODE32K)
    # first: long rows (the several-workgroups-per-row selection and its scratch state) and a
    # short one; second: a smaller batch over the scratch the first one left behind
    cases = [([40000, 33000, 5000], [1, 1, 1]), ([3000, 2100], [1, 1])]
    for lens, q in cases:
        inp = synth.make(synth.reduced(base, lens, q), mode)
        note(f"case noalloc {mode} lens={lens}")
        ri, rv, gi, gv = _both(inp, base.shape.K)
        assert np.array_equal(ri, gi), lens
        assert np.array_equal(rv, gv), lens


def test_noalloc_prefill_chunks():
    """A prefill batch whose score rows exceed the scratch in one piece runs in token chunks
    (the same chunked loop as the workspace call, with smaller chunks): same selection."""
    wl = synth.reduced(synth.workload(synth.PREFILL64K), [5000], [5000])
    inp = synth.make(wl, "continuous")
    note("case noalloc prefill 5000 tokens (two chunks of score rows)")
    ri, rv, gi, gv = _both(inp, wl.shape.K)
    assert np.array_equal(ri, gi) and np.array_equal(rv, gv)
