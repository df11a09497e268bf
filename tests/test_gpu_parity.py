"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle on seeded inputs.

Gates: Top-K bit-exact in the exact input mode; otherwise recall >= 0.999 with every
mismatch within 1e-3 relative of the k-th score; fused == unfused bit for bit; attention
max-abs error <= 1e-2 (bf16 / fp32 cache) or 2e-2 (e4m3 cache) against the oracle on the
GPU's selected set; lse within 1e-3."""
import numpy as np
import pytest
import torch

import synth
from synth.device import to_device
from oracle import Oracle
from tests.gpu_path import (attend, check_attention, check_scores, check_topk, note, run_path,
                            run_path_sampled, sample_tokens)

pytestmark = pytest.mark.gpu


def _common(inp, r, tokens, exact, also_bf16=False, qmode=None):
    """Fused == unfused, emitted values, scores, Top-K and attention gates.  also_bf16: the
    attention call is run again with a bf16 output (the benchmarked form for e4m3 caches)
    and gated as well.  qmode: the oracle's query mode ('fp8' or 'none')."""
    orc = Oracle(inp, qmode=qmode)
    # fused and unfused chains agree exactly
    assert np.array_equal(r.idx, r.idx2), "fused vs unfused Top-K"
    assert np.array_equal(r.val, r.val2), "fused vs unfused Top-K values"
    # the emitted values are the scores of the emitted positions
    for t in tokens[:8]:
        sel = r.idx[t][r.idx[t] >= 0]
        assert np.array_equal(r.val[t][: sel.size], r.scores[t, sel]), t
    serr = check_scores(inp, orc, r.scores, tokens)
    rec = check_topk(inp, orc, r.idx, tokens, exact)
    aerr = check_attention(inp, orc, r, tokens)
    note(f"  {inp.wl.name}/{inp.mode}: score rel err {serr:.2e}, recall {rec}, "
         f"attn err {aerr[0]:.2e}, lse err {aerr[1]:.2e}")
    if also_bf16 and not r.out_bf16:
        rb = attend(inp, r, "bf16")
        berr = check_attention(inp, orc, rb, tokens)
        note(f"  {inp.wl.name}/{inp.mode}: bf16 output: attn err {berr[0]:.2e}, "
             f"lse err {berr[1]:.2e}")
    return serr


@pytest.mark.parametrize("mode", ["continuous", "exact"])
def test_tiny_fp32(mode):
    inp = synth.make(synth.workload(synth.TINY), mode)
    note(f"case tiny mode={mode}")
    r = run_path(inp)
    serr = _common(inp, r, list(range(inp.T)), mode == "exact")
    if mode == "exact":
        assert serr == 0.0


@pytest.mark.parametrize("mode", ["continuous", "exact"])
def test_decode_shapes_small(mode):
    # decode32k shapes; one request shorter than K selects everything; one ragged tail page
    wl = synth.reduced(synth.workload(synth.DECODE32K), [4096, 1500, 5000, 2049], [1, 1, 2, 1])
    inp = synth.make(wl, mode)
    note(f"case decode-small mode={mode} T={inp.T}")
    r = run_path(inp)
    serr = _common(inp, r, list(range(inp.T)), mode == "exact")
    if mode == "exact":
        assert serr == 0.0
    else:
        assert serr < 1e-4


def test_decode_shapes_random_pages():
    wl = synth.reduced(synth.workload(synth.DECODE32K), [3000, 6000, 2500], [1, 1, 1])
    a = synth.make(wl, "continuous", random_pages=False)
    b = synth.make(wl, "continuous", random_pages=True)
    note("case decode page-permutation invariance")
    ra, rb = run_path(a, unfused=False), run_path(b, unfused=False)
    assert np.array_equal(ra.idx, rb.idx)
    assert np.array_equal(ra.out, rb.out) and np.array_equal(ra.lse, rb.lse)


@pytest.mark.parametrize("mode", ["continuous", "exact"])
def test_prefill_shapes_small(mode):
    # prefill64k shapes (e4m3 latent cache, heavy hitters): every token queries its prefix
    wl = synth.reduced(synth.workload(synth.PREFILL64K), [2600], [2600])
    inp = synth.make(wl, mode)
    note(f"case prefill-small mode={mode} T={inp.T}")
    r = run_path(inp)
    toks = sample_tokens(inp, 120)
    _common(inp, r, toks, mode == "exact", also_bf16=True)


def test_decode1m_shapes_small():
    wl = synth.reduced(synth.workload(synth.DECODE1M), [70000, 40000], [1, 1])
    inp = synth.make(wl, "continuous")
    note("case decode1m-small (16 key splits per token)")
    r = run_path(inp)
    _common(inp, r, list(range(inp.T)), False, also_bf16=True)
    # the planted block dominates the selection
    for b in range(inp.B):
        off = inp.info["planted"][b]
        sel = r.idx[b][r.idx[b] >= 0]
        frac = np.mean((sel >= off) & (sel < off + 4096))
        note(f"  request {b}: {frac:.3f} of the selection inside the planted block")
        assert frac > 0.5


@pytest.mark.parametrize("mode", ["continuous", "exact"])
def test_ragged_small(mode):
    L = [1024, 3000, 700, 5000, 64, 2100]
    q = [1, 300, 1, 1, 64, 1]
    wl = synth.reduced(synth.workload(synth.RAGGED), L, q)
    inp = synth.make(wl, mode)
    note(f"case ragged-small mode={mode} T={inp.T}")
    r = run_path(inp)
    _common(inp, r, sample_tokens(inp, 80), mode == "exact", also_bf16=True)


@pytest.mark.parametrize("mode", ["continuous", "exact"])
def test_decode_shapes_e4m3_cache(mode):
    """decode32k shapes over an e4m3 latent cache: 32 tokens, so each token's keys are split
    in four and merged (fp16 partials for a bf16 output, fp32 partials for an fp32 one)."""
    import dataclasses
    base = synth.workload(synth.DECODE32K)
    L = [4096, 3000, 2500, 5000] * 8
    wl = synth.reduced(base, L, [1] * 32, shape=dataclasses.replace(base.shape, kv_fp8=True))
    inp = synth.make(wl, mode)
    note(f"case decode-shapes e4m3 cache mode={mode} T={inp.T}")
    r = run_path(inp)
    _common(inp, r, list(range(inp.T)), mode == "exact", also_bf16=True)


def test_many_requests_with_empty_ones():
    """150 requests (more than one 64-request window of the token locator), some with no query
    tokens (cu_q repeats), some with several."""
    rng = np.random.default_rng(5)
    B = 150
    L = rng.integers(40, 700, size=B).tolist()
    q = [0 if i % 17 == 3 else (5 if i % 23 == 0 else 1) for i in range(B)]
    q[0] = q[-1] = 0
    wl = synth.reduced(synth.workload(synth.DECODE32K), L, q)
    inp = synth.make(wl, "continuous")
    note(f"case many-requests B={B} T={inp.T}")
    r = run_path(inp, out_f32=True)  # |O| reaches 4+ over a few hundred keys
    _common(inp, r, list(range(inp.T)), False)


def test_attention_workspace_reuse():
    """One workspace reused by calls of different batch sizes gives the results of fresh
    workspaces."""
    import top_indexed_sparse_amd as tis
    note("case attention workspace reuse")
    wl = synth.reduced(synth.workload(synth.DECODE32K), [5000, 3000, 4096, 2100], [1, 1, 1, 1])
    inp = synth.make(wl, "continuous")
    sh = inp.wl.shape
    ref = run_path(inp, unfused=False)
    d, bt = ref.dev, ref.batch
    idx = torch.tensor(ref.idx, device="cuda")
    big = tis.sparse_mla_attn_workspace_size(bt, sh.K, sh.H, sh.D_qk, sh.D_v, tis.TIS_BF16)
    assert big > 0
    ws = torch.full((big + 4096,), 0x7F, dtype=torch.uint8, device="cuda")
    for rnd in range(3):
        out = torch.empty((inp.T, sh.H, sh.D_v), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((inp.T, sh.H), dtype=torch.float32, device="cuda")
        tis.sparse_mla_attn(bt, d.q, d.kv_pool, d.kv_scale, idx, sh.softmax_scale, out, lse, ws=ws)
        torch.cuda.synchronize()
        assert np.array_equal(out.float().cpu().numpy().astype(np.float64), ref.out), rnd
        assert np.array_equal(lse.cpu().numpy().astype(np.float64), ref.lse), rnd
        # a smaller batch through the same workspace
        bt1 = tis.Batch(inp.seq_lens[:1], inp.cu_q[:2], inp.page_table[:1], inp.n_pages)
        out1 = torch.empty((1, sh.H, sh.D_v), dtype=torch.bfloat16, device="cuda")
        tis.sparse_mla_attn(bt1, d.q[:1], d.kv_pool, d.kv_scale, idx[:1].contiguous(),
                            sh.softmax_scale, out1, None, ws=ws)
        torch.cuda.synchronize()
        # (another split count: same values up to rounding)
        assert np.abs(out1.float().cpu().numpy()[0].astype(np.float64) - ref.out[0]).max() < 1e-2


def test_split_merge_for_long_batches():
    """Many tokens with K above the 2048-key split limit: every token is split and merged."""
    import dataclasses
    base = synth.workload(synth.DECODE32K)
    wl = synth.reduced(base, [6000], [4100], shape=dataclasses.replace(base.shape, K=2560))
    inp = synth.make(wl, "continuous")
    note(f"case separate split merge T={inp.T} K={inp.wl.shape.K}")
    r = run_path(inp, unfused=False, out_f32=True)
    orc = Oracle(inp)
    toks = [0, 1, 2047, 2048, 3000, inp.T - 1]
    check_topk(inp, orc, r.idx, toks, False)
    check_attention(inp, orc, r, toks)


def test_determinism():
    wl = synth.reduced(synth.workload(synth.DECODE32K), [4096, 3000], [1, 1])
    inp = synth.make(wl, "continuous")
    note("case determinism")
    a, b = run_path(inp, unfused=False), run_path(inp, unfused=False)
    assert np.array_equal(a.idx, b.idx) and np.array_equal(a.val, b.val)
    assert np.array_equal(a.out, b.out) and np.array_equal(a.lse, b.lse)


def test_k_edge_cases():
    wl = synth.reduced(synth.workload(synth.DECODE32K), [3000, 100], [1, 1])
    inp = synth.make(wl, "exact")
    orc = Oracle(inp)
    note("case K in {1, 100, 5000}")
    for K in (1, 100, 5000):
        r = run_path(inp, K=K)
        assert np.array_equal(r.idx, r.idx2)
        check_topk(inp, orc, r.idx, list(range(inp.T)), True, K=K)
        check_attention(inp, orc, r, list(range(inp.T)))


def test_out_of_range_pages_are_skipped():
    import top_indexed_sparse_amd as tis
    from tests.gpu_path import make_batch
    from synth.device import to_device
    wl = synth.reduced(synth.workload(synth.DECODE32K), [4096], [1])
    inp = synth.make(wl, "continuous")
    inp.page_table = inp.page_table.copy()
    inp.page_table[0, 3] = inp.n_pages + 7        # logical page 3 -> out of range
    note("case out-of-range page entry")
    d, bt = to_device(inp), make_batch(inp)
    scores = torch.zeros((1, 4096), dtype=torch.float32, device="cuda")
    tis.index_score(bt, d.q_idx, d.w, d.k_pool, d.k_scale, scores)
    s = scores.cpu().numpy()[0]
    assert np.all(np.isneginf(s[192:256])) and np.all(np.isfinite(s[:192]))
    idx = torch.tensor(np.arange(150, 350, dtype=np.int32)[None, :], device="cuda")
    out = torch.empty((1, 128, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, 128), dtype=torch.float32, device="cuda")
    tis.sparse_mla_attn(bt, d.q, d.kv_pool, d.kv_scale, idx, inp.wl.shape.softmax_scale, out, lse)
    orc = Oracle(inp)
    keep = np.array([s for s in range(150, 350) if not (192 <= s < 256)])
    o, l = orc.attention(0, keep)
    assert np.abs(out.float().cpu().numpy()[0] - o).max() < 1e-2


def test_topk_crafted_rows():
    """Top-K on crafted score rows: one value everywhere (the short list overflows and the
    exact whole-row select runs), four distinct values, the largest scores crowded at the
    end or the start of the row, signed zeros and -inf, mostly exact zeros, and lengths that
    end inside a block of four.  Every row equals the oracle's Top-K, values included."""
    import top_indexed_sparse_amd as tis
    from oracle.method import topk_token
    rng = np.random.default_rng(20261202)
    lens = [32768, 32768, 32768, 32768, 20001, 4097, 8190, 32768, 3000]
    B, K, ld = len(lens), 2048, 32768
    S = np.zeros((B, ld), np.float32)
    S[0] = 1.5
    S[1] = rng.integers(0, 4, ld)
    S[2] = np.linspace(-1.0, 1.0, ld)
    S[3] = np.linspace(1.0, -1.0, ld)
    S[4] = rng.standard_normal(ld)
    S[4][::7] = -0.0
    S[4][::11] = 0.0
    S[4][::13] = -np.inf
    S[5] = rng.standard_normal(ld)
    S[6] = rng.exponential(size=ld) * (rng.random(ld) < 0.3)
    S[7] = rng.standard_normal(ld)
    S[8] = rng.standard_normal(ld)
    note("case Top-K on crafted rows")
    bt = tis.Batch(np.array(lens, np.int32), np.arange(B + 1, dtype=np.int32),
                   np.zeros((B, 512), np.int32), 1)
    scores = torch.from_numpy(S).cuda()
    idx = torch.full((B, K), -7, dtype=torch.int32, device="cuda")
    val = torch.full((B, K), 7.0, dtype=torch.float32, device="cuda")
    tis.topk_select(bt, scores, K, idx, val)
    idx, val = idx.cpu().numpy(), val.cpu().numpy()
    for b in range(B):
        ref = topk_token(S[b, :lens[b]].astype(np.float64), K)[0]
        assert np.array_equal(idx[b], ref), b
        k = int((ref >= 0).sum())
        assert np.array_equal(val[b, :k], S[b, ref[:k]]), b
        assert np.all(val[b, k:] == 0.0)


def test_topk_crafted_long_rows():
    """Top-K over a few rows longer than 32768 positions (selected by several workgroups per
    row): unique, tied (the candidate list overflows and the one-workgroup select finishes the
    row), signed-zero / -inf, sparse and short rows, a 1M-position row, for K = 1, 2048 and 4096
    (the largest K of that path) and 4100 (the one-workgroup path).  Every row equals the
    oracle's Top-K, values included."""
    import top_indexed_sparse_amd as tis
    from oracle.method import topk_token
    rng = np.random.default_rng(20261203)
    lens = [100000, 100000, 70001, 65537, 40000, 50000, 40000, 2000, 1000000]
    B, ld = len(lens), 1000000
    S = np.zeros((B, ld), np.float32)
    S[0] = 1.5
    S[1] = rng.integers(0, 4, ld)
    S[2] = np.linspace(-1.0, 1.0, ld)
    S[3] = np.linspace(1.0, -1.0, ld)
    S[4] = rng.standard_normal(ld)
    S[4][::7] = -0.0
    S[4][::11] = 0.0
    S[4][::13] = -np.inf
    S[5] = rng.standard_normal(ld)
    S[5][lens[5] - 3000:lens[5]] += 4.0
    S[6] = rng.exponential(size=ld) * (rng.random(ld) < 0.3)
    S[7] = rng.standard_normal(ld)
    S[8] = rng.standard_normal(ld)
    bt = tis.Batch(np.array(lens, np.int32), np.arange(B + 1, dtype=np.int32),
                   np.zeros((B, -(-ld // 64)), np.int32), 1)
    scores = torch.from_numpy(S).cuda()
    refs = {}
    for K in (1, 2048, 4096, 4100):
        note(f"case Top-K on crafted long rows, K={K}")
        idx = torch.full((B, K), -7, dtype=torch.int32, device="cuda")
        val = torch.full((B, K), 7.0, dtype=torch.float32, device="cuda")
        tis.topk_select(bt, scores, K, idx, val)
        idx, val = idx.cpu().numpy(), val.cpu().numpy()
        for b in range(B):
            if (b, K) not in refs:
                refs[b, K] = topk_token(S[b, :lens[b]].astype(np.float64), K)[0]
            ref = refs[b, K]
            assert np.array_equal(idx[b], ref), (b, K)
            k = int((ref >= 0).sum())
            assert np.array_equal(val[b, :k], S[b, ref[:k]]), (b, K)
            assert np.all(val[b, k:] == 0.0), (b, K)


def test_topk_streamed_rows():
    """Top-K over more than 64 rows longer than 32768 positions (one workgroup per row, the row
    streamed): the one-pass candidate list over a uniform sample's bound, with ties at the
    threshold (scores rounded to 1/8), sparse rows, signed zeros and -inf, a rising ramp, and
    rows whose candidates overflow the list (a constant row, four distinct values), which the
    exact streamed radix select finishes.  Every row equals the oracle's Top-K, values
    included, for K = 1, 100, 2048 and 4096."""
    import top_indexed_sparse_amd as tis
    from oracle.method import topk_token
    rng = np.random.default_rng(20261204)
    B = 66
    lens = rng.integers(32769, 90001, B)
    lens[:4] = [32769, 65536, 90000, 40001]
    ld = 90000
    S = np.zeros((B, ld), np.float32)
    for b in range(B):
        kind = b % 7
        x = rng.standard_normal(ld).astype(np.float32)
        if kind == 1:
            x = np.round(x * 8.0) / 8.0
        elif kind == 2:
            x = (rng.exponential(size=ld) * (rng.random(ld) < 0.2)).astype(np.float32)
        elif kind == 3:
            x[::7] = -0.0
            x[::11] = 0.0
            x[::13] = -np.inf
        elif kind == 4:
            x = rng.integers(0, 4, ld).astype(np.float32)
        elif kind == 5:
            x += np.linspace(0.0, 6.0, ld, dtype=np.float32)
        elif kind == 6 and b == 6:
            x[:] = 2.5
        S[b] = x
    bt = tis.Batch(np.array(lens, np.int32), np.arange(B + 1, dtype=np.int32),
                   np.zeros((B, -(-ld // 64)), np.int32), 1)
    scores = torch.from_numpy(S).cuda()
    for K in (1, 100, 2048, 4096):
        note(f"case Top-K on streamed rows, K={K}")
        idx = torch.full((B, K), -7, dtype=torch.int32, device="cuda")
        val = torch.full((B, K), 7.0, dtype=torch.float32, device="cuda")
        tis.topk_select(bt, scores, K, idx, val)
        idx, val = idx.cpu().numpy(), val.cpu().numpy()
        for b in range(B):
            ref = topk_token(S[b, :lens[b]].astype(np.float64), K)[0]
            assert np.array_equal(idx[b], ref), (b, K)
            k = int((ref >= 0).sum())
            assert np.array_equal(val[b, :k], S[b, ref[:k]] + np.float32(0.0)), (b, K)


def test_fused_call_crafted_scores():
    """index_score_topk on crafted score rows made by the scorer itself: every key page holds
    the same codes, so a token's score at position s is the key scale of s times one per-token
    constant, and the scales shape the rows: one value everywhere (the short list overflows and
    the exact whole-row select runs), eight values (ties at the threshold), rising and falling
    ramps, mostly exact zeros, a row no longer than K, a 65536-position row (several
    workgroups per row) and one that ends one position into a 4096-position block.  Fused ==
    unfused bit for bit, every row equals the oracle's Top-K of the scores the scorer wrote,
    and those scores pass the score gate."""
    from oracle.method import topk_token
    lens = [32768, 32768, 32768, 32768, 20001, 1500, 65536, 4097]
    wl = synth.reduced(synth.workload(synth.DECODE32K), lens, [1] * len(lens))
    inp = synth.make(wl, "continuous")
    rng = np.random.default_rng(20261204)
    inp.k_pool = np.ascontiguousarray(
        np.broadcast_to(inp.k_pool[inp.page_table[0, 0]], inp.k_pool.shape))
    ks = inp.k_scale.copy()
    for b, n in enumerate(lens):
        pos = np.arange(n)
        v = {0: np.full(n, 0.75), 1: rng.integers(1, 9, n) / 8.0,
             2: np.linspace(0.5, 2.0, n), 3: np.linspace(2.0, 0.5, n),
             4: rng.exponential(size=n) * (rng.random(n) < 0.05)}.get(b)
        if v is None:
            v = rng.exponential(size=n) + 0.01
        ks[inp.page_table[b, pos // 64], pos % 64] = v.astype(np.float32)
    inp.k_scale = ks
    note(f"case fused call on crafted score rows T={inp.T}")
    r = run_path(inp)
    assert np.array_equal(r.idx, r.idx2), "fused vs unfused Top-K"
    assert np.array_equal(r.val, r.val2), "fused vs unfused Top-K values"
    K = inp.wl.shape.K
    for t, n in enumerate(lens):
        ref = topk_token(r.scores[t, :n].astype(np.float64), K)[0]
        assert np.array_equal(r.idx[t], ref), t
        k = int((ref >= 0).sum())
        assert np.array_equal(r.val[t, :k], r.scores[t, ref[:k]]), t
    check_scores(inp, Oracle(inp), r.scores, [0, 1, 4, 5, 7])


@pytest.mark.parametrize("lens", [[40000, 5000], [8000, 3000, 12000]])
def test_graph_capture_replays(lens):
    """The fused selection and the attention call captured in a HIP graph: every replay, with
    eager calls and synchronisations in between, equals the eager result bit for bit (the path
    allocates nothing and clears memory with kernels, not memsets).  [40000, 5000] takes the
    several-workgroups-per-row selection."""
    import top_indexed_sparse_amd as tis
    wl = synth.reduced(synth.workload(synth.DECODE32K), lens, [1] * len(lens))
    inp = synth.make(wl, "continuous")
    note(f"case graph capture, lens {lens}")
    sh, K, T = wl.shape, wl.shape.K, inp.T
    d = to_device(inp)
    bt = tis.Batch(inp.seq_lens, inp.cu_q, inp.page_table, inp.n_pages)
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    val = torch.empty((T, K), dtype=torch.float32, device="cuda")
    out = torch.empty((T, sh.H, sh.D_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, sh.H), dtype=torch.float32, device="cuda")
    ws_i = torch.empty(max(1, tis.index_score_topk_workspace_size(bt, sh.H_I, sh.D_I, K)),
                       dtype=torch.uint8, device="cuda")
    ws_a = torch.empty(max(1, tis.sparse_mla_attn_workspace_size(bt, K, sh.H, sh.D_qk, sh.D_v,
                                                                 tis.TIS_BF16)),
                       dtype=torch.uint8, device="cuda")

    def step():
        tis.index_score_topk(bt, d.q_idx, d.w, d.k_pool, d.k_scale, K, idx, val, ws=ws_i)
        tis.sparse_mla_attn(bt, d.q, d.kv_pool, d.kv_scale, idx, sh.softmax_scale, out, lse,
                            ws=ws_a)

    step()
    torch.cuda.synchronize()
    ref = [x.clone() for x in (idx, val, out, lse)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        idx.fill_(-5)
        val.zero_()
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for x, y in zip((idx, val, out, lse), ref):
            assert torch.equal(x, y), f"replay {rep} differs"
        step()  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("mode", ["continuous", "exact"])
def test_decode32k_full_size(mode):
    """The benchmarked workload itself: 32 x 32768, K = 2048, bf16 latent cache (exact mode:
    integer scores, Top-K bit-exact)."""
    inp = synth.make(synth.workload(synth.DECODE32K), mode)
    note(f"case decode32k full size, {mode}")
    r = run_path(inp)
    _common(inp, r, list(range(inp.T)), mode == "exact")


def _full_size(cfg, n_sample, mode="continuous"):
    """A workload at its full size: every token through the fused and unfused chains and the
    attention call (e4m3 caches: with a bf16 output, the benchmarked form, and with an fp32
    one); sampled tokens against the oracle (Top-K bit-exact in exact mode)."""
    wl = synth.workload(cfg, mode)
    note(f"case {wl.name} full size, {mode}: generating inputs")
    inp = synth.make(wl, mode)
    tokens = sample_tokens(inp, n_sample)
    note(f"case {wl.name} full size: T={inp.T} B={inp.B} max L={int(inp.seq_lens.max())}, "
         f"{len(tokens)} sampled tokens; running")
    outs = ["bf16", "f32"] if wl.shape.kv_fp8 else ["bf16"]
    r = run_path_sampled(inp, tokens, outs)
    note(f"case {wl.name} full size: checking against the oracle")
    assert r.fused_equal, "fused vs unfused Top-K"
    for name, a in r.att.items():
        assert a.out_finite and a.lse_finite, f"non-finite attention output ({name})"
    for t in tokens[:8]:
        sel = r.idx[t][r.idx[t] >= 0]
        assert np.array_equal(r.val[t][: sel.size], r.scores[t, sel]), t
    orc = Oracle(inp)
    serr = check_scores(inp, orc, r.scores, tokens)
    rec = check_topk(inp, orc, r.idx, tokens, mode == "exact")
    for name, a in r.att.items():
        aerr = check_attention(inp, orc, a, tokens)
        note(f"  {wl.name}/{mode}: score rel err {serr:.2e}, recall {rec}, {name} output: "
             f"attn err {aerr[0]:.2e}, lse err {aerr[1]:.2e}")
    if mode == "exact":
        assert serr == 0.0, "exact-mode scores must be exact"
    return inp, r, tokens


@pytest.mark.timeout(900)
@pytest.mark.parametrize("mode", ["continuous", "exact"])
def test_decode1m_full_size(mode):
    """4 x 1,048,576 context, e4m3 caches, planted blocks (continuous mode): every token
    checked.  Exact mode: integer scores with heavy ties, selected bit-exact."""
    inp, r, tokens = _full_size(synth.DECODE1M, 4, mode)
    assert tokens == list(range(inp.T))
    if mode == "exact":
        return
    for b in range(inp.B):
        off = inp.info["planted"][b]
        sel = r.idx[b][r.idx[b] >= 0]
        assert np.mean((sel >= off) & (sel < off + 4096)) > 0.5


@pytest.mark.timeout(900)
@pytest.mark.parametrize("mode", ["continuous", "exact"])
def test_prefill64k_full_size(mode):
    """One 65,536-token causal prefill, e4m3 latent cache with heavy rows (exact mode:
    integer scores, Top-K bit-exact on the sampled tokens)."""
    _full_size(synth.PREFILL64K, 96, mode)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("mode", ["continuous", "exact"])
def test_ragged_full_size(mode):
    """64 requests of 1K..256K context, 48 decoding and 16 in a 4096-token prefill slice,
    random page table over a poisoned pool (exact mode: Top-K bit-exact)."""
    _full_size(synth.RAGGED, 96, mode)


def test_tiny_query_heads():
    """Query heads whose largest |q_I| is below 2^-119 get a power-of-two scale below 2^-127
    (no reciprocal overflow: finite scores that match the oracle).  Token 0 has one such head,
    token 1 has all 64; their values stay in bf16's normal range."""
    from synth.gen import to_bf16_bits
    wl = synth.reduced(synth.workload(synth.DECODE32K), [3000, 2500, 4096], [1, 1, 1])
    inp = synth.make(wl, "continuous")
    qf = (inp.q_idx.astype(np.uint32) << 16).view(np.float32).copy()
    mag = np.float32(0.5) + np.abs(qf)                   # |q| >= 0.5 before scaling
    tiny = np.sign(qf) * mag * np.float32(2.0 ** -123)
    qf[0, 5] = tiny[0, 5]
    qf[1] = tiny[1]
    assert np.all(np.abs(qf[0, 5]) >= 2.0 ** -126) and np.all(np.abs(qf[1]) >= 2.0 ** -126)
    inp.q_idx = to_bf16_bits(qf)
    note("case tiny query heads")
    r = run_path(inp)
    assert np.all(np.isfinite(r.scores[0, :3000])) and np.all(np.isfinite(r.scores[1, :2500]))
    orc = Oracle(inp)
    serr = check_scores(inp, orc, r.scores, [0, 1, 2])
    check_topk(inp, orc, r.idx, [0, 1, 2], False)
    assert np.array_equal(r.idx, r.idx2)
    note(f"  tiny query heads: score rel err {serr:.2e}")
    assert serr < 1e-3


@pytest.mark.parametrize("mode", ["continuous", "exact"])
@pytest.mark.parametrize("shape", ["decode", "prefill"])
def test_bf16_query_mode(shape, mode):
    """TIS_QMODE_BF16: q_I as stored on bf16 matrix cores over the exactly widened e4m3 keys,
    against the oracle with no query quantisation (exact mode: scores and Top-K bit-exact);
    decode shapes (8-wave workgroups, one token each) and prefill shapes (four tokens per
    workgroup)."""
    import top_indexed_sparse_amd as tis
    if shape == "decode":
        wl = synth.reduced(synth.workload(synth.DECODE32K), [4096, 1500, 5000, 2049], [1, 1, 2, 1])
    else:
        wl = synth.reduced(synth.workload(synth.PREFILL64K), [2600], [2600])
    inp = synth.make(wl, mode)
    note(f"case bf16 query mode, {shape} shapes, mode={mode} T={inp.T}")
    r = run_path(inp, qmode=tis.TIS_QMODE_BF16)
    toks = list(range(inp.T)) if inp.T <= 64 else sample_tokens(inp, 100)
    serr = _common(inp, r, toks, mode == "exact", qmode="none")
    if mode == "exact":
        assert serr == 0.0
    else:
        assert serr < 1e-4
