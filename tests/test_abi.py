"""The C ABI library on the CPU: it loads, exports every symbol include/topidx.h declares,
and rejects bad arguments on the host before any launch (no GPU calls are made)."""
import ctypes
import os
import re
import struct
import subprocess
import tempfile

import numpy as np
import pytest

import top_indexed_sparse_amd as tis
from top_indexed_sparse_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "topidx.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(\w+)\s*\(", src)) - {"if", "sizeof"})


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(L.EXPORTS), names
    lib = tis.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert lib.tis_abi_version() == 6


LLVM = "/opt/rocm/llvm/bin"


def _device_kernel_names(lib_path):
    """Kernel symbols of every gfx950 code object in the library's offload bundles (one bundle
    per source file in the .hip_fatbin section)."""
    with tempfile.TemporaryDirectory() as d:
        fat = os.path.join(d, "fat.bin")
        subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section",
                        f".hip_fatbin={fat}", lib_path, os.path.join(d, "copy.so")], check=True)
        data = open(fat, "rb").read()
        names = set()
        magic = b"__CLANG_OFFLOAD_BUNDLE__"
        for i, m in enumerate(re.finditer(re.escape(magic), data)):
            st = m.start()
            n = struct.unpack_from("<Q", data, st + 24)[0]
            p = st + 32
            for _ in range(n):
                off, size, tl = struct.unpack_from("<QQQ", data, p)
                triple = data[p + 24:p + 24 + tl].decode()
                p += 24 + tl
                if triple.endswith("gfx950"):
                    obj = os.path.join(d, f"dev{i}.o")
                    open(obj, "wb").write(data[st + off:st + off + size])
                    out = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "--symbols",
                                          "--wide", obj], capture_output=True, text=True,
                                         check=True).stdout
                    names |= set(re.findall(r"(_ZN3tis\S+)\.kd\b", out))
        return names


def _registered_kernel_names(lib_path):
    """Mangled kernel names the host side registers (string literals in .rodata)."""
    out = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "-p", ".rodata", lib_path],
                         capture_output=True, text=True, check=True).stdout
    return set(re.findall(r"\]\s+(_ZN3tis\S+)", out))


def test_registered_kernels_exist_in_the_code_object():
    """Every kernel the host registers by mangled name exists in the gfx950 code objects, and
    the other way round.  A name that the host and device compilation passes mangle
    differently (e.g. a kernel signature naming a type that depends on an unnamed enum) leaves
    the launch without a kernel, and the runtime aborts the process at its first launch."""
    tools = ("llvm-objcopy", "llvm-readelf")
    if not all(os.path.exists(os.path.join(LLVM, t)) for t in tools):
        pytest.skip("ROCm llvm tools not found")
    host = _registered_kernel_names(L.LIB_PATH)
    dev = _device_kernel_names(L.LIB_PATH)
    assert len(host) >= 20
    assert host == dev, (sorted(host - dev), sorted(dev - host))


class FakeBatch:
    """Host-side view of a batch with dummy (never dereferenced) device pointers."""

    def __init__(self, seq_lens, cu_q, pt_stride=None, page_size=64, n_pages=100):
        self.sl = np.asarray(seq_lens, np.int32)
        self.cq = np.asarray(cu_q, np.int32)
        stride = pt_stride or max(1, -(-int(self.sl.max()) // 64))
        dummy = 0x100000
        self.c = L.TisBatch(len(self.sl), int(self.cq[-1]), dummy, dummy, self.sl.ctypes.data,
                            self.cq.ctypes.data, dummy, stride, page_size, n_pages)

    @property
    def ref(self):
        return ctypes.byref(self.c)


D = 0x200000  # dummy 16-byte aligned "device" address, never touched on error paths


def call_index(b, **kw):
    a = dict(q=D, qdt=L.TIS_BF16, w=D, k=D, kdt=L.TIS_E4M3, ks=D, H=64, Dd=128,
             qm=L.TIS_QMODE_FP8, sc=D, ld=1024)
    a.update(kw)
    return tis.lib().index_score(b.ref, a["q"], a["qdt"], a["w"], a["k"], a["kdt"], a["ks"],
                                 a["H"], a["Dd"], a["qm"], a["sc"], a["ld"], None, 0, None)


def call_attn(b, **kw):
    a = dict(q=D, qdt=L.TIS_BF16, kv=D, kvdt=L.TIS_BF16, kvs=None, idx=D, K=64, H=128, Dqk=576,
             Dv=512, scale=0.1, out=D, odt=L.TIS_BF16, ws=None, wsb=0)
    a.update(kw)
    return tis.lib().sparse_mla_attn(b.ref, a["q"], a["qdt"], a["kv"], a["kvdt"], a["kvs"],
                                     a["idx"], a["K"], a["H"], a["Dqk"], a["Dv"], a["scale"],
                                     a["out"], a["odt"], None, a["ws"], a["wsb"], None)


def last_error():
    return tis.lib().tis_last_error().decode()


def test_batch_validation():
    lib = tis.lib()
    assert lib.index_score(None, D, 1, D, D, 2, D, 64, 128, 0, D, 1024, None, 0, None) == 1
    assert "NULL" in last_error()
    bad = [
        FakeBatch([100], [0, 1], page_size=32),              # page size must be 64
        FakeBatch([100], [1, 2]),                            # cu_q[0] != 0
        FakeBatch([100, 50], [0, 3, 2]),                     # decreasing cu_q
        FakeBatch([2], [0, 3]),                              # more queries than positions
        FakeBatch([1000], [0, 1], pt_stride=2),              # page table too narrow
        FakeBatch([(1 << 28) + 1], [0, 1]),                  # longer than 2^28 positions
        FakeBatch([1000], [0, 1], n_pages=(1 << 24) + 1),    # more than 2^24 pages
    ]
    for b in bad:
        assert call_index(b) == L.TIS_ERR_INVALID, last_error()
    # the largest sizes themselves pass the batch check (seen through a size query, which
    # launches nothing: 0 would mean a rejected batch)
    big = FakeBatch([1 << 28], [0, 1], n_pages=1 << 24)
    assert lib.topk_select_workspace_size(big.ref, 2048) > 0
    for b in bad[-2:]:
        assert lib.topk_select_workspace_size(b.ref, 2048) == 0


def test_index_argument_validation():
    b = FakeBatch([1000, 600], [0, 1, 3])
    assert call_index(b, ld=999) == L.TIS_ERR_INVALID         # ld < max seq len
    assert call_index(b, ld=1002) == L.TIS_ERR_INVALID        # ld not a multiple of 4
    assert call_index(b, q=D + 4) == L.TIS_ERR_INVALID        # misaligned
    assert call_index(b, ks=None) == L.TIS_ERR_INVALID        # e4m3 keys need scales
    assert call_index(b, H=32) == L.TIS_ERR_UNSUPPORTED
    assert call_index(b, qdt=L.TIS_F32) == L.TIS_ERR_UNSUPPORTED
    assert call_index(b, qdt=L.TIS_F32, kdt=L.TIS_F32, qm=L.TIS_QMODE_BF16, ks=None, H=64,
                      Dd=256) == L.TIS_ERR_UNSUPPORTED   # 64*256 > 8192
    lib = tis.lib()
    assert lib.topk_select(b.ref, D, 1024, 0, D, None, None, 0, None) == L.TIS_ERR_INVALID
    assert lib.topk_select(b.ref, D, 1000, 10, None, None, None, 0, None) == L.TIS_ERR_INVALID
    need = lib.index_score_topk_workspace_size(b.ref, 64, 128, 16)
    assert need == 12032                 # T=3 rows of ld=1000 scores, rounded up to 256 bytes
    assert lib.index_score_topk(b.ref, D, L.TIS_BF16, D, D, L.TIS_E4M3, D, 64, 128,
                                L.TIS_QMODE_FP8, 16, D, None, D, need - 1, None) == L.TIS_ERR_INVALID
    assert "workspace" in last_error()


def test_long_row_selection_workspace():
    """Few tokens over rows longer than 32768 positions are selected by several workgroups per
    row, through a workspace that the size query reports and the call checks."""
    lib = tis.lib()
    b = FakeBatch([40000, 1000], [0, 1, 2])
    need = lib.topk_select_workspace_size(b.ref, 2048)
    # per row: 8192 (key, position) candidates, state (16 bytes), (offset, count) of each
    # 16384-position slice
    assert need == 2 * (8 * 8192 + 16 + 8 * 3)
    assert lib.topk_select_workspace_size(b.ref, 5000) == 0           # K above 4096
    assert lib.topk_select_workspace_size(FakeBatch([30000], [0, 1]).ref, 2048) == 0
    assert lib.topk_select(b.ref, D, 40000, 2048, D, None, D, need - 1, None) == L.TIS_ERR_INVALID
    assert "workspace" in last_error()
    assert lib.topk_select(b.ref, D, 40000, 2048, D, None, None, need, None) == L.TIS_ERR_INVALID
    fused = lib.index_score_topk_workspace_size(b.ref, 64, 128, 2048)
    assert fused == 2 * 40000 * 4 + need  # two score rows (256-byte multiple) + the selection's


def test_attention_argument_validation():
    b = FakeBatch([1000], [0, 32])
    assert call_attn(b, Dv=600) == L.TIS_ERR_INVALID
    assert call_attn(b, K=0) == L.TIS_ERR_INVALID
    assert call_attn(b, scale=float("nan")) == L.TIS_ERR_INVALID
    assert call_attn(b, kvdt=L.TIS_E4M3) == L.TIS_ERR_INVALID      # needs kv_scale
    assert call_attn(b, kvs=D) == L.TIS_ERR_INVALID                # bf16 takes no scale
    assert call_attn(b, H=64) == L.TIS_ERR_UNSUPPORTED
    assert call_attn(b, qdt=L.TIS_F32) == L.TIS_ERR_UNSUPPORTED    # fp32 q, bf16 cache
    need = tis.lib().sparse_mla_attn_workspace_size(b.ref, 64, 128, 576, 512, L.TIS_BF16)
    if need:
        assert call_attn(b, ws=D, wsb=need - 16) == L.TIS_ERR_INVALID
    # tiny fp32 path needs no workspace
    assert tis.lib().sparse_mla_attn_workspace_size(b.ref, 64, 8, 80, 64, L.TIS_F32) == 0


def test_noalloc_rejects_rows_beyond_its_scratch():
    """index_score_topk_noalloc holds a 64 MiB scratch per device: a batch whose score row
    does not fit is rejected on the host, before the scratch is looked up or anything runs."""
    lib = tis.lib()
    b = FakeBatch([20_000_000], [0, 1])
    st = lib.index_score_topk_noalloc(b.ref, D, L.TIS_BF16, D, D, L.TIS_E4M3, D, 64, 128,
                                      L.TIS_QMODE_FP8, 2048, D, None, None)
    assert st == L.TIS_ERR_INVALID and "scratch" in last_error()
    # argument errors come first, as for index_score_topk
    assert lib.index_score_topk_noalloc(b.ref, D, L.TIS_BF16, D, D, L.TIS_E4M3, D, 64, 128,
                                        L.TIS_QMODE_FP8, 0, D, None, None) == L.TIS_ERR_INVALID


def test_query_modes():
    """The three indexer query modes of the header: FP8 (dynamic e4m3 query) = 0, BF16 (the
    query as stored) = 1 and MXFP8 (group-32 scales, with MXFP8 keys) = 2; combinations
    outside the supported ones are refused on the host."""
    src = open(os.path.join(ROOT, "include", "topidx.h")).read()
    assert re.search(r"TIS_QMODE_FP8\s*=\s*0", src) and re.search(r"TIS_QMODE_BF16\s*=\s*1", src)
    assert re.search(r"TIS_QMODE_MXFP8\s*=\s*2", src) and re.search(r"TIS_MXFP8\s*=\s*3", src)
    assert (L.TIS_QMODE_FP8, L.TIS_QMODE_BF16, L.TIS_QMODE_MXFP8) == (0, 1, 2)
    assert L.TIS_MXFP8 == 3
    b = FakeBatch([1000, 600], [0, 1, 3])
    # fp32 queries and keys: only "as stored"
    assert call_index(b, qdt=L.TIS_F32, kdt=L.TIS_F32, qm=L.TIS_QMODE_FP8, ks=None, H=4,
                      Dd=32) == L.TIS_ERR_UNSUPPORTED
    assert call_index(b, qm=7) == L.TIS_ERR_UNSUPPORTED
    assert call_index(b, qm=L.TIS_QMODE_BF16, H=32) == L.TIS_ERR_UNSUPPORTED
    assert call_index(b, qm=L.TIS_QMODE_BF16, ks=None) == L.TIS_ERR_INVALID
    # MXFP8 queries go with MXFP8 keys only, and MXFP8 keys with MXFP8 queries only
    assert call_index(b, qm=L.TIS_QMODE_MXFP8) == L.TIS_ERR_UNSUPPORTED          # e4m3 keys
    assert call_index(b, kdt=L.TIS_MXFP8) == L.TIS_ERR_UNSUPPORTED               # FP8 query
    assert call_index(b, kdt=L.TIS_MXFP8, qm=L.TIS_QMODE_BF16) == L.TIS_ERR_UNSUPPORTED
    assert call_index(b, kdt=L.TIS_MXFP8, qm=L.TIS_QMODE_MXFP8, ks=None) == L.TIS_ERR_INVALID
    assert call_index(b, kdt=L.TIS_MXFP8, qm=L.TIS_QMODE_MXFP8, ks=D + 4) == L.TIS_ERR_INVALID
    assert call_index(b, kdt=L.TIS_MXFP8, qm=L.TIS_QMODE_MXFP8, H=32) == L.TIS_ERR_UNSUPPORTED
    # the attention call takes no MXFP8 cache
    assert call_attn(FakeBatch([1000], [0, 32]), kvdt=L.TIS_MXFP8, kvs=D) == L.TIS_ERR_UNSUPPORTED


def test_cache_append_argument_validation():
    """cache_append: rows and pool set and aligned, D a multiple of 16 in [16, 2048], fp32 or
    bf16 rows, an e4m3 or MXFP8 cache with (a bf16 cache without) its scale array."""
    lib = tis.lib()
    b = FakeBatch([1000, 600], [0, 1, 3])

    def call(rows=D, rdt=L.TIS_F32, Dd=576, pool=D, pdt=L.TIS_E4M3, ps=D):
        return lib.cache_append(b.ref, rows, rdt, Dd, pool, pdt, ps, None)

    assert call(rows=None) == L.TIS_ERR_INVALID
    assert call(pool=D + 8) == L.TIS_ERR_INVALID
    assert call(Dd=100) == L.TIS_ERR_INVALID
    assert call(Dd=4096) == L.TIS_ERR_INVALID
    assert call(ps=None) == L.TIS_ERR_INVALID
    assert call(pdt=L.TIS_BF16) == L.TIS_ERR_INVALID          # bf16 cache takes no scale
    assert call(rdt=L.TIS_E4M3) == L.TIS_ERR_UNSUPPORTED
    assert call(pdt=L.TIS_F32, ps=None) == L.TIS_ERR_UNSUPPORTED
    # MXFP8 caches: scale bytes required, D a multiple of 32
    assert call(pdt=L.TIS_MXFP8, ps=None) == L.TIS_ERR_INVALID
    assert call(pdt=L.TIS_MXFP8, Dd=80) == L.TIS_ERR_INVALID
    assert "multiple of 32" in last_error()
    assert lib.cache_append(None, D, 0, 576, D, 2, D, None) == L.TIS_ERR_INVALID


def test_block_selection_argument_validation():
    """Block-granular calls: K_blocks >= 1, block_idx set, an aligned expansion buffer, block
    rows of at least ceil(n / 64) entries, matrix-core scorer only; the workspace queries
    follow the block row length."""
    lib = tis.lib()
    b = FakeBatch([1000, 600], [0, 1, 3])          # 16 blocks at most

    def sel(ld=16, K=4, bi=D, bv=None, ti=D, ws=None, wsb=0):
        return lib.topk_block_select(b.ref, D, ld, K, bi, bv, ti, ws, wsb, None)

    assert sel(K=0) == L.TIS_ERR_INVALID
    assert sel(bi=None) == L.TIS_ERR_INVALID
    assert sel(ti=D + 4) == L.TIS_ERR_INVALID
    assert sel(ld=12) == L.TIS_ERR_INVALID         # < 16 blocks
    assert sel(ld=18) == L.TIS_ERR_INVALID         # not a multiple of 4
    assert sel(K=(1 << 18) + 1) == L.TIS_ERR_INVALID
    assert lib.topk_block_select_workspace_size(b.ref, 4) == 0
    # a 3M-position row: 46,875 blocks, above the one-workgroup limit -> multi-workgroup rows
    big = FakeBatch([3_000_000], [0, 1])
    assert lib.topk_block_select_workspace_size(big.ref, 32) > 0

    def blk(**kw):
        a = dict(q=D, qdt=L.TIS_BF16, w=D, k=D, kdt=L.TIS_E4M3, ks=D, H=64, Dd=128,
                 qm=L.TIS_QMODE_FP8, sc=D, ld=16)
        a.update(kw)
        return lib.index_score_block(b.ref, a["q"], a["qdt"], a["w"], a["k"], a["kdt"], a["ks"],
                                     a["H"], a["Dd"], a["qm"], a["sc"], a["ld"], None)

    assert blk(ld=8) == L.TIS_ERR_INVALID
    assert blk(sc=D + 4) == L.TIS_ERR_INVALID
    assert blk(qdt=L.TIS_F32, kdt=L.TIS_F32, qm=L.TIS_QMODE_BF16, ks=None, H=4,
               Dd=32) == L.TIS_ERR_UNSUPPORTED
    need = lib.index_score_topk_block_workspace_size(b.ref, 64, 128, 4)
    assert need == 3 * 16 * 4 + (256 - 3 * 16 * 4 % 256) % 256   # T=3 rows of 16 block scores
    assert lib.index_score_topk_block(b.ref, D, L.TIS_BF16, D, D, L.TIS_E4M3, D, 64, 128,
                                      L.TIS_QMODE_FP8, 4, D, None, D, D, need - 1,
                                      None) == L.TIS_ERR_INVALID
    assert "workspace" in last_error()


def test_dense_attention_argument_validation():
    """sparse_mla_attn_dense: the attention call's argument checks, matrix-core shapes only, and
    a workspace for the split partials of long causal ranges."""
    lib = tis.lib()
    b = FakeBatch([9000], [0, 300])

    def call(**kw):
        a = dict(q=D, qdt=L.TIS_BF16, kv=D, kvdt=L.TIS_BF16, kvs=None, idx=D, K=64, H=128,
                 Dqk=576, Dv=512, scale=0.1, out=D, odt=L.TIS_BF16, ws=None, wsb=0)
        a.update(kw)
        return lib.sparse_mla_attn_dense(b.ref, a["q"], a["qdt"], a["kv"], a["kvdt"], a["kvs"],
                                         a["idx"], a["K"], a["H"], a["Dqk"], a["Dv"], a["scale"],
                                         a["out"], a["odt"], None, a["ws"], a["wsb"], None)

    assert call(Dv=600) == L.TIS_ERR_INVALID
    assert call(qdt=L.TIS_F32, kvdt=L.TIS_F32, odt=L.TIS_F32, H=8, Dqk=80,
                Dv=64) == L.TIS_ERR_UNSUPPORTED
    need = lib.sparse_mla_attn_dense_workspace_size(b.ref, 64, 128, 576, 512, L.TIS_BF16)
    assert need == 256 * 5 * 128 * 516 * 4          # chunks of 256 tokens, five 1,824-position splits
    assert call() == L.TIS_ERR_INVALID and "workspace" in last_error()
    short = FakeBatch([2000], [0, 300])
    assert lib.sparse_mla_attn_dense_workspace_size(short.ref, 64, 128, 576, 512,
                                                    L.TIS_BF16) == 0
