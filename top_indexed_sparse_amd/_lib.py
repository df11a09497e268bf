"""ctypes binding of libtopidx.so (include/topidx.h).  Argument marshalling only: every step
of the computation runs in the library's HIP kernels; PyTorch supplies device memory and the
current stream.  Raises if the library is not built."""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtopidx.so")

TIS_OK, TIS_ERR_INVALID, TIS_ERR_UNSUPPORTED, TIS_ERR_HIP = 0, 1, 2, 3
TIS_F32, TIS_BF16, TIS_E4M3, TIS_MXFP8 = 0, 1, 2, 3
TIS_QMODE_FP8, TIS_QMODE_BF16, TIS_QMODE_MXFP8 = 0, 1, 2
PAGE_SIZE = 64

EXPORTS = ("index_score", "topk_select", "index_score_topk", "index_score_topk_noalloc",
           "sparse_mla_attn", "cache_append",
           "index_score_block", "topk_block_select", "index_score_topk_block",
           "sparse_mla_attn_dense", "sparse_mla_attn_dense_workspace_size",
           "index_score_workspace_size", "topk_select_workspace_size",
           "index_score_topk_workspace_size", "sparse_mla_attn_workspace_size",
           "topk_block_select_workspace_size", "index_score_topk_block_workspace_size",
           "tis_last_error", "tis_abi_version")


class TisBatch(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32),
                ("seq_lens", ctypes.c_void_p), ("cu_q", ctypes.c_void_p),
                ("seq_lens_host", ctypes.c_void_p), ("cu_q_host", ctypes.c_void_p),
                ("page_table", ctypes.c_void_p), ("pt_stride", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("n_pages", ctypes.c_int32)]


class TisError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"status {status}: {msg}")
        self.status = status


_lib = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_F = ctypes.c_float
_BP = ctypes.POINTER(TisBatch)


def lib():
    """Load libtopidx.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m top_indexed_sparse_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    L.tis_abi_version.restype = _I32
    L.tis_last_error.restype = ctypes.c_char_p
    L.index_score.argtypes = [_BP, _P, _I32, _P, _P, _I32, _P, _I32, _I32, _I32, _P, _I64, _P,
                              _SZ, _P]
    L.topk_select.argtypes = [_BP, _P, _I64, _I32, _P, _P, _P, _SZ, _P]
    L.index_score_topk.argtypes = [_BP, _P, _I32, _P, _P, _I32, _P, _I32, _I32, _I32, _I32, _P,
                                   _P, _P, _SZ, _P]
    L.index_score_topk_noalloc.argtypes = [_BP, _P, _I32, _P, _P, _I32, _P, _I32, _I32, _I32,
                                           _I32, _P, _P, _P]
    L.sparse_mla_attn.argtypes = [_BP, _P, _I32, _P, _I32, _P, _P, _I32, _I32, _I32, _I32, _F,
                                  _P, _I32, _P, _P, _SZ, _P]
    L.cache_append.argtypes = [_BP, _P, _I32, _I32, _P, _I32, _P, _P]
    L.sparse_mla_attn_dense.argtypes = [_BP, _P, _I32, _P, _I32, _P, _P, _I32, _I32, _I32,
                                        _I32, _F, _P, _I32, _P, _P, _SZ, _P]
    L.sparse_mla_attn_dense_workspace_size.argtypes = [_BP, _I32, _I32, _I32, _I32, _I32]
    L.sparse_mla_attn_dense_workspace_size.restype = _SZ
    L.index_score_block.argtypes = [_BP, _P, _I32, _P, _P, _I32, _P, _I32, _I32, _I32, _P, _I64,
                                    _P]
    L.topk_block_select.argtypes = [_BP, _P, _I64, _I32, _P, _P, _P, _P, _SZ, _P]
    L.index_score_topk_block.argtypes = [_BP, _P, _I32, _P, _P, _I32, _P, _I32, _I32, _I32,
                                         _I32, _P, _P, _P, _P, _SZ, _P]
    for f in ("index_score", "topk_select", "index_score_topk", "index_score_topk_noalloc",
              "sparse_mla_attn", "cache_append", "index_score_block", "topk_block_select",
              "index_score_topk_block", "sparse_mla_attn_dense"):
        getattr(L, f).restype = _I32
    L.index_score_workspace_size.argtypes = [_BP, _I32, _I32]
    L.topk_select_workspace_size.argtypes = [_BP, _I32]
    L.index_score_topk_workspace_size.argtypes = [_BP, _I32, _I32, _I32]
    L.sparse_mla_attn_workspace_size.argtypes = [_BP, _I32, _I32, _I32, _I32, _I32]
    L.topk_block_select_workspace_size.argtypes = [_BP, _I32]
    L.index_score_topk_block_workspace_size.argtypes = [_BP, _I32, _I32, _I32]
    for f in ("index_score_workspace_size", "topk_select_workspace_size",
              "index_score_topk_workspace_size", "sparse_mla_attn_workspace_size",
              "topk_block_select_workspace_size", "index_score_topk_block_workspace_size"):
        getattr(L, f).restype = _SZ
    if L.tis_abi_version() != 6:
        raise RuntimeError("libtopidx ABI version mismatch")
    _lib = L
    return L


def _check(status: int):
    if status != TIS_OK:
        raise TisError(status, lib().tis_last_error().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dtype(t) -> int:
    if t.dtype == torch.float32:
        return TIS_F32
    if t.dtype == torch.bfloat16:
        return TIS_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return TIS_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _cache_dtype(pool, scale) -> int:
    """A cache's format: uint8 codes with uint8 scale bytes are MXFP8, with fp32 scales e4m3."""
    if pool.dtype == torch.uint8 and scale is not None and scale.dtype == torch.uint8:
        return TIS_MXFP8
    return _dtype(pool)


def _qmode(q_idx, k_dt, qmode):
    if qmode is not None:
        return qmode
    if q_idx.dtype == torch.float32:
        return TIS_QMODE_BF16
    return TIS_QMODE_MXFP8 if k_dt == TIS_MXFP8 else TIS_QMODE_FP8


def _stream():
    return torch.cuda.current_stream().cuda_stream


class Batch:
    """A ragged paged batch in the form the C ABI takes: device arrays plus host copies.

    seq_lens[B], cu_q[B+1] (host int arrays), page_table[B, pt_stride] (host or device),
    n_pages = pages in each cache pool."""

    def __init__(self, seq_lens, cu_q, page_table, n_pages: int, device="cuda"):
        self.seq_lens_h = np.ascontiguousarray(seq_lens, dtype=np.int32)
        self.cu_q_h = np.ascontiguousarray(cu_q, dtype=np.int32)
        self.seq_lens = torch.from_numpy(self.seq_lens_h).to(device)
        self.cu_q = torch.from_numpy(self.cu_q_h).to(device)
        if isinstance(page_table, torch.Tensor):
            self.page_table = page_table.to(device=device, dtype=torch.int32).contiguous()
        else:
            self.page_table = torch.from_numpy(np.ascontiguousarray(page_table, np.int32)).to(device)
        self.B = int(self.seq_lens_h.shape[0])
        self.T = int(self.cu_q_h[-1])
        self.n_pages = int(n_pages)
        self.c = TisBatch(self.B, self.T, self.seq_lens.data_ptr(), self.cu_q.data_ptr(),
                          self.seq_lens_h.ctypes.data, self.cu_q_h.ctypes.data,
                          self.page_table.data_ptr(), int(self.page_table.shape[1]), PAGE_SIZE,
                          self.n_pages)

    @property
    def ref(self):
        return ctypes.byref(self.c)

    @property
    def max_n(self) -> int:
        q = np.diff(self.cu_q_h)
        return int(self.seq_lens_h[q > 0].max())


def _ws(nbytes: int, ws, device):
    if nbytes == 0:
        return None, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"workspace needs {nbytes} bytes")
    return ws, ws.numel() * ws.element_size()


def index_score(batch: Batch, q_idx, w, k_pool, k_scale, scores, qmode=None):
    """scores[t, s] for s <= p_t (see index_score in topidx.h).  Keys are MXFP8 when k_scale
    holds uint8 scale bytes; qmode defaults to the key format's quantised mode."""
    H_I, D_I = int(q_idx.shape[1]), int(q_idx.shape[2])
    kd = _cache_dtype(k_pool, k_scale)
    qmode = _qmode(q_idx, kd, qmode)
    _check(lib().index_score(batch.ref, _ptr(q_idx), _dtype(q_idx), _ptr(w), _ptr(k_pool),
                             kd, _ptr(k_scale), H_I, D_I, qmode, _ptr(scores),
                             int(scores.stride(0)), None, 0, _stream()))
    return scores


def topk_select_workspace_size(batch: Batch, K: int) -> int:
    return int(lib().topk_select_workspace_size(batch.ref, int(K)))


def topk_select(batch: Batch, scores, K: int, topk_idx, topk_val=None, ws=None):
    need = topk_select_workspace_size(batch, K)
    ws, nb = _ws(need, ws, scores.device)
    _check(lib().topk_select(batch.ref, _ptr(scores), int(scores.stride(0)), int(K),
                             _ptr(topk_idx), _ptr(topk_val), _ptr(ws), nb, _stream()))
    return topk_idx


def index_score_topk_workspace_size(batch: Batch, H_I: int, D_I: int, K: int) -> int:
    return int(lib().index_score_topk_workspace_size(batch.ref, H_I, D_I, int(K)))


def index_score_topk(batch: Batch, q_idx, w, k_pool, k_scale, K: int, topk_idx, topk_val=None,
                     ws=None, qmode=None):
    H_I, D_I = int(q_idx.shape[1]), int(q_idx.shape[2])
    kd = _cache_dtype(k_pool, k_scale)
    qmode = _qmode(q_idx, kd, qmode)
    need = index_score_topk_workspace_size(batch, H_I, D_I, K)
    ws, nb = _ws(need, ws, q_idx.device)
    _check(lib().index_score_topk(batch.ref, _ptr(q_idx), _dtype(q_idx), _ptr(w), _ptr(k_pool),
                                  kd, _ptr(k_scale), H_I, D_I, qmode, int(K),
                                  _ptr(topk_idx), _ptr(topk_val), _ptr(ws), nb, _stream()))
    return topk_idx


def index_score_topk_noalloc(batch: Batch, q_idx, w, k_pool, k_scale, K: int, topk_idx,
                             topk_val=None, qmode=None):
    """index_score_topk with the library's own per-device scratch (allocates nothing)."""
    H_I, D_I = int(q_idx.shape[1]), int(q_idx.shape[2])
    kd = _cache_dtype(k_pool, k_scale)
    qmode = _qmode(q_idx, kd, qmode)
    _check(lib().index_score_topk_noalloc(batch.ref, _ptr(q_idx), _dtype(q_idx), _ptr(w),
                                          _ptr(k_pool), kd, _ptr(k_scale), H_I, D_I,
                                          qmode, int(K), _ptr(topk_idx), _ptr(topk_val),
                                          _stream()))
    return topk_idx


def sparse_mla_attn_workspace_size(batch: Batch, K: int, H: int, D_qk: int, D_v: int,
                                   kv_dtype: int) -> int:
    return int(lib().sparse_mla_attn_workspace_size(batch.ref, int(K), H, D_qk, D_v, kv_dtype))


def sparse_mla_attn(batch: Batch, q, kv_pool, kv_scale, topk_idx, softmax_scale: float, out,
                    lse=None, ws=None):
    H, D_qk = int(q.shape[1]), int(q.shape[2])
    D_v = int(out.shape[2])
    K = int(topk_idx.shape[1])
    kvd = _dtype(kv_pool)
    need = sparse_mla_attn_workspace_size(batch, K, H, D_qk, D_v, kvd)
    ws, nb = _ws(need, ws, q.device)
    _check(lib().sparse_mla_attn(batch.ref, _ptr(q), _dtype(q), _ptr(kv_pool), kvd,
                                 _ptr(kv_scale), _ptr(topk_idx), K, H, D_qk, D_v,
                                 float(softmax_scale), _ptr(out), _dtype(out), _ptr(lse),
                                 _ptr(ws), nb, _stream()))
    return out


def cache_append(batch: Batch, rows, pool, pool_scale=None):
    """Write rows [T][D] (fp32 or bf16) of the batch's query tokens into their slots of a paged
    cache pool [n_pages][64][D] (uint8 e4m3 codes with pool_scale [n_pages][64] fp32, uint8
    MXFP8 codes with pool_scale [n_pages][64][D/32] uint8, or bf16 with pool_scale None)."""
    D = int(rows.shape[-1])
    _check(lib().cache_append(batch.ref, _ptr(rows), _dtype(rows), D, _ptr(pool),
                              _cache_dtype(pool, pool_scale), _ptr(pool_scale), _stream()))
    return pool


def blocks_of(n: int) -> int:
    """Blocks (64-position pages) of a causal range of n positions."""
    return -(-int(n) // PAGE_SIZE)


def index_score_block(batch: Batch, q_idx, w, k_pool, k_scale, block_scores, qmode=None):
    """block_scores[t, j]: the largest score of token t over the causal positions of page j
    (see index_score_block in topidx.h)."""
    H_I, D_I = int(q_idx.shape[1]), int(q_idx.shape[2])
    kd = _cache_dtype(k_pool, k_scale)
    qmode = _qmode(q_idx, kd, qmode)
    _check(lib().index_score_block(batch.ref, _ptr(q_idx), _dtype(q_idx), _ptr(w), _ptr(k_pool),
                                   kd, _ptr(k_scale), H_I, D_I, qmode, _ptr(block_scores),
                                   int(block_scores.stride(0)), _stream()))
    return block_scores


def topk_block_select_workspace_size(batch: Batch, K_blocks: int) -> int:
    return int(lib().topk_block_select_workspace_size(batch.ref, int(K_blocks)))


def topk_block_select(batch: Batch, block_scores, K_blocks: int, block_idx, block_val=None,
                      topk_idx=None, ws=None):
    """The K_blocks best pages per token (block_idx), optionally expanded to the positions
    the attention reads (topk_idx [T][64 * K_blocks])."""
    need = topk_block_select_workspace_size(batch, K_blocks)
    ws, nb = _ws(need, ws, block_scores.device)
    _check(lib().topk_block_select(batch.ref, _ptr(block_scores), int(block_scores.stride(0)),
                                   int(K_blocks), _ptr(block_idx), _ptr(block_val),
                                   _ptr(topk_idx), _ptr(ws), nb, _stream()))
    return block_idx


def index_score_topk_block_workspace_size(batch: Batch, H_I: int, D_I: int, K_blocks: int) -> int:
    return int(lib().index_score_topk_block_workspace_size(batch.ref, H_I, D_I, int(K_blocks)))


def index_score_topk_block(batch: Batch, q_idx, w, k_pool, k_scale, K_blocks: int, block_idx,
                           block_val=None, topk_idx=None, ws=None, qmode=None):
    """index_score_block + topk_block_select in one call (block scores in the workspace)."""
    H_I, D_I = int(q_idx.shape[1]), int(q_idx.shape[2])
    kd = _cache_dtype(k_pool, k_scale)
    qmode = _qmode(q_idx, kd, qmode)
    need = index_score_topk_block_workspace_size(batch, H_I, D_I, K_blocks)
    ws, nb = _ws(need, ws, q_idx.device)
    _check(lib().index_score_topk_block(batch.ref, _ptr(q_idx), _dtype(q_idx), _ptr(w),
                                        _ptr(k_pool), kd, _ptr(k_scale), H_I, D_I, qmode,
                                        int(K_blocks), _ptr(block_idx), _ptr(block_val),
                                        _ptr(topk_idx), _ptr(ws), nb, _stream()))
    return block_idx


def sparse_mla_attn_dense_workspace_size(batch: Batch, K: int, H: int, D_qk: int, D_v: int,
                                         kv_dtype: int) -> int:
    return int(lib().sparse_mla_attn_dense_workspace_size(batch.ref, int(K), H, D_qk, D_v,
                                                          kv_dtype))


def sparse_mla_attn_dense(batch: Batch, q, kv_pool, kv_scale, topk_idx, softmax_scale: float,
                          out, lse=None, ws=None):
    """sparse_mla_attn computed the dense-masked way (every causal row read and multiplied,
    the selection as a mask)."""
    H, D_qk = int(q.shape[1]), int(q.shape[2])
    D_v = int(out.shape[2])
    K = int(topk_idx.shape[1])
    kvd = _dtype(kv_pool)
    need = sparse_mla_attn_dense_workspace_size(batch, K, H, D_qk, D_v, kvd)
    ws, nb = _ws(need, ws, q.device)
    _check(lib().sparse_mla_attn_dense(batch.ref, _ptr(q), _dtype(q), _ptr(kv_pool), kvd,
                                       _ptr(kv_scale), _ptr(topk_idx), K, H, D_qk, D_v,
                                       float(softmax_scale), _ptr(out), _dtype(out), _ptr(lse),
                                       _ptr(ws), nb, _stream()))
    return out
