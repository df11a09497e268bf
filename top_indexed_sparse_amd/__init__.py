"""MI355X-native indexer-driven Top-K sparse attention (libtopidx, gfx950).

The Python surface mirrors the C ABI in include/topidx.h one to one: index_score,
topk_select, index_score_topk (and its allocation-free variant), the block-granular
index_score_block / topk_block_select / index_score_topk_block, sparse_mla_attn and
cache_append, plus workspace-size queries.  All
computation happens in the HIP kernels of libtopidx.so."""
from ._lib import (Batch, TisError, cache_append, index_score, index_score_topk, index_score_topk_noalloc,
                   index_score_block, topk_block_select, topk_block_select_workspace_size,
                   index_score_topk_block, index_score_topk_block_workspace_size, blocks_of,
                   sparse_mla_attn_dense, sparse_mla_attn_dense_workspace_size,
                   index_score_topk_workspace_size,
                   lib, sparse_mla_attn, sparse_mla_attn_workspace_size, topk_select,
                   topk_select_workspace_size,
                   TIS_F32, TIS_BF16, TIS_E4M3, TIS_MXFP8, TIS_QMODE_FP8, TIS_QMODE_BF16,
                   TIS_QMODE_MXFP8, LIB_PATH, EXPORTS)

__all__ = ["Batch", "TisError", "cache_append", "index_score", "index_score_topk", "index_score_topk_noalloc",
           "index_score_block", "topk_block_select", "topk_block_select_workspace_size",
           "index_score_topk_block", "index_score_topk_block_workspace_size", "blocks_of",
           "sparse_mla_attn_dense", "sparse_mla_attn_dense_workspace_size",
           "index_score_topk_workspace_size", "lib", "sparse_mla_attn",
           "sparse_mla_attn_workspace_size", "topk_select", "topk_select_workspace_size",
           "TIS_F32", "TIS_BF16", "TIS_E4M3", "TIS_MXFP8", "TIS_QMODE_FP8", "TIS_QMODE_BF16",
           "TIS_QMODE_MXFP8", "LIB_PATH", "EXPORTS"]
