// Host-side launchers of the gfx950 kernels (internal to libtopidx).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"

namespace tis {

hipError_t launch_index_score_f32(const DevBatch& bt, int t_begin, int t_count, int max_n,
                                  const float* q, const float* w, const float* kpool, int H,
                                  int D, float* scores, int64_t ld, hipStream_t st);
// qmode: 0 = e4m3 query with per-head scales (per-token fp32 key scales), 1 = bf16 query
// (per-token fp32 key scales), 2 = MXFP8 query and keys (kscale: four scale bytes per key).
// block: one score per 64-key page (the largest causal key score) instead of one per key.
// np (decode only, 1..64): key pages per wave of a workgroup's chunk (512 * np keys).
hipError_t launch_index_score_fp8(const DevBatch& bt, int t_begin, int t_count, int max_n,
                                  bool prefill_like, int np, int qmode, bool block, const uint16_t* q_idx,
                                  const float* w, const uint8_t* kpool, const void* kscale,
                                  float* scores, int64_t ld, hipStream_t st);
hipError_t launch_topk(const DevBatch& bt, int t_begin, int t_count, int max_n,
                       const float* scores, int64_t ld, int K, int32_t* idx, float* val,
                       void* ws, hipStream_t st);
// workspace bytes of launch_topk over up to `rows` rows of up to max_n positions (0 when the
// selection needs none)
size_t topk_ws_bytes(int rows, int max_n, int K);
hipError_t launch_mla_attn_f32(const DevBatch& bt, int t_begin, int t_count, const float* q,
                               const float* kv, const int32_t* idx, int K, int H, int Dqk,
                               int Dv, float scale, float* out, float* lse, hipStream_t st);
hipError_t launch_mla_attn(const DevBatch& bt, int t_begin, int t_count, bool fp8,
                           const uint16_t* q, const uint8_t* kv, const float* kvscale,
                           const int32_t* idx, int K, float softmax_scale, int nsplit,
                           void* out, bool out_f32, float* lse, float* part_o, float* part_ml,
                           hipStream_t st, int dense_n = 0);
// topk_idx[t][64*i + r] = 64*block_idx[t][i] + r for causal positions of kept pages, else -1
hipError_t launch_expand_blocks(const DevBatch& bt, int t_begin, int t_count,
                                const int32_t* block_idx, int K_blocks, int32_t* topk_idx,
                                hipStream_t st);
int attn_split_count(int t_count, int K);
int attn_keys_per_split(int K, int nsplit);
size_t attn_smem_bytes(bool fp8, int kps);
// pool_fmt: 0 = bf16, 1 = e4m3 with one fp32 scale per token, 2 = MXFP8 (one scale byte per
// 32 elements)
hipError_t launch_cache_append(const DevBatch& bt, const void* rows, bool rows_bf16, int D,
                               void* pool, int pool_fmt, void* pool_scale, hipStream_t st);

}  // namespace tis
