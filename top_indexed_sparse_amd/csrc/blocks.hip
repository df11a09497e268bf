// Block-granular selection, last step: the kept pages of each token expanded to the positions
// the attention reads.
//
// Method: "Day-0 Adaptation for Trillion-Parameter Models" (the index selection returns
// blocks of the cache layout, which the attention then fetches whole) and "Achieving Day-0
// Readiness ... Million-Token Context", section 2.2 (the cache is cut into fixed-size blocks
// located through a block index table, so a block comes in through one indirect lookup).
// Here a block is a 64-position page; a kept page contributes its causal positions, the rest
// of its 64 entries (past the token's position) and every padding page's entries are -1,
// which the attention skips.
//
// One workgroup per token (its causal length is looked up once); consecutive threads write
// consecutive entries, four per thread as one 16-byte store.
#include "common.h"
#include "launch.h"

namespace tis {

__global__ __launch_bounds__(256) void expand_blocks_kernel(DevBatch bt, int t_begin,
    const int32_t* __restrict__ block_idx, int K_blocks, int32_t* __restrict__ topk_idx) {
  const int tl = blockIdx.x;
  const int t = t_begin + tl;
  __shared__ int n_sh;
  if (threadIdx.x < 64) {
    const TokLoc loc = locate(bt, t);  // (one wave, all of its lanes)
    if (threadIdx.x == 0) n_sh = loc.n;
  }
  __syncthreads();
  const int n = n_sh;
  const int32_t* bi = block_idx + (int64_t)t * K_blocks;
  int4* out = (int4*)(topk_idx + (int64_t)t * K_blocks * kPage);
  const int nq = K_blocks * (kPage / 4);  // 16-byte pieces of the row
  for (int q = threadIdx.x; q < nq; q += blockDim.x) {
    const int i = q >> 4;                 // the page entry
    const int r = (q & 15) * 4;           // its first position within the page
    const int b = bi[i];
    int v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int pos = b * kPage + r + e;
      v[e] = (b >= 0 && pos < n) ? pos : -1;
    }
    out[q] = make_int4(v[0], v[1], v[2], v[3]);
  }
}

hipError_t launch_expand_blocks(const DevBatch& bt, int t_begin, int t_count,
                                const int32_t* block_idx, int K_blocks, int32_t* topk_idx,
                                hipStream_t st) {
  if (t_count < 1) return hipSuccess;
  hipLaunchKernelGGL(expand_blocks_kernel, dim3(t_count), dim3(256), 0, st, bt, t_begin,
                     block_idx, K_blocks, topk_idx);
  return hipGetLastError();
}

}  // namespace tis
