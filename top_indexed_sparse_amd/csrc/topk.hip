// Per-query Top-K over the scores of positions 0..p_t.
//
// Method: "Day 0 Support for New LLM Architectures", Step 1 and Key Optimization 1 (the
// Top-K positions of the indexer scores are selected on the device); "Achieving Day-0
// Readiness ... Million-Token Context" 2.1 (selection is an operator of its own, run on
// the GPU with the index kept resident).  Selection is exact: the k_t = min(K, n_t) largest
// scores under the total order (score descending, position ascending), -0.0 == +0.0,
// emitted in ascending position order and padded with -1.
//
// One 1024-thread workgroup per row.  Scores map to order-preserving uint32 keys.  The key
// range [kmin, kmax] of the row is measured first; radix select then walks the bits of
// (key - kmin) from the top in 11-bit digits, so the first digit already splits the
// occupied range into 2048 bins instead of spending it on the (nearly constant) sign and
// exponent bits.  Each pass histograms the elements that still match the selected prefix
// (LDS atomics) and picks the bin holding the k-th largest.  The result is a threshold key
// T and the number r of elements equal to T that are taken; the compaction keeps every
// element > T and the first r elements == T in position order, via two block scans.
// Each thread owns NPT consecutive positions per 1024*NPT chunk; rows that fit one chunk
// keep their keys in registers, longer rows are re-read per pass.
#include "common.h"
#include "launch.h"

namespace tis {

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0.0 ties with +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// Exclusive scan over the 1024 threads; `sh` holds >= 17 words.  Ends with a barrier.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh, uint32_t& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint32_t inc = wave_incl_scan(v, lane);
  if (lane == 63) sh[wid] = inc;
  __syncthreads();
  if (wid == 0) {
    uint32_t x = lane < 16 ? sh[lane] : 0u;
    uint32_t xi = wave_incl_scan(x, lane);
    if (lane < 16) sh[lane] = xi - x;
    if (lane == 15) sh[16] = xi;
  }
  __syncthreads();
  uint32_t r = sh[wid] + inc - v;
  total = sh[16];
  __syncthreads();
  return r;
}

__device__ __forceinline__ void block_minmax(uint32_t& mn, uint32_t& mx, uint32_t* sh) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor(mn, o));
    mx = max(mx, (uint32_t)__shfl_xor(mx, o));
  }
  if (lane == 0) { sh[wid] = mn; sh[16 + wid] = mx; }
  __syncthreads();
  if (wid == 0) {
    uint32_t a = lane < 16 ? sh[lane] : ~0u, c = lane < 16 ? sh[16 + lane] : 0u;
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) {
      a = min(a, (uint32_t)__shfl_xor(a, o));
      c = max(c, (uint32_t)__shfl_xor(c, o));
    }
    if (lane == 0) { sh[32] = a; sh[33] = c; }
  }
  __syncthreads();
  mn = sh[32];
  mx = sh[33];
  __syncthreads();
}

template <int NPT>
__global__ __launch_bounds__(1024) void topk_stream_kernel(DevBatch bt, int t_begin,
    const float* __restrict__ scores, int64_t ld, int K, int32_t* __restrict__ out_idx,
    float* __restrict__ out_val) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t sh[40];
  __shared__ uint32_t pick[2];
  const int tid = threadIdx.x;
  const int tl = blockIdx.x;
  const int t = t_begin + tl;
  const int n = locate(bt, t).n;
  const float* row = scores + (int64_t)tl * ld;
  int32_t* oi = out_idx + (int64_t)t * K;
  float* ov = out_val ? out_val + (int64_t)t * K : nullptr;

  if (n <= K) {  // everything is selected
    for (int i = tid; i < K; i += 1024) {
      oi[i] = i < n ? i : -1;
      if (ov) ov[i] = i < n ? row[i] : 0.f;
    }
    return;
  }
  const int k = K;
  constexpr int CH = 1024 * NPT;
  const bool cached = n <= CH;
  uint32_t key[NPT];

  auto load_chunk = [&](int c0) {
    const int p0 = c0 + tid * NPT;
#pragma unroll
    for (int j = 0; j < NPT; j += 4) {
      const int p = p0 + j;
      if (p + 3 < n) {
        float4 f = *(const float4*)(row + p);
        key[j] = order_key(f.x); key[j + 1] = order_key(f.y);
        key[j + 2] = order_key(f.z); key[j + 3] = order_key(f.w);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) key[j + e] = (p + e < n) ? order_key(row[p + e]) : 0u;
      }
    }
  };
  auto valid_count = [&](int c0) { return max(0, min(NPT, n - (c0 + tid * NPT))); };

  if (cached) load_chunk(0);

  // ---- key range of the row
  uint32_t kmin = ~0u, kmax = 0u;
  for (int c0 = 0; c0 < n; c0 += CH) {
    if (!cached) load_chunk(c0);
    const int nv = valid_count(c0);
#pragma unroll
    for (int j = 0; j < NPT; ++j)
      if (j < nv) { kmin = min(kmin, key[j]); kmax = max(kmax, key[j]); }
  }
  block_minmax(kmin, kmax, sh);
  const uint32_t span = kmax - kmin;
  int hi = span ? 32 - __clz(span) : 0;

  // ---- radix select on r = key - kmin, digits of up to 11 bits from bit `hi` down
  uint32_t prefix = 0u;
  uint32_t krem = (uint32_t)k;
  while (hi > 0) {
    const int lo = max(0, hi - 11);
    const uint32_t dmask = (1u << (hi - lo)) - 1u;
    hist[tid] = 0u;
    hist[tid + 1024] = 0u;
    __syncthreads();
    for (int c0 = 0; c0 < n; c0 += CH) {
      if (!cached) load_chunk(c0);
      const int nv = valid_count(c0);
#pragma unroll
      for (int j = 0; j < NPT; ++j) {
        const uint32_t r = key[j] - kmin;
        const uint32_t top = hi >= 32 ? 0u : (r >> hi);
        if (j < nv && top == prefix) atomicAdd(&hist[(r >> lo) & dmask], 1u);
      }
    }
    __syncthreads();
    // bins in descending order: thread i owns bins 2047-2i and 2046-2i
    const uint32_t ch = hist[2047 - 2 * tid], cl = hist[2046 - 2 * tid];
    uint32_t tot;
    const uint32_t above_h = block_excl_scan(ch + cl, sh, tot);
    const uint32_t above_l = above_h + ch;
    if (ch && above_h < krem && krem <= above_h + ch) { pick[0] = 2047 - 2 * tid; pick[1] = above_h; }
    if (cl && above_l < krem && krem <= above_l + cl) { pick[0] = 2046 - 2 * tid; pick[1] = above_l; }
    __syncthreads();
    prefix = (prefix << (hi - lo)) | pick[0];
    krem -= pick[1];
    hi = lo;
    __syncthreads();
  }
  const uint32_t T = kmin + prefix;  // threshold key; krem elements equal to T are taken

  // ---- order-preserving compaction
  uint32_t run_eq = 0u, run_sel = 0u;
  for (int c0 = 0; c0 < n; c0 += CH) {
    if (!cached) load_chunk(c0);
    const int nv = valid_count(c0);
    uint32_t ceq = 0u;
#pragma unroll
    for (int j = 0; j < NPT; ++j) ceq += (j < nv && key[j] == T) ? 1u : 0u;
    uint32_t tot_eq;
    uint32_t eq_before = block_excl_scan(ceq, sh, tot_eq) + run_eq;
    run_eq += tot_eq;
    uint32_t csel = 0u;
    uint32_t e = eq_before;
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      if (j < nv) {
        const bool eq = key[j] == T;
        csel += (key[j] > T || (eq && e < krem)) ? 1u : 0u;
        e += eq ? 1u : 0u;
      }
    }
    uint32_t tot_sel;
    uint32_t o = block_excl_scan(csel, sh, tot_sel) + run_sel;
    run_sel += tot_sel;
    e = eq_before;
    const int p0 = c0 + tid * NPT;
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      if (j < nv) {
        const bool eq = key[j] == T;
        if (key[j] > T || (eq && e < krem)) {
          oi[o] = p0 + j;
          if (ov) ov[o] = key_value(key[j]);
          ++o;
        }
        e += eq ? 1u : 0u;
      }
    }
  }
  for (int i = k + tid; i < K; i += 1024) {
    oi[i] = -1;
    if (ov) ov[i] = 0.f;
  }
}

// ---------------------------------------------------------------- LDS-resident rows
// Rows of up to kLdsRow candidates live in LDS as keys.  One 12-bit histogram pass over the
// occupied key range finds the bin that holds the k-th largest; if that bin holds at most
// kCand elements they are ranked against each other directly (the exact total order, ties by
// position) and the chosen ones are marked in place; otherwise further radix passes narrow
// the bin down to one key value and ties are taken in position order.  The compaction walks
// each thread's 32 consecutive positions (bank-rotated LDS reads) and writes the selected
// positions in ascending order.
constexpr int kLdsRow = 32768;
constexpr int kBins = 4096;
constexpr int kCand = 2048;
constexpr uint32_t kSel = 0xffffffffu;   // marks a chosen candidate (no float maps here)
constexpr uint32_t kRej = 0u;            // marks a rejected candidate (no float maps here)

struct TopkSmem {
  uint32_t keys[kLdsRow];
  uint32_t hist[kBins];  // reused as the candidate list (pos, key) after the bin is found
  uint32_t sh[40];
  uint32_t pick[4];
};

__global__ __launch_bounds__(1024) void topk_lds_kernel(DevBatch bt, int t_begin,
    const float* __restrict__ scores, int64_t ld, int K, int32_t* __restrict__ out_idx,
    float* __restrict__ out_val) {
  extern __shared__ __attribute__((aligned(16))) char smraw[];
  TopkSmem& S = *(TopkSmem*)smraw;
  const int tid = threadIdx.x;
  const int tl = blockIdx.x;
  const int t = t_begin + tl;
  const int n = locate(bt, t).n;
  const float* row = scores + (int64_t)tl * ld;
  int32_t* oi = out_idx + (int64_t)t * K;
  float* ov = out_val ? out_val + (int64_t)t * K : nullptr;
  if (n <= K) {
    for (int i = tid; i < K; i += 1024) {
      oi[i] = i < n ? i : -1;
      if (ov) ov[i] = i < n ? row[i] : 0.f;
    }
    return;
  }

  // ---- coalesced load into LDS, key range
  uint32_t kmin = ~0u, kmax = 0u;
  for (int p = 4 * tid; p < n; p += 4096) {
    uint32_t k4[4];
    if (p + 3 < n) {
      const float4 f = *(const float4*)(row + p);
      k4[0] = order_key(f.x); k4[1] = order_key(f.y); k4[2] = order_key(f.z);
      k4[3] = order_key(f.w);
    } else {
      for (int e = 0; e < 4; ++e) k4[e] = p + e < n ? order_key(row[p + e]) : 0u;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (p + e < n) { kmin = min(kmin, k4[e]); kmax = max(kmax, k4[e]); }
    *(i32x4*)&S.keys[p] = i32x4{(int)k4[0], (int)k4[1], (int)k4[2], (int)k4[3]};
  }
  block_minmax(kmin, kmax, S.sh);
  const uint32_t span = kmax - kmin;
  int hi = span ? 32 - __clz(span) : 0;

  uint32_t krem = (uint32_t)K;  // still to choose among the elements matching `prefix`
  uint32_t prefix = 0u;         // bits [hi, 32) of (key - kmin) of the surviving bin
  bool marked = false;          // candidates ranked and marked in place
  int lo = hi;
  // ---- radix passes (the first one usually suffices)
  for (int pass = 0; hi > 0; ++pass) {
    lo = max(0, hi - (pass == 0 ? 12 : 11));
    const uint32_t dmask = (1u << (hi - lo)) - 1u;
    for (int i = tid; i < kBins; i += 1024) S.hist[i] = 0u;
    __syncthreads();
    for (int p = tid; p < n; p += 1024) {
      const uint32_t r = S.keys[p] - kmin;
      const uint32_t top = hi >= 32 ? 0u : (r >> hi);
      if (top == prefix) atomicAdd(&S.hist[(r >> lo) & dmask], 1u);
    }
    __syncthreads();
    // bins in descending order: thread i owns bins 4095-4i .. 4092-4i
    uint32_t c[4], sum = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) { c[e] = S.hist[kBins - 1 - 4 * tid - e]; sum += c[e]; }
    uint32_t tot;
    uint32_t above = block_excl_scan(sum, S.sh, tot);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (c[e] && above < krem && krem <= above + c[e]) {
        S.pick[0] = kBins - 1 - 4 * tid - e;
        S.pick[1] = above;
        S.pick[2] = c[e];
      }
      above += c[e];
    }
    __syncthreads();
    const uint32_t bin = S.pick[0], nabove = S.pick[1], cnt = S.pick[2];
    prefix = (prefix << (hi - lo)) | bin;
    krem -= nabove;
    hi = lo;
    __syncthreads();
    if (lo > 0 && cnt <= (uint32_t)kCand) {
      // rank the bin's elements against each other and mark the chosen ones
      uint32_t* cpos = S.hist;
      uint32_t* ckey = S.hist + kCand;
      if (tid == 0) S.pick[3] = 0u;
      __syncthreads();
      for (int p = tid; p < n; p += 1024) {
        const uint32_t k = S.keys[p];
        if (((k - kmin) >> lo) == prefix) {
          const uint32_t slot = atomicAdd(&S.pick[3], 1u);
          cpos[slot] = (uint32_t)p;
          ckey[slot] = k;
        }
      }
      __syncthreads();
      for (uint32_t ci = tid; ci < cnt; ci += 1024) {
        const uint32_t k = ckey[ci], p = cpos[ci];
        uint32_t rank = 0u;
        for (uint32_t cj = 0; cj < cnt; ++cj) {
          const uint32_t k2 = ckey[cj];
          rank += (k2 > k || (k2 == k && cpos[cj] < p)) ? 1u : 0u;
        }
        S.keys[p] = rank < krem ? kSel : kRej;
      }
      __syncthreads();
      marked = true;
      break;
    }
  }
  // Selection predicate: marked -> (key == kSel) or (unmarked key above the surviving bin);
  // otherwise -> key above T = kmin + prefix, or equal to T (first krem in position order).
  const uint32_t T = kmin + prefix;
  const int base = 32 * tid;
  uint32_t gtmask = 0u, eqmask = 0u;
#pragma unroll 8
  for (int j = 0; j < 32; ++j) {
    const int jj = (j + tid) & 31;
    const int p = base + jj;
    if (p < n) {
      const uint32_t k = S.keys[p];
      bool gt, eq = false;
      if (marked) {
        gt = k == kSel || (k != kRej && ((k - kmin) >> lo) > prefix);
      } else {
        gt = k > T;
        eq = k == T;
      }
      gtmask |= (gt ? 1u : 0u) << jj;
      eqmask |= (eq ? 1u : 0u) << jj;
    }
  }
  uint32_t selmask = gtmask;
  if (!marked) {
    uint32_t tot_eq;
    const uint32_t eq_before = block_excl_scan(__popc(eqmask), S.sh, tot_eq);
    uint32_t take = eq_before < krem ? min(krem - eq_before, (uint32_t)__popc(eqmask)) : 0u;
    uint32_t m = eqmask;
    while (take--) { selmask |= m & (~m + 1u); m &= m - 1u; }
  }
  uint32_t tot_sel;
  uint32_t o = block_excl_scan(__popc(selmask), S.sh, tot_sel);
  while (selmask) {
    const int jj = __ffs(selmask) - 1;
    selmask &= selmask - 1u;
    oi[o] = base + jj;
    if (ov) ov[o] = row[base + jj];
    ++o;
  }
}

hipError_t launch_topk(const DevBatch& bt, int t_begin, int t_count, int max_n,
                       const float* scores, int64_t ld, int K, int32_t* idx, float* val,
                       hipStream_t st) {
  if (max_n <= kLdsRow) {
    const size_t shm = sizeof(TopkSmem);
    hipError_t e = hipFuncSetAttribute((const void*)topk_lds_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_lds_kernel, dim3(t_count), dim3(1024), shm, st, bt, t_begin, scores,
                       ld, K, idx, val);
  } else {
    hipLaunchKernelGGL(topk_stream_kernel<32>, dim3(t_count), dim3(1024), 0, st, bt, t_begin,
                       scores, ld, K, idx, val);
  }
  return hipGetLastError();
}

}  // namespace tis
