// Per-query Top-K over the scores of positions 0..p_t.
//
// Method: "Day 0 Support for New LLM Architectures", Step 1 and Key Optimization 1 (the
// Top-K positions of the indexer scores are selected on the device); "Achieving Day-0
// Readiness ... Million-Token Context" 2.1 (selection is an operator of its own, run on
// the GPU with the index kept resident).  Selection is exact: the k_t = min(K, n_t) largest
// scores under the total order (score descending, position ascending), -0.0 == +0.0,
// emitted in ascending position order and padded with -1.
//
// One 1024-thread workgroup per row.  Scores map to order-preserving uint32 keys and the
// key range [kmin, kmax] of the row is measured.  Radix select walks the bits of
// (key - base) from the top in 11-bit digits, so the first digit already splits the occupied
// range into 2048 bins instead of spending it on the (nearly constant) sign and exponent
// bits; each pass histograms the keys that still match the chosen prefix (LDS atomics) and
// picks the bin holding the k-th largest.  For rows held in registers a sampled lower bound
// first cuts the keys to a short list, so the radix passes run over ~1.4 K keys instead of
// the row.  The result is a threshold key T and the number r of keys equal to T that are
// taken; the compaction keeps every key > T and the first r keys == T in position order,
// via block scans.
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

// Wave-wide inclusive scan on the DPP network (gfx9 wave64 pattern): shifts by 1, 2, 4, 8
// within each 16-lane row, then row 15 -> rows 1 and 3 and lane 31 -> rows 2 and 3.  Lanes
// whose source is outside the row receive 0 (max: receive the identity given).
template <typename Op>
__device__ __forceinline__ uint32_t wave_incl(uint32_t x, uint32_t id, Op op) {
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x111, 0xf, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x112, 0xf, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x114, 0xf, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x118, 0xf, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x142, 0xa, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x143, 0xc, 0xf, false));
  return x;
}
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  return wave_incl(x, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}

// Exclusive scan over the 1024 threads; `sh` holds >= 17 words.  Ends with a barrier.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh, uint32_t& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v);
  if (lane == 63) sh[wid] = inc;
  __syncthreads();
  if (wid == 0) {
    const uint32_t x = lane < 16 ? sh[lane] : 0u;
    const uint32_t xi = wave_incl_scan(x);
    if (lane < 16) sh[lane] = xi - x;
    if (lane == 15) sh[16] = xi;
  }
  __syncthreads();
  const uint32_t r = sh[wid] + inc - v;
  total = sh[16];
  __syncthreads();
  return r;
}

__device__ __forceinline__ void block_minmax(uint32_t& mn, uint32_t& mx, uint32_t* sh) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  auto fmin_ = [](uint32_t a, uint32_t b) { return min(a, b); };
  auto fmax_ = [](uint32_t a, uint32_t b) { return max(a, b); };
  mn = __builtin_amdgcn_readlane(wave_incl(mn, ~0u, fmin_), 63);
  mx = __builtin_amdgcn_readlane(wave_incl(mx, 0u, fmax_), 63);
  if (lane == 0) { sh[wid] = mn; sh[16 + wid] = mx; }
  __syncthreads();
  if (wid == 0) {
    uint32_t a = lane < 16 ? sh[lane] : ~0u, c = lane < 16 ? sh[16 + lane] : 0u;
    a = __builtin_amdgcn_readlane(wave_incl(a, ~0u, fmin_), 63);
    c = __builtin_amdgcn_readlane(wave_incl(c, 0u, fmax_), 63);
    if (lane == 0) { sh[32] = a; sh[33] = c; }
  }
  __syncthreads();
  mn = sh[32];
  mx = sh[33];
  __syncthreads();
}

// LDS of the selection kernel: histogram, scan scratch, picks and the candidate list.
constexpr int kCandMax = 8192;
struct SelSmem {
  uint32_t hist[2048];
  uint32_t sh[40];
  uint32_t pick[4];
  uint32_t candk[kCandMax];
};

// Radix select of the krem-th largest key among the keys produced by `each` (called with a
// visitor), over r = key - base with digits of up to 11 bits from bit `hi` down.  Returns the
// threshold key; krem is left as the number of keys equal to it that are taken.
template <typename Each>
__device__ __forceinline__ uint32_t radix_select(uint32_t base, int hi, uint32_t& krem,
                                                 SelSmem& S, Each each) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0u;
  while (hi > 0) {
    const int lo = max(0, hi - 11);
    const uint32_t dmask = (1u << (hi - lo)) - 1u;
    S.hist[tid] = 0u;
    S.hist[tid + 1024] = 0u;
    __syncthreads();
    each([&](uint32_t key) {
      const uint32_t r = key - base;
      const uint32_t top = hi >= 32 ? 0u : (r >> hi);
      if (top == prefix) atomicAdd(&S.hist[(r >> lo) & dmask], 1u);
    });
    __syncthreads();
    // bins in descending order: thread i owns bins 2047-2i and 2046-2i
    const uint32_t ch = S.hist[2047 - 2 * tid], cl = S.hist[2046 - 2 * tid];
    uint32_t tot;
    const uint32_t above_h = block_excl_scan(ch + cl, S.sh, tot);
    const uint32_t above_l = above_h + ch;
    if (ch && above_h < krem && krem <= above_h + ch) {
      S.pick[0] = 2047 - 2 * tid;
      S.pick[1] = above_h;
    }
    if (cl && above_l < krem && krem <= above_l + cl) {
      S.pick[0] = 2046 - 2 * tid;
      S.pick[1] = above_l;
    }
    __syncthreads();
    prefix = (prefix << (hi - lo)) | S.pick[0];
    krem -= S.pick[1];
    hi = lo;
    __syncthreads();
  }
  return base + prefix;
}

// One 1024-thread workgroup per row; thread i owns NPT consecutive positions per chunk of
// 1024*NPT (rows that fit one chunk keep their keys in registers).
// Threshold search, rows held in registers: a sample (2 keys per thread, at a fixed stride)
// is histogrammed over the row's key range; the bin where the sample count from the top
// reaches 1.25x the expected share of K (plus 16) gives a lower bound T_lo, and the keys
// >= T_lo (normally ~1.4 K of them) are listed in LDS and radix-selected exactly.  When the
// list holds fewer than K keys or would overflow (heavy ties, adversarial orders), the exact
// radix select runs over the whole row instead; both give the same threshold.
template <int NPT>
__global__ __launch_bounds__(1024) void topk_select_kernel(DevBatch bt, int t_begin,
    const float* __restrict__ scores, int64_t ld, int K, int32_t* __restrict__ out_idx,
    float* __restrict__ out_val) {
  extern __shared__ __attribute__((aligned(16))) char smraw[];
  SelSmem& S = *(SelSmem*)smraw;
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
  // Positions past the row hold key 0, which no score maps to (the smallest key, of -inf,
  // is 0x007fffff): validity is key != 0, and every threshold below is above 0.
  // visits every valid key of the row (from registers when cached)
  auto each_row = [&](auto&& f) {
    for (int c0 = 0; c0 < n; c0 += CH) {
      if (!cached) load_chunk(c0);
#pragma unroll
      for (int j = 0; j < NPT; ++j)
        if (key[j] != 0u) f(key[j]);
    }
  };

  if (cached) load_chunk(0);

  // ---- key range of the row
  uint32_t kmin = ~0u, kmax = 0u;
  each_row([&](uint32_t kk) { kmin = min(kmin, kk); kmax = max(kmax, kk); });
  block_minmax(kmin, kmax, S.sh);
  const uint32_t span = kmax - kmin;
  const int hi = span ? 32 - __clz(span) : 0;

  uint32_t krem = (uint32_t)k;
  uint32_t T = 0u;
  bool found = false;
  if (cached && hi > 0) {
    // ---- sampled lower bound of the threshold
    const int shift = max(0, hi - 11);
    S.hist[tid] = 0u;
    S.hist[tid + 1024] = 0u;
    __syncthreads();
    if (key[0] != 0u) atomicAdd(&S.hist[(key[0] - kmin) >> shift], 1u);
    if (key[NPT / 2] != 0u) atomicAdd(&S.hist[(key[NPT / 2] - kmin) >> shift], 1u);
    __syncthreads();
    const uint32_t nsamp = (uint32_t)((n + NPT - 1) / NPT + (n + NPT / 2 - 1) / NPT);
    const uint32_t want = min(nsamp, (uint32_t)(((uint64_t)k * nsamp * 5) / (4ull * n)) + 16u);
    {
      const uint32_t ch = S.hist[2047 - 2 * tid], cl = S.hist[2046 - 2 * tid];
      uint32_t tot;
      const uint32_t above_h = block_excl_scan(ch + cl, S.sh, tot);
      const uint32_t above_l = above_h + ch;
      if (ch && above_h < want && want <= above_h + ch) S.pick[2] = 2047 - 2 * tid;
      if (cl && above_l < want && want <= above_l + cl) S.pick[2] = 2046 - 2 * tid;
      __syncthreads();
    }
    const uint32_t tlo = kmin + (S.pick[2] << shift);
    // ---- list the keys >= tlo
    uint32_t c = 0u;
#pragma unroll
    for (int j = 0; j < NPT; ++j) c += key[j] >= tlo ? 1u : 0u;
    uint32_t C;
    uint32_t o = block_excl_scan(c, S.sh, C);
    if (C >= (uint32_t)k && C <= (uint32_t)kCandMax) {
#pragma unroll
      for (int j = 0; j < NPT; ++j)
        if (key[j] >= tlo) S.candk[o++] = key[j];
      __syncthreads();
      const uint32_t cspan = kmax - tlo;
      T = radix_select(tlo, cspan ? 32 - __clz(cspan) : 0, krem, S, [&](auto&& f) {
        for (uint32_t i = tid; i < C; i += 1024) f(S.candk[i]);
      });
      found = true;
    }
  }
  if (!found) T = radix_select(kmin, hi, krem, S, each_row);
  // T is the threshold key; krem elements equal to T are taken (in position order)

  // ---- order-preserving compaction: one scan of the per-thread counts of keys > T (low 16
  // bits) and == T (high 16 bits; both totals stay below 2^16 per chunk)
  uint32_t run_gt = 0u, run_eq = 0u;
  for (int c0 = 0; c0 < n; c0 += CH) {
    if (!cached) load_chunk(c0);
    uint32_t cgt = 0u, ceq = 0u;
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      cgt += key[j] > T ? 1u : 0u;
      ceq += key[j] == T ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t before = block_excl_scan(cgt | (ceq << 16), S.sh, tot);
    uint32_t e = (before >> 16) + run_eq;  // ties before this thread
    uint32_t o = (before & 0xffffu) + run_gt + min(e, krem);
    run_gt += tot & 0xffffu;
    run_eq += tot >> 16;
    const int p0 = c0 + tid * NPT;
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      const bool eq = key[j] == T;
      if (key[j] > T || (eq && e < krem)) {
        oi[o] = p0 + j;
        if (ov) ov[o] = key_value(key[j]);
        ++o;
      }
      e += eq ? 1u : 0u;
    }
  }
  for (int i = k + tid; i < K; i += 1024) {
    oi[i] = -1;
    if (ov) ov[i] = 0.f;
  }
}

hipError_t launch_topk(const DevBatch& bt, int t_begin, int t_count, int max_n,
                       const float* scores, int64_t ld, int K, int32_t* idx, float* val,
                       hipStream_t st) {
  // keys per thread: the smallest power of two (>= 4) that keeps the longest row in registers,
  // up to 32 (32768 positions); longer rows stream through 1024*32-key chunks per pass
  int npt = 4;
  while (npt < 32 && 1024 * npt < max_n) npt *= 2;
  auto* fn = npt == 4 ? topk_select_kernel<4>
             : npt == 8 ? topk_select_kernel<8>
             : npt == 16 ? topk_select_kernel<16> : topk_select_kernel<32>;
  const size_t shm = sizeof(SelSmem);
  hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)shm);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3(t_count), dim3(1024), shm, st, bt, t_begin, scores, ld, K, idx,
                     val);
  return hipGetLastError();
}

}  // namespace tis
