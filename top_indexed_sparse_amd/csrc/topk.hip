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

// Entries of token t's selection row: its n causal positions, or ceil(n / 64) page scores for
// block-granular selection (row_shift 6).
__device__ __forceinline__ int row_len(const DevBatch& bt, int t) {
  const int n = locate(bt, t).n;
  return (n + (1 << bt.row_shift) - 1) >> bt.row_shift;
}


__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  u = u == 0x80000000u ? 0u : u;  // -0.0 ties with +0.0
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);  // negative: ~u, else u | sign
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

// Exclusive scan over the 1024 threads with one barrier: the 16 wave totals go to sh[0..15];
// lane l of every wave reads total l & 15 and scans them on the DPP network.  sh must not be
// written again before the next barrier after this call (every caller has one in between).
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh, uint32_t& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v);
  if (lane == 63) sh[wid] = inc;
  __syncthreads();
  const uint32_t w = wave_incl_scan(lane < 16 ? sh[lane] : 0u);
  total = __builtin_amdgcn_readlane(w, 15);
  const uint32_t before = wid ? __builtin_amdgcn_readlane(w, wid - 1) : 0u;
  return before + inc - v;
}

// The same scan, also returning the maximum of m over the threads (sh: 32 words).
__device__ __forceinline__ uint32_t block_excl_scan_max(uint32_t v, uint32_t& m, uint32_t* sh,
                                                        uint32_t& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  auto fmax_ = [](uint32_t a, uint32_t b) { return max(a, b); };
  const uint32_t inc = wave_incl_scan(v);
  const uint32_t wm = __builtin_amdgcn_readlane(wave_incl(m, 0u, fmax_), 63);
  if (lane == 63) sh[wid] = inc;
  if (lane == 0) sh[16 + wid] = wm;
  __syncthreads();
  const uint32_t w = wave_incl_scan(lane < 16 ? sh[lane] : 0u);
  total = __builtin_amdgcn_readlane(w, 15);
  m = __builtin_amdgcn_readlane(wave_incl(lane < 16 ? sh[16 + lane] : 0u, 0u, fmax_), 15);
  const uint32_t before = wid ? __builtin_amdgcn_readlane(w, wid - 1) : 0u;
  return before + inc - v;
}

// Row minimum and maximum over the 1024 threads with one barrier (sh: 32 words, same rule).
__device__ __forceinline__ void block_minmax(uint32_t& mn, uint32_t& mx, uint32_t* sh) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  auto fmin_ = [](uint32_t a, uint32_t b) { return min(a, b); };
  auto fmax_ = [](uint32_t a, uint32_t b) { return max(a, b); };
  mn = __builtin_amdgcn_readlane(wave_incl(mn, ~0u, fmin_), 63);
  mx = __builtin_amdgcn_readlane(wave_incl(mx, 0u, fmax_), 63);
  if (lane == 0) { sh[wid] = mn; sh[16 + wid] = mx; }
  __syncthreads();
  mn = __builtin_amdgcn_readlane(wave_incl(lane < 16 ? sh[lane] : ~0u, ~0u, fmin_), 15);
  mx = __builtin_amdgcn_readlane(wave_incl(lane < 16 ? sh[16 + lane] : 0u, 0u, fmax_), 15);
}

// LDS of the selection kernel: histogram, scan scratch, picks and the candidate list.
constexpr int kCandMax = 8192;
constexpr int kListMax = kCandMax / 2;  // candidate list: keys and positions
struct SelSmem {
  uint32_t hist[2048];
  uint32_t hist2[2048];
  uint32_t sh[48];    // scan totals (0..15), row min/max (16..47)
  uint32_t pick[4];
  uint32_t candk[kCandMax];
};

// Long-row selection state per row, words [mode, bin, candidates, keys above the bin]
constexpr uint32_t kLongCand = 0u, kLongAll = 1u, kLongOver = 2u;
constexpr int kLongCap = 8192;      // candidates per row (8 per thread of the last step)
constexpr int kLongRows = 64;       // at most this many rows per launch take the long-row path
constexpr int kLongSlices = 1024;   // slices per row at most

// Radix select of the krem-th largest key among the keys produced by `each` (called with a
// visitor), over r = key - base with digits of up to 11 bits from bit `hi` down.  Returns the
// threshold key; krem is left as the number of keys equal to it that are taken.  The two
// histograms alternate, the next one being cleared while the current one fills: three
// barriers per digit.
template <typename Each>
__device__ __forceinline__ uint32_t radix_select(uint32_t base, int hi, uint32_t& krem,
                                                 SelSmem& S, Each each) {
  const int tid = threadIdx.x;
  uint32_t* hb[2] = {S.hist, S.hist2};
  int cur = 0;
  uint32_t prefix = 0u;
  hb[0][tid] = 0u;
  hb[0][tid + 1024] = 0u;
  __syncthreads();
  while (hi > 0) {
    const int lo = max(0, hi - 11);
    const uint32_t dmask = (1u << (hi - lo)) - 1u;
    uint32_t* h = hb[cur];
    each([&](uint32_t key) {
      const uint32_t r = key - base;
      const uint32_t top = hi >= 32 ? 0u : (r >> hi);
      if (top == prefix) atomicAdd(&h[(r >> lo) & dmask], 1u);
    });
    hb[cur ^ 1][tid] = 0u;
    hb[cur ^ 1][tid + 1024] = 0u;
    __syncthreads();
    // bins in descending order: thread i owns bins 2047-2i and 2046-2i
    const uint32_t ch = h[2047 - 2 * tid], cl = h[2046 - 2 * tid];
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
    cur ^= 1;
  }
  return base + prefix;
}

// One 1024-thread workgroup per row; thread i owns NPT consecutive positions per chunk of
// 1024*NPT (rows that fit one chunk keep their keys in registers, loaded before the token's
// causal length is known and masked after).
// Threshold search, rows held in registers: a sample (2 keys per thread, at a fixed stride)
// is histogrammed over the row's key range; the bin where the sample count from the top
// reaches 1.25x the expected share of K (plus 16) gives a lower bound T_lo.  The keys >= T_lo
// (normally ~1.4 K of them) are histogrammed again over their own range, which puts the
// k-th largest key in a bin of a few keys: those are ranked by one wave (or, for larger bins,
// radix-selected).  When fewer than K keys reach T_lo, or the bin would overflow the list
// (heavy ties, adversarial orders), the exact radix select runs over the whole row instead;
// every path gives the same threshold.
template <int NPT>
__global__ __launch_bounds__(1024) void topk_select_kernel(DevBatch bt, int t_begin,
    const float* __restrict__ scores, int64_t ld, int K, const uint32_t* __restrict__ only,
    int32_t* __restrict__ out_idx,
    float* __restrict__ out_val) {
  extern __shared__ __attribute__((aligned(16))) char smraw[];
  SelSmem& S = *(SelSmem*)smraw;
  const int tid = threadIdx.x;
  const int tl = blockIdx.x;
  const int t = t_begin + tl;
  const float* row = scores + (int64_t)tl * ld;
  // (after the long-row selection: only the rows it left over)
  if (only && only[4 * tl] != kLongOver) return;
  constexpr int CH = 1024 * NPT;
  uint32_t key[NPT];  // the raw score bits until to_keys, then the order keys

  // scores of chunk c0 at positions < lim (positions past it read nothing)
  auto load_raw = [&](int c0, int lim) {
    const int p0 = c0 + tid * NPT;
#pragma unroll
    for (int j = 0; j < NPT; j += 4) {
      const int p = p0 + j;
      if (p + 3 < lim) {
        const uint4 f = *(const uint4*)(row + p);
        key[j] = f.x; key[j + 1] = f.y; key[j + 2] = f.z; key[j + 3] = f.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) key[j + e] = (p + e < lim) ? __float_as_uint(row[p + e]) : 0u;
      }
    }
  };
  // Positions past the row hold key 0, which no score maps to (the smallest key, of -inf,
  // is 0x007fffff): validity is key != 0, and every threshold below is above 0.
  int n = 0;
  auto to_keys = [&](int c0) {
    const int p0 = c0 + tid * NPT;
    if (__all(p0 + NPT <= n)) {  // (the wave is inside the row: no position test)
#pragma unroll
      for (int j = 0; j < NPT; ++j) key[j] = order_key(__uint_as_float(key[j]));
    } else {
#pragma unroll
      for (int j = 0; j < NPT; ++j)
        key[j] = p0 + j < n ? order_key(__uint_as_float(key[j])) : 0u;
    }
  };
  auto load_chunk = [&](int c0) {
    load_raw(c0, n);
    to_keys(c0);
  };
  // The first chunk arrives through LDS: each wave reads its 256*NPT bytes with coalesced
  // 1 KB loads (16-byte piece P = 64i + lane of the wave's span belongs to thread P / Q of the
  // wave, Q = NPT/4 pieces per thread), stores them swizzled (piece q of thread u at slot
  // u*Q + (q ^ ((u >> sw) & (Q-1))), which keeps both the stores and the reads below on 16
  // distinct 4-bank groups per 16 lanes) and reads its own Q pieces back.  Read directly, each
  // load instruction would touch 64 lines for 16 bytes of each.  The buffer overlaps S.
  auto load_first = [&](int lim) {
    if constexpr (NPT == 4) {
      load_raw(0, lim);  // (one piece per thread: already coalesced)
    } else {
      constexpr int Q = NPT / 4;
      constexpr int sw = Q == 8 ? 1 : Q == 4 ? 2 : 3;  // log2(16 / Q)
      const int lane = tid & 63;
      const int wb = (tid >> 6) * 64 * NPT;  // the wave's first position
      uint4 v[Q];
#pragma unroll
      for (int i = 0; i < Q; ++i) {
        const int p = wb + 256 * i + 4 * lane;  // (lim and p are multiples of 4)
        v[i] = *(const uint4*)(row + min(p, lim - 4));
        if (p >= lim) v[i] = make_uint4(0u, 0u, 0u, 0u);
      }
      char* wbuf = smraw + (tid >> 6) * 64 * NPT * 4;
#pragma unroll
      for (int i = 0; i < Q; ++i) {
        const int u = (64 * i + lane) / Q, q = lane % Q;
        *(uint4*)(wbuf + 16 * (u * Q + (q ^ ((u >> sw) & (Q - 1))))) = v[i];
      }
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const uint4 x = *(const uint4*)(wbuf + 16 * (lane * Q + (q ^ ((lane >> sw) & (Q - 1)))));
        key[4 * q] = x.x; key[4 * q + 1] = x.y; key[4 * q + 2] = x.z; key[4 * q + 3] = x.w;
      }
    }
  };

  // the first chunk goes out before the token lookup (up to the row stride, which bounds
  // every causal length), so the two memory latencies overlap
  const LocLoads lw = locate_issue(bt);
  load_first((int)min<int64_t>(ld, (int64_t)CH));
  n = locate_finish(bt, t, lw).n;
  n = (n + (1 << bt.row_shift) - 1) >> bt.row_shift;  // (block rows: pages, not positions)
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
  const bool cached = n <= CH;
  // visits every valid key of the row (from registers when cached)
  auto each_row = [&](auto&& f) {
    for (int c0 = 0; c0 < n; c0 += CH) {
      if (!cached) load_chunk(c0);
#pragma unroll
      for (int j = 0; j < NPT; ++j)
        if (key[j] != 0u) f(key[j]);
    }
  };

  __syncthreads();  // (every wave has read its first chunk back before S is written)
  to_keys(0);
  S.hist[tid] = 0u;
  S.hist[tid + 1024] = 0u;
  S.hist2[tid] = 0u;
  S.hist2[tid + 1024] = 0u;
  if (tid == 0) S.pick[3] = 0u;

  uint32_t krem = (uint32_t)k;
  uint32_t T = 0u;
  if (cached) {
    // ---- sampled lower bound of the threshold, over the key range of the sample (keys above
    // it are all candidates anyway); its barrier also orders the clears above
    uint32_t smin1 = min(key[0] - 1u, key[NPT / 2] - 1u);  // (invalid key 0 -> 0xffffffff)
    uint32_t smax = max(key[0], key[NPT / 2]);
    block_minmax(smin1, smax, S.sh + 16);
    const uint32_t smin = smin1 + 1u;
    const uint32_t sspan = smax - smin;
    const int shift = max(0, (sspan ? 32 - __clz(sspan) : 0) - 11);
    if (key[0] != 0u) atomicAdd(&S.hist[(key[0] - smin) >> shift], 1u);
    if (key[NPT / 2] != 0u) atomicAdd(&S.hist[(key[NPT / 2] - smin) >> shift], 1u);
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
    const uint32_t tlo = smin + (S.pick[2] << shift);
    // ---- list the keys >= tlo with their positions, in position order (~1.4 K of them)
    uint32_t c = 0u, kmax = 0u;
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      c += key[j] >= tlo ? 1u : 0u;
      kmax = max(kmax, key[j]);
    }
    uint32_t C;
    uint32_t o = block_excl_scan_max(c, kmax, S.sh, C);
    if (C >= (uint32_t)k && C <= (uint32_t)kListMax) {
      uint32_t* lk = S.candk;              // keys
      uint32_t* lp = S.candk + kListMax;   // positions
      {
        const uint32_t p0 = (uint32_t)(tid * NPT);
#pragma unroll
        for (int j = 0; j < NPT; ++j)
          if (key[j] >= tlo) {
            lk[o] = key[j];
            lp[o] = p0 + j;
            ++o;
          }
      }
      __syncthreads();
      // ---- histogram of the list over [tlo, kmax]: the k-th largest lies in one bin
      const uint32_t cspan = kmax - tlo;
      const int shift2 = max(0, (cspan ? 32 - __clz(cspan) : 0) - 11);
      for (uint32_t i = tid; i < C; i += 1024) atomicAdd(&S.hist2[(lk[i] - tlo) >> shift2], 1u);
      __syncthreads();
      {
        const uint32_t ch = S.hist2[2047 - 2 * tid], cl = S.hist2[2046 - 2 * tid];
        uint32_t tot;
        const uint32_t above_h = block_excl_scan(ch + cl, S.sh, tot);
        const uint32_t above_l = above_h + ch;
        if (ch && above_h < (uint32_t)k && (uint32_t)k <= above_h + ch) {
          S.pick[0] = 2047 - 2 * tid;
          S.pick[1] = above_h;
        }
        if (cl && above_l < (uint32_t)k && (uint32_t)k <= above_l + cl) {
          S.pick[0] = 2046 - 2 * tid;
          S.pick[1] = above_l;
        }
        __syncthreads();
      }
      const uint32_t b2 = S.pick[0];
      const uint32_t tb = tlo + (b2 << shift2);  // the bin holds keys tb .. tb + 2^shift2 - 1
      const uint32_t cb = S.hist2[b2];
      krem = (uint32_t)k - S.pick[1];            // keys of the bin that are taken
      if (cb == krem) {  // the whole bin: every key >= tb, none equal to the threshold
        T = tb - 1u;
        krem = 0u;
      } else if (cb <= 64u) {
        // one wave ranks the bin: the key with (# greater) < krem <= (# greater or equal)
        const uint32_t bhi =
            (uint32_t)min<uint64_t>((uint64_t)tb + ((1u << shift2) - 1u), 0xffffffffull);
        uint32_t* bl = S.hist;  // (free since the sample)
        for (uint32_t i = tid; i < C; i += 1024)
          if (lk[i] >= tb && lk[i] <= bhi) bl[atomicAdd(&S.pick[3], 1u)] = lk[i];
        __syncthreads();
        if (tid < 64) {
          const uint32_t mine = tid < (int)cb ? bl[tid] : 0u;
          uint32_t gt = 0u, ge = 0u;
          for (uint32_t j = 0; j < cb; ++j) {
            const uint32_t ot = bl[j];
            gt += ot > mine ? 1u : 0u;
            ge += ot >= mine ? 1u : 0u;
          }
          const uint64_t hit = __ballot(tid < (int)cb && gt < krem && krem <= ge);
          const int src = (int)__builtin_ctzll(hit);  // (never empty: ranks cover 1..cb)
          if (tid == 0) {
            S.pick[0] = __builtin_amdgcn_readlane(mine, src);
            S.pick[1] = krem - __builtin_amdgcn_readlane(gt, src);
          }
        }
        __syncthreads();
        T = S.pick[0];
        krem = S.pick[1];
      } else {
        // a larger bin: radix select within it (list keys outside the bin fall outside the
        // digit prefix and are not counted)
        T = radix_select(tb, shift2, krem, S, [&](auto&& f) {
          for (uint32_t i = tid; i < C; i += 1024) f(lk[i]);
        });
      }
      // ---- compaction over the list (position order): an entry is taken if its key is > T,
      // or == T with fewer than krem earlier entries == T.  Thread i owns entries E*i ..
      const uint32_t E = (C + 1023u) / 1024u;
      uint32_t cgt = 0u, ceq = 0u;
      for (uint32_t e = 0; e < E; ++e) {
        const uint32_t i = (uint32_t)tid * E + e;
        if (i < C) {
          cgt += lk[i] > T ? 1u : 0u;
          ceq += lk[i] == T ? 1u : 0u;
        }
      }
      uint32_t tot;
      const uint32_t before = block_excl_scan(cgt | (ceq << 16), S.sh, tot);
      uint32_t eqb = before >> 16;
      uint32_t oo = (before & 0xffffu) + min(eqb, krem);
      for (uint32_t e = 0; e < E; ++e) {
        const uint32_t i = (uint32_t)tid * E + e;
        if (i < C) {
          const uint32_t kk = lk[i];
          const bool eq = kk == T;
          if (kk > T || (eq && eqb < krem)) {
            oi[oo] = (int32_t)lp[i];
            if (ov) ov[oo] = key_value(kk);
            ++oo;
          }
          eqb += eq ? 1u : 0u;
        }
      }
      return;
    }
  }
  {  // whole-row radix select (streamed rows, or a short list that failed)
    uint32_t kmin = ~0u, kmax = 0u;
    each_row([&](uint32_t kk) { kmin = min(kmin, kk); kmax = max(kmax, kk); });
    __syncthreads();  // (the list path may still be reading sh)
    block_minmax(kmin, kmax, S.sh + 16);
    const uint32_t span = kmax - kmin;
    krem = (uint32_t)k;
    T = radix_select(kmin, span ? 32 - __clz(span) : 0, krem, S, each_row);
  }
  // T is the threshold key; krem elements equal to T are taken (in position order)

  // ---- order-preserving compaction: one scan of the per-thread counts of keys > T (low 16
  // bits) and == T (high 16 bits; both totals stay below 2^16 per chunk).  Rows held in
  // registers stage the k positions and keys in LDS and write them out coalesced.
  if (cached && k <= kCandMax) {
    uint32_t cgt = 0u, ceq = 0u;
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      cgt += key[j] > T ? 1u : 0u;
      ceq += key[j] == T ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t before = block_excl_scan(cgt | (ceq << 16), S.sh, tot);
    uint32_t e = before >> 16;  // ties before this thread
    uint32_t o = (before & 0xffffu) + min(e, krem);
    uint32_t sel = 0u;  // bit j: position p0 + j is taken
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      const bool eq = key[j] == T;
      sel |= (key[j] > T || (eq && e < krem)) ? (1u << j) : 0u;
      e += eq ? 1u : 0u;
    }
    const uint32_t p0 = (uint32_t)(tid * NPT);
    for (; sel; sel &= sel - 1u) S.candk[o++] = p0 + (uint32_t)__builtin_ctz(sel);
    __syncthreads();
    for (int i = tid; i < k; i += 1024) {
      const int32_t p = (int32_t)S.candk[i];
      oi[i] = p;
      if (ov) ov[i] = row[p] + 0.f;  // (+ 0: -0.0 comes out as +0.0, as from a key)
    }
    return;
  }
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


// ---------------------------------------------------------------- long rows, few of them
// With few rows of many positions, one workgroup per row leaves most of the chip idle and
// streams each row through one CU.  Then every row is cut into slices:
//   0. the row's histogram and state words are cleared;
//   1. each slice histograms the top 11 bits of its keys in LDS and adds the non-empty bins to
//      the row's histogram;
//   2. one workgroup per row finds the bin b holding the k-th largest key: the keys in bins
//      >= b (at least k of them) are the candidates;
//   3. each slice counts its candidates, then writes them (key, position) to the row's list
//      at the offset of the slices before it, so the list is in position order;
//   4. one workgroup per row holds the list in registers, radix-selects the threshold key T
//      among the keys of the picked bin (the keys above it are all taken) and keeps the keys
//      > T and the first ones == T, in list (= position) order.
// Rows with n <= K take every position in step 4.  A row whose list would exceed kLongCap
// (many equal or nearly equal scores) is marked in step 2 and selected afterwards by the
// one-workgroup kernel, which skips every other row.  The result is the same selection.

__global__ __launch_bounds__(256) void topk_long_zero_kernel(uint32_t* __restrict__ hist,
                                                             uint32_t* __restrict__ state) {
  const int tl = blockIdx.x;
  for (int i = threadIdx.x; i < 2048; i += 256) hist[(int64_t)tl * 2048 + i] = 0u;
  if (threadIdx.x < 4) state[4 * tl + threadIdx.x] = 0u;
}

__global__ __launch_bounds__(256) void topk_long_hist_kernel(DevBatch bt, int t_begin,
    const float* __restrict__ scores, int64_t ld, int K, int slice,
    uint32_t* __restrict__ hist) {
  __shared__ uint32_t h[2048];
  const int tid = threadIdx.x, tl = blockIdx.y;
  for (int i = tid; i < 2048; i += 256) h[i] = 0u;
  const int n = row_len(bt, t_begin + tl);
  const float* row = scores + (int64_t)tl * ld;
  const int p0 = blockIdx.x * slice, p1 = min(n, p0 + slice);
  __syncthreads();
  if (n > K) {
    for (int p = p0 + 4 * tid; p < p1; p += 1024) {
      float v[4];
      if (p + 3 < p1) {
        const float4 f = *(const float4*)(row + p);
        v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = p + e < p1 ? row[p + e] : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {  // (key 0 is never listed: it is not counted either)
        const uint32_t k = order_key(v[e]);
        if (p + e < p1 && k != 0u) atomicAdd(&h[k >> 21], 1u);
      }
    }
  }
  __syncthreads();
  uint32_t* gh = hist + (int64_t)tl * 2048;
  for (int i = tid; i < 2048; i += 256)
    if (h[i]) atomicAdd(&gh[i], h[i]);
}

__global__ __launch_bounds__(1024) void topk_long_pick_kernel(DevBatch bt, int t_begin, int K,
    const uint32_t* __restrict__ hist, uint32_t* __restrict__ state) {
  __shared__ uint32_t sh[48];
  __shared__ uint32_t pick[3];
  const int tid = threadIdx.x, tl = blockIdx.x;
  const int n = row_len(bt, t_begin + tl);
  uint32_t* st = state + 4 * tl;
  if (n <= K) {  // (uniform over the workgroup)
    if (tid == 0) st[0] = kLongAll;
    return;
  }
  // bins in descending order: thread i owns bins 2047 - 2i and 2046 - 2i
  const uint32_t* hr = hist + (int64_t)tl * 2048;
  const uint32_t ch = hr[2047 - 2 * tid], cl = hr[2046 - 2 * tid];
  if (tid == 0) {  // (no bin reaches K only when keys 0 were left out: overflow, as for ties)
    pick[0] = 0u;
    pick[1] = ~0u;
    pick[2] = 0u;
  }
  uint32_t tot;
  const uint32_t above_h = block_excl_scan(ch + cl, sh, tot);
  const uint32_t above_l = above_h + ch;
  const uint32_t k = (uint32_t)K;
  if (ch && above_h < k && k <= above_h + ch) {
    pick[0] = 2047 - 2 * tid;
    pick[1] = above_h + ch;
    pick[2] = above_h;
  }
  if (cl && above_l < k && k <= above_l + cl) {
    pick[0] = 2046 - 2 * tid;
    pick[1] = above_l + cl;
    pick[2] = above_l;
  }
  __syncthreads();
  if (tid == 0) {
    st[0] = pick[1] > (uint32_t)kLongCap ? kLongOver : kLongCand;
    st[1] = pick[0];
    st[2] = pick[1];
    st[3] = pick[2];
  }
}

// keys of positions p .. p + 3 of a slice ending at p1 (key 0 past it)
__device__ __forceinline__ void long_keys4(const float* row, int p, int p1, uint32_t key[4]) {
  float v[4];
  if (p + 3 < p1) {
    const float4 f = *(const float4*)(row + p);
    v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = p + e < p1 ? row[p + e] : 0.f;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) key[e] = p + e < p1 ? order_key(v[e]) : 0u;
}

__global__ __launch_bounds__(256) void topk_long_count_kernel(DevBatch bt, int t_begin,
    const float* __restrict__ scores, int64_t ld, int slice, const uint32_t* __restrict__ state,
    uint32_t* __restrict__ counts) {
  __shared__ uint32_t c_sh;
  const int tid = threadIdx.x, tl = blockIdx.y;
  const uint32_t* st = state + 4 * tl;
  if (st[0] != kLongCand) return;
  const uint32_t thr = st[1] << 21;  // the candidates: keys in bins >= the picked one
  const int n = row_len(bt, t_begin + tl);
  const float* row = scores + (int64_t)tl * ld;
  const int p0 = blockIdx.x * slice, p1 = min(n, p0 + slice);
  if (tid == 0) c_sh = 0u;
  __syncthreads();
  uint32_t c = 0u;
  for (int p = p0 + 4 * tid; p < p1; p += 1024) {
    uint32_t key[4];
    long_keys4(row, p, p1, key);
#pragma unroll
    for (int e = 0; e < 4; ++e) c += key[e] >= thr && key[e] != 0u ? 1u : 0u;
  }
  if (c) atomicAdd(&c_sh, c);
  __syncthreads();
  if (tid == 0) counts[(int64_t)tl * kLongSlices + blockIdx.x] = c_sh;
}

__global__ __launch_bounds__(1024) void topk_long_write_kernel(DevBatch bt, int t_begin,
    const float* __restrict__ scores, int64_t ld, int slice, const uint32_t* __restrict__ state,
    const uint32_t* __restrict__ counts, uint64_t* __restrict__ cand) {
  __shared__ uint32_t sh[48];
  const int tid = threadIdx.x, tl = blockIdx.y, s = blockIdx.x;
  const uint32_t* st = state + 4 * tl;
  if (st[0] != kLongCand) return;  // (uniform over the workgroup)
  const uint32_t thr = st[1] << 21;
  const int n = row_len(bt, t_begin + tl);
  const float* row = scores + (int64_t)tl * ld;
  uint64_t* out = cand + (int64_t)tl * kLongCap;
  const int p0 = s * slice, p1 = min(n, p0 + slice);
  // this slice's offset: the candidates of the slices before it (s < 1024 threads)
  uint32_t base;
  block_excl_scan(tid < s ? counts[(int64_t)tl * kLongSlices + tid] : 0u, sh, base);
  const int iters = p1 > p0 ? (p1 - p0 + 4095) / 4096 : 0;
  for (int it = 0; it < iters; ++it) {
    const int p = p0 + 4096 * it + 4 * tid;
    uint32_t key[4];
    long_keys4(row, p, p1, key);
    uint32_t c = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) c += key[e] >= thr && key[e] != 0u ? 1u : 0u;
    __syncthreads();  // (sh of the previous scan has been read)
    uint32_t tot;
    uint32_t o = base + block_excl_scan(c, sh, tot);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (key[e] >= thr && key[e] != 0u) {
        if (o < (uint32_t)kLongCap) out[o] = ((uint64_t)key[e] << 32) | (uint32_t)(p + e);
        ++o;
      }
    }
    base += tot;
  }
}

__global__ __launch_bounds__(1024) void topk_long_final_kernel(DevBatch bt, int t_begin,
    const float* __restrict__ scores, int64_t ld, int K, const uint32_t* __restrict__ state,
    const uint64_t* __restrict__ cand, int32_t* __restrict__ out_idx,
    float* __restrict__ out_val) {
  extern __shared__ __attribute__((aligned(16))) char smraw[];
  SelSmem& S = *(SelSmem*)smraw;
  const int tid = threadIdx.x, tl = blockIdx.x;
  const int t = t_begin + tl;
  const uint32_t* st = state + 4 * tl;
  // the list, 8 consecutive entries per thread (position order), requested with the state
  // (entries past the list's end are not used)
  uint64_t cv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) cv[j] = cand[(int64_t)tl * kLongCap + 8 * tid + j];
  const uint32_t mode = st[0];
  if (mode == kLongOver) return;
  const float* row = scores + (int64_t)tl * ld;
  int32_t* oi = out_idx + (int64_t)t * K;
  float* ov = out_val ? out_val + (int64_t)t * K : nullptr;
  if (mode == kLongAll) {
    const int n = row_len(bt, t);
    for (int i = tid; i < K; i += 1024) {
      oi[i] = i < n ? i : -1;
      if (ov) ov[i] = i < n ? row[i] : 0.f;
    }
    return;
  }
  // key 0 past the list's end
  const uint32_t cnt = min(st[2], (uint32_t)kLongCap);
  uint32_t key[8], pos[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint64_t c = 8u * tid + j < cnt ? cv[j] : 0ull;
    key[j] = (uint32_t)(c >> 32);
    pos[j] = (uint32_t)c;
  }
  // the keys above the picked bin are all taken; the rest come from within it
  uint32_t krem = (uint32_t)K - st[3];
  const uint32_t T = radix_select(st[1] << 21, 21, krem, S, [&](auto&& f) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (key[j] != 0u) f(key[j]);
  });
  uint32_t gt = 0u, eq = 0u;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    gt += key[j] > T ? 1u : 0u;
    eq += key[j] == T ? 1u : 0u;
  }
  uint32_t tot;
  uint32_t er = block_excl_scan(eq, S.sh, tot);  // ties before this thread's
  const uint32_t teq = er < krem ? min(eq, krem - er) : 0u;
  __syncthreads();
  uint32_t o = block_excl_scan(gt + teq, S.sh, tot);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    bool sel = key[j] > T;
    if (key[j] == T) {
      sel = er < krem;
      ++er;
    }
    if (sel && o < (uint32_t)K) {  // (exactly K are selected; the bound keeps it in the row)
      oi[o] = (int32_t)pos[j];
      if (ov) ov[o] = key_value(key[j]);  // (the score; -0.0 comes out as +0.0)
      ++o;
    }
  }
}

bool topk_long_rows(int max_n, int K) { return max_n > 32768 && K <= kLongCap / 2; }
constexpr size_t kLongRowBytes = (size_t)kLongCap * 8 + 2048 * 4 + kLongSlices * 4 + 16;

// workspace of a launch over up to `rows` rows (any smaller launch fits in it too)
size_t topk_ws_bytes(int rows, int max_n, int K) {
  return topk_long_rows(max_n, K) ? (size_t)std::min(rows, kLongRows) * kLongRowBytes : 0;
}

hipError_t launch_topk(const DevBatch& bt, int t_begin, int t_count, int max_n,
                       const float* scores, int64_t ld, int K, int32_t* idx, float* val,
                       void* ws, hipStream_t st) {
  const uint32_t* only = nullptr;
  if (t_count <= kLongRows && topk_long_rows(max_n, K)) {
    // ws: candidates [t_count][kLongCap] | histograms [t_count][2048] |
    //     slice counts [t_count][kLongSlices] | state [t_count][4]
    uint64_t* cand = (uint64_t*)ws;
    uint32_t* hist = (uint32_t*)(cand + (size_t)t_count * kLongCap);
    uint32_t* counts = hist + (size_t)t_count * 2048;
    uint32_t* state = counts + (size_t)t_count * kLongSlices;
    // slices of a multiple of 4096 positions, about 1024 workgroups in all (at most
    // kLongSlices per row)
    const int S = std::min((max_n + 8191) / 8192, std::max(1, kLongSlices / t_count));
    const int slice = ((max_n + S - 1) / S + 4095) / 4096 * 4096;
    const int nsl = (max_n + slice - 1) / slice;
    hipLaunchKernelGGL(topk_long_zero_kernel, dim3(t_count), dim3(256), 0, st, hist, state);
    hipLaunchKernelGGL(topk_long_hist_kernel, dim3(nsl, t_count), dim3(256), 0, st, bt, t_begin,
                       scores, ld, K, slice, hist);
    hipLaunchKernelGGL(topk_long_pick_kernel, dim3(t_count), dim3(1024), 0, st, bt, t_begin, K,
                       hist, state);
    hipLaunchKernelGGL(topk_long_count_kernel, dim3(nsl, t_count), dim3(256), 0, st, bt,
                       t_begin, scores, ld, slice, state, counts);
    hipLaunchKernelGGL(topk_long_write_kernel, dim3(nsl, t_count), dim3(1024), 0, st, bt,
                       t_begin, scores, ld, slice, state, counts, cand);
    const size_t fshm = sizeof(SelSmem);
    hipError_t e = hipFuncSetAttribute((const void*)topk_long_final_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)fshm);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_long_final_kernel, dim3(t_count), dim3(1024), fshm, st, bt, t_begin,
                       scores, ld, K, state, cand, idx, val);
    only = state;  // the one-workgroup kernel below finishes the rows marked as overflowing
  }
  // keys per thread: the smallest power of two (>= 4) that keeps the longest row in registers,
  // up to 32 (32768 positions); longer rows stream through 1024*32-key chunks per pass
  int npt = 4;
  while (npt < 32 && 1024 * npt < max_n) npt *= 2;
  auto* fn = npt == 4 ? topk_select_kernel<4>
             : npt == 8 ? topk_select_kernel<8>
             : npt == 16 ? topk_select_kernel<16> : topk_select_kernel<32>;
  // dynamic LDS: the selection's, or the first chunk's transposition if larger
  const size_t shm = std::max(sizeof(SelSmem), (size_t)4096 * (size_t)npt);
  hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)shm);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3(t_count), dim3(1024), shm, st, bt, t_begin, scores, ld, K, only,
                     idx, val);
  return hipGetLastError();
}

}  // namespace tis
