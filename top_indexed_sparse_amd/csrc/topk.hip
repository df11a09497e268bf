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

// LDS of the streamed selection (rows longer than one chunk) and of the long-row final step:
// two histograms, scan scratch and picks.
struct SelSmem {
  uint32_t hist[2048];
  uint32_t hist2[2048];
  uint32_t sh[48];    // scan totals (0..15), row min/max (16..47)
  uint32_t pick[4];
};

// Long-row selection state per row, words [mode, tlo, candidates reserved, -]
constexpr uint32_t kLongCand = 0u, kLongAll = 1u;
constexpr int kLongCap = 8192;      // candidate positions per row (8 per thread of the last step)
constexpr int kLongRows = 64;       // at most this many rows per launch take the long-row path
constexpr int kLongSlice = 16384;   // entries per slice

// Radix select of the krem-th largest key among the keys produced by `each` (called with a
// visitor), over r = key - base with digits of up to 11 bits from bit `hi` down.  Returns the
// threshold key; krem is left as the number of keys equal to it that are taken.  The two
// 2048-bin histograms h0 and h1 alternate, the next one being cleared while the current one
// fills: three barriers per digit.  sh: 16 words of scan scratch; pick: 2 words.
template <typename Each>
__device__ __forceinline__ uint32_t radix_select(uint32_t base, int hi, uint32_t& krem,
                                                 uint32_t* h0, uint32_t* h1, uint32_t* sh,
                                                 uint32_t* pick, Each each) {
  const int tid = threadIdx.x;
  uint32_t* hb[2] = {h0, h1};
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
    const uint32_t above_h = block_excl_scan(ch + cl, sh, tot);
    const uint32_t above_l = above_h + ch;
    if (ch && above_h < krem && krem <= above_h + ch) {
      pick[0] = 2047 - 2 * tid;
      pick[1] = above_h;
    }
    if (cl && above_l < krem && krem <= above_l + cl) {
      pick[0] = 2046 - 2 * tid;
      pick[1] = above_l;
    }
    __syncthreads();
    prefix = (prefix << (hi - lo)) | pick[0];
    krem -= pick[1];
    hi = lo;
    cur ^= 1;
  }
  return base + prefix;
}
template <typename Each>
__device__ __forceinline__ uint32_t radix_select(uint32_t base, int hi, uint32_t& krem,
                                                 SelSmem& S, Each each) {
  return radix_select(base, hi, krem, S.hist, S.hist2, S.sh, S.pick, each);
}

// Bin of the want-th largest count over 2048 bins, counted from the top (thread i owns bins
// 2047-2i and 2046-2i).  The thread whose bins hold it writes [bin, count above it, its
// count] to pick[0..2]; one barrier inside the scan, none after (the caller's follows).
__device__ __forceinline__ void pick_bin(const uint32_t* h, uint32_t want, uint32_t* sh,
                                         uint32_t* pick) {
  const int tid = threadIdx.x;
  const uint32_t ch = h[2047 - 2 * tid], cl = h[2046 - 2 * tid];
  uint32_t tot;
  const uint32_t above_h = block_excl_scan(ch + cl, sh, tot);
  const uint32_t above_l = above_h + ch;
  if (ch && above_h < want && want <= above_h + ch) {
    pick[0] = 2047 - 2 * tid;
    pick[1] = above_h;
    pick[2] = ch;
  }
  if (cl && above_l < want && want <= above_l + cl) {
    pick[0] = 2046 - 2 * tid;
    pick[1] = above_l;
    pick[2] = cl;
  }
}

// ---------------------------------------------------------------- rows held on chip
// A row of at most 1024*NPT entries stays on the CU.  Thread (wave w, lane l) keeps the
// 16-byte pieces it loaded, piece i = scores of positions 64*NPT*w + 256*i + 4*l .. + 3
// (coalesced loads, no transposition), and the row is also written to LDS in position
// order.  Entries past the row are NaN (scores are never NaN), so no comparison selects them.
//  1. Sample: two scores per thread, lane l taking the first score of pieces l mod (NPT/8)
//     and l mod (NPT/8) + NPT/8 (positions at a stride of NPT/2 over the row), histogrammed
//     over the sample's key range; the bin where the count from the top reaches 1.25x the
//     expected share of K (+16) gives a lower bound tlo of the K-th largest key.
//  2. One pass over the registers: each score is compared with tlo's value and the result
//     shifted into a per-thread bit mask; the row maximum comes along.
//  3. Each wave reserves room in an LDS list with one atomic and writes its candidates'
//     positions (the set bits of the masks), in no particular order.
//  4. The candidates' keys (read from the LDS row) are histogrammed over [tlo, max]; a scan
//     finds the bin of the K-th largest.  Keys above the bin are taken.  A bin taken whole
//     ends the search; a bin of at most 64 keys is ranked by one wave; a larger one is
//     histogrammed again over its own range, down to single key values.  The result is the
//     threshold key T and the number of keys equal to T that are taken.
//  5. Taken positions are set in an LDS bitmap, the ties at T in a second one.  Thread i
//     emits the set bits of word i at its offset from one scan of (taken, tie) counts, with
//     ties in position order up to their quota: the output is in ascending position order.
// When fewer than K, or more than the list holds, reach tlo (heavy ties, adversarial orders),
// an exact radix select over the registers gives T, and the bitmaps come from the registers.
constexpr int kResListMax = 3904;  // candidate positions of a row held on chip
constexpr int kResRankMax = 64;    // keys of a bin ranked by one wave

template <int NPT>
struct ResLds {  // byte offsets in the dynamic LDS
  static constexpr int CH = 1024 * NPT;
  static constexpr size_t row = 0;                        // float[CH], position order
  static constexpr size_t hA = row + 4 * (size_t)CH;      // u32[2048]: sample histogram, bitmaps
  static constexpr size_t hB = hA + 8192;                 // u32[2048]: candidate histogram
  static constexpr size_t list = hB + 8192;               // u32[kResListMax]: positions
  static constexpr size_t rank = list + 4 * kResListMax;  // u32[2][kResRankMax]: (key, position)
  static constexpr size_t sh = rank + 8 * kResRankMax;    // u32[48]: scan scratch, min/max
  static constexpr size_t misc = sh + 192;                // u32[8]: picks, counters
  static constexpr size_t bytes = misc + 32;
};
static_assert(ResLds<32>::bytes <= 160 * 1024, "a row held on chip fits the CU's LDS");

template <int NPT>
__device__ __forceinline__ void select_resident(const uint4 (&v)[NPT / 4], int n, int k,
                                                char* smraw, int32_t* __restrict__ oi,
                                                float* __restrict__ ov) {
  using L = ResLds<NPT>;
  constexpr int Q = NPT / 4, CH = L::CH, NW = CH / 32;  // pieces per thread, bitmap words
  const int tid = threadIdx.x, lane = tid & 63;
  float* rowf = (float*)(smraw + L::row);
  uint32_t* hA = (uint32_t*)(smraw + L::hA);
  uint32_t* hB = (uint32_t*)(smraw + L::hB);
  uint32_t* list = (uint32_t*)(smraw + L::list);
  uint32_t* rk = (uint32_t*)(smraw + L::rank);
  uint32_t* sh = (uint32_t*)(smraw + L::sh);
  uint32_t* pick = (uint32_t*)(smraw + L::misc);  // [bin, above, count, tie quota]
  uint32_t* cnt = pick + 4;                       // [list length, max key, rank fill]
  const int pl = (tid >> 6) * 64 * NPT + 4 * lane;  // position of piece 0's first score

  float x[NPT];  // x[4i + e]: position pl + 256i + e
#pragma unroll
  for (int i = 0; i < Q; ++i) {
    x[4 * i] = __uint_as_float(v[i].x);
    x[4 * i + 1] = __uint_as_float(v[i].y);
    x[4 * i + 2] = __uint_as_float(v[i].z);
    x[4 * i + 3] = __uint_as_float(v[i].w);
  }
  if (!__all(pl - 4 * lane + 64 * NPT <= n)) {  // (the wave's span crosses the row's end)
#pragma unroll
    for (int j = 0; j < NPT; ++j)
      if (pl + 256 * (j >> 2) + (j & 3) >= n) x[j] = __uint_as_float(0x7fc00000u);
  }
#pragma unroll
  for (int i = 0; i < Q; ++i)
    *(float4*)(rowf + pl + 256 * i) = make_float4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
  hA[tid] = 0u;
  hA[tid + 1024] = 0u;
  hB[tid] = 0u;
  hB[tid + 1024] = 0u;
  if (tid < 8) pick[tid] = 0u;  // (picks and counters)

  // ---- 1. sampled lower bound (the sample's min/max barrier also orders the clears above)
  float sa, sb;
  if constexpr (Q == 1) {
    sa = x[0];
    sb = x[2];
  } else {
    constexpr int H = Q / 2;
    const int r = lane & (H - 1);
    sa = x[0];
    sb = x[4 * H];
#pragma unroll
    for (int i = 1; i < H; ++i)
      if (r == i) {
        sa = x[4 * i];
        sb = x[4 * (i + H)];
      }
  }
  const uint32_t ka = sa == sa ? order_key(sa) : 0u, kb = sb == sb ? order_key(sb) : 0u;
  uint32_t smin1 = min(ka - 1u, kb - 1u), smax = max(ka, kb);  // (invalid key 0 -> ~0u)
  block_minmax(smin1, smax, sh + 16);
  const uint32_t smin = smin1 + 1u;
  const uint32_t sspan = smax - smin;
  const int shift = max(0, (sspan ? 32 - __clz(sspan) : 0) - 11);
  if (ka) atomicAdd(&hA[(ka - smin) >> shift], 1u);
  if (kb) atomicAdd(&hA[(kb - smin) >> shift], 1u);
  __syncthreads();
  {
    const uint32_t ch = hA[2047 - 2 * tid], cl = hA[2046 - 2 * tid];
    uint32_t tot;  // valid samples
    const uint32_t above_h = block_excl_scan(ch + cl, sh, tot);
    const uint32_t want =
        min(tot, (uint32_t)(((uint64_t)k * tot * 5u) / (4ull * (uint64_t)n)) + 16u);
    const uint32_t above_l = above_h + ch;
    if (ch && above_h < want && want <= above_h + ch) pick[2] = 2047 - 2 * tid;
    if (cl && above_l < want && want <= above_l + cl) pick[2] = 2046 - 2 * tid;
    __syncthreads();
  }
  const uint32_t tlo = smin + (pick[2] << shift);

  // ---- 2. candidate masks (bit NPT-1-j: score j reaches tlo) and the row maximum
  const float tf = key_value(tlo);  // (x >= tf exactly when order_key(x) >= tlo)
  uint32_t m = 0u;
  float rmax = -INFINITY;
#pragma unroll
  for (int j = 0; j < NPT; ++j) {
    // m = 2m + (x >= tf): the compare's lane mask is the carry-in of one add (with the two
    // wait states a carry read needs after the compare writes it)
    asm("v_cmp_le_f32_e32 vcc, %2, %1\n\ts_nop 1\n\tv_addc_co_u32_e32 %0, vcc, %3, %3, vcc"
        : "=v"(m) : "v"(x[j]), "s"(tf), "v"(m) : "vcc");
    rmax = fmaxf(rmax, x[j]);  // (NaN entries are skipped)
  }
  // ---- 3. the wave's candidates into the list
  {
    const uint32_t c = __popc(m);
    const uint32_t inc = wave_incl_scan(c);
    uint32_t base = 0u;
    if (lane == 63) base = atomicAdd(&cnt[0], inc);
    uint32_t o = __builtin_amdgcn_readlane(base, 63) + inc - c;
    for (uint32_t mm = m; mm; mm &= mm - 1u, ++o) {
      const int j = NPT - 1 - __builtin_ctz(mm);
      if (o < (uint32_t)kResListMax) list[o] = (uint32_t)(pl + 256 * (j >> 2) + (j & 3));
    }
    auto fmax_ = [](uint32_t a, uint32_t b) { return max(a, b); };
    const uint32_t wm = wave_incl(order_key(rmax), 0u, fmax_);
    if (lane == 63) atomicMax(&cnt[1], wm);
  }
  __syncthreads();
  const uint32_t C = cnt[0];
  uint32_t* taken;
  uint32_t* ties;
  uint32_t quota;  // keys equal to the threshold that are taken (first in position order)

  if (C >= (uint32_t)k && C <= (uint32_t)kResListMax) {
    // ---- 4. histogram of the candidates over [tlo, max]
    const uint32_t kmax = cnt[1];
    const uint32_t cspan = kmax - tlo;
    const int shift2 = max(0, (cspan ? 32 - __clz(cspan) : 0) - 11);
    constexpr int E = (kResListMax + 1023) / 1024;
    uint32_t lk[E], lp[E];  // entry tid + 1024e: key (0 past the list) and position
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t i = (uint32_t)tid + 1024u * e;
      lp[e] = i < C ? list[i] : 0u;
      lk[e] = i < C ? order_key(rowf[lp[e]]) : 0u;
      if (i < C) atomicAdd(&hB[(lk[e] - tlo) >> shift2], 1u);
    }
    hA[tid] = 0u;  // (the bitmaps; the sample histogram was last read before tlo's barrier)
    hA[tid + 1024] = 0u;
    __syncthreads();
    pick_bin(hB, (uint32_t)k, sh, pick);
    __syncthreads();
    uint32_t lo = tlo + (pick[0] << shift2);  // the bin: keys lo .. lo + 2^s - 1
    int s = shift2;
    uint32_t cb = pick[2];
    uint32_t krem = (uint32_t)k - pick[1];    // keys of the bin that are taken
    taken = hA;
    ties = hA + NW;
    auto mark = [&](uint32_t* w, uint32_t p) { atomicOr(&w[p >> 5], 1u << (p & 31)); };
    auto top_of = [](uint32_t l, int sb) {
      return (uint32_t)min<uint64_t>((uint64_t)l + ((1ull << sb) - 1ull), 0xffffffffull);
    };
    if (cb != krem && cb <= (uint32_t)kResRankMax && s > 0) {
      // a few keys in the bin: keys above it are taken now, the bin's keys are collected
      // and ranked by one wave, which takes them or marks the ties
      const uint32_t hi = top_of(lo, s);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (lk[e] > hi) mark(taken, lp[e]);
        else if (lk[e] >= lo) {
          const uint32_t sl = atomicAdd(&cnt[2], 1u);  // (< cb <= kResRankMax)
          rk[2 * sl] = lk[e];
          rk[2 * sl + 1] = lp[e];
        }
      }
      __syncthreads();
      if (tid < 64) {
        const bool has = (uint32_t)tid < cb;
        const uint32_t mine = has ? rk[2 * tid] : 0u, mp = has ? rk[2 * tid + 1] : 0u;
        uint32_t gt = 0u, ge = 0u;
        for (uint32_t j = 0; j < cb; ++j) {  // (lane j holds key j)
          const uint32_t ot = __builtin_amdgcn_readlane(mine, j);
          gt += ot > mine ? 1u : 0u;
          ge += ot >= mine ? 1u : 0u;
        }
        if (has && ge <= krem) mark(taken, mp);  // (every key >= this one fits)
        else if (has && gt < krem) {             // this key is the threshold: a tie
          mark(ties, mp);
          pick[3] = krem - gt;                   // (the same value from every tie)
        }
      }
      __syncthreads();
      quota = pick[3];
    } else {
      // threshold (T, quota): the bin taken whole, a bin of one key value, or narrower bins
      // (histograms alternating between hB and hA) down to a rank by one wave
      uint32_t T;
      uint32_t* hc = hA;
      uint32_t* hn = hB;
      bool used_a = false;
      while (true) {
        if (cb == krem) {  // the whole bin: every key >= lo, no ties
          T = lo - 1u;
          quota = 0u;
          break;
        }
        if (s == 0) {  // every key of the bin equals lo
          T = lo;
          quota = krem;
          break;
        }
        const uint32_t hi = top_of(lo, s);
        if (cb <= (uint32_t)kResRankMax) {
#pragma unroll
          for (int e = 0; e < E; ++e)
            if (lk[e] >= lo && lk[e] <= hi) {
              const uint32_t sl = atomicAdd(&cnt[2], 1u);
              rk[2 * sl] = lk[e];
            }
          __syncthreads();
          if (tid < 64) {
            const bool has = (uint32_t)tid < cb;
            const uint32_t mine = has ? rk[2 * tid] : 0u;
            uint32_t gt = 0u, ge = 0u;
            for (uint32_t j = 0; j < cb; ++j) {
              const uint32_t ot = __builtin_amdgcn_readlane(mine, j);
              gt += ot > mine ? 1u : 0u;
              ge += ot >= mine ? 1u : 0u;
            }
            if (has && gt < krem && krem <= ge) {  // the krem-th largest of the bin
              pick[0] = mine;
              pick[1] = krem - gt;
            }
          }
          __syncthreads();
          T = pick[0];
          quota = pick[1];
          break;
        }
        const int s2 = max(0, s - 11);
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (lk[e] >= lo && lk[e] <= hi) atomicAdd(&hc[(lk[e] - lo) >> s2], 1u);
        hn[tid] = 0u;
        hn[tid + 1024] = 0u;
        used_a = true;
        __syncthreads();
        pick_bin(hc, krem, sh, pick);
        __syncthreads();
        lo += pick[0] << s2;
        krem -= pick[1];
        cb = pick[2];
        s = s2;
        uint32_t* t0 = hc;
        hc = hn;
        hn = t0;
      }
      if (used_a) {  // (the bitmaps held a histogram)
        __syncthreads();
        hA[tid] = 0u;
        hA[tid + 1024] = 0u;
      }
      __syncthreads();
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (lk[e] > T) mark(taken, lp[e]);
        else if (lk[e] == T && lk[e] != 0u) mark(ties, lp[e]);
      }
      __syncthreads();
    }
  } else {
    // ---- exact radix select over the registers (keys; 0 for entries past the row)
    uint32_t kk[NPT];
#pragma unroll
    for (int j = 0; j < NPT; ++j) kk[j] = x[j] == x[j] ? order_key(x[j]) : 0u;
    uint32_t kmin = ~0u, kmx = 0u;
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      kmin = min(kmin, kk[j] - 1u);
      kmx = max(kmx, kk[j]);
    }
    block_minmax(kmin, kmx, sh + 16);
    kmin += 1u;
    taken = list;  // (the list is not used on this path)
    ties = list + NW;
    for (int i = tid; i < 2 * NW; i += 1024) list[i] = 0u;
    const uint32_t span = kmx - kmin;
    quota = (uint32_t)k;
    const uint32_t T = radix_select(kmin, span ? 32 - __clz(span) : 0, quota, hA, hB, sh, pick,
                                    [&](auto&& f) {
#pragma unroll
                                      for (int j = 0; j < NPT; ++j)
                                        if (kk[j] != 0u) f(kk[j]);
                                    });
#pragma unroll
    for (int i = 0; i < Q; ++i) {
      uint32_t g = 0u, q = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t kx = kk[4 * i + e];
        g |= (kx > T ? 1u : 0u) << e;
        q |= (kx == T && kx != 0u ? 1u : 0u) << e;
      }
      const int p = pl + 256 * i;  // (the piece's four positions share a bitmap word)
      if (g) atomicOr(&taken[p >> 5], g << (p & 31));
      if (q) atomicOr(&ties[p >> 5], q << (p & 31));
    }
    __syncthreads();
  }

  // ---- 5. emission: thread i owns bitmap word i (positions 32i .. 32i + 31)
  uint32_t tw = 0u, ew = 0u;
  if (tid < NW) {
    tw = taken[tid];
    ew = ties[tid];
  }
  uint32_t tot;
  const uint32_t before = block_excl_scan(__popc(tw) | ((uint32_t)__popc(ew) << 16), sh, tot);
  const uint32_t eb = before >> 16;  // ties before this thread's
  uint32_t o = (before & 0xffffu) + min(eb, quota);
  for (uint32_t a = quota > eb ? quota - eb : 0u; a && ew; --a) {
    tw |= ew & (0u - ew);  // the lowest remaining tie
    ew &= ew - 1u;
  }
  while (tw) {  // four positions at a time, their values read together
    int pp[4];
    float vv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pp[e] = tw ? 32 * tid + __builtin_ctz(tw) : -1;
      tw &= tw - 1u;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) vv[e] = pp[e] >= 0 ? rowf[pp[e]] : 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (pp[e] >= 0 && o < (uint32_t)k) {  // (exactly k are set; the bound keeps every
        oi[o] = pp[e];                      //  store in the row)
        if (ov) ov[o] = vv[e] + 0.f;        // (+ 0: -0.0 comes out as +0.0, as from a key)
        ++o;
      }
  }
}

// ---------------------------------------------------------------- rows longer than a chunk
// Rows longer than 1024*32 entries, first attempt: the threshold search of rows held on chip,
// with the row read once.
//  1. A uniform sample of 2048 scores (positions floor(s n / 2048)) gives tlo as above.
//  2. One pass over the row in 32K-entry chunks of coalesced pieces (thread (w, l), piece i:
//     positions c0 + 2048w + 256i + 4l .. + 3) lists the positions of the scores >= tlo in
//     position order: per piece a wave scan of the lanes' counts, per chunk a scan of the
//     waves' totals.
//  3. The candidates' keys are read back by position (thread i owns list entries 8i .. 8i + 7);
//     the threshold key T and the quota of ties at T come from the candidate histogram, bins
//     narrowed down to a rank by one wave or to a single key value.
//  4. A block scan of (> T, == T) counts compacts the list in position order.
// Returns false, having written nothing, when fewer than K or more than the list holds reach
// tlo; the caller then runs the exact streamed radix select.
constexpr int kStreamListMax = 8192;  // candidate positions of a streamed row
struct StreamLds {
  uint32_t hA[2048];
  uint32_t hB[2048];
  uint32_t list[kStreamListMax];
  uint32_t rk[64];
  uint32_t sh[48];   // scan totals (0..15), min/max (16..47)
  uint32_t pick[4];  // [bin or T, above or quota, count, -]
  uint32_t cnt[4];   // [rank fill]
};

// Threshold and compaction over a position-ordered candidate list: thread i holds entries
// E*i .. E*i + E - 1 (keys, 0 past the list, and positions); every listed key is >= tlo and kmax
// is the largest.  The candidate histogram over [tlo, kmax] puts the K-th largest in one bin;
// the bin taken whole ends the search, a bin of one key value fixes it, a bin of at most 64
// keys is ranked by one wave (lane j holds key j, the others read with readlane), a larger bin
// is histogrammed again over its own range.  Then one block scan of (> T, == T) counts writes
// the keys > T and the first `quota` keys == T in list order.  S.hB and S.cnt[0] must be zero,
// and visible to every thread, on entry.
template <int E>
__device__ __forceinline__ void select_listed(const uint32_t (&lk)[E], const uint32_t (&lp)[E],
                                              uint32_t tlo, uint32_t kmax, int k, StreamLds& S,
                                              int32_t* __restrict__ oi, float* __restrict__ ov) {
  const int tid = threadIdx.x;
  const uint32_t cspan = kmax - tlo;
  const int shift2 = max(0, (cspan ? 32 - __clz(cspan) : 0) - 11);
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (lk[e] != 0u) atomicAdd(&S.hB[(lk[e] - tlo) >> shift2], 1u);
  S.hA[tid] = 0u;  // (hA's earlier contents were last read before the caller's last barrier)
  S.hA[tid + 1024] = 0u;
  __syncthreads();
  pick_bin(S.hB, (uint32_t)k, S.sh, S.pick);
  __syncthreads();
  uint32_t lo = tlo + (S.pick[0] << shift2);  // the bin: keys lo .. lo + 2^s - 1
  int s = shift2;
  uint32_t cb = S.pick[2];
  uint32_t krem = (uint32_t)k - S.pick[1];
  uint32_t T, quota;
  uint32_t* hc = S.hA;
  uint32_t* hn = S.hB;
  while (true) {
    if (cb == krem) {  // the whole bin: every key >= lo, no ties
      T = lo - 1u;
      quota = 0u;
      break;
    }
    if (s == 0) {  // every key of the bin equals lo
      T = lo;
      quota = krem;
      break;
    }
    const uint32_t hi =
        (uint32_t)min<uint64_t>((uint64_t)lo + ((1ull << s) - 1ull), 0xffffffffull);
    if (cb <= 64u) {  // one wave ranks the bin's keys (lane j holds key j)
      __syncthreads();  // (the previous level's picks have been read)
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (lk[e] >= lo && lk[e] <= hi) S.rk[atomicAdd(&S.cnt[0], 1u)] = lk[e];
      __syncthreads();
      if (tid < 64) {
        const bool has = (uint32_t)tid < cb;
        const uint32_t mine = has ? S.rk[tid] : 0u;
        uint32_t gt = 0u, ge = 0u;
        for (uint32_t j = 0; j < cb; ++j) {
          const uint32_t ot = __builtin_amdgcn_readlane(mine, j);
          gt += ot > mine ? 1u : 0u;
          ge += ot >= mine ? 1u : 0u;
        }
        if (has && gt < krem && krem <= ge) {  // the krem-th largest of the bin
          S.pick[0] = mine;
          S.pick[1] = krem - gt;
        }
      }
      __syncthreads();
      T = S.pick[0];
      quota = S.pick[1];
      break;
    }
    const int s2 = max(0, s - 11);
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (lk[e] >= lo && lk[e] <= hi) atomicAdd(&hc[(lk[e] - lo) >> s2], 1u);
    hn[tid] = 0u;
    hn[tid + 1024] = 0u;
    __syncthreads();
    pick_bin(hc, krem, S.sh, S.pick);
    __syncthreads();
    lo += S.pick[0] << s2;
    krem -= S.pick[1];
    cb = S.pick[2];
    s = s2;
    uint32_t* t0 = hc;
    hc = hn;
    hn = t0;
  }

  // ---- 4. compaction in list (= position) order
  uint32_t cgt = 0u, ceq = 0u;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    cgt += lk[e] > T ? 1u : 0u;
    ceq += lk[e] == T && lk[e] != 0u ? 1u : 0u;
  }
  uint32_t tot;
  __syncthreads();  // (sh: the last pick's scan)
  const uint32_t bsc = block_excl_scan(cgt | (ceq << 16), S.sh, tot);
  uint32_t eb = bsc >> 16;  // ties before this thread's
  uint32_t o = (bsc & 0xffffu) + min(eb, quota);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool eq = lk[e] == T && lk[e] != 0u;
    if ((lk[e] > T || (eq && eb < quota)) && o < (uint32_t)k) {
      oi[o] = (int32_t)lp[e];
      if (ov) ov[o] = key_value(lk[e]);  // (the score; -0.0 comes out as +0.0)
      ++o;
    }
    eb += eq ? 1u : 0u;
  }
}

__device__ __forceinline__ bool select_stream_list(const float* __restrict__ row, int n, int k,
                                                   char* smraw, int32_t* __restrict__ oi,
                                                   float* __restrict__ ov) {
  constexpr int CH = 1024 * 32, E = kStreamListMax / 1024;
  StreamLds& S = *(StreamLds*)smraw;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  S.hA[tid] = 0u;
  S.hA[tid + 1024] = 0u;
  S.hB[tid] = 0u;
  S.hB[tid + 1024] = 0u;
  if (tid < 4) S.pick[tid] = 0u;
  else if (tid < 8) S.cnt[tid - 4] = 0u;

  // ---- 1. sampled lower bound (the min/max barrier also orders the clears above)
  const uint32_t ka = order_key(row[(int)(((int64_t)tid * n) >> 11)]);
  const uint32_t kb = order_key(row[(int)(((int64_t)(tid + 1024) * n) >> 11)]);
  uint32_t smin = min(ka, kb), smax = max(ka, kb);
  block_minmax(smin, smax, S.sh + 16);
  const uint32_t sspan = smax - smin;
  const int shift = max(0, (sspan ? 32 - __clz(sspan) : 0) - 11);
  atomicAdd(&S.hA[(ka - smin) >> shift], 1u);
  atomicAdd(&S.hA[(kb - smin) >> shift], 1u);
  __syncthreads();
  {
    const uint32_t want = min(2048u, (uint32_t)(((uint64_t)k * 2048u * 5u) / (4ull * n)) + 16u);
    pick_bin(S.hA, want, S.sh, S.pick);
    __syncthreads();
  }
  const uint32_t tlo = smin + (S.pick[0] << shift);
  const float tf = key_value(tlo);  // (x >= tf exactly when order_key(x) >= tlo)

  // ---- 2. the candidates' positions, in position order, and the row maximum
  uint32_t run = 0u;  // entries listed so far
  float rmax = -INFINITY;
  const int pl = wave * 2048 + 4 * lane;
  for (int c0 = 0; c0 < n; c0 += CH) {
    float x[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = c0 + pl + 256 * i;
      if (p + 3 < n) {
        const float4 f = *(const float4*)(row + p);
        x[4 * i] = f.x; x[4 * i + 1] = f.y; x[4 * i + 2] = f.z; x[4 * i + 3] = f.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          x[4 * i + e] = p + e < n ? row[p + e] : __uint_as_float(0x7fc00000u);  // (NaN)
      }
    }
    uint32_t bits[8], ex[8], wbase[8];
    uint32_t wtot = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      bits[i] = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bits[i] |= (x[4 * i + e] >= tf ? 1u : 0u) << e;
        rmax = fmaxf(rmax, x[4 * i + e]);  // (NaN entries are skipped)
      }
      const uint32_t c = __popc(bits[i]);
      const uint32_t inc = wave_incl_scan(c);
      ex[i] = inc - c;
      wbase[i] = wtot;
      wtot += __builtin_amdgcn_readlane(inc, 63);
    }
    if (lane == 0) S.sh[wave] = wtot;
    __syncthreads();
    const uint32_t ws = wave_incl_scan(lane < 16 ? S.sh[lane] : 0u);
    const uint32_t before = wave ? __builtin_amdgcn_readlane(ws, wave - 1) : 0u;
    const uint32_t ctot = __builtin_amdgcn_readlane(ws, 15);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t o = run + before + wbase[i] + ex[i];
      const uint32_t p = (uint32_t)(c0 + pl + 256 * i);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((bits[i] >> e) & 1u) {
          if (o < (uint32_t)kStreamListMax) S.list[o] = p + e;
          ++o;
        }
    }
    run += ctot;
    __syncthreads();  // (the next chunk's scan writes sh)
  }
  const uint32_t C = run;  // (uniform)
  uint32_t kmin_unused = ~0u, kmax = order_key(rmax);
  block_minmax(kmin_unused, kmax, S.sh + 16);  // (its barrier also publishes the list)
  if (C < (uint32_t)k || C > (uint32_t)kStreamListMax) return false;

  // ---- 3. keys by position; histogram over [tlo, max]; the threshold
  uint32_t lk[E], lp[E];  // entries E*tid .. : key (0 past the list) and position
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t i = (uint32_t)(E * tid + e);
    lp[e] = i < C ? S.list[i] : 0u;
    lk[e] = i < C ? order_key(row[lp[e]]) : 0u;
  }
  select_listed<E>(lk, lp, tlo, kmax, k, S, oi, ov);
  return true;
}

// Exact fallback: each pass streams the row through registers, thread i holding 32
// consecutive positions of each chunk.  The key range is measured, then a radix select
// over the whole row gives T; the compaction keeps keys > T and the first krem keys == T
// chunk by chunk, one block scan per chunk.
__device__ __forceinline__ void select_streamed(const float* __restrict__ row, int n, int k,
                                                int K, char* smraw, int32_t* __restrict__ oi,
                                                float* __restrict__ ov) {
  constexpr int NPT = 32, CH = 1024 * NPT;
  SelSmem& S = *(SelSmem*)smraw;
  const int tid = threadIdx.x;
  uint32_t key[NPT];
  auto load_chunk = [&](int c0) {
    const int p0 = c0 + tid * NPT;
#pragma unroll
    for (int j = 0; j < NPT; j += 4) {
      const int p = p0 + j;
      if (p + 3 < n) {
        const uint4 f = *(const uint4*)(row + p);
        key[j] = f.x; key[j + 1] = f.y; key[j + 2] = f.z; key[j + 3] = f.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) key[j + e] = (p + e < n) ? __float_as_uint(row[p + e]) : 0u;
      }
    }
    // positions past the row hold key 0, which no score maps to (the smallest key, of -inf,
    // is 0x007fffff)
    if (__all(p0 + NPT <= n)) {
#pragma unroll
      for (int j = 0; j < NPT; ++j) key[j] = order_key(__uint_as_float(key[j]));
    } else {
#pragma unroll
      for (int j = 0; j < NPT; ++j)
        key[j] = p0 + j < n ? order_key(__uint_as_float(key[j])) : 0u;
    }
  };
  auto each_row = [&](auto&& f) {
    for (int c0 = 0; c0 < n; c0 += CH) {
      load_chunk(c0);
#pragma unroll
      for (int j = 0; j < NPT; ++j)
        if (key[j] != 0u) f(key[j]);
    }
  };
  uint32_t kmin = ~0u, kmax = 0u;
  each_row([&](uint32_t kk) { kmin = min(kmin, kk); kmax = max(kmax, kk); });
  block_minmax(kmin, kmax, S.sh + 16);
  const uint32_t span = kmax - kmin;
  uint32_t krem = (uint32_t)k;
  const uint32_t T = radix_select(kmin, span ? 32 - __clz(span) : 0, krem, S, each_row);
  // T is the threshold key; krem elements equal to T are taken (in position order).
  // Order-preserving compaction: one scan of the per-thread counts of keys > T (low 16 bits)
  // and == T (high 16 bits; both totals stay below 2^16 per chunk).
  uint32_t run_gt = 0u, run_eq = 0u;
  for (int c0 = 0; c0 < n; c0 += CH) {
    load_chunk(c0);
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
    __syncthreads();  // (the next chunk's scan writes sh)
  }
  for (int i = k + tid; i < K; i += 1024) {
    oi[i] = -1;
    if (ov) ov[i] = 0.f;
  }
}

// One 1024-thread workgroup per row of at most 1024*NPT entries (longer rows are left to
// topk_stream_kernel).  The first 1024*NPT entries are requested as coalesced 16-byte pieces
// before the token's causal length is known (up to the row stride, which bounds every causal
// length), so the two memory latencies overlap.
template <int NPT>
__global__ __launch_bounds__(1024) void topk_select_kernel(DevBatch bt, int t_begin,
    const float* __restrict__ scores, int64_t ld, int K, int32_t* __restrict__ out_idx,
    float* __restrict__ out_val) {
  extern __shared__ __attribute__((aligned(16))) char smraw[];
  const int tid = threadIdx.x;
  const int tl = blockIdx.x;
  const int t = t_begin + tl;
  const float* row = scores + (int64_t)tl * ld;
  constexpr int CH = 1024 * NPT, Q = NPT / 4;

  const LocLoads lw = locate_issue(bt);
  uint4 v[Q];
  {
    const int lim = (int)min<int64_t>(ld, (int64_t)CH);  // (ld is a multiple of 4)
    const int pl = (tid >> 6) * 64 * NPT + 4 * (tid & 63);
#pragma unroll
    for (int i = 0; i < Q; ++i) {
      const int p = pl + 256 * i;
      v[i] = *(const uint4*)(row + min(p, lim - 4));
      if (p >= lim) v[i] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  int n = locate_finish(bt, t, lw).n;
  n = (n + (1 << bt.row_shift) - 1) >> bt.row_shift;  // (block rows: pages, not positions)
  int32_t* oi = out_idx + (int64_t)t * K;
  float* ov = out_val ? out_val + (int64_t)t * K : nullptr;

  if (n > CH) return;
  if (n <= K) {  // everything is selected
    for (int i = tid; i < K; i += 1024) {
      oi[i] = i < n ? i : -1;
      if (ov) ov[i] = i < n ? row[i] : 0.f;
    }
    return;
  }
  select_resident<NPT>(v, n, K, smraw, oi, ov);
}

// One 1024-thread workgroup per row longer than 1024*32 entries (the others return at once).
__global__ __launch_bounds__(1024) void topk_stream_kernel(DevBatch bt, int t_begin,
    const float* __restrict__ scores, int64_t ld, int K, int32_t* __restrict__ out_idx,
    float* __restrict__ out_val) {
  extern __shared__ __attribute__((aligned(16))) char smraw[];
  const int tid = threadIdx.x;
  const int tl = blockIdx.x;
  const int t = t_begin + tl;
  const int n = row_len(bt, t);  // (each wave looks it up)
  if (n <= 1024 * 32) return;
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
  if (!select_stream_list(row, n, K, smraw, oi, ov)) select_streamed(row, n, K, K, smraw, oi, ov);
}


// ---------------------------------------------------------------- long rows, few of them
// With few rows of many positions (at most kLongRows per launch, rows over 32K entries,
// K <= 4096), one workgroup per row would leave most of the chip idle and read each row through
// one CU.  Three launches instead:
//   1. one workgroup per row: 8192 scores in 512 runs of 16 at uniform sites give the lower
//      bound tlo of the K-th largest key (as for streamed rows); the row's candidate count is
//      reset;
//   2. one workgroup per 16384-entry slice (coalesced 16-byte pieces): the slice's scores
//      >= tlo are counted, room for them is reserved in the row's candidate list (at most
//      kLongCap positions) with one atomic per slice (few slices per row: the atomics of one
//      row serialise), and their (key, position) pairs are written there in position order,
//      with the slice's (offset, count);
//   3. one workgroup per row: thread i fetches list entries 8i .. 8i + 7 of the slices'
//      candidates in slice (= position) order, and the threshold and compaction of streamed
//      rows finish the row.  A row whose candidates overflow the list or fall short of K (many equal
//      scores) is selected by the exact streamed select in the same workgroup.
// Rows with n <= K take every position in step 3.

__global__ __launch_bounds__(1024) void topk_long_sample_kernel(DevBatch bt, int t_begin,
    const float* __restrict__ scores, int64_t ld, int K, uint32_t* __restrict__ state) {
  __shared__ uint32_t h[2048];
  __shared__ uint32_t sh[48];
  __shared__ uint32_t pick[4];
  const int tid = threadIdx.x, tl = blockIdx.x;
  const int n = row_len(bt, t_begin + tl);  // (each wave looks it up)
  uint32_t* s = state + 4 * tl;
  if (n <= K) {
    if (tid == 0) {
      s[0] = kLongAll;
      s[2] = 0u;
    }
    return;
  }
  const float* row = scores + (int64_t)tl * ld;
  h[tid] = 0u;
  h[tid + 1024] = 0u;
  if (tid < 4) pick[tid] = 0u;
  // 8192 scores: 512 runs of 16 consecutive positions at uniform sites (a run starts at
  // floor(r (n - 16) / 511) rounded down to a multiple of 4, so each of a run's four threads
  // reads one 16-byte piece, the last ending at n - 1 at most); two runs per group of four
  // threads.  (Rows shorter than 16 read their positions clamped to the row.)
  uint32_t kk[8];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = (tid >> 2) + 256 * j;
    const int base = n >= 16 ? (int)(((int64_t)r * (n - 16)) / 511) & ~3 : 0;
    const int p = base + 4 * (tid & 3);
    float f[4];
    if (p + 3 < n) {
      const float4 v = *(const float4*)(row + p);
      f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) f[e] = row[min(p + e, n - 1)];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) kk[4 * j + e] = order_key(f[e]);
  }
  uint32_t mn = ~0u, mx = 0u;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    mn = min(mn, kk[j]);
    mx = max(mx, kk[j]);
  }
  block_minmax(mn, mx, sh + 16);  // (its barrier also orders the clears above)
  const uint32_t span = mx - mn;
  const int shift = max(0, (span ? 32 - __clz(span) : 0) - 11);
#pragma unroll
  for (int j = 0; j < 8; ++j) atomicAdd(&h[(kk[j] - mn) >> shift], 1u);
  __syncthreads();
  const uint32_t want = min(8192u, (uint32_t)(((uint64_t)K * 8192u * 5u) / (4ull * n)) + 16u);
  pick_bin(h, want, sh, pick);
  __syncthreads();
  if (tid == 0) {
    s[0] = kLongCand;
    s[1] = mn + (pick[0] << shift);
    s[2] = 0u;
  }
}

__global__ __launch_bounds__(1024) void topk_long_list_kernel(DevBatch bt, int t_begin,
    const float* __restrict__ scores, int64_t ld, int nsl, uint32_t* __restrict__ state,
    uint32_t* __restrict__ slices, uint64_t* __restrict__ cand) {
  __shared__ uint32_t wt[16];
  __shared__ uint32_t base_sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sl = blockIdx.x, tl = blockIdx.y;
  uint32_t* s = state + 4 * tl;
  if (s[0] != kLongCand) return;
  const int n = row_len(bt, t_begin + tl);  // (each wave looks it up)
  const int s0 = sl * kLongSlice;
  uint32_t* so = slices + ((int64_t)tl * nsl + sl) * 2;
  if (s0 >= n) {
    if (tid == 0) {
      so[0] = 0u;
      so[1] = 0u;
    }
    return;
  }
  const float tf = key_value(s[1]);  // (x >= tf exactly when order_key(x) >= tlo)
  const float* row = scores + (int64_t)tl * ld;
  const int pl = s0 + 1024 * wave + 4 * lane;  // piece i: positions pl + 256 i .. + 3
  uint32_t bits[4], ex[4], wb[4];
  float xk[4][4];
  uint32_t wtot = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = pl + 256 * i;
    float x[4];
    if (p + 3 < n) {
      const float4 f = *(const float4*)(row + p);
      x[0] = f.x; x[1] = f.y; x[2] = f.z; x[3] = f.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = p + e < n ? row[p + e] : __uint_as_float(0x7fc00000u);
    }
    bits[i] = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bits[i] |= (x[e] >= tf ? 1u : 0u) << e;
      xk[i][e] = x[e];
    }
    const uint32_t c = __popc(bits[i]);
    const uint32_t inc = wave_incl_scan(c);
    ex[i] = inc - c;
    wb[i] = wtot;
    wtot += __builtin_amdgcn_readlane(inc, 63);
  }
  if (lane == 0) wt[wave] = wtot;
  __syncthreads();
  const uint32_t ws = wave_incl_scan(lane < 16 ? wt[lane] : 0u);
  const uint32_t before = wave ? __builtin_amdgcn_readlane(ws, wave - 1) : 0u;
  const uint32_t total = __builtin_amdgcn_readlane(ws, 15);
  if (tid == 0) base_sh = total ? atomicAdd(&s[2], total) : 0u;
  __syncthreads();
  const uint32_t base = base_sh;
  if (tid == 0) {
    so[0] = base;
    so[1] = total;
  }
  uint64_t* cl = cand + (int64_t)tl * kLongCap;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t o = base + before + wb[i] + ex[i];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if ((bits[i] >> e) & 1u) {
        if (o < (uint32_t)kLongCap)
          cl[o] = ((uint64_t)order_key(xk[i][e]) << 32) | (uint32_t)(pl + 256 * i + e);
        ++o;
      }
  }
}

__global__ __launch_bounds__(1024) void topk_long_final_kernel(DevBatch bt, int t_begin,
    const float* __restrict__ scores, int64_t ld, int K, int nsl,
    const uint32_t* __restrict__ state, const uint32_t* __restrict__ slices,
    const uint64_t* __restrict__ cand, int32_t* __restrict__ out_idx,
    float* __restrict__ out_val) {
  extern __shared__ __attribute__((aligned(16))) char smraw[];
  constexpr int E = kLongCap / 1024;
  StreamLds& S = *(StreamLds*)smraw;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, tl = blockIdx.x;
  const int t = t_begin + tl;
  const int n = row_len(bt, t);
  const float* row = scores + (int64_t)tl * ld;
  int32_t* oi = out_idx + (int64_t)t * K;
  float* ov = out_val ? out_val + (int64_t)t * K : nullptr;
  const uint32_t* s = state + 4 * tl;
  if (s[0] == kLongAll) {
    for (int i = tid; i < K; i += 1024) {
      oi[i] = i < n ? i : -1;
      if (ov) ov[i] = i < n ? row[i] : 0.f;
    }
    return;
  }
  const uint32_t tlo = s[1], C = s[2];
  if (C < (uint32_t)K || C > (uint32_t)kLongCap) {  // (many equal scores: the exact select)
    select_streamed(row, n, K, K, smraw, oi, ov);
    return;
  }
  // list entries E*tid .. E*tid + E - 1 of the slices' candidates in slice (= position)
  // order, 1024 slices at a time: the slices' source offsets and destinations are staged in
  // hA, and each entry of the group finds its slice by binary search over the destinations
  // (all of a thread's loads in flight together)
  uint32_t* src = S.hA;
  uint32_t* dst = S.hA + 1024;
  uint32_t lk[E], lp[E];
#pragma unroll
  for (int e = 0; e < E; ++e) lk[e] = lp[e] = 0u;  // (key 0 past the list)
  uint32_t run = 0u;
  for (int g = 0; g < nsl; g += 1024) {
    const int sl = g + tid;
    const uint32_t* so = slices + ((int64_t)tl * nsl + sl) * 2;
    const uint32_t c = sl < nsl ? so[1] : 0u;
    const uint32_t o = sl < nsl ? so[0] : 0u;
    uint32_t tot;
    const uint32_t pre = block_excl_scan(c, S.sh, tot);
    src[tid] = o;
    dst[tid] = run + pre;
    __syncthreads();
    const int ng = min(1024, nsl - g);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t d = (uint32_t)(E * tid + e);
      if (d >= run && d < run + tot) {
        int lo = 0, hi = ng - 1;  // the last slice whose destination is <= d
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (dst[mid] <= d) lo = mid;
          else hi = mid - 1;
        }
        const uint32_t q = src[lo] + (d - dst[lo]);
        if (q < (uint32_t)kLongCap) {
          const uint64_t pr = cand[(int64_t)tl * kLongCap + q];
          lk[e] = (uint32_t)(pr >> 32);
          lp[e] = (uint32_t)pr;
        }
      }
    }
    run += tot;
    __syncthreads();  // (the staging and sh are reused)
  }
  uint32_t kmn = ~0u, kmx = 0u;
#pragma unroll
  for (int e = 0; e < E; ++e) kmx = max(kmx, lk[e]);
  S.hB[tid] = 0u;
  S.hB[tid + 1024] = 0u;
  if (tid < 4) S.cnt[tid] = 0u;
  block_minmax(kmn, kmx, S.sh + 16);  // (its barrier also publishes the clears)
  select_listed<E>(lk, lp, tlo, kmx, K, S, oi, ov);
}

bool topk_long_rows(int max_n, int K) { return max_n > 32768 && K <= kLongCap / 2; }
// long-row workspace per row: the candidate list of (key, position) pairs, state, the slices'
// (offset, count)
size_t long_row_bytes(int max_n) {
  const size_t nsl = ((size_t)max_n + kLongSlice - 1) / kLongSlice;
  return 8 * (size_t)kLongCap + 16 + 8 * nsl;
}

// workspace of a launch over up to `rows` rows (any smaller launch fits in it too)
size_t topk_ws_bytes(int rows, int max_n, int K) {
  return topk_long_rows(max_n, K) ? (size_t)std::min(rows, kLongRows) * long_row_bytes(max_n)
                                  : 0;
}

hipError_t launch_topk(const DevBatch& bt, int t_begin, int t_count, int max_n,
                       const float* scores, int64_t ld, int K, int32_t* idx, float* val,
                       void* ws, hipStream_t st) {
  if (t_count <= kLongRows && topk_long_rows(max_n, K)) {
    // ws: candidates [t_count][kLongCap] (key, position) | state [t_count][4] |
    //     slices [t_count][nsl][2]
    const int nsl = (max_n + kLongSlice - 1) / kLongSlice;
    uint64_t* cand = (uint64_t*)ws;
    uint32_t* state = (uint32_t*)(cand + (size_t)t_count * kLongCap);
    uint32_t* slices = state + 4 * (size_t)t_count;
    hipLaunchKernelGGL(topk_long_sample_kernel, dim3(t_count), dim3(1024), 0, st, bt, t_begin,
                       scores, ld, K, state);
    hipLaunchKernelGGL(topk_long_list_kernel, dim3(nsl, t_count), dim3(1024), 0, st, bt,
                       t_begin, scores, ld, nsl, state, slices, cand);
    const size_t fshm = std::max(sizeof(SelSmem), sizeof(StreamLds));
    hipError_t e = hipFuncSetAttribute((const void*)topk_long_final_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)fshm);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_long_final_kernel, dim3(t_count), dim3(1024), fshm, st, bt, t_begin,
                       scores, ld, K, nsl, state, slices, cand, idx, val);
    return hipGetLastError();  // (every row is finished by the final kernel)
  }
  // keys per thread: the smallest power of two (>= 4) that keeps the longest row in registers,
  // up to 32 (32768 positions); longer rows stream through 1024*32-key chunks per pass
  int npt = 4;
  while (npt < 32 && 1024 * npt < max_n) npt *= 2;
  auto* fn = npt == 4 ? topk_select_kernel<4>
             : npt == 8 ? topk_select_kernel<8>
             : npt == 16 ? topk_select_kernel<16> : topk_select_kernel<32>;
  // dynamic LDS: a row held on chip (row, histograms, list, bitmaps), or the streamed
  // selection's histograms if larger
  const size_t res = npt == 4 ? ResLds<4>::bytes
                     : npt == 8 ? ResLds<8>::bytes
                     : npt == 16 ? ResLds<16>::bytes : ResLds<32>::bytes;
  const size_t shm = std::max(sizeof(SelSmem), res);
  hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)shm);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3(t_count), dim3(1024), shm, st, bt, t_begin, scores, ld, K, idx,
                     val);
  if (max_n > 1024 * 32) {  // rows longer than one chunk
    const size_t sshm = std::max(sizeof(SelSmem), sizeof(StreamLds));
    e = hipFuncSetAttribute((const void*)topk_stream_kernel,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)sshm);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_stream_kernel, dim3(t_count), dim3(1024), sshm, st, bt, t_begin,
                       scores, ld, K, idx, val);
  }
  return hipGetLastError();
}

}  // namespace tis
