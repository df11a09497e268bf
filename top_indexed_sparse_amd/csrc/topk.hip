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

// Long-row selection state per row, words [mode, bin, candidates, keys above the bin]
constexpr uint32_t kLongCand = 0u, kLongAll = 1u, kLongOver = 2u;
constexpr int kLongCap = 8192;      // candidates per row (8 per thread of the last step)
constexpr int kLongRows = 64;       // at most this many rows per launch take the long-row path
constexpr int kLongSlices = 1024;   // slices per row at most

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
  const uint32_t cspan = kmax - tlo;
  const int shift2 = max(0, (cspan ? 32 - __clz(cspan) : 0) - 11);
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (lk[e] != 0u) atomicAdd(&S.hB[(lk[e] - tlo) >> shift2], 1u);
  S.hA[tid] = 0u;  // (the sample histogram was last read before tlo's barrier)
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
    const float* __restrict__ scores, int64_t ld, int K, const uint32_t* __restrict__ only,
    int32_t* __restrict__ out_idx,
    float* __restrict__ out_val) {
  extern __shared__ __attribute__((aligned(16))) char smraw[];
  const int tid = threadIdx.x;
  const int tl = blockIdx.x;
  const int t = t_begin + tl;
  const float* row = scores + (int64_t)tl * ld;
  // (after the long-row selection: only the rows it left over)
  if (only && only[4 * tl] != kLongOver) return;
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
    const float* __restrict__ scores, int64_t ld, int K, const uint32_t* __restrict__ only,
    int32_t* __restrict__ out_idx, float* __restrict__ out_val) {
  extern __shared__ __attribute__((aligned(16))) char smraw[];
  const int tid = threadIdx.x;
  const int tl = blockIdx.x;
  const int t = t_begin + tl;
  if (only && only[4 * tl] != kLongOver) return;
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
  // dynamic LDS: a row held on chip (row, histograms, list, bitmaps), or the streamed
  // selection's histograms if larger
  const size_t res = npt == 4 ? ResLds<4>::bytes
                     : npt == 8 ? ResLds<8>::bytes
                     : npt == 16 ? ResLds<16>::bytes : ResLds<32>::bytes;
  const size_t shm = std::max(sizeof(SelSmem), res);
  hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)shm);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3(t_count), dim3(1024), shm, st, bt, t_begin, scores, ld, K, only,
                     idx, val);
  if (max_n > 1024 * 32) {  // rows longer than one chunk
    const size_t sshm = std::max(sizeof(SelSmem), sizeof(StreamLds));
    e = hipFuncSetAttribute((const void*)topk_stream_kernel,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)sshm);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_stream_kernel, dim3(t_count), dim3(1024), sshm, st, bt, t_begin,
                       scores, ld, K, only, idx, val);
  }
  return hipGetLastError();
}

}  // namespace tis
