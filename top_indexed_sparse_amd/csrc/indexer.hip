// Indexer scorer: score[t][s] = sum_h w[t][h] * max(0, q_I[t][h] . k_I[s]) for s <= p_t.
//
// Method: "Day 0 Support for New LLM Architectures", Step 1 (a light indexer scores every
// earlier position) and Key Optimization 1 (scoring and head-weight application read the
// paged K cache directly).  Key Optimization 2 quantises the indexer query dynamically;
// here each (token, head) row of q_I gets the smallest power-of-two scale s with
// max|q|/s <= 448, q/s is rounded to e4m3 (RNE) and s is folded into the head weight, so the
// dot products run on the FP8 matrix cores with exact products and fp32 accumulation.
//
// FP8 kernel layout (one wave = one token over a key range; 64 heads x 128 dims):
//   MFMA v_mfma_f32_16x16x128_f8f6f4, A = q8 (16 heads x 128 dims, 4 tiles for 64 heads),
//   B = k8 (128 dims x 16 keys).  Lane l holds head/key (l & 15) and 32 of the 128 dims,
//   chosen by g = l >> 4: bytes [16g, 16g+16) and [64+16g, 64+16g+16) of the row, so each
//   load instruction reads the first (or second) 64 bytes of 16 key rows.  The same dim
//   permutation is applied to q and k, so the dot products are unchanged.
//   The accumulator of tile m holds heads 16m + 4g + i (i < 4) of key (l & 15): ReLU and
//   head weights are applied in-lane, and two permlane swaps finish the head sum while
//   transposing four 16-key tiles so that lane l ends with the score of key base + l.
#include "common.h"
#include "launch.h"

namespace tis {

// ---------------------------------------------------------------- fp32 (small shapes)
__global__ __launch_bounds__(256) void idx_score_f32_kernel(DevBatch bt, int t_begin,
    const float* __restrict__ q, const float* __restrict__ w, const float* __restrict__ kpool,
    int H, int D, float* __restrict__ scores, int64_t ld) {
  extern __shared__ float sq[];  // [H*D] query, [H] weights
  const int t = t_begin + blockIdx.x;
  const TokLoc loc = locate(bt, t);
  const int b = loc.b;
  const int p = loc.n - 1;
  const int s = blockIdx.y * blockDim.x + threadIdx.x;
  if ((int)(blockIdx.y * blockDim.x) > p) return;  // whole block beyond the causal range
  for (int i = threadIdx.x; i < H * D; i += blockDim.x) sq[i] = q[(int64_t)t * H * D + i];
  for (int i = threadIdx.x; i < H; i += blockDim.x) sq[H * D + i] = w[(int64_t)t * H + i];
  __syncthreads();
  if (s > p) return;
  const int64_t slot = slot_of(bt, b, s);
  float tot;
  if (slot < 0) {
    tot = -INFINITY;
  } else {
    const float* k = kpool + slot * D;
    tot = 0.f;
    for (int h = 0; h < H; ++h) {
      float dot = 0.f;
      for (int d = 0; d < D; ++d) dot = fmaf(sq[h * D + d], k[d], dot);
      tot = fmaf(sq[H * D + h], fmaxf(dot, 0.f), tot);
    }
  }
  scores[(int64_t)(t - t_begin) * ld + s] = tot;
}

// ---------------------------------------------------------------- FP8 matrix-core scorer
constexpr int kIH = 64;   // indexer heads
constexpr int kID = 128;  // indexer head dim

// The token's query rows and head weights in the lanes that quantise them: lane (n, g) holds
// dims [16g, 16g+16) and [64+16g, 64+16g+16) of heads 16m + n, and the weights of heads
// 16m + 4g + i.  Loading is split from quantising so the loads can be issued early.
struct QRaw {
  i32x4 r[4][4];
  float w[4][4];
};

__device__ __forceinline__ void a0_load_tile(const uint16_t* __restrict__ qrow,
                                             const float* __restrict__ wrow, int lane, int m,
                                             i32x4 (&r)[4], float (&wr)[4]) {
  const int n = lane & 15, g = lane >> 4;
  const uint16_t* hrow = qrow + (16 * m + n) * kID;
  r[0] = *(const i32x4*)(hrow + 16 * g);
  r[1] = *(const i32x4*)(hrow + 16 * g + 8);
  r[2] = *(const i32x4*)(hrow + 64 + 16 * g);
  r[3] = *(const i32x4*)(hrow + 64 + 16 * g + 8);
#pragma unroll
  for (int i = 0; i < 4; ++i) wr[i] = wrow[16 * m + 4 * g + i];
}
__device__ __forceinline__ void a0_load(const uint16_t* __restrict__ qrow,
                                        const float* __restrict__ wrow, int lane, QRaw& qr) {
#pragma unroll
  for (int m = 0; m < 4; ++m) a0_load_tile(qrow, wrow, lane, m, qr.r[m], qr.w[m]);
}

// Quantise head tile m of the query (heads 16m .. 16m+15) to e4m3 in the MFMA A layout and
// build the lane's head weights w'[16m + 4g + i] = w * s (s = power-of-two scale of the head).
__device__ __forceinline__ void a0_tile(const i32x4 (&r)[4], const float (&wr)[4], int lane,
                                        i32x8& A, float (&wp)[4]) {
  const int g = lane >> 4;
  {
    uint32_t wd[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) wd[j] = (uint32_t)r[j >> 2][j & 3];
    float v[32];
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      v[2 * j] = __uint_as_float(wd[j] << 16);
      v[2 * j + 1] = __uint_as_float(wd[j] & 0xffff0000u);
      amax = fmaxf(amax, fmaxf(fabsf(v[2 * j]), fabsf(v[2 * j + 1])));
    }
    // max over the four lanes that share this head (g = 0..3)
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    int E;
    float mant = frexpf(amax, &E);
    int e = (mant <= 0.875f) ? E - 9 : E - 8;
    if (amax == 0.f) e = 0;
    const float s_q = ldexpf(1.f, e);
    const float inv_s = ldexpf(1.f, -e);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int word = 0;
      word = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * j] * inv_s, v[4 * j + 1] * inv_s, word,
                                             false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * j + 2] * inv_s, v[4 * j + 3] * inv_s, word,
                                             true);
      A[j] = word;
    }
    // w'[16m + 4g + i]: the scale of head 16m + r lives in lane r (any g)
#pragma unroll
    for (int i = 0; i < 4; ++i) wp[i] = wr[i] * __shfl(s_q, 4 * g + i);
  }
}

// All four head tiles.
__device__ __forceinline__ void a0_prologue(const QRaw& qr, int lane, i32x8 (&A)[4],
                                            float (&wp)[4][4]) {
#pragma unroll
  for (int m = 0; m < 4; ++m) a0_tile(qr.r[m], qr.w[m], lane, A[m], wp[m]);
}

struct KTile4 {
  i32x4 lo[4], hi[4];
};

__device__ __forceinline__ void load_ktile4(const uint8_t* __restrict__ page_base, int lane,
                                            KTile4& kt) {
  const int n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint8_t* row = page_base + (16 * j + n) * kID;
    kt.lo[j] = *(const i32x4*)(row + 16 * g);
    kt.hi[j] = *(const i32x4*)(row + 64 + 16 * g);
  }
}

// Scores of the 64 keys of one page-aligned group; lane l returns key base + l (unscaled).
__device__ __forceinline__ float score_group(const i32x8 (&A)[4], const float (&wp)[4][4],
                                             const KTile4& kt) {
  float v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    i32x8 B;
    B[0] = kt.lo[j][0]; B[1] = kt.lo[j][1]; B[2] = kt.lo[j][2]; B[3] = kt.lo[j][3];
    B[4] = kt.hi[j][0]; B[5] = kt.hi[j][1]; B[6] = kt.hi[j][2]; B[7] = kt.hi[j][3];
    float acc = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
      c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[m], B, c, 0, 0, 0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = fmaf(wp[m][i], fmaxf(c[i], 0.f), acc);
    }
    v[j] = acc;
  }
  // head sum over g and 4x4 transpose: lane l ends with tile (l >> 4), key (l & 15)
  float k0 = pair32_sum(v[0], v[2]);
  float k1 = pair32_sum(v[1], v[3]);
  return pair16_sum(k0, k1);
}

// group_mode == 0: one token per workgroup (blockIdx.x), its waves split the key chunk
//                  blockIdx.y.
// group_mode == 1: four consecutive tokens per workgroup, one per wave, same key chunk.
__global__ __launch_bounds__(512) void idx_score_fp8_kernel(DevBatch bt, int t_begin,
    int t_count, const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint8_t* __restrict__ kpool, const float* __restrict__ kscale,
    float* __restrict__ scores, int64_t ld, int group_mode, int chunk) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int tl, k0, k1;
  if (group_mode) {
    tl = blockIdx.x * 4 + wave;
    k0 = blockIdx.y * chunk;
    k1 = k0 + chunk;
  } else {
    tl = blockIdx.x;
    const int part = chunk / (int)(blockDim.x >> 6);
    k0 = blockIdx.y * chunk + wave * part;
    k1 = k0 + part;
  }
  if (tl >= t_count) return;  // (decode: the same for every wave of the workgroup)
  const int t = t_begin + tl;
  // The query goes out first: it needs the token only.  Decode: the eight waves share the
  // token, so waves 0..3 each quantise one 16-head tile and hand it over through LDS.
  const uint16_t* qrow = q_idx + (int64_t)t * kIH * kID;
  const float* wrow = w + (int64_t)t * kIH;
  QRaw qr;
  if (group_mode) a0_load(qrow, wrow, lane, qr);
  else if (wave < 4) a0_load_tile(qrow, wrow, lane, wave, qr.r[0], qr.w[0]);
  const TokLoc loc = locate(bt, t);
  const int b = loc.b;
  const int n = loc.n;
  k1 = min(k1, n);
  const bool active = k0 < k1;

  const int32_t* pt = bt.page_table + (int64_t)b * bt.pt_stride;
  float* out = scores + (int64_t)tl * ld;

  // Start-up order matters: everything waits on the page ids, and loads complete in issue
  // order, so the page ids are requested before the first key groups; the query is quantised
  // while those groups are in flight.
  // Page ids of this wave's range, one per lane, fetched once (a scalar page-table load per
  // group would stall every prefetch on a scalar round trip).
  const int pg0 = k0 >> 6;
  const int npg = active ? (k1 - 1) / 64 - pg0 + 1 : 0;  // <= 64 pages per wave
  const int my_page = lane < npg ? pt[pg0 + lane] : 0;

  // three-slot ring of 64-key groups: while one group is scored the next two are in flight
  struct Slot {
    KTile4 kt;
    float ks;
    bool ok;
  };
  auto fetch = [&](int base, Slot& sl) {
    if (base < k1) {
      const int page = __builtin_amdgcn_readlane(my_page, (base >> 6) - pg0);
      sl.ok = page >= 0 && page < bt.n_pages;
      const int64_t pg = sl.ok ? page : 0;
      load_ktile4(kpool + pg * kPage * kID, lane, sl.kt);
      sl.ks = kscale[pg * kPage + lane];
    }
  };
  Slot s0, s1, s2;
  fetch(k0, s0);
  fetch(k0 + 64, s1);
  i32x8 A[4];
  float wp[4][4];
  if (group_mode) {
    if (!active) return;
    a0_prologue(qr, lane, A, wp);
  } else {
    __shared__ i32x8 a_sh[4][64];
    __shared__ f32x4 w_sh[4][64];
    if (wave < 4) {
      i32x8 at;
      float wt[4];
      a0_tile(qr.r[0], qr.w[0], lane, at, wt);
      a_sh[wave][lane] = at;
      w_sh[wave][lane] = f32x4{wt[0], wt[1], wt[2], wt[3]};
    }
    __syncthreads();
    if (!active) return;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      A[m] = a_sh[m][lane];
      const f32x4 wv = w_sh[m][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) wp[m][i] = wv[i];
    }
  }
  auto consume = [&](int base, const Slot& sl) {
    if (base < k1) {
      float sc = score_group(A, wp, sl.kt) * sl.ks;
      if (!sl.ok) sc = -INFINITY;
      if (base + lane < k1) out[base + lane] = sc;
    }
  };
  for (int base = k0; base < k1; base += 192) {
    fetch(base + 128, s2);
    consume(base, s0);
    fetch(base + 192, s0);
    consume(base + 64, s1);
    fetch(base + 256, s1);
    consume(base + 128, s2);
  }
}

// ---------------------------------------------------------------- launchers
hipError_t launch_index_score_f32(const DevBatch& bt, int t_begin, int t_count, int max_n,
                                  const float* q, const float* w, const float* kpool, int H,
                                  int D, float* scores, int64_t ld, hipStream_t st) {
  dim3 grid(t_count, (max_n + 255) / 256);
  size_t shm = (size_t)(H * D + H) * sizeof(float);
  hipLaunchKernelGGL(idx_score_f32_kernel, grid, dim3(256), shm, st, bt, t_begin, q, w, kpool,
                     H, D, scores, ld);
  return hipGetLastError();
}

hipError_t launch_index_score_fp8(const DevBatch& bt, int t_begin, int t_count, int max_n,
                                  bool prefill_like, const uint16_t* q_idx, const float* w,
                                  const uint8_t* kpool, const float* kscale, float* scores,
                                  int64_t ld, hipStream_t st) {
  const int group = prefill_like ? 1 : 0;
  const int chunk = prefill_like ? 1024 : 4096;
  dim3 grid(group ? (t_count + 3) / 4 : t_count, (max_n + chunk - 1) / chunk);
  // decode: one 8-wave workgroup per 4096-key chunk of a token (512 keys per wave); prefill:
  // four tokens per 4-wave workgroup sharing a 1024-key chunk
  hipLaunchKernelGGL(idx_score_fp8_kernel, grid, dim3(group ? 256 : 512), 0, st, bt, t_begin,
                     t_count, q_idx, w, kpool, kscale, scores, ld, group, chunk);
  return hipGetLastError();
}

}  // namespace tis
