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
//
// MXFP8 mode (Key Optimization 2 of the same page: the indexer fully quantised as MXFP8, every
// 32 consecutive elements of Q and K sharing one power-of-two scale): keys carry one scale
// byte 127 + X per 32 dims, and the query is quantised in the prologue per (head, 32 dims)
// with X = floor(log2 amax) - 8 (clamped to [-127, 127]) and codes RNE(q / 2^X) clamped to
// +-448.  Both scales go to the matrix instruction's block-scale operands, which apply to
// K blocks [32b, 32b+32): the lane layout above puts K index 16g+i (i < 16) in the first half
// of lane (n, g)'s operand and 64+16g+i in the second, i.e. the dims in their own order, so
// block b is dim group b and the scale byte of lane (n, g) is that of head/key n, group g.
//
// bf16 query mode (the quantisation-free implementation kept beside the quantised one, as in
// Key Optimization 1): the same kernel with q_I used as stored on v_mfma_f32_16x16x32_bf16.
// The 32 query dims a lane holds are already the four 8-dim k-steps of that instruction's A
// layout (dims 16g.., 16g+8.., 64+16g.., 64+16g+8..), and each staged 16-byte run of key
// bytes widens exactly (every e4m3 value is a bf16 value) into two B operands of the same
// dims; the weights are used as given.
#include <type_traits>

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
    // q / 2^e by exponent adjustment (exact: the quotient is at most 448); a reciprocal scale
    // would overflow to inf for heads with max |q| below about 2^-118
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int word = 0;
      word = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4 * j], -e), ldexpf(v[4 * j + 1], -e),
                                             word, false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4 * j + 2], -e), ldexpf(v[4 * j + 3], -e),
                                             word, true);
      A[j] = word;
    }
    // w'[16m + 4g + i] = w * 2^e: the exponent of head 16m + r lives in lane r (any g); for
    // such tiny heads w' is subnormal (gradual underflow, never inf or NaN)
#pragma unroll
    for (int i = 0; i < 4; ++i) wp[i] = ldexpf(wr[i], __shfl(e, 4 * g + i));
  }
}

// All four head tiles.
__device__ __forceinline__ void a0_prologue(const QRaw& qr, int lane, i32x8 (&A)[4],
                                            float (&wp)[4][4]) {
#pragma unroll
  for (int m = 0; m < 4; ++m) a0_tile(qr.r[m], qr.w[m], lane, A[m], wp[m]);
}

// Quantise head tile m to MXFP8 in the MFMA A layout.  Lane (n, g) holds dims [16g, 16g+16)
// (half of group g >> 1) and [64+16g, 64+16g+16) (half of group 2 + (g >> 1)); the other half
// of each group sits in lane (n, g ^ 1).  sa = the scale byte of head n, group g, which lane
// (n, g & 1 ? 2 : 0) computed for its first (g < 2) or second (g >= 2) half.  The weights are
// used as given.
__device__ __forceinline__ void mx_tile(const i32x4 (&r)[4], const float (&wr)[4], int lane,
                                        i32x8& A, int& sa, float (&wp)[4]) {
  const int n = lane & 15, g = lane >> 4;
  uint32_t wd[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) wd[j] = (uint32_t)r[j >> 2][j & 3];
  float v[32];
  float am[2] = {0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    v[2 * j] = __uint_as_float(wd[j] << 16);
    v[2 * j + 1] = __uint_as_float(wd[j] & 0xffff0000u);
    am[j >> 3] = fmaxf(am[j >> 3], fmaxf(fabsf(v[2 * j]), fabsf(v[2 * j + 1])));
  }
  int X[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) X[h] = mx_exponent(fmaxf(am[h], __shfl_xor(am[h], 16)));
  // q / 2^X by exponent adjustment (exact), saturated to the largest finite e4m3 magnitude
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int e = -X[j >> 2];
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = fminf(fmaxf(ldexpf(v[4 * j + i], e), -448.f), 448.f);
    int word = 0;
    word = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], word, false);
    word = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], word, true);
    A[j] = word;
  }
  const int src = n + 32 * (g & 1);
  const int lo = __shfl(X[0], src), hi = __shfl(X[1], src);
  sa = (g < 2 ? lo : hi) + 127;
#pragma unroll
  for (int i = 0; i < 4; ++i) wp[i] = wr[i];
}

struct KTile4 {
  i32x4 lo[4], hi[4];
};

// Cache-policy bits of a buffer load: the non-temporal bit (the one __builtin_nontemporal_load
// sets).
constexpr int kAuxNT = 2;

// One 8 KB page of keys (64 rows of 128 bytes) in eight non-temporal loads of 1 KB each,
// through a buffer resource based at the page (offsets past its record count read nothing and
// return zeros): load i, lane l gets bytes [1024i + 16l, +16), i.e. row 8i + (l >> 3), bytes
// 16(l & 7)... (whole rows per instruction stream better than the MFMA layout's 64-byte half
// rows).
struct KPage {
  i32x4 r[8];
};
__device__ __forceinline__ void load_kpage_rsrc(__amdgpu_buffer_rsrc_t r, int lane, KPage& kp) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
    kp.r[i] = __builtin_bit_cast(
        i32x4, __builtin_amdgcn_raw_buffer_load_b128(r, 1024 * i + 16 * lane, 0, kAuxNT));
}

// A key page in LDS: 64 rows of 128 bytes, the 16-byte column c of row r stored at column
// c ^ ((r >> 1) & 7).  With 64 banks of 4 bytes, each 16-lane quarter of a 16-byte access
// covers 256 bytes: a quarter of a row write (two rows, all eight columns) and of a
// matrix-layout read (sixteen rows, one column each) then falls on 64 distinct banks.
constexpr int kRowB = 128;
constexpr int kStage = 64 * kRowB;  // bytes per page
__device__ __forceinline__ int swz(int r, int c) { return r * kRowB + 16 * (c ^ ((r >> 1) & 7)); }

// load i of a page (see load_kpage_rsrc) into the page buffer: lane l holds row 8i + (l >> 3),
// column l & 7
__device__ __forceinline__ void put_load(uint8_t* st, int i, int lane, i32x4 v) {
  *(i32x4*)(st + swz(8 * i + (lane >> 3), lane & 7)) = v;
}

// The four 16-key tiles of a page buffer in the MFMA B layout: lane (n = l & 15, g = l >> 4)
// takes bytes [16g, 16g+16) and [64+16g, 64+16g+16) of row 16j + n.
__device__ __forceinline__ void read_ktile4(const uint8_t* st, int lane, KTile4& kt) {
  const int n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    kt.lo[j] = *(const i32x4*)(st + swz(16 * j + n, g));
    kt.hi[j] = *(const i32x4*)(st + swz(16 * j + n, 4 + g));
  }
}

// Through the wave's own page buffer into the MFMA B layout.  (LDS operations of one wave
// complete in order, so the buffer can be rewritten by the next page without a wait.)
__device__ __forceinline__ void stage_ktile4(uint8_t* stage, int lane, const KPage& kp,
                                             KTile4& kt) {
#pragma unroll
  for (int i = 0; i < 8; ++i) put_load(stage, i, lane, kp.r[i]);
  read_ktile4(stage, lane, kt);
}

// Query modes of the matrix-core scorer: e4m3 with one power-of-two scale per head folded
// into the weights, bf16 as stored, or MXFP8 (e4m3 with one scale byte per 32 dims).
enum QMode : int { kQFp8 = 0, kQBf16 = 1, kQMx = 2 };

// The query's A operands for the four 16-head tiles: e4m3 (one 16x16x128 step per tile, MXFP8
// with the lane's block-scale byte) or bf16 as stored (four 16x16x32 steps per tile, each the
// i32x4 of 8 dims the lane loaded).
template <int QM>
struct QOps {
  i32x8 a[4];
};
template <>
struct QOps<kQBf16> {
  i32x4 a[4][4];
};
template <>
struct QOps<kQMx> {
  i32x8 a[4];
  int sa[4];
};

// The key scale word a lane loads for key `lane` of a page: the fp32 per-token scale, or
// (MXFP8) the key's four scale bytes, group g in bits [8g, 8g+8).
template <int QM>
using KScale = typename std::conditional<QM == kQMx, uint32_t, float>::type;

// All four head tiles in the mode's A layout.
template <int QM>
__device__ __forceinline__ void q_prologue(const QRaw& qr, int lane, QOps<QM>& A,
                                           float (&wp)[4][4]) {
  if constexpr (QM == kQBf16) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        A.a[m][i] = qr.r[m][i];
        wp[m][i] = qr.w[m][i];
      }
  } else if constexpr (QM == kQMx) {
#pragma unroll
    for (int m = 0; m < 4; ++m) mx_tile(qr.r[m], qr.w[m], lane, A.a[m], A.sa[m], wp[m]);
  } else {
    a0_prologue(qr, lane, A.a, wp);
  }
}

// 8 e4m3 codes (two dwords) widened to bf16, exactly (scale 1)
__device__ __forceinline__ bf16x8 widen8_bf16(int lo, int hi) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, false);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, true);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, false);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, true);
  return __builtin_shufflevector(__builtin_shufflevector(p0, p1, 0, 1, 2, 3),
                                 __builtin_shufflevector(p2, p3, 0, 1, 2, 3), 0, 1, 2, 3, 4, 5,
                                 6, 7);
}

// max(0, x) in one instruction (median of x, 0 and the largest float; scores are finite)
__device__ __forceinline__ float relu(float x) { return __builtin_amdgcn_fmed3f(x, 0.f, 3.402823466e38f); }

// The head-weighted ReLU sum of key tile j (16 keys) on the FP8 matrix instruction, from the
// tile's two 16-byte halves in the MFMA B layout (lo: bytes [16g, 16g+16) of row 16j + n, hi:
// bytes [64+16g, 64+16g+16)).  The four head tiles' products go out before the first is read
// (one accumulator reused would make each wait for the previous one's result).  MXFP8: the B
// block-scale byte of lane (n, g) is group g of key 16j + n.
template <int QM>
__device__ __forceinline__ float fp8_tile_sum(const QOps<QM>& A, const float (&wp)[4][4],
                                              i32x4 lo, i32x4 hi, KScale<QM> ks, int j) {
  const int lane = threadIdx.x & 63;
  const i32x8 B = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  int sb = 0;
  if constexpr (QM == kQMx)
    sb = __builtin_amdgcn_ubfe((uint32_t)__shfl((int)ks, 16 * j + (lane & 15)), 8 * (lane >> 4),
                               8);
  f32x4 c[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    c[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (QM == kQMx)
      c[m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A.a[m], B, c[m], 0, 0, 0, A.sa[m],
                                                              0, sb);
    else
      c[m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A.a[m], B, c[m], 0, 0, 0, 0, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  float acc = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = fmaf(wp[m][i], relu(c[m][i]), acc);
  return acc;
}

// Head sum over g and 4x4 transpose of the four tiles' partial sums: lane l ends with the score
// of key 16 (l >> 4) + (l & 15), times the key's scale (MXFP8: its scales entered the products).
template <int QM>
__device__ __forceinline__ float group_finish(const float (&v)[4], KScale<QM> ks) {
  float k0 = pair32_sum(v[0], v[2]);
  float k1 = pair32_sum(v[1], v[3]);
  const float r = pair16_sum(k0, k1);
  if constexpr (QM == kQMx) return r;
  else return r * ks;
}

// Scores of the 64 keys of one page-aligned group; lane l returns key base + l, times the
// key's scale word ks (the key's fp32 scale; MXFP8: its scale bytes enter the products).
template <int QM>
__device__ __forceinline__ float score_group(const QOps<QM>& A, const float (&wp)[4][4],
                                             const KTile4& kt, KScale<QM> ks) {
  float v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (QM == kQBf16) {
      bf16x8 B[4];
      B[0] = widen8_bf16(kt.lo[j][0], kt.lo[j][1]);
      B[1] = widen8_bf16(kt.lo[j][2], kt.lo[j][3]);
      B[2] = widen8_bf16(kt.hi[j][0], kt.hi[j][1]);
      B[3] = widen8_bf16(kt.hi[j][2], kt.hi[j][3]);
      float acc = 0.f;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st)
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A.a[m][st]),
                                                      B[st], c, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = fmaf(wp[m][i], relu(c[i]), acc);
      }
      v[j] = acc;
    } else {
      v[j] = fp8_tile_sum<QM>(A, wp, kt.lo[j], kt.hi[j], ks, j);
    }
  }
  return group_finish<QM>(v, ks);
}

// The same for an FP8 mode straight from a page buffer in LDS, each key tile read just before
// its products (the four tiles held at once would cost 24 more registers per lane).
template <int QM>
__device__ __forceinline__ float score_group_lds(const QOps<QM>& A, const float (&wp)[4][4],
                                                 const uint8_t* st, KScale<QM> ks) {
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  float v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    v[j] = fp8_tile_sum<QM>(A, wp, *(const i32x4*)(st + swz(16 * j + n, g)),
                            *(const i32x4*)(st + swz(16 * j + n, 4 + g)), ks, j);
  return group_finish<QM>(v, ks);
}

// Decode scoring: one token per workgroup (blockIdx.x) and key chunk blockIdx.y of 8 * np pages
// (np pages per wave, np <= 64); the pages are dealt round-robin to the eight waves (wave w
// scores pages w, w+8, ... of the chunk), so that at each step the workgroup reads 64 KB of
// consecutive pages when the request's pages are consecutive.  The host picks np so that the
// grid still covers the chip: long rows at few tokens take large chunks, which pays the
// token's set-up (request lookup, query quantisation, filling the page ring) once per chunk.
// (kernel signatures name no type that depends on the mode: the key scales come in untyped)
// BLK: block-granular scoring: instead of one score per key, one per 64-key page, the largest
// score among the page's causal keys (-inf for a page whose table entry is out of range),
// written to scores[tl][page]; the wave reduces the page's 64 scores and stores once.
template <int QM, bool BLK>
__global__ __launch_bounds__(512) void idx_score_fp8_kernel(DevBatch bt, int t_begin,
    int t_count, const uint16_t* q_idx, const float* w, const uint8_t* kpool,
    const void* kscale_raw, float* __restrict__ scores, int64_t ld, int np) {
  constexpr bool BQ = QM == kQBf16;
  const KScale<QM>* kscale = (const KScale<QM>*)kscale_raw;
  // (the wave index through readfirstlane, so that the ranges derived from it are scalars)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  constexpr int kStep = 8;  // page stride of a wave within the chunk
  const int tl = blockIdx.x;
  const int poff = wave;    // the wave's first page within the chunk
  const int chunk = 64 * kStep * np;
  const int k0 = blockIdx.y * chunk;
  if (tl >= t_count) return;  // (the same for every wave of the workgroup)
  const int t = t_begin + tl;
  // The wave's page ids, lane g holding that of its page g (chunk page poff + 8g), fetched
  // once (a scalar page-table load per page would stall every prefetch on a scalar round
  // trip).  Everything waits on them, so they are requested first, together with the token's
  // request lookup, for request min(t, B - 1) (the request of token t when every request has
  // one token), and again if that was not it.  The query goes out behind them (loads complete
  // in issue order, so the first pages need not wait for it).  The eight waves share the
  // token, so waves 0..3 each quantise one 16-head tile and hand it over through LDS (every
  // wave loads tile wave & 3: a load under a branch would make the compiler wait for the
  // query before the first pages).
  const int pg0 = k0 >> 6;
  const int pcol = min(pg0 + poff + kStep * min(lane, np - 1), bt.pt_stride - 1);
  const int bguess = min(t, bt.B - 1);
  int my_page = bt.page_table[(int64_t)bguess * bt.pt_stride + pcol];
  const LocLoads lw = locate_issue(bt);
  asm volatile("" ::: "memory");  // (the query loads stay behind these)
  const uint16_t* qrow = q_idx + (int64_t)t * kIH * kID;
  const float* wrow = w + (int64_t)t * kIH;
  i32x4 qr[4];
  float qw[4];
  a0_load_tile(qrow, wrow, lane, wave & 3, qr, qw);
  const TokLoc loc = locate_finish(bt, t, lw);
  const int k1 = min(k0 + chunk, loc.n);                 // the chunk's keys in range
  const int npg = k0 < k1 ? (k1 - 1 - k0) / 64 + 1 : 0;  // its pages in range (<= 8 np)
  const int gn = npg > poff ? (npg - poff + kStep - 1) / kStep : 0;  // the wave's, in range
  // A wave with no keys leaves now, unless it quantises a query tile for the others (it
  // then scores nothing and its page fetches read nothing).  (An ended wave no longer takes
  // part in the workgroup's barriers.)
  if (gn == 0 && wave >= 4) return;
  if (loc.b != bguess) my_page = bt.page_table[(int64_t)loc.b * bt.pt_stride + pcol];
  float* out = scores + (int64_t)tl * ld;

  // Page g of the wave is in range while g < gn.  A four-slot ring of pages keeps three in
  // flight while one is scored.  Nothing in the page loop branches around a load or a store
  // (under a branch the compiler waits for every outstanding load, which would leave one page
  // in flight): a page and its key scales are fetched through buffer resources whose record
  // count is zero past the wave's last page (or for a table entry out of range), so those
  // fetches return zeros without reading memory, and scores go out through a buffer resource
  // that ends at the chunk's last key in range, so the hardware drops stores past it.
  struct Slot {
    KPage kp;
    KScale<QM> ks;
    bool ok;
  };
  auto fetch = [&](int g, Slot& sl) {
    const int page = __builtin_amdgcn_readlane(my_page, g & 63);
    sl.ok = page >= 0 && page < bt.n_pages;
    const bool on = sl.ok && g < gn;
    const int64_t pg = on ? page : 0;
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kpool + pg * kPage * kID), 0, on ? kPage * kID : 0, kBufDword3);
    const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kscale + pg * kPage), 0, on ? kPage * (int)sizeof(KScale<QM>) : 0, kBufDword3);
    // (the key scale first: one short read ahead of the page's eight, so that waiting for a
    // scale never waits for a page)
    sl.ks = __builtin_bit_cast(KScale<QM>, __builtin_amdgcn_raw_buffer_load_b32(sr, 4 * lane, 0, 0));
    load_kpage_rsrc(kr, lane, sl.kp);
  };
  // (kept in this order by the empty asm statements: each wait in the loop counts the loads
  // issued after the page it waits for, and one moved behind later pages would make it wait
  // for those too)
  Slot sl[4];
#pragma unroll
  for (int g = 0; g < 3; ++g) {
    fetch(g, sl[g]);
    asm volatile("" ::: "memory");
  }
  __shared__ __attribute__((aligned(16))) uint8_t stage_sh[8 * kStage];
  uint8_t* stage = stage_sh + wave * kStage;
  QOps<QM> A;
  float wp[4][4];
  {
    // (e4m3: one 32-byte operand per lane and tile, plus the MXFP8 scale byte; bf16: the 64
    // loaded bytes as they are)
    __shared__ i32x4 a_sh[4][BQ ? 4 : 2][64];
    __shared__ f32x4 w_sh[4][64];
    __shared__ int s_sh[4][QM == kQMx ? 64 : 1];
    if (wave < 4) {
      float wt[4];
      if constexpr (BQ) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a_sh[wave][i][lane] = qr[i];
          wt[i] = qw[i];
        }
      } else {
        i32x8 at;
        if constexpr (QM == kQMx) {
          int sa;
          mx_tile(qr, qw, lane, at, sa, wt);
          s_sh[wave][lane] = sa;
        } else {
          a0_tile(qr, qw, lane, at, wt);
        }
        a_sh[wave][0][lane] = i32x4{at[0], at[1], at[2], at[3]};
        a_sh[wave][1][lane] = i32x4{at[4], at[5], at[6], at[7]};
      }
      w_sh[wave][lane] = f32x4{wt[0], wt[1], wt[2], wt[3]};
    }
    __syncthreads();
    if (gn == 0) return;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if constexpr (BQ) {
#pragma unroll
        for (int i = 0; i < 4; ++i) A.a[m][i] = a_sh[m][i][lane];
      } else {
        const i32x4 lo = a_sh[m][0][lane], hi = a_sh[m][1][lane];
        A.a[m] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        if constexpr (QM == kQMx) A.sa[m] = s_sh[m][lane];
      }
      const f32x4 wv = w_sh[m][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) wp[m][i] = wv[i];
    }
  }
  // stores at byte offset 4*s of the row, kept for s < k1 (BLK: 4*page, for pages below k1)
  const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
      out, 0, BLK ? ((k1 + 63) >> 6) * 4 : k1 * 4, kBufDword3);
  // page g from ring slot u: fetch page g + 3 into the slot freed last, then score page g
  auto step = [&](int g, int u) {
    fetch(g + 3, sl[(u + 3) & 3]);
    asm volatile("" ::: "memory");  // (the loads go out before this page is scored)
    const Slot& c = sl[u];
    KTile4 kt;
    stage_ktile4(stage, lane, c.kp, kt);
    float sc = score_group<QM>(A, wp, kt, c.ks);
    if (!c.ok) sc = -INFINITY;
    const int pos = k0 + 64 * (poff + g * kStep) + lane;
    if constexpr (BLK) {
      // the page's largest causal score, stored by lane 0 (the other lanes' offsets lie past
      // the resource's end, so the hardware drops their stores)
      const float m = wave_max(pos < k1 ? sc : -INFINITY);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m), orsrc,
                                            lane == 0 ? (pos >> 6) * 4 : 0x40000000, 0, 0);
    } else {
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), orsrc, pos * 4, 0, 0);
    }
  };
  // four pages per iteration, so that every ring slot is a fixed register set.  The loop has
  // one exit, at its end (an exit between its pages would make the compiler's wait insertion
  // assume that path could loop as well, and wait for a page more); the pages of the last
  // iteration past the wave's range read nothing and store nothing.
  for (int g0 = 0; g0 < gn; g0 += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) step(g0 + u, u);
  }
}

// Prefill scoring with shared key pages: four consecutive tokens per 4-wave workgroup (one per
// wave) over one 4096-key chunk (64 pages, so that the query's load and quantisation are paid
// once per 64 pages).  The tokens of one request read the same pages:
// the four waves split each page's eight 1 KB loads (wave w: loads 2w, 2w + 1), write them
// once into a double-buffered LDS page (one barrier per page, the next page written while the
// current one is scored), and every wave scores its own token from it, so a page crosses the
// memory path and the LDS transpose once per workgroup instead of once per token.  A ring of
// four pieces keeps three pages in flight per wave.  Tokens of the group that belong to
// different requests are scored in one pass per request (every wave loads and waits in every
// pass; a wave stores only in its own request's pass, through a buffer resource whose record
// count is zero otherwise).  A wave without a token (the batch's last group) only loads.
// (FP8 modes: at most 128 registers, four waves per SIMD, so that one wave's vector epilogue
// overlaps another's matrix products; the bf16 query mode needs more)
template <int QM, bool BLK>
__global__ __launch_bounds__(256, QM == kQBf16 ? 1 : 4) void idx_score_group_kernel(DevBatch bt, int t_begin,
    int t_count, const uint16_t* q_idx, const float* w, const uint8_t* kpool,
    const void* kscale_raw, float* __restrict__ scores, int64_t ld) {
  constexpr int kChunk = 4096;
  const KScale<QM>* kscale = (const KScale<QM>*)kscale_raw;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int tl = blockIdx.x * 4 + wave;
  const bool has = tl < t_count;
  const int tc = min(tl, t_count - 1);  // (a wave without a token reads a valid query)
  const int t = t_begin + tc;
  const int k0 = blockIdx.y * kChunk;
  const LocLoads lw = locate_issue(bt);
  asm volatile("" ::: "memory");
  QRaw qr;
  a0_load(q_idx + (int64_t)t * kIH * kID, w + (int64_t)t * kIH, lane, qr);
  const TokLoc loc = locate_finish(bt, t, lw);
  __shared__ int req_sh[4], n_sh[4];
  __shared__ __attribute__((aligned(16))) uint8_t pg_sh[2][kStage];
  if (lane == 0) {
    req_sh[wave] = has ? loc.b : -1;
    n_sh[wave] = has ? loc.n : 0;
  }
  QOps<QM> A;
  float wp[4][4];
  q_prologue<QM>(qr, lane, A, wp);
  __syncthreads();
  int rq[4], nn[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    rq[i] = __builtin_amdgcn_readfirstlane(req_sh[i]);
    nn[i] = __builtin_amdgcn_readfirstlane(n_sh[i]);
  }
  float* out = scores + (int64_t)tc * ld;
  const int my_k1 = has ? min(k0 + kChunk, loc.n) : 0;  // the token's keys below this bound
  struct Piece {
    i32x4 r[2];
    KScale<QM> ks;
    bool ok;
  };
#pragma unroll 1
  for (int r = 0; r < 4; ++r) {
    const int b = rq[r];
    bool first = b >= 0;
#pragma unroll
    for (int r2 = 0; r2 < 4; ++r2)
      if (r2 < r && rq[r2] == b) first = false;
    if (!first) continue;  // (uniform: each request once)
    int nmax = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (rq[i] == b) nmax = max(nmax, nn[i]);
    const int k1 = min(k0 + kChunk, nmax);
    const int npg = k0 < k1 ? (k1 - 1 - k0) / 64 + 1 : 0;
    if (npg == 0) continue;  // (uniform)
    // stores at byte offset 4*s of the token's row, kept for s < my_k1 in its own request's pass
    // (BLK: 4*page, for pages below my_k1)
    const bool mine = has && loc.b == b;
    const int rec = BLK ? ((my_k1 + 63) >> 6) * 4 : my_k1 * 4;
    const __amdgpu_buffer_rsrc_t orsrc =
        __builtin_amdgcn_make_buffer_rsrc(out, 0, mine ? rec : 0, kBufDword3);
    const int pcol = min((k0 >> 6) + lane, bt.pt_stride - 1);
    const int my_page = bt.page_table[(int64_t)b * bt.pt_stride + pcol];
    // (no branch around a load: a page past the range is fetched through buffer resources
    // whose record count is zero, which return zeros without reading memory)
    auto fetch = [&](int g, Piece& pc) {
      const int page = __builtin_amdgcn_readlane(my_page, g & 63);
      pc.ok = page >= 0 && page < bt.n_pages;
      const bool on = pc.ok && g < npg;
      const int64_t pg = on ? page : 0;
      const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(kpool + pg * kPage * kID), 0, on ? kPage * kID : 0, kBufDword3);
      const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(kscale + pg * kPage), 0, on ? kPage * (int)sizeof(KScale<QM>) : 0, kBufDword3);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        pc.r[i] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                kr, 1024 * (2 * wave + i) + 16 * lane, 0, kAuxNT));
      pc.ks = __builtin_bit_cast(KScale<QM>, __builtin_amdgcn_raw_buffer_load_b32(sr, 4 * lane, 0, 0));
    };
    // the wave's two loads of a page into its rows of LDS page buffer u
    auto put = [&](int u, const Piece& pc) {
#pragma unroll
      for (int i = 0; i < 2; ++i) put_load(pg_sh[u], 2 * wave + i, lane, pc.r[i]);
    };
    Piece ring[4];
#pragma unroll
    for (int g = 0; g < 3; ++g) {
      fetch(g, ring[g]);
      asm volatile("" ::: "memory");
    }
    __syncthreads();  // (the previous pass's readers are done with the buffers)
    put(0, ring[0]);
    __syncthreads();
    // page g from buffer g & 1 (ring slot g & 3): fetch page g + 3, write page g + 1 into the
    // other buffer, score page g, wait for every wave.  Four pages per iteration and one exit,
    // at its end (an exit between pages would make the compiler's wait insertion assume that
    // path could loop as well, and drain the ring at every iteration); the last iteration's
    // pages past the range read nothing and store nothing.
#pragma unroll 1
    for (int g0 = 0; g0 < npg; g0 += 4) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int g = g0 + u;
        fetch(g + 3, ring[(u + 3) & 3]);
        asm volatile("" ::: "memory");
        put((u + 1) & 1, ring[(u + 1) & 3]);
        float sc;
        if constexpr (QM == kQBf16) {
          KTile4 kt;
          read_ktile4(pg_sh[u & 1], lane, kt);
          sc = score_group<QM>(A, wp, kt, ring[u].ks);
        } else {
          sc = score_group_lds<QM>(A, wp, pg_sh[u & 1], ring[u].ks);
        }
        if (!ring[u].ok) sc = -INFINITY;
        const int pos = k0 + 64 * g + lane;
        if constexpr (BLK) {
          const float m = wave_max(pos < my_k1 ? sc : -INFINITY);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m), orsrc,
                                                lane == 0 ? (pos >> 6) * 4 : 0x40000000, 0, 0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), orsrc, pos * 4, 0, 0);
        }
        __syncthreads();
      }
    }
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

template <int QM, bool BLK>
static hipError_t launch_mma(const DevBatch& bt, int t_begin, int t_count, int max_n,
                             bool prefill_like, int np, const uint16_t* q_idx, const float* w,
                             const uint8_t* kpool, const void* kscale, float* scores, int64_t ld,
                             hipStream_t st) {
  // decode: one 8-wave workgroup per chunk of 512 * np keys of a token (64 np keys per wave);
  // prefill: four tokens per 4-wave workgroup sharing a 4096-key chunk
  if (prefill_like) {
    const int chunk = 4096;
    dim3 grid((t_count + 3) / 4, (max_n + chunk - 1) / chunk);
    auto* gfn = idx_score_group_kernel<QM, BLK>;
    hipLaunchKernelGGL(gfn, grid, dim3(256), 0, st, bt, t_begin, t_count,
                       q_idx, w, kpool, kscale, scores, ld);
    return hipGetLastError();
  }
  if (np < 1 || np > 64) return hipErrorInvalidValue;  // (lane g holds page g of a wave)
  const int chunk = 512 * np;
  dim3 grid(t_count, (max_n + chunk - 1) / chunk);
  auto* fn = idx_score_fp8_kernel<QM, BLK>;
  hipLaunchKernelGGL(fn, grid, dim3(512), 0, st, bt, t_begin, t_count,
                     q_idx, w, kpool, kscale, scores, ld, np);
  return hipGetLastError();
}

template <bool BLK>
static hipError_t launch_mode(const DevBatch& bt, int t_begin, int t_count, int max_n,
                              bool prefill_like, int np, int qmode, const uint16_t* q_idx,
                              const float* w, const uint8_t* kpool, const void* kscale,
                              float* scores, int64_t ld, hipStream_t st) {
  switch (qmode) {
    case kQBf16:
      return launch_mma<kQBf16, BLK>(bt, t_begin, t_count, max_n, prefill_like, np, q_idx, w,
                                     kpool, kscale, scores, ld, st);
    case kQMx:
      return launch_mma<kQMx, BLK>(bt, t_begin, t_count, max_n, prefill_like, np, q_idx, w, kpool,
                                   kscale, scores, ld, st);
    default:
      return launch_mma<kQFp8, BLK>(bt, t_begin, t_count, max_n, prefill_like, np, q_idx, w,
                                    kpool, kscale, scores, ld, st);
  }
}

hipError_t launch_index_score_fp8(const DevBatch& bt, int t_begin, int t_count, int max_n,
                                  bool prefill_like, int np, int qmode, bool block, const uint16_t* q_idx,
                                  const float* w, const uint8_t* kpool, const void* kscale,
                                  float* scores, int64_t ld, hipStream_t st) {
  return block ? launch_mode<true>(bt, t_begin, t_count, max_n, prefill_like, np, qmode, q_idx, w,
                                   kpool, kscale, scores, ld, st)
               : launch_mode<false>(bt, t_begin, t_count, max_n, prefill_like, np, qmode, q_idx, w,
                                    kpool, kscale, scores, ld, st);
}

}  // namespace tis
