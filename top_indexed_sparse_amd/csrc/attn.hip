// Sparse MLA attention over the selected rows of a paged latent cache.
//
// Method: "Day 0 Support for New LLM Architectures", Step 1 (the sparse-attention kernel
// reads only the selected entries of the low-rank KV cache and computes exact attention)
// and Key Optimization 1 (after selection, the attention kernel gathers from the main KV
// by index).  "Day-0 Support for Large Model Inference", Core Operator Optimization 2
// (gather the non-contiguous rows, compute blockwise with fused normalisation, balance
// variable lengths).  Every head reads the same latent row: keys are the full 576-wide row
// (512 latent + 64 RoPE), values are its first 512 dims.
//
// Matrix-core kernel (bf16 or e4m3 cache), one 4-wave workgroup per (token, key split,
// group of 64 heads); wave (hh, dv) owns 32 heads (half hh of the group) and value dims
// 256dv .. 256dv + 255 over every key of the split:
//   * the split's positions are translated through the page table once into LDS;
//   * 32-row stages are gathered with 16-byte loads (each wave a fixed eight rows) into a
//     one-stage register queue and written into a three-stage LDS ring; the value part of an
//     e4m3 row is widened exactly to fp16 as it is written (once per workgroup), its RoPE part
//     stays e4m3 and is widened per fragment; the matrix cores then run on fp16 (Q rounded to
//     fp16 once), and on bf16 for a bf16 cache;
//   * each wave multiplies its half of the 576 contracted dims, S^T = K . Q^T on
//     v_mfma_f32_16x16x32 (all of its Q^T in registers), and the two waves of a head half
//     add their partial logits through LDS;
//   * O^T[vdim][head] += V^T . P^T on v_mfma_f32_32x32x16: P reaches the B layout with one
//     permlane16 swap, and V^T fragments come from the row-major tile via
//     ds_read_b64_tr_b16 (bf16 / fp16);
//   * the stages are software pipelined (QK^T of stage st beside the softmax of stage
//     st - 1, then PV of st - 1 beside the ring writes and gathers), with the order of
//     matrix and vector work pinned by scheduling fences;
//   * the running max is raised lazily, only when a stage's P would exceed 2^15 (fp16 P of an
//     e4m3 cache: below the format's largest value) or 2^30 (bf16 P), so rescaling the
//     accumulators is rare even where the logits grow along the selected positions;
//   * e4m3: per-token scales go into the logits in fp32 and into P relative to the split's
//     largest scale; P then is fp16 (11-bit significand) so that heavy rows stay accurate,
//     and the normaliser is accumulated from the same rounded P values;
//   * each wave writes its own O (through LDS, in whole lines); with several splits per
//     token, the (m, l, O) partials are merged by mla_combine_kernel with log-sum-exp
//     weights.
#include "common.h"
#include "launch.h"

#include <algorithm>
#include <type_traits>
#include <utility>

namespace tis {

// ---------------------------------------------------------------- fp32 (small shapes)
__global__ __launch_bounds__(256) void mla_attn_f32_kernel(DevBatch bt, int t_begin,
    const float* __restrict__ q, const float* __restrict__ kv, const int32_t* __restrict__ idx,
    int K, int H, int Dqk, int Dv, float scale, float* __restrict__ out,
    float* __restrict__ lse) {
  extern __shared__ float smf[];  // q[Dqk], logits[K], slots (as int) [K]
  float* sq = smf;
  float* z = smf + Dqk;
  int* slots = (int*)(z + K);
  __shared__ float red[64];
  const int t = t_begin + blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const TokLoc loc = locate(bt, t);
  const int b = loc.b;
  const int L = loc.L;
  for (int d = tid; d < Dqk; d += blockDim.x) sq[d] = q[((int64_t)t * H + h) * Dqk + d];
  for (int i = tid; i < K; i += blockDim.x) {
    const int s = idx[(int64_t)t * K + i];
    int64_t slot = (s >= 0 && s < L) ? slot_of(bt, b, s) : -1;
    slots[i] = (int)slot;
  }
  __syncthreads();
  float mloc = -INFINITY;
  for (int i = tid; i < K; i += blockDim.x) {
    float v = -INFINITY;
    if (slots[i] >= 0) {
      const float* r = kv + (int64_t)slots[i] * Dqk;
      float acc = 0.f;
      for (int d = 0; d < Dqk; ++d) acc = fmaf(sq[d], r[d], acc);
      v = acc * scale;
    }
    z[i] = v;
    mloc = fmaxf(mloc, v);
  }
  for (int o = 32; o > 0; o >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, o));
  if ((tid & 63) == 0) red[tid >> 6] = mloc;
  __syncthreads();
  float m = -INFINITY;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) m = fmaxf(m, red[w]);
  __syncthreads();
  float lloc = 0.f;
  for (int i = tid; i < K; i += blockDim.x) {
    const float p = (z[i] == -INFINITY) ? 0.f : expf(z[i] - m);
    z[i] = p;
    lloc += p;
  }
  for (int o = 32; o > 0; o >>= 1) lloc += __shfl_xor(lloc, o);
  if ((tid & 63) == 0) red[tid >> 6] = lloc;
  __syncthreads();
  float l = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) l += red[w];
  const float inv = l > 0.f ? 1.f / l : 0.f;
  for (int d = tid; d < Dv; d += blockDim.x) {
    float acc = 0.f;
    for (int i = 0; i < K; ++i)
      if (slots[i] >= 0) acc = fmaf(z[i], kv[(int64_t)slots[i] * Dqk + d], acc);
    out[((int64_t)t * H + h) * Dv + d] = acc * inv;
  }
  if (lse && tid == 0) lse[(int64_t)t * H + h] = l > 0.f ? m + logf(l) : -INFINITY;
}

// ---------------------------------------------------------------- matrix-core kernel
constexpr int kH = 128, kDqk = 576, kDv = 512;
constexpr int kHB = 32;        // heads per wave
constexpr int kHW = 2 * kHB;   // heads per workgroup
constexpr int kWT = 16;        // rows (keys) per tile
constexpr int kSR = 2 * kWT;   // rows per stage: the tiles of the two key halves
constexpr int kMaxKps = 2048;  // keys per split (bounds the LDS index table)
constexpr float kMFloor = -1e30f;  // running max before the first live key (log2 units)
// 16-row tiles are gathered with 16-byte loads into registers and written to LDS (a load
// straight to LDS costs its wave about twice the issue time of a load plus an LDS write); the
// two waves that read a tile (the two head halves of one key half) issue half of its loads
// each.  A tile has two regions: A holds the value part of each row (its first 512 dims) at
// a padded row stride, one load instruction per row (every lane a 16-byte chunk of that row,
// so the source is a per-row scalar base plus the lane offset: no per-lane address
// arithmetic); B holds the 64 RoPE dims of the 16 rows (bf16: two loads, e4m3: one).  The A stride is 8 dwords more
// than a multiple of the 64 LDS banks and the B stride 4 more than a multiple of 16 (both
// measured fastest for the reads below), and the rows are consumed in the order
// pi(8h + j) = 8h + 2j (j < 4), 8h + 2(j - 4) + 1 (j >= 4), which makes both the 16-byte
// key-fragment reads and the transposed value reads nearly free of bank conflicts.  Region A
// holds 16-bit values in both cases (an e4m3 row's value part is widened exactly to fp16 as it
// is written, once per workgroup, instead of at every fragment read); region B holds the RoPE
// dims as cached (bf16, or e4m3, widened per fragment: one fragment of nine), which keeps the
// e4m3 kernel's LDS, with its row-scale table, within the 160 KB.
template <bool FP8>
struct KvFmt {
  static constexpr int kRowBytes = FP8 ? kDqk : 2 * kDqk;   // cached row (global memory)
  static constexpr int kVBytes = FP8 ? kDv : 2 * kDv;       // its value part
  static constexpr int kRBytes = kRowBytes - kVBytes;       // its RoPE part: 64 / 128
  static constexpr int kAStride = 2 * kDv + 32;             // row stride, region A (16-bit)
  static constexpr int kRStride = kRBytes + 16;             // row stride, region B (as cached)
  static constexpr int kABytes = kWT * kAStride;
  static constexpr int kBBytes = kWT * kRStride;
  static constexpr int kWBytes = kABytes + kBBytes;         // one wave tile
};
__host__ __device__ constexpr int tile_row(int m) {  // pi: consumption order -> tile row
  return (m & 8) + ((m & 4) ? 2 * (m & 3) + 1 : 2 * (m & 3));
}

// Q^T per wave: 9 fragments of 32 dims (8 of value dims, 1 of RoPE dims) per 16 heads, the
// wave's half of the contracted dims, all in registers.
constexpr int kNQ2 = 9;
constexpr int kDvW = kDv / 2;  // value dims per wave
constexpr int kRing = 3;       // stages in the LDS ring
// LDS reads in flight per wave: one wave per SIMD keeps the LDS busy only with many reads
// outstanding (K fragments read this many steps ahead, V^T this many dim tiles ahead)
constexpr int kKPre = 6, kVPre = 3;
constexpr int kOStage = kDvW + 4;  // floats per head row when O is staged for the stores

// Dynamic LDS: ring of three stages (two tiles each) | rows[kMaxKps] | masks[kMaxKps/16] |
// scl[kMaxKps] (e4m3) | partial logits [2][4 waves][4 tiles][64 lanes] f32x4 | red/anyv/lastv.
template <bool FP8>
struct AttnSmem {
  static constexpr int rows = kRing * 2 * KvFmt<FP8>::kWBytes;
  static constexpr int masks = rows + kMaxKps * 4;
  static constexpr int scl = masks + kMaxKps / 16 * 2;
  static constexpr int xs = scl + (FP8 ? kMaxKps * 4 : 0);
  static constexpr int red = xs + 2 * 4 * 4096;
  // after the loop the whole area holds the waves' O, staged for whole-line stores
  static constexpr int ostage = 4 * kHB * kOStage * 4;
  static constexpr int total = red + 64 > ostage ? red + 64 : ostage;
  static_assert(xs % 16 == 0 && total <= 160 * 1024, "LDS budget");
};

// Split partials of a bf16 output: the split's normalised O in fp16 scaled by 2^-8, i.e.
// 11 significant bits for |O| up to 1.6e7 (saturating beyond), half the bytes of fp32 and
// 8 times finer than bf16 (a bf16 partial adds an error the size of the output rounding).
constexpr float kPartScale = 1.f / 256.f, kPartUnscale = 256.f;

// Eight consecutive partials as fp16 (one 16-byte store).
__device__ __forceinline__ void store_part16x8(void* part, int64_t off, f32x4 lo, f32x4 hi) {
  f16x8 h;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = (_Float16)fminf(fmaxf(lo[i] * kPartScale, -65504.f), 65504.f);
    h[4 + i] = (_Float16)fminf(fmaxf(hi[i] * kPartScale, -65504.f), 65504.f);
  }
  *(f16x8*)((uint16_t*)part + off) = h;
}

// Eight consecutive outputs at element offset `off`: fp32 (two 16-byte stores) or bf16
// (round to nearest even; one 16-byte store).
template <bool OUT_F32>
__device__ __forceinline__ void store_out8(void* out, int64_t off, f32x4 lo, f32x4 hi) {
  if (OUT_F32) {
    *(f32x4*)((float*)out + off) = lo;
    *(f32x4*)((float*)out + off + 4) = hi;
  } else {
    i32x4 w;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      w[i] = (int)((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo[2 * i]) |
                   ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo[2 * i + 1]) << 16));
      w[2 + i] = (int)((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi[2 * i]) |
                       ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi[2 * i + 1]) << 16));
    }
    *(i32x4*)((uint16_t*)out + off) = w;
  }
}

// One accumulator element times alpha, into a VGPR (the accumulator is left as it is).
__device__ __forceinline__ float acc_read_scaled(float x, float alpha) {
  float r;
  asm volatile("v_accvgpr_read_b32 %0, %1\n\tv_mul_f32 %0, %0, %2" : "=&v"(r) : "a"(x), "v"(alpha));
  return r;
}

// Scale an accumulator tile in place, element by element through one VGPR.  Written out so
// that the tile never leaves the accumulator registers: a plain multiply makes the register
// allocator move all 256 accumulators of a wave into VGPRs and spill.
__device__ __forceinline__ void acc_scale(f32x16& acc, float alpha) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float x = acc[i];
    float tmp;
    asm volatile(
        "v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
        : "+a"(x), "=&v"(tmp)
        : "v"(alpha));
    acc[i] = x;
  }
}

// Sum / max over the four 16-lane rows (lanes c, c+16, c+32, c+48).
__device__ __forceinline__ float rows4_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return xor32_max(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ __forceinline__ float rows4_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return xor32_sum(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

// One workgroup per (token, key split, group of 64 heads).  Wave w = (hh, dv) = (w & 1, w >> 1)
// owns heads 32hh .. 32hh + 31 of the group and value dims 256dv .. 256dv + 255, over every key
// of the split; its QK^T covers one half of the 576 contracted dims (value dims 256dv.. and RoPE
// dims 512 + 32dv..), and the two waves of a head half (w and w ^ 2) add their partial logits
// through LDS.  Per 32-key stage (two 16-row tiles) and wave:
//   S^T[16 keys][16 heads] x 2 x 2 = K . Q^T on v_mfma_f32_16x16x32_bf16 (fp16 for e4m3) over 9 fragments of 32
//     dims (K fragments from LDS, all of the wave's Q^T resident in registers; e4m3 rows are
//     widened exactly: value dims to fp16 as the row is written, RoPE dims per fragment);
//   the partial logits go to LDS; after the next barrier each wave adds its partner's and runs
//   the online softmax per head (lane-local over 8 keys, then across the four 16-lane rows);
//   one permlane16 swap per tile moves P^T into the B layout of v_mfma_f32_32x32x16, and
//   O^T[32 dims][32 heads] += V^T . P^T for the wave's 8 dim tiles, V^T read by
//   ds_read_b64_tr_b16 (bf16 / fp16).
// The stages are software pipelined.  In the iteration of stage st a wave computes its partial
// QK^T of stage st while it finishes the softmax of stage st - 1 (whose logits its partner
// completed before the barrier), then runs PV of stage st - 1 while it writes the gathered rows
// of stage st + 1 into the LDS ring (three stages) and issues the gathers of stage st + 2 (one
// stage of rows in flight in registers).  The running max is raised lazily (only when a
// stage's P would exceed 2^15 with fp16 P, 2^30 with bf16 P), by recomputing the stage's
// softmax.  e4m3: per-row scales enter the fp32
// logits and P relative to the split's largest scale; P is fp16 and the normaliser sums the same
// rounded values.  Each wave writes its own heads' dims of O (or, with several splits, the
// partials that mla_combine_kernel merges), transposed through LDS into whole lines.
// DENSE: the same attention computed the dense-masked way ("Achieving Day-0 Readiness ...
// Million-Token Context", section 2.3: the prefill path multiplies over the full key range with
// a row-wise sparse mask): split j covers the token's causal positions [j*kps, (j+1)*kps), every
// one of them is gathered and multiplied, and the selection (the K entries of idx, built into an
// LDS bitmask of the split's positions) only decides which rows' P is kept; the rest are masked
// exactly as unselected rows (P = 0).  A position listed twice counts once.
// Token order of a launch: v -> token, a bijection of [0, n): the first 16*S positions
// (S = n / 16) are 16 segments of S, segment g taking the place of segment g/2 (g even) or
// 15 - g/2 (g odd); the rest stay where they are.
__device__ __forceinline__ int zigzag16(int v, int n) {
  const int S = n >> 4;
  if (S == 0 || v >= 16 * S) return v;
  const int g = v / S, j = v - g * S;
  const int seg = (g & 1) ? 15 - (g >> 1) : (g >> 1);
  return seg * S + j;
}

template <bool FP8, bool OUT_F32, bool DENSE = false>
__device__ __forceinline__ void mla_attn_body(DevBatch bt, int t_begin, int t_count,
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv,
    const float* __restrict__ kvscale, const int32_t* __restrict__ idx, int K, float c2,
    int nsplit, int kps, void* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_ml) {
  using F = KvFmt<FP8>;
  using SM = AttnSmem<FP8>;
  extern __shared__ __attribute__((aligned(16))) char sm[];
  char* ring = sm;
  int* rows = (int*)(sm + SM::rows);
  uint16_t* masks = (uint16_t*)(sm + SM::masks);
  float* scl = (float*)(sm + SM::scl);
  char* xs = sm + SM::xs;  // partial logits [2 buffers][4 waves][4 tiles][64 lanes] f32x4
  float* red = (float*)(sm + SM::red);
  int* anyv = (int*)(red + 4);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c16 = lane & 15, g4 = lane >> 4;  // 16x16 layouts
  const int c32 = lane & 31, h2 = lane >> 5;  // 32x32 layouts
  const int hh = wave & 1, dv = wave >> 1;    // head half, value-dim half
  const int partner = wave ^ 2;

  // workgroup -> (token, split, head group); the workgroups of one token sit on one XCD
  // (workgroups are dealt to the 8 XCDs round-robin), so its rows are fetched from HBM once
  // and served to the other head group from that XCD's L2.  Each XCD takes a contiguous range
  // of virtual tokens, and the virtual tokens are the launch's tokens in zigzag order ("Day 0
  // Support for New LLM Architectures", Key Optimization 3, applied to the XCDs): cut into 16
  // segments, XCD x gets segments x and 15 - x, so that in a causal batch (work growing with
  // the token's position) no XCD holds all of the longest tokens.
  const int nblk = gridDim.x;
  const int xcd = blockIdx.x & 7, slot8 = blockIdx.x >> 3;
  const int per = nblk >> 3, extra = nblk & 7;
  const int pidx = xcd * per + min(xcd, extra) + slot8;
  const int hg = pidx & 1;
  const int split = (pidx >> 1) % nsplit;
  const int tl = zigzag16((pidx >> 1) / nsplit, t_count);
  const int t = t_begin + tl;
  const int h0 = hg * kHW + hh * kHB;  // this wave's first head

  const int kbeg = split * kps;

  // ---- positions -> physical slots (and e4m3 row scales); masked keys read slot 0.  Each
  // thread translates up to kPer rows with its loads batched per step: the positions (they
  // only need the token) go out together with the token's request lookup, then the pages,
  // then the scales, so the chain costs three memory latencies however many rows there are.
  constexpr int kPer = kMaxKps / 256;
  int pos[kPer];
  bool sel[kPer];  // (dense: the row is selected)
  int nk;
  TokLoc loc;
  if constexpr (DENSE) {
    uint32_t* bits = (uint32_t*)xs;  // (the logit exchange area is free until the loop)
    if (tid < kMaxKps / 32) bits[tid] = 0u;
    const LocLoads lw = locate_issue(bt);
    loc = locate_finish(bt, t, lw);
    nk = max(0, min(kps, loc.n - kbeg));  // the token's causal positions in this split
    __syncthreads();
    for (int i = tid; i < K; i += 256) {
      const int e = idx[(int64_t)t * K + i] - kbeg;
      if (e >= 0 && e < nk) atomicOr(&bits[e >> 5], 1u << (e & 31));
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = tid + 256 * j;
      pos[j] = i < nk ? kbeg + i : -1;
      sel[j] = i < nk && ((bits[i >> 5] >> (i & 31)) & 1u) != 0u;
    }
  } else {
    nk = max(0, min(kps, K - kbeg));
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = tid + 256 * j;
      pos[j] = i < nk ? idx[(int64_t)t * K + kbeg + i] : -1;
      sel[j] = true;
    }
    const LocLoads lw = locate_issue(bt);
    loc = locate_finish(bt, t, lw);
  }
  const int nstage = (nk + kSR - 1) / kSR;
  const int nrows = nstage * kSR;
  const int b = loc.b;
  const int Lb = loc.L;
  const int32_t* ptb = bt.page_table + (int64_t)b * bt.pt_stride;
  int slot[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int sp = pos[j];
    slot[j] = (sp >= 0 && sp < Lb) ? ptb[sp >> 6] : -1;
  }
  // The wave's Q^T fragments (B operand of 16x16x32: head 16ht + c16, dims 8g4.. of fragment
  // ks = value dims 256dv + 32ks (ks < 8) or RoPE dims 512 + 32dv (ks = 8)), issued after the
  // page lookups: loads complete in issue order, so the slots below wait for the page entries
  // only, and Q arrives while the slots and the first tiles are in flight.
  // (e4m3 cache: the matrix cores run on fp16, and Q is rounded to fp16 once, before the first
  // stage; bf16 -> fp16 is exact for |q| in [2^-14, 65504])
  using QOp = typename std::conditional<FP8, f16x8, bf16x8>::type;
  bf16x8 qb[2][kNQ2];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const uint16_t* qr = q + ((int64_t)t * kH + h0 + 16 * ht + c16) * kDqk + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < kNQ2; ++ks)
      qb[ht][ks] = *(const bf16x8*)(qr + (ks < kNQ2 - 1 ? 256 * dv + 32 * ks : kDv + 32 * dv));
  }
  QOp qf[2][kNQ2];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int pg = slot[j];
    slot[j] = (pg >= 0 && pg < bt.n_pages) ? pg * kPage + (pos[j] & (kPage - 1)) : -1;
  }
  float smax = 0.f;
  float scv[kPer];
  if (FP8) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) scv[j] = slot[j] >= 0 ? kvscale[slot[j]] : 0.f;
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = tid + 256 * j;
    if (i < nrows) {
      rows[i] = slot[j];
      if (FP8) {  // scales in consumption order: entry 16*tile + m is row pi(m) of the tile
        const int r = i & (kWT - 1);
        scl[(i & ~(kWT - 1)) + ((r & 8) | ((r & 1) << 2) | ((r >> 1) & 3))] = scv[j];
        smax = fmaxf(smax, sel[j] ? scv[j] : 0.f);
      }
    }
  }
  if (FP8) {
    for (int o = 32; o > 0; o >>= 1) smax = fmaxf(smax, __shfl_xor(smax, o));
    if (lane == 0) red[wave] = smax;
  }
  int* lastv = anyv + 4;
  {  // some selected row of the wave's rows (-1 if there is none): one ballot; and the last row
     // that is read at all (the stages past it hold only padding and are skipped)
    int v = -1;
#pragma unroll
    for (int j = 0; j < kPer; ++j) v = max(v, slot[j]);
    const uint64_t bb = __ballot(v >= 0);
    int last = -1;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const uint64_t bv = __ballot(slot[j] >= 0);
      if (bv) last = 256 * j + 64 * wave + 63 - __builtin_clzll(bv);
    }
    if (lane == 0) {
      anyv[wave] = bb ? __builtin_amdgcn_readlane(v, __builtin_ctzll(bb)) : -1;
      lastv[wave] = last;
    }
  }
  // per 16-row tile: bit m = row pi(m) selected (the order in which the keys are consumed),
  // from one ballot per row step: rows 256j + 64wave + l, four tiles, lane q < 4 writes
  // tile q's mask.  Row r of a tile is consumed as m = (r & 8) | (r & 1) << 2 | (r >> 1) & 3:
  // within each byte the even rows' bits go to the low nibble and the odd rows' to the high
  // one, an unzip of each byte in three mask-and-shift steps per half.
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const uint64_t bj = __ballot(slot[j] >= 0 && sel[j]);
    if (lane < 4) {
      const uint32_t nat = (uint32_t)(bj >> (16 * lane)) & 0xffffu;
      uint32_t e = nat & 0x5555u, o = (nat >> 1) & 0x5555u;
      e = (e | (e >> 1)) & 0x3333u;
      o = (o | (o >> 1)) & 0x3333u;
      e = (e | (e >> 2)) & 0x0f0fu;
      o = (o | (o >> 2)) & 0x0f0fu;
      masks[(256 * j + 64 * wave) / kWT + lane] = (uint16_t)(e | (o << 4));
    }
  }
  // (LDS only: the wave's Q loads stay in flight across the barrier, under the first gathers)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (FP8) smax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  // Rows that are not selected are gathered from a selected row of the split (finite data,
  // whose P is zero: exactly nothing is added).  A split without any selected row skips
  // the loop, leaving O = 0 and l = 0.
  const int fill = __builtin_amdgcn_readfirstlane(max(max(anyv[0], anyv[1]), max(anyv[2], anyv[3])));
  const int lastrow =
      __builtin_amdgcn_readfirstlane(max(max(lastv[0], lastv[1]), max(lastv[2], lastv[3])));
  const int nst = fill >= 0 ? min(nstage, lastrow / kSR + 1) : 0;
  const float inv_smax = smax > 0.f ? 1.f / smax : 0.f;

  // ---- gathers: wave w loads rows 8w .. 8w + 7 of each stage, i.e. rows 8(w & 1) .. of tile
  // w >> 1.  bf16: one load per row for its 1 KB value part (lane l: bytes 16l ..; the row
  // base is a scalar), one load for the eight rows' RoPE parts (lane l: row l >> 3, chunk
  // l & 7).  e4m3: one load per two rows' 512-byte value parts (lane l: row 2k + (l >> 5),
  // bytes 16(l & 31)), one load for the eight rows' RoPE parts (lane l: row (l >> 2) & 7, chunk
  // l & 3; lanes 32.. repeat lanes 0..31: same bytes to the same place).
  constexpr int kNL = FP8 ? 5 : 9;  // loads per wave and stage
  struct Gath {
    int s[kNL];  // slot read by load k (per lane)
  };
  auto gath_rows = [&](int st) {
    Gath g;
    const int* rr = rows + st * kSR + 8 * wave;
    if constexpr (FP8) {
#pragma unroll
      for (int k = 0; k < 4; ++k) g.s[k] = rr[2 * k + (lane >> 5)];
      g.s[4] = rr[(lane >> 2) & 7];
    } else {
      const int mine = rr[lane & 7];
#pragma unroll
      for (int k = 0; k < 8; ++k) g.s[k] = __builtin_amdgcn_readlane(mine, k);
      g.s[8] = rr[lane >> 3];
    }
#pragma unroll
    for (int k = 0; k < kNL; ++k) g.s[k] = g.s[k] >= 0 ? g.s[k] : fill;
    return g;
  };
  auto gload = [&](const Gath& g, int k) -> i32x4 {
    if (FP8) {
      const uint64_t rb = (uint64_t)(uintptr_t)kv + (uint64_t)(uint32_t)g.s[k] * F::kRowBytes;
      return *GLOBAL_PTR(const i32x4, rb + (k < 4 ? 16u * (uint32_t)(lane & 31)
                                                  : F::kVBytes + 16u * (uint32_t)(lane & 3)));
    }
    if (k < 8) {  // the row base in scalar registers: the scalar-base form of the load
      const uint64_t rb = (uint64_t)(uintptr_t)kv + (uint64_t)(uint32_t)g.s[k] * F::kRowBytes;
      const uint32_t blo = __builtin_amdgcn_readfirstlane((uint32_t)rb);
      const uint32_t bhi = __builtin_amdgcn_readfirstlane((uint32_t)(rb >> 32));
      return *GLOBAL_PTR(const i32x4, (((uint64_t)bhi << 32) | blo) + 16u * (uint32_t)lane);
    }
    const uint64_t rb = (uint64_t)(uintptr_t)kv + (uint64_t)(uint32_t)g.s[k] * F::kRowBytes;
    return *GLOBAL_PTR(const i32x4, rb + F::kVBytes + 16u * (uint32_t)(lane & 7));
  };
  // LDS byte offset of load k's 16 bytes within a ring slot (the wave's tile and rows)
  const int wtile = (wave >> 1) * F::kWBytes;
  const int rw0 = 8 * (wave & 1);
  auto gofs = [&](int k) -> int {
    if (FP8) {  // (value loads: the 32 bytes their 16 codes widen to)
      if (k < 4) return wtile + (rw0 + 2 * k + (lane >> 5)) * F::kAStride + 32 * (lane & 31);
      return wtile + F::kABytes + (rw0 + ((lane >> 2) & 7)) * F::kRStride + 16 * (lane & 3);
    }
    if (k < 8) return wtile + (rw0 + k) * F::kAStride + 16 * lane;
    return wtile + F::kABytes + (rw0 + (lane >> 3)) * F::kRStride + 16 * (lane & 7);
  };
  constexpr int kSlot = 2 * F::kWBytes;
  // load k's data into its place in the ring slot at offset so (e4m3 value loads: the 16
  // codes widened exactly to fp16, two 16-byte writes)
  auto put = [&](int so, int k, const i32x4& v) {
    char* dst = ring + so + gofs(k);
    if constexpr (FP8) {
      if (k < 4) {
        i32x4 h[2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v[i], 1.f, false);
          const f16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v[i], 1.f, true);
          h[i >> 1][2 * (i & 1)] = __builtin_bit_cast(int, lo);
          h[i >> 1][2 * (i & 1) + 1] = __builtin_bit_cast(int, hi);
        }
        *(i32x4*)dst = h[0];
        *(i32x4*)(dst + 16) = h[1];
        return;
      }
    }
    *(i32x4*)dst = v;
  };

  // ---- register state
  f32x16 o[kDvW / 32];  // O^T: dims 256dv + 32mt + 8(i/4) + 4h2 + i%4, head h0 + c32
#pragma unroll
  for (int mt = 0; mt < kDvW / 32; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[mt][i] = 0.f;
  // per lane two heads, 16ht + c16; le sums P unrounded (for lse, and to normalise O with a
  // bf16 cache), l sums the fp16 P of an e4m3 cache as rounded for the matrix cores
  float m_run[2] = {kMFloor, kMFloor}, l_run[2] = {0.f, 0.f}, le_run[2] = {0.f, 0.f};
  const bool hsel = (lane & 16) != 0;  // the O^T column c32 is head 16*hsel + c16
  i32x4 qq[kNL];                       // the gathered rows of the next stage to write
  f32x4 sp[2][2];                      // partial logits of the stage being multiplied
  f32x4 prev[2][2];                    // partial logits of the stage in softmax
  const int qrow = tile_row(c16);
  using KRaw = typename std::conditional<FP8, i32x4, bf16x8>::type;

  // K fragment f = 2ks + kt of the stage at ring offset so: lane (m = c16, g4): row pi(m),
  // dims 8g4 .. + 7 of the wave's fragment ks (value dims: 16 bytes of 16-bit values; e4m3
  // RoPE dims: 8 codes, in the low half)
  auto kread = [&](int so, int f) -> KRaw {
    const int ks = f >> 1, kt = f & 1;
    const char* tb = ring + so + kt * F::kWBytes;
    if (ks < kNQ2 - 1) return *(const KRaw*)(tb + qrow * F::kAStride + 2 * (256 * dv + 32 * ks + 8 * g4));
    const char* pb = tb + F::kABytes + qrow * F::kRStride;
    if constexpr (FP8) {
      const i32x2 c = *(const i32x2*)(pb + 32 * dv + 8 * g4);
      return i32x4{c[0], c[1], 0, 0};
    } else {
      return *(const KRaw*)(pb + 2 * (32 * dv + 8 * g4));
    }
  };
  auto widen = [&](KRaw cur, int ks) -> QOp {
    if constexpr (FP8) {
      if (ks < kNQ2 - 1) return __builtin_bit_cast(f16x8, cur);
      const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cur[0], 1.f, false);
      const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cur[0], 1.f, true);
      const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cur[1], 1.f, false);
      const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cur[1], 1.f, true);
      return __builtin_shufflevector(__builtin_shufflevector(p0, p1, 0, 1, 2, 3),
                                     __builtin_shufflevector(p2, p3, 0, 1, 2, 3), 0, 1, 2, 3, 4,
                                     5, 6, 7);
    } else {
      return cur;
    }
  };
  auto qkmma = [&](QOp a, QOp b, f32x4 c) -> f32x4 {
    if constexpr (FP8) return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    else return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  };
  // partial QK^T of the stage at ring offset so into sp
  auto qk = [&](int so) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) sp[kt][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int kPre = 3;  // fragments read ahead of their use
    constexpr int kNF = 2 * kNQ2;
    KRaw kr[kPre];
#pragma unroll
    for (int f = 0; f < kPre; ++f) kr[f] = kread(so, f);
#pragma unroll
    for (int f = 0; f < kNF; ++f) {
      const KRaw cur = kr[f % kPre];
      if (f + kPre < kNF) kr[f % kPre] = kread(so, f + kPre);
      const QOp a = widen(cur, f >> 1);
      const int ks = f >> 1, kt = f & 1;
#pragma unroll
      for (int ht = 0; ht < 2; ++ht)
        sp[kt][ht] = qkmma(a, qf[ht][ks], sp[kt][ht]);
    }
  };

  // ---- softmax of stage st: logits s = own partial (prev) + the partner's (LDS buffer xo);
  // t = z - m_run with z = s * zsc (zsc = softmax scale * log2 e, times the row scale for e4m3),
  // p = 2^t.  Masked keys get t = -inf, hence p = 0; m_run starts at a finite floor so this
  // holds before the first live key too.  Returns whether the running max must be raised
  // (some t of the stage above kRaiseAt: a lane-local test, uniform through __any).  P = 2^t is
  // then at most 2^15 as fp16 (largest finite value 65504) or 2^30 as bf16, summed in fp32; the
  // formats' relative precision does not depend on the magnitude.  A threshold of 8 raised the
  // max in 26 of 63 stages of prefill rows whose logits grow along the positions.
  constexpr float kRaiseAt = FP8 ? 15.f : 30.f;
  float pv[2][2][4];
  uint32_t mk[2];
  f32x4 zsc[2];
  // logits of stage st: own partial (prev) + the partner's (LDS buffer xo)
  auto logits = [&](int xo, f32x4 (&sf)[2][2]) {
    const char* xb = xs + xo + partner * 4096 + 16 * lane;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ht = 0; ht < 2; ++ht)
        sf[kt][ht] = prev[kt][ht] + *(const f32x4*)(xb + (2 * kt + ht) * 1024);
  };
  auto soft1 = [&](int st, int xo) {
    f32x4 sf[2][2];
    logits(xo, sf);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      mk[kt] = ((uint32_t)masks[st * 2 + kt] >> (4 * g4)) & 0xFu;
      zsc[kt] = f32x4{c2, c2, c2, c2};
      if (FP8) zsc[kt] = *(const f32x4*)(scl + st * kSR + kt * kWT + 4 * g4) * c2;
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ht = 0; ht < 2; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = fmaf(sf[kt][ht][i], zsc[kt][i], -m_run[ht]);
          const float tzv = ((mk[kt] >> i) & 1u) ? v : -INFINITY;
          tmax = fmaxf(tmax, tzv);
          pv[kt][ht][i] = __builtin_amdgcn_exp2f(tzv);
        }
    return tmax > kRaiseAt;
  };
  // raise the running max of each head to the stage's, rescale l, le and O, recompute p
  auto raise = [&](int xo) {
    f32x4 s_full[2][2];
    logits(xo, s_full);
    float alpha[2];
    const float m_old[2] = {m_run[0], m_run[1]};
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      float zm = -INFINITY;  // (from z itself: t loses z next to the floor)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if ((mk[kt] >> i) & 1u) zm = fmaxf(zm, s_full[kt][ht][i] * zsc[kt][i]);
      const float m_new = fmaxf(m_run[ht], rows4_max(zm));
      alpha[ht] = __builtin_amdgcn_exp2f(m_run[ht] - m_new);
      l_run[ht] *= alpha[ht];
      le_run[ht] *= alpha[ht];
      m_run[ht] = m_new;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          pv[kt][ht][i] = ((mk[kt] >> i) & 1u)
                              ? __builtin_amdgcn_exp2f(fmaf(s_full[kt][ht][i], zsc[kt][i], -m_new))
                              : 0.f;
    }
    // O is rescaled only once some head has seen a live key before: on the first live stage
    // (every running max still at the floor) O is zero and the factor is 0
    if (__any(m_old[0] > kMFloor || m_old[1] > kMFloor)) {
      const float a_sel = hsel ? alpha[1] : alpha[0];
#pragma unroll
      for (int mi = 0; mi < kDvW / 32; ++mi) acc_scale(o[mi], a_sel);
    }
  };
  // normaliser terms of the stage (added to le / l by commit) and P^T in the 32x32x16 B
  // layout per tile: lane l gets keys 8h2 + j of head c32
  i32x4 pb[2];
  float le_add[2], l_add[2];
  // P^T of tile kt (and, e4m3, its normaliser terms as rounded for the matrix cores)
  auto pack_tile = [&](int kt) {
    uint32_t pk[2][2];  // [ht][pair]: packed 16-bit P of keys 4g4 + 2*pair + {0,1}
    if (FP8) {
      const f32x4 sc = zsc[kt] * (1.f / c2);
      f32x4 rs, sn;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sn[i] = sc[i] * inv_smax;
        // (the normaliser's weight smax/scale through the hardware reciprocal: within 1 ulp,
        // far below the fp16 rounding of P it multiplies)
        rs[i] = sc[i] > 0.f ? smax * __builtin_amdgcn_rcpf(sc[i]) : 0.f;
      }
#pragma unroll
      for (int ht = 0; ht < 2; ++ht)
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          const _Float16 v0 = (_Float16)(pv[kt][ht][2 * pr] * sn[2 * pr]);
          const _Float16 v1 = (_Float16)(pv[kt][ht][2 * pr + 1] * sn[2 * pr + 1]);
          l_add[ht] = fmaf((float)v0, rs[2 * pr], l_add[ht]);
          l_add[ht] = fmaf((float)v1, rs[2 * pr + 1], l_add[ht]);
          pk[ht][pr] = (uint32_t)__builtin_bit_cast(uint16_t, v0) |
                       ((uint32_t)__builtin_bit_cast(uint16_t, v1) << 16);
        }
    } else {
      // one packed round-to-nearest-even conversion per pair; O is normalised by the sum of
      // the unrounded P (le), the rounding of each P being far below the output precision
#pragma unroll
      for (int ht = 0; ht < 2; ++ht)
#pragma unroll
        for (int pr = 0; pr < 2; ++pr)
          pk[ht][pr] = __builtin_bit_cast(
              uint32_t,
              __builtin_convertvector(f32x2{pv[kt][ht][2 * pr], pv[kt][ht][2 * pr + 1]}, bf16x2));
    }
    // lanes of the low 16-row of each half keep tile 0 and take tile 0 of the row above;
    // lanes of the high 16-row take tile 1 of the row below and keep their tile 1
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      auto r = __builtin_amdgcn_permlane16_swap(pk[0][pr], pk[1][pr], false, false);
      pb[kt][pr] = (int)r[0];      // keys 8h2 + 2pr + {0,1}
      pb[kt][2 + pr] = (int)r[1];  // keys 8h2 + 4 + 2pr + {0,1}
    }
  };
  auto soft2 = [&]() {
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      le_add[ht] = l_add[ht] = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) le_add[ht] += pv[kt][ht][i];
    }
    pack_tile(0);
    pack_tile(1);
  };
  auto commit = [&]() {
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      le_run[ht] += le_add[ht];
      l_run[ht] += l_add[ht];
    }
  };
  // ---- region 1 of an iteration: the partial QK^T of the stage at ring offset so (36 matrix
  // ops, two per fragment step) with the softmax of stage sst cut into slices between them,
  // so that the vector work runs while the matrix cores are busy.  The order is pinned with
  // scheduling fences (left alone, the scheduler issues the matrix ops back to back and the
  // softmax after them).  Returns whether the running max must be raised.
  auto qk_soft = [&](int so, int sst, int xo) -> bool {
    // the partner's logits, masks and row scales of stage sst go out first
    const char* xb = xs + xo + partner * 4096 + 16 * lane;
    f32x4 px[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) px[kt][ht] = *(const f32x4*)(xb + (2 * kt + ht) * 1024);
    const uint32_t mraw = *(const uint32_t*)(masks + sst * 2);  // both tiles' masks
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      zsc[kt] = f32x4{c2, c2, c2, c2};
      if (FP8) zsc[kt] = *(const f32x4*)(scl + sst * kSR + kt * kWT + 4 * g4) * c2;
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) sp[kt][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int kNF = 2 * kNQ2;
    KRaw kr[kKPre];
#pragma unroll
    for (int f = 0; f < kKPre; ++f) kr[f] = kread(so, f);
    float tmax = -INFINITY;
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) le_add[ht] = l_add[ht] = 0.f;
    // softmax slice after fragment step j: for j = 2 .. 17 the logit, exponential and sum of
    // value v = j - 2 (tile v >> 3, head tile (v >> 2) & 1, key i = v & 3); at j = 10 the P^T
    // operand of tile 0 (tile 1's follows the last step)
    auto slice = [&](int j) {
      if (j >= 2) {
        const int v = j - 2, kt = v >> 3, ht = (v >> 2) & 1, i = v & 3;
        if ((v & 7) == 0) mk[kt] = (mraw >> (16 * kt + 4 * g4)) & 0xFu;
        const float sf = prev[kt][ht][i] + px[kt][ht][i];
        const float z = fmaf(sf, zsc[kt][i], -m_run[ht]);
        const float tzv = ((mk[kt] >> i) & 1u) ? z : -INFINITY;
        tmax = fmaxf(tmax, tzv);
        pv[kt][ht][i] = __builtin_amdgcn_exp2f(tzv);
        le_add[ht] += pv[kt][ht][i];
      }
      if (j == 10) pack_tile(0);
    };
#pragma unroll
    for (int f = 0; f < kNF; ++f) {
      const KRaw cur = kr[f % kKPre];
      if (f + kKPre < kNF) kr[f % kKPre] = kread(so, f + kKPre);
      const QOp a = widen(cur, f >> 1);
      const int ks = f >> 1, kt = f & 1;
#pragma unroll
      for (int ht = 0; ht < 2; ++ht)
        sp[kt][ht] = qkmma(a, qf[ht][ks], sp[kt][ht]);
      __builtin_amdgcn_sched_barrier(0);
      slice(f);
      __builtin_amdgcn_sched_barrier(0);
    }
    pack_tile(1);
    return tmax > kRaiseAt;
  };

  // ---- O^T[32 dims][32 heads] += V^T[32 dims][16 keys] . P^T over the wave's 8 dim tiles of
  // the stage at ring offset so; `side(mi)` runs after the products of dim tile mi are issued
  using VOp = typename std::conditional<FP8, f16x8, bf16x8>::type;
  auto vread = [&](int so, int mi, int kt) -> VOp {
    const int G = g4;
    const int d0 = 256 * dv + 32 * mi + 16 * (G & 1);
    const char* sb = ring + so + kt * F::kWBytes;
    // lane k of the 16-row group: keys j = k / 4 (row pi(8h + j) = 8h + 2j) and j + 4 (the
    // next row), dims d0 + 4 (k % 4).  Whole-vector moves only: element-wise assembly of this
    // operand from the two 64-bit halves was mistranslated by the compiler.
    const int kr = 8 * (G >> 1) + 2 * (c16 >> 2);
    const char* base = sb + kr * F::kAStride + 2 * (d0 + 4 * (c16 & 3));
    if constexpr (FP8) {  // (16-bit values in LDS for both caches; fp16 for an e4m3 one)
      typedef __fp16 h4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
      const f16x4 lo = __builtin_bit_cast(
          f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16(LDS_PTR(h4, base)));
      const f16x4 hi = __builtin_bit_cast(
          f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16(LDS_PTR(h4, base + F::kAStride)));
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    } else {
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, base));
      const bf16x4 hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, base + F::kAStride));
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };
  auto vmma = [&](int mi, VOp a, int kt) {
    if constexpr (FP8)
      o[mi] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, __builtin_bit_cast(f16x8, pb[kt]), o[mi],
                                                     0, 0, 0);
    else
      o[mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, pb[kt]),
                                                      o[mi], 0, 0, 0);
  };
  // ---- O^T[32 dims][32 heads] += V^T[32 dims][16 keys] . P^T over the wave's 8 dim tiles of
  // the stage at ring offset so, V^T read one dim tile ahead; side_a(mi) / side_b(mi) run
  // between the two products of dim tile mi (the order pinned as in region 1)
  auto pv_mul = [&](int so, auto&& side_a, auto&& side_b) {
    constexpr int kNM = kDvW / 32;
    VOp vq[kVPre][2];  // V^T of dim tiles mi .. mi + kVPre - 1 in flight
#pragma unroll
    for (int m = 0; m < kVPre; ++m) {
      vq[m][0] = vread(so, m, 0);
      vq[m][1] = vread(so, m, 1);
    }
#pragma unroll
    for (int mi = 0; mi < kNM; ++mi) {
      const VOp c0 = vq[mi % kVPre][0], c1 = vq[mi % kVPre][1];
      if (mi + kVPre < kNM) {
        vq[mi % kVPre][0] = vread(so, mi + kVPre, 0);
        vq[mi % kVPre][1] = vread(so, mi + kVPre, 1);
      }
      vmma(mi, c0, 0);
      __builtin_amdgcn_sched_barrier(0);
      side_a(mi);
      __builtin_amdgcn_sched_barrier(0);
      vmma(mi, c1, 1);
      __builtin_amdgcn_sched_barrier(0);
      side_b(mi);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto write_xs = [&](int xo) {
    char* xb = xs + xo + wave * 4096 + 16 * lane;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) *(f32x4*)(xb + (2 * kt + ht) * 1024) = sp[kt][ht];
  };
  auto copy_prev = [&]() {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) prev[kt][ht] = sp[kt][ht];
  };
  // One iteration for stage st >= 1.  Ring slots rotate as (so_pv, so_qk, so_wr) = slots of
  // stages st - 1, st, st + 1; the logits buffers alternate with the parity of the stage.
  int so_pv = 0, so_qk = kSlot, so_wr = 2 * kSlot;
  auto iteration = [&](int st) {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const Gath g2 = gath_rows(min(st + 2, nst - 1));
    const int xo_prev = ((st - 1) & 1) * 4 * 4096, xo_cur = (st & 1) * 4 * 4096;
    // region 1: softmax of stage st - 1 (speculating that the running max holds) interleaved
    // with the partial QK^T of stage st
    const bool up = qk_soft(so_qk, st - 1, xo_prev);
    if (__any(up)) {  // (rare: the running max is raised and the stage's softmax redone)
      raise(xo_prev);
      soft2();
    }
    // region 2: PV of stage st - 1, with the rows of stage st + 1 written from the queue, the
    // gathers of stage st + 2 issued into it, and this stage's partial logits to LDS
    commit();
    write_xs(xo_cur);
    copy_prev();
    pv_mul(
        so_pv,
        [&](int mi) {  // the queued rows of stage st + 1 into their ring slot
          if (mi < kNL) put(so_wr, mi < kNL ? mi : 0, qq[mi < kNL ? mi : 0]);
          if (mi == kDvW / 32 - 1 && kNL > kDvW / 32)  // (bf16: the ninth load)
            put(so_wr, kNL - 1, qq[kNL - 1]);
        },
        [&](int mi) {  // the gathers of stage st + 2 into the queue
          if (mi < kNL) qq[mi < kNL ? mi : 0] = gload(g2, mi < kNL ? mi : 0);
          if (mi == kDvW / 32 - 1 && kNL > kDvW / 32) qq[kNL - 1] = gload(g2, kNL - 1);
        });
    const int t0 = so_pv;
    so_pv = so_qk;
    so_qk = so_wr;
    so_wr = t0;
  };

  if (nst > 0) {
    // prologue: stage 0 straight into slot 0, stage 1 into the queue; after the barrier,
    // stage 1 into slot 1, stage 2 into the queue, and QK^T of stage 0
    {
      // (both stages' gathers go out before the first is waited for)
      const Gath g0 = gath_rows(0);
      const Gath g1 = gath_rows(min(1, nst - 1));
      i32x4 q0[kNL];
#pragma unroll
      for (int k = 0; k < kNL; ++k) q0[k] = gload(g0, k);
#pragma unroll
      for (int k = 0; k < kNL; ++k) qq[k] = gload(g1, k);
#pragma unroll
      for (int k = 0; k < kNL; ++k) put(0, k, q0[k]);
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    {
#pragma unroll
      for (int k = 0; k < kNL; ++k) put(kSlot, k, qq[k]);
      const Gath g2 = gath_rows(min(2, nst - 1));
#pragma unroll
      for (int k = 0; k < kNL; ++k) qq[k] = gload(g2, k);
#pragma unroll
      for (int ht = 0; ht < 2; ++ht)
#pragma unroll
        for (int ks = 0; ks < kNQ2; ++ks) {
          if constexpr (FP8) {
#pragma unroll
            for (int i = 0; i < 8; ++i) qf[ht][ks][i] = (_Float16)(float)qb[ht][ks][i];
          } else {
            qf[ht][ks] = qb[ht][ks];
          }
        }
      qk(0);
      write_xs(0);
      copy_prev();
    }
    // slots: stage 0 in slot 0 (PV next), stage 1 in slot 1 (QK next), stage 2 goes to slot 2
    for (int st = 1; st < nst; ++st) iteration(st);
    // softmax and PV of the last stage
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const int xo_last = ((nst - 1) & 1) * 4 * 4096;
    const bool up = soft1(nst - 1, xo_last);
    if (__any(up)) raise(xo_last);
    soft2();
    commit();
    pv_mul(so_pv, [](int) {}, [](int) {});
  }

  // ---- per head: normaliser and lse over the four 16-lane rows; lane l holds head c32's
  // (the two waves of a head half computed the same values)
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    le_run[ht] = rows4_sum(le_run[ht]);
    l_run[ht] = FP8 ? rows4_sum(l_run[ht]) : le_run[ht];
  }
  const float M = hsel ? m_run[1] : m_run[0];
  const float Ls = hsel ? l_run[1] : l_run[0];
  const float LEs = hsel ? le_run[1] : le_run[0];
  const int head = h0 + c32;
  const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
  // O was accumulated relative to the largest row scale (e4m3)
  const float fo = FP8 ? smax : 1.f;
  if (dv == 0 && h2 == 0) {
    if (nsplit == 1) {
      if (lse) lse[(int64_t)t * kH + head] = LEs > 0.f ? (M + log2f(LEs)) * kLn2 : -INFINITY;
    } else {
      const int64_t pr = ((int64_t)tl * nsplit + split) * kH + head;
      *(f32x4*)(part_ml + pr * 4) = f32x4{M, Ls, LEs, 0.f};
    }
  }
  // ---- the wave's O (its 32 heads x 256 dims) through LDS into whole lines: each lane stores
  // its four dims of head c32 (scaled) into a per-wave [32 heads][256 dims] fp32 staging area
  // over the ring, then each store instruction writes 16 bytes per lane of two heads' rows
  __syncthreads();  // (every wave is done with the ring)
  float* xw = (float*)(sm + wave * (kHB * kOStage * 4));
  const float f = (nsplit > 1 && OUT_F32) ? fo : fo * inv;  // fp32 partials stay unnormalised
#pragma unroll
  for (int mi = 0; mi < kDvW / 32; ++mi)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const f32x4 v = {acc_read_scaled(o[mi][4 * q4], f), acc_read_scaled(o[mi][4 * q4 + 1], f),
                       acc_read_scaled(o[mi][4 * q4 + 2], f),
                       acc_read_scaled(o[mi][4 * q4 + 3], f)};
      *(f32x4*)(xw + c32 * kOStage + 32 * mi + 8 * q4 + 4 * h2) = v;
    }
  // (the wave reads back only what it wrote: LDS operations of a wave complete in order)
  const int64_t obase = ((int64_t)t * kH + h0) * kDv + 256 * dv;
  const int64_t pbase = (((int64_t)tl * nsplit + split) * kH + h0) * kDv + 256 * dv;
  if (OUT_F32) {
    // 64 lanes x 16 bytes = one head's 256 dims per store
#pragma unroll 4
    for (int hr = 0; hr < kHB; ++hr) {
      const f32x4 v = *(const f32x4*)(xw + hr * kOStage + 4 * lane);
      if (nsplit == 1) *(f32x4*)((float*)out + obase + (int64_t)hr * kDv + 4 * lane) = v;
      else *(f32x4*)(part_o + pbase + (int64_t)hr * kDv + 4 * lane) = v;
    }
  } else {
    // 32 lanes x 8 dims (16 bytes of bf16 / fp16) per head, two heads per store
#pragma unroll 4
    for (int hr = 0; hr < kHB; hr += 2) {
      const int hx = hr + (lane >> 5);
      const float* src = xw + hx * kOStage + 8 * (lane & 31);
      const f32x4 lo = *(const f32x4*)src, hi = *(const f32x4*)(src + 4);
      const int64_t off = (int64_t)hx * kDv + 8 * (lane & 31);
      if (nsplit == 1) store_out8<false>(out, obase + off, lo, hi);
      else store_part16x8(part_o, pbase + off, lo, hi);
    }
  }
}

#define MLA_ATTN_ARGS                                                                       \
  DevBatch bt, int t_begin, int t_count, const uint16_t* __restrict__ q,                      \
      const uint8_t* __restrict__ kv, const float* __restrict__ kvscale,                      \
      const int32_t* __restrict__ idx, int K, float c2, int nsplit, int kps,                  \
      void* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,            \
      float* __restrict__ part_ml
#define MLA_ATTN_PASS \
  bt, t_begin, t_count, q, kv, kvscale, idx, K, c2, nsplit, kps, out, lse, part_o, part_ml

__global__ __launch_bounds__(256, 1) void mla_attn_bf16_kernel(MLA_ATTN_ARGS) {
  mla_attn_body<false, false>(MLA_ATTN_PASS);
}
__global__ __launch_bounds__(256, 1) void mla_attn_bf16_o32_kernel(MLA_ATTN_ARGS) {
  mla_attn_body<false, true>(MLA_ATTN_PASS);
}
__global__ __launch_bounds__(256, 1) void mla_attn_fp8_kernel(MLA_ATTN_ARGS) {
  mla_attn_body<true, false>(MLA_ATTN_PASS);
}
__global__ __launch_bounds__(256, 1) void mla_attn_fp8_o32_kernel(MLA_ATTN_ARGS) {
  mla_attn_body<true, true>(MLA_ATTN_PASS);
}
// the dense-masked form (kps: the causal positions per split; K: the selection's width)
__global__ __launch_bounds__(256, 1) void mla_attn_bf16_dense_kernel(MLA_ATTN_ARGS) {
  mla_attn_body<false, false, true>(MLA_ATTN_PASS);
}
__global__ __launch_bounds__(256, 1) void mla_attn_bf16_o32_dense_kernel(MLA_ATTN_ARGS) {
  mla_attn_body<false, true, true>(MLA_ATTN_PASS);
}
__global__ __launch_bounds__(256, 1) void mla_attn_fp8_dense_kernel(MLA_ATTN_ARGS) {
  mla_attn_body<true, false, true>(MLA_ATTN_PASS);
}
__global__ __launch_bounds__(256, 1) void mla_attn_fp8_o32_dense_kernel(MLA_ATTN_ARGS) {
  mla_attn_body<true, true, true>(MLA_ATTN_PASS);
}

// Merge split partials (m in log2 units; l = the normaliser of O, le = unrounded sum of P):
// O = sum_j 2^(m_j - M) O_j / sum_j 2^(m_j - M) l_j,  lse = M + log2 sum_j 2^(m_j - M) le_j.
// fp32 output: O_j is the split's unnormalised fp32 sum.  bf16 output: O_j is stored
// normalised (O_j / l_j) as fp16 (see store_part16), and is weighted by l_j here.
// One split's partial O for 8 consecutive dims (fp32 unnormalised, or fp16 normalised).
template <bool OUT_F32>
__device__ __forceinline__ void load_part8(const float* part_o, int64_t off, f32x4& lo,
                                           f32x4& hi) {
  if (OUT_F32) {
    lo = *(const f32x4*)(part_o + off);
    hi = *(const f32x4*)(part_o + off + 4);
  } else {
    const f16x8 h = *(const f16x8*)((const uint16_t*)part_o + off);
    lo = f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]} * kPartUnscale;
    hi = f32x4{(float)h[4], (float)h[5], (float)h[6], (float)h[7]} * kPartUnscale;
  }
}

// Up to N splits: unconditional loads (the split index clamped; the extra copies get weight
// 0), so that they all go out before the first use.
template <bool OUT_F32, int N>
__device__ __forceinline__ void combine_splits(int nsplit, int64_t pr0, int d0,
                                               const float* __restrict__ part_o,
                                               const float* __restrict__ part_ml, float& M,
                                               float& Lsum, float& LEsum, f32x4& alo,
                                               f32x4& ahi) {
  f32x4 ml[N], vlo[N], vhi[N];
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const int64_t pr = pr0 + min(j, nsplit - 1) * kH;
    ml[j] = *(const f32x4*)(part_ml + pr * 4);
    load_part8<OUT_F32>(part_o, pr * kDv + d0, vlo[j], vhi[j]);
  }
#pragma unroll
  for (int j = 0; j < N; ++j)
    if (j < nsplit && ml[j][1] > 0.f) M = fmaxf(M, ml[j][0]);
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const bool use = j < nsplit && ml[j][1] > 0.f;
    const float wgt = use ? exp2f(ml[j][0] - M) : 0.f;
    Lsum = fmaf(wgt, ml[j][1], Lsum);
    LEsum = fmaf(wgt, ml[j][2], LEsum);
    const float f = OUT_F32 ? wgt : wgt * ml[j][1];
    alo += f * vlo[j];
    ahi += f * vhi[j];
  }
}

// One wave per (token, head), lane l owning dims 8l .. 8l+7 (16-byte partial loads and
// output stores); four heads per workgroup.
template <bool OUT_F32>
__global__ __launch_bounds__(256) void mla_combine_kernel(int t_begin, int t_count, int nsplit,
    const float* __restrict__ part_o, const float* __restrict__ part_ml,
    void* __restrict__ out, float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);  // (token, head)
  const int tl = pair / kH, head = pair % kH;
  if (tl >= t_count) return;
  const int t = t_begin + tl;
  const int d0 = 8 * lane;
  const int64_t pr0 = (int64_t)tl * nsplit * kH + head;  // split j: pr0 + j * kH
  float M = -INFINITY, Lsum = 0.f, LEsum = 0.f;
  f32x4 alo = {0.f, 0.f, 0.f, 0.f}, ahi = {0.f, 0.f, 0.f, 0.f};
  if (nsplit <= 2) {
    combine_splits<OUT_F32, 2>(nsplit, pr0, d0, part_o, part_ml, M, Lsum, LEsum, alo, ahi);
  } else if (nsplit <= 4) {
    combine_splits<OUT_F32, 4>(nsplit, pr0, d0, part_o, part_ml, M, Lsum, LEsum, alo, ahi);
  } else if (nsplit <= 8) {
    combine_splits<OUT_F32, 8>(nsplit, pr0, d0, part_o, part_ml, M, Lsum, LEsum, alo, ahi);
  } else {
    // eight splits at a time (their loads all in flight), each group merged into the running
    // sums with the factors 2^(M - M') and 2^(Mc - M') of the new maximum M'
    for (int j0 = 0; j0 < nsplit; j0 += 8) {
      float Mc = -INFINITY, Lc = 0.f, LEc = 0.f;
      f32x4 clo = {0.f, 0.f, 0.f, 0.f}, chi = {0.f, 0.f, 0.f, 0.f};
      combine_splits<OUT_F32, 8>(min(8, nsplit - j0), pr0 + (int64_t)j0 * kH, d0, part_o,
                                 part_ml, Mc, Lc, LEc, clo, chi);
      const float Mn = fmaxf(M, Mc);
      const float fa = M > -INFINITY ? exp2f(M - Mn) : 0.f;
      const float fc = Mc > -INFINITY ? exp2f(Mc - Mn) : 0.f;
      Lsum = Lsum * fa + Lc * fc;
      LEsum = LEsum * fa + LEc * fc;
      alo = alo * fa + clo * fc;
      ahi = ahi * fa + chi * fc;
      M = Mn;
    }
  }
  const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
  const int64_t orow = ((int64_t)t * kH + head) * kDv + d0;
  store_out8<OUT_F32>(out, orow, alo * inv, ahi * inv);
  if (lse && lane == 0)
    lse[(int64_t)t * kH + head] = LEsum > 0.f ? (M + log2f(LEsum)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------- launchers
hipError_t launch_mla_attn_f32(const DevBatch& bt, int t_begin, int t_count, const float* q,
                               const float* kv, const int32_t* idx, int K, int H, int Dqk,
                               int Dv, float scale, float* out, float* lse, hipStream_t st) {
  size_t shm = (size_t)(Dqk + 2 * K) * sizeof(float);
  hipLaunchKernelGGL(mla_attn_f32_kernel, dim3(t_count, H), dim3(256), shm, st, bt, t_begin, q,
                     kv, idx, K, H, Dqk, Dv, scale, out, lse);
  return hipGetLastError();
}

int attn_keys_per_split(int K, int nsplit) {
  int kps = (K + nsplit - 1) / nsplit;
  return (kps + kSR - 1) / kSR * kSR;
}

int attn_split_count(int t_count, int K) {
  // enough workgroups (2 head groups per token and split) to cover the 256 CUs, at least four
  // stages of keys per split (a workgroup's prologue and epilogue cost about as much as four
  // stages: shorter splits only add partials), at most kMaxKps; recomputed from the rounded
  // split length so that no split is empty
  int s = (256 + 2 * t_count - 1) / (2 * t_count);
  s = std::max(1, std::min(s, (K + 4 * kSR - 1) / (4 * kSR)));
  s = std::max(s, (K + kMaxKps - 1) / kMaxKps);
  const int kps = attn_keys_per_split(K, s);
  return (K + kps - 1) / kps;
}

size_t attn_smem_bytes(bool fp8, int kps) {
  (void)kps;
  return fp8 ? (size_t)AttnSmem<true>::total : (size_t)AttnSmem<false>::total;
}

hipError_t launch_mla_attn(const DevBatch& bt, int t_begin, int t_count, bool fp8,
                           const uint16_t* q, const uint8_t* kv, const float* kvscale,
                           const int32_t* idx, int K, float softmax_scale, int nsplit,
                           void* out, bool out_f32, float* lse, float* part_o, float* part_ml,
                           hipStream_t st, int dense_n) {
  // dense_n > 0: the dense-masked form over causal ranges of at most dense_n positions
  const bool dense = dense_n > 0;
  const int kps = attn_keys_per_split(dense ? dense_n : K, nsplit);
  const float c2 = softmax_scale * kLog2e;
  const size_t shm = attn_smem_bytes(fp8, kps);
  auto* fn = dense ? (fp8 ? (out_f32 ? mla_attn_fp8_o32_dense_kernel : mla_attn_fp8_dense_kernel)
                          : (out_f32 ? mla_attn_bf16_o32_dense_kernel
                                     : mla_attn_bf16_dense_kernel))
                   : (fp8 ? (out_f32 ? mla_attn_fp8_o32_kernel : mla_attn_fp8_kernel)
                          : (out_f32 ? mla_attn_bf16_o32_kernel : mla_attn_bf16_kernel));
  // above 64 KB the kernel's dynamic LDS limit has to be raised before the launch (a
  // host-side attribute; set on every such launch so it holds on whichever device is current)
  if (shm > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)shm);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(fn, dim3(t_count * nsplit * 2), dim3(256), shm, st, bt, t_begin, t_count, q, kv,
                     kvscale, idx, K, c2, nsplit, kps, out, lse, part_o, part_ml);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  auto* cfn = out_f32 ? mla_combine_kernel<true> : mla_combine_kernel<false>;
  hipLaunchKernelGGL(cfn, dim3(t_count * kH / 4), dim3(256), 0, st, t_begin, t_count, nsplit,
                     part_o, part_ml, out, lse);
  return hipGetLastError();
}

}  // namespace tis
