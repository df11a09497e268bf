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
// group of 64 heads); wave (hh, kh) owns 32 heads (half hh of the group) and key half kh
// of every 32-key stage:
//   * the split's positions are translated through the page table once into LDS;
//   * 16-row tiles are gathered with 16-byte loads into a one-stage register queue and
//     written into a two-stage LDS ring, interleaved with the QK matrix ops; e4m3 rows stay
//     e4m3 in LDS and are widened per fragment;
//   * S^T = K_tile . Q^T on v_mfma_f32_16x16x32 over 18 fragments of 32 dims, most of Q^T in
//     registers and the rest in LDS (one copy per head half, loaded half by each of its two
//     waves);
//   * O^T[vdim][head] += V^T . P^T on v_mfma_f32_32x32x16: P reaches the B layout with one
//     permlane16 swap, and V^T fragments come from the row-major tile via
//     ds_read_b64_tr_b16 (bf16) / ds_read_b64_tr_b8 (e4m3);
//   * the running max is raised lazily (only when a tile exceeds it by 2^8), so rescaling
//     the 256 accumulator registers is rare;
//   * e4m3: per-token scales go into the logits in fp32 and into P relative to the split's
//     largest scale; P then is fp16 (11-bit significand) so that heavy rows stay accurate,
//     and the normaliser is accumulated from the same rounded P values;
//   * the two key halves are merged through LDS; with several splits per token, each split
//     writes (m, l, O) partials that mla_combine_kernel merges with log-sum-exp weights.
#include "common.h"
#include "launch.h"

#include <algorithm>
#include <type_traits>

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
// Q^T per wave: 18 fragments of 32 dims per 16 heads; the first kQR stay in registers, the
// last kQL are read from LDS one step ahead, which leaves the registers for the queue of
// gathered rows.  The two waves of a head half (the two key halves) need the same Q: each
// loads the fragments of one parity from HBM and takes the others from the copy its partner
// leaves in LDS (one copy per head half, in the lane order of the operand), which halves the
// Q traffic of the prologue.  So that every register index stays static, the key-half-1
// wave contracts the dims of each fragment pair in swapped order: its step ks uses fragment
// ks ^ 1 of both K and Q (the pairs never straddle the value/RoPE boundary).
constexpr int kNQ = kDqk / 32, kQL = 4, kQR = kNQ - kQL;
static_assert(kNQ % 2 == 0 && kQR % 2 == 0 && (kDv / 32) % 2 == 0, "fragment pairs");

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
// key-fragment reads and the transposed value reads nearly free of bank conflicts.  bf16:
// 1056-byte A rows, 18 loads per tile; e4m3: 544-byte A rows, 17 loads (one of them issued
// by both waves).
template <bool FP8>
struct KvFmt {
  static constexpr int kRowBytes = FP8 ? kDqk : 2 * kDqk;   // cached row
  static constexpr int kVBytes = FP8 ? kDv : 2 * kDv;       // value part (region A)
  static constexpr int kRBytes = kRowBytes - kVBytes;       // RoPE part (region B): 64 / 128
  static constexpr int kAStride = kVBytes + 32;             // row stride, region A
  static constexpr int kRStride = kRBytes + 16;             // row stride, region B
  static constexpr int kABytes = kWT * kAStride;
  static constexpr int kBBytes = kWT * kRStride;
  static constexpr int kWBytes = kABytes + kBBytes;         // one wave tile
  static constexpr int kBLoads = kWT * kRBytes / 1024;      // 64 lanes x 16 bytes each
  static constexpr int kIssue = kWT + kBLoads;              // loads per tile
  static constexpr int kIssueW = (kIssue + 1) / 2;          // loads per tile and wave
  static constexpr int kBufs = 2;                           // stages in the ring
  static constexpr int kTiles = kBufs * 2 * kWBytes;        // LDS bytes of the ring
};
__host__ __device__ constexpr int tile_row(int m) {  // pi: consumption order -> tile row
  return (m & 8) + ((m & 4) ? 2 * (m & 3) + 1 : 2 * (m & 3));
}

// Dynamic LDS: ring (or the exchange) | rows[kMaxKps] | masks[kMaxKps/16] | scl[kMaxKps] (e4m3) | xm[4][3][32].
// After the main loop the ring area holds the cross-wave exchange of O (4 x 32 x 132 floats).
constexpr int kXPitch = 132;  // floats per head row of the exchange (128 dims + pad)
template <bool FP8>
struct AttnSmem {
  static constexpr int kXBytes = 4 * kHB * kXPitch * 4;  // the exchange of O
  static constexpr int rows = KvFmt<FP8>::kTiles > kXBytes ? KvFmt<FP8>::kTiles : kXBytes;
  static constexpr int masks = rows + kMaxKps * 4;
  static constexpr int scl = masks + kMaxKps / 16 * 2;
  static constexpr int xm = scl + (FP8 ? kMaxKps * 4 : 0);
  static constexpr int qlds = xm + 4 * 3 * kHB * 4 + 2 * 3 * kHB * 4;
  static constexpr int total = qlds + 2 * 2 * kNQ * 1024;  // Q: [head half][ht][fragment]
  static_assert(total <= 160 * 1024, "LDS budget");
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

// One workgroup per (token, key split, group of 64 heads); wave w takes heads 32(w%2) .. +31
// of the group and the 16-key tiles 2i + w/2 of the split, which it shares with the wave of
// the other head half.  Per wave tile:
//   S^T[16 keys][16 heads] x 2 = K . Q^T on v_mfma_f32_16x16x32_bf16 (K fragments from LDS,
//     Q^T resident in registers; e4m3 rows are widened exactly per fragment);
//   online softmax per head (lane-local over 4 keys, then across the four 16-lane rows);
//   one permlane16 swap moves P^T into the B layout of v_mfma_f32_32x32x16 (keys 8(l/32)+j,
//     head l%32), and O^T[32 dims][32 heads] += V^T . P^T with V^T read by
//     ds_read_b64_tr_b16 (bf16) / ds_read_b64_tr_b8 (e4m3, widened to fp16).
// The running max is raised lazily (only when a tile exceeds it by 2^8).  e4m3: per-row scales
// enter the fp32 logits and P relative to the split's largest scale; P is fp16 and the
// normaliser sums the same rounded values.  The two key halves' (m, l, O) of each head are
// merged through LDS; with several splits the workgroup writes fp32 partials for
// mla_combine_kernel.
template <bool FP8, bool OUT_F32>
__device__ __forceinline__ void mla_attn_body(DevBatch bt, int t_begin, int t_count,
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv,
    const float* __restrict__ kvscale, const int32_t* __restrict__ idx, int K, float c2,
    int nsplit, int kps, void* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_ml) {
  using F = KvFmt<FP8>;
  using SM = AttnSmem<FP8>;
  extern __shared__ __attribute__((aligned(16))) char sm[];
  char* tiles = sm;
  int* rows = (int*)(sm + SM::rows);
  uint16_t* masks = (uint16_t*)(sm + SM::masks);
  float* scl = (float*)(sm + SM::scl);
  float* xm = (float*)(sm + SM::xm);          // [wave][m, l, le][32 heads]
  float* xf = xm + 4 * 3 * kHB;               // [head half][M, L, LE][32 heads]
  __shared__ float red[4];
  __shared__ int anyv[4];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c16 = lane & 15, g4 = lane >> 4;  // 16x16 layouts
  const int c32 = lane & 31, h2 = lane >> 5;  // 32x32 layouts
  const int hh = wave & 1, kh = wave >> 1;    // head half, key half
  // this lane's slot in the head half's copy of Q; fragment f of head tile ht at
  // (ht * kNQ + f) KB.  qxe / qxo address fragment ks ^ kh for even / odd ks.
  char* const qx = sm + SM::qlds + hh * (2 * kNQ * 1024) + 16 * lane;
  char* const qxe = qx + 1024 * kh;
  char* const qxo = qx - 1024 * kh;

  // workgroup -> (token, split, head group); the workgroups of one token sit on one XCD
  // (workgroups are dealt to the 8 XCDs round-robin), so its rows are fetched from HBM once
  // and served to the other head groups from that XCD's L2
  const int nblk = gridDim.x;
  const int xcd = blockIdx.x & 7, slot8 = blockIdx.x >> 3;
  const int per = nblk >> 3, extra = nblk & 7;
  const int pidx = xcd * per + min(xcd, extra) + slot8;
  const int hg = pidx & 1;
  const int split = (pidx >> 1) % nsplit;
  const int tl = (pidx >> 1) / nsplit;
  const int t = t_begin + tl;
  const int h0 = hg * kHW + hh * kHB;  // this wave's first head

  const int kbeg = split * kps;
  const int nk = max(0, min(kps, K - kbeg));
  const int nstage = (nk + kSR - 1) / kSR;
  const int nrows = nstage * kSR;

  // ---- positions -> physical slots (and e4m3 row scales); masked keys read slot 0.  Each
  // thread translates up to kPer rows with its loads batched per step: the positions (they
  // only need the token) go out together with the token's request lookup, then the pages,
  // then the scales, so the chain costs three memory latencies however many rows there are.
  constexpr int kPer = kMaxKps / 256;
  int pos[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = tid + 256 * j;
    pos[j] = i < nk ? idx[(int64_t)t * K + kbeg + i] : -1;
  }
  const LocLoads lw = locate_issue(bt);
  const TokLoc loc = locate_finish(bt, t, lw);
  const int b = loc.b;
  const int Lb = loc.L;
  const int32_t* ptb = bt.page_table + (int64_t)b * bt.pt_stride;
  int slot[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int sp = pos[j];
    slot[j] = (sp >= 0 && sp < Lb) ? ptb[sp >> 6] : -1;
  }
  // This wave's half of the Q^T fragments of its 32 heads (B operand of 16x16x32: head c16,
  // dims 32f + 8g4 of fragment f = 2i + kh), issued after the page lookups: loads complete
  // in issue order, so the slots below wait for the page entries only, and Q arrives while
  // the slots and the first tiles are in flight.  Register slot ks holds fragment ks ^ kh:
  // the even slots are loaded here, the odd ones come from the partner's copy.
  bf16x8 qf[2][kQR], qtl[2][kQL / 2];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const uint16_t* qr = q + ((int64_t)t * kH + h0 + 16 * ht + c16) * kDqk + 8 * g4 + 32 * kh;
#pragma unroll
    for (int i = 0; i < kNQ / 2; ++i) {
      const bf16x8 v = *(const bf16x8*)(qr + 64 * i);
      if (2 * i < kQR) qf[ht][2 * i] = v;
      else qtl[ht][i - kQR / 2] = v;
    }
  }
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
        smax = fmaxf(smax, scv[j]);
      }
    }
  }
  if (FP8) {
    for (int o = 32; o > 0; o >>= 1) smax = fmaxf(smax, __shfl_xor(smax, o));
    if (lane == 0) red[wave] = smax;
  }
  {  // some selected row of the wave's rows (-1 if there is none): one ballot
    int v = -1;
#pragma unroll
    for (int j = 0; j < kPer; ++j) v = max(v, slot[j]);
    const uint64_t b = __ballot(v >= 0);
    if (lane == 0) anyv[wave] = b ? __builtin_amdgcn_readlane(v, __builtin_ctzll(b)) : -1;
  }
  // per 16-row tile: bit m = row pi(m) selected (the order in which the keys are consumed),
  // from one ballot per row step: rows 256j + 64wave + l, four tiles, lane q < 4 writes
  // tile q's mask (row r of a tile is consumed as m = (r & 8) | (r & 1) << 2 | (r >> 1) & 3)
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const uint64_t bj = __ballot(slot[j] >= 0);
    if (lane < 4) {
      const uint32_t nat = (uint32_t)(bj >> (16 * lane)) & 0xffffu;
      uint32_t m = 0u;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        m |= ((nat >> r) & 1u) << ((r & 8) | ((r & 1) << 2) | ((r >> 1) & 3));
      masks[(256 * j + 64 * wave) / kWT + lane] = (uint16_t)m;
    }
  }
  __syncthreads();
  if (FP8) smax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  // Rows that are not selected are gathered from a selected row of the split (finite data,
  // whose P is zero: exactly nothing is added).  A split without any selected row skips
  // the loop, leaving O = 0 and l = 0.
  const int fill = __builtin_amdgcn_readfirstlane(max(max(anyv[0], anyv[1]), max(anyv[2], anyv[3])));
  const int nst = fill >= 0 ? nstage : 0;
  const float inv_smax = smax > 0.f ? 1.f / smax : 0.f;

  // ---- this wave's tile of stage st: rows st*32 + 16*kh .. +15
  // wave-uniform pieces of the gather addresses live in scalar registers: the row base of
  // each A-region load is kv + slot * rowbytes (a scalar), the lane adds 16 * lane, and the
  // LDS destination (M0) is a scalar too
  const int kh_u = __builtin_amdgcn_readfirstlane(kh);
  const int jlo = __builtin_amdgcn_readfirstlane(hh) ? F::kIssue - F::kIssueW : 0;
  const uint32_t lane16 = 16u * (uint32_t)lane;
  // the slots of the wave's tile of stage st: lane r of each 16 holds row r (region A), and
  // bslot[j] the row of region-B chunk l % C of load j (C = RoPE chunks per row)
  constexpr int kRC = F::kRBytes / 16;
  struct TileRows {
    int my;
    int bslot[F::kBLoads];
  };
  auto tile_rows = [&](int st) {
    TileRows tr;
    const int* rw = rows + st * kSR + kh_u * kWT;
    tr.my = rw[lane & (kWT - 1)];
#pragma unroll
    for (int j = 0; j < F::kBLoads; ++j) tr.bslot[j] = rw[(64 * j + lane) / kRC];
    return tr;
  };
  // load j (< kIssue) of the tile of stage st: j < kWT is row j of region A (one load per
  // row), the rest are the region-B loads.  Head half 0 issues loads 0 .. kIssueW - 1, head
  // half 1 the last kIssueW (with 17 loads, load 8 is issued twice: same bytes, same place)
  // load j of a tile, into registers: j < kWT is row j of region A (lane l: bytes 16l ..
  // 16l + 15 of the row), the rest are region-B loads; it goes to LDS one stage later
  auto load_one = [&](const TileRows& tr, int j) -> i32x4 {
    if (j < kWT) {
      const int sj = __builtin_amdgcn_readlane(tr.my, j);
      const uint32_t sr = (uint32_t)(sj >= 0 ? sj : fill);
      // the row base in scalar registers: the scalar-base form of the load
      const uint64_t base = (uint64_t)(uintptr_t)kv + (uint64_t)sr * F::kRowBytes;
      const uint32_t blo = __builtin_amdgcn_readfirstlane((uint32_t)base);
      const uint32_t bhi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
      const uint64_t rowp = ((uint64_t)bhi << 32) | blo;
      // (global, not generic: a generic load would also count against the LDS counter; all
      // lanes load, e4m3 lanes 32..63 a copy of lane - 32's chunk, so that no lane-predicated
      // write of the queue registers makes the counters wait)
      return *GLOBAL_PTR(const i32x4, rowp + (FP8 ? 16u * (uint32_t)(lane & 31) : lane16));
    }
    const int jb = j - kWT;  // (a run-time index: select, do not index the array)
    const int bs = (F::kBLoads == 1 || jb == 0) ? tr.bslot[0] : tr.bslot[F::kBLoads - 1];
    const int c = (64 * jb + lane) % kRC;
    return *GLOBAL_PTR(const i32x4, (uintptr_t)kv + (uint64_t)(uint32_t)(bs >= 0 ? bs : fill) *
                                            F::kRowBytes + F::kVBytes + 16 * c);
  };
  auto write_one = [&](int st, int j, i32x4 v) {
    char* ta = tiles + ((st % F::kBufs) * 2 + kh) * F::kWBytes;
    if (j < kWT) {
      if (!FP8 || lane < F::kVBytes / 16) *(i32x4*)(ta + j * F::kAStride + lane16) = v;
    } else {
      const int e = 64 * (j - kWT) + lane;  // chunk e % C of row e / C
      *(i32x4*)(ta + F::kABytes + (e / kRC) * F::kRStride + 16 * (e % kRC)) = v;
    }
  };

  f32x16 o[kDv / 32];  // O^T: dims 32mt + 8(i/4) + 4h2 + i%4, head h0 + c32
#pragma unroll
  for (int mt = 0; mt < kDv / 32; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[mt][i] = 0.f;
  // per lane two heads, 16ht + c16; le sums P unrounded (for lse, and to normalise O with a
  // bf16 cache), l sums the fp16 P of an e4m3 cache as rounded for the matrix cores
  float m_run[2] = {kMFloor, kMFloor}, l_run[2] = {0.f, 0.f}, le_run[2] = {0.f, 0.f};
  const bool hsel = (lane & 16) != 0;  // the O^T column c32 is head 16*hsel + c16

  // The gathers go through registers: during stage st the loads of the tile of stage st + 2
  // are issued and the loaded rows of the tile of stage st + 1 are written to LDS, one of each
  // every other step of the QK loop (a one-stage queue of kIssueW loads per wave).  Each
  // stage starts with a barrier: the tile of the stage has been written by both of its waves,
  // and the ring slot written during the stage has been read by both.
  i32x4 stg[F::kIssueW];
  // (one guarded block from the first gather to the end of the loop: the gathers read `fill`,
  // and a single path into the loop keeps the counter waits exact)
  if (nst > 0) {
    const TileRows tr0 = tile_rows(0);
#pragma unroll
    for (int j = 0; j < F::kIssueW; ++j) stg[j] = load_one(tr0, jlo + j);
#pragma unroll
    for (int j = 0; j < F::kIssueW; ++j) write_one(0, jlo + j, stg[j]);
    const TileRows tr1 = tile_rows(min(1, nst - 1));
#pragma unroll
    for (int j = 0; j < F::kIssueW; ++j) stg[j] = load_one(tr1, jlo + j);
  // Q has landed on every path into the loop (otherwise the waits for Q placed inside the loop
  // would also hold back the queued gathers): the loaded half goes to the shared copy, and
  // after a barrier the partner's half of the register fragments comes back from it
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
#pragma unroll
    for (int i = 0; i < kNQ / 2; ++i)
      *(bf16x8*)(qxe + (ht * kNQ + 2 * i) * 1024) =
          2 * i < kQR ? qf[ht][2 * i < kQR ? 2 * i : 0] : qtl[ht][2 * i < kQR ? 0 : i - kQR / 2];
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
#pragma unroll
    for (int i = 0; i < kQR / 2; ++i)
      qf[ht][2 * i + 1] = *(const bf16x8*)(qxo + (ht * kNQ + 2 * i + 1) * 1024);
  }
  for (int st = 0; st < nst; ++st) {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const TileRows trn = tile_rows(min(st + 2, nst - 1));
    const uint32_t mask = masks[st * 2 + kh];
    const char* sb = tiles + ((st % F::kBufs) * 2 + kh) * F::kWBytes;
    const int rbase = st * kSR + kh * kWT;

    // S^T[key 4g4 + i][head 16ht + c16]
    f32x4 s[2];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) s[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
    // K fragments are read kPre steps ahead of their use (the latency of an LDS read is
    // several MFMA steps)
    constexpr int kPre = 3;
    using KRaw = typename std::conditional<FP8, i32x2, bf16x8>::type;
    KRaw kr[kPre];
    // lane (m = c16, g4): row pi(m), dims 32f + 8g4 .. +7 of fragment f = ks ^ kh (region A
    // below dim 512, B above)
    const int qr = tile_row(c16);
    auto kread = [&](int ks) -> KRaw {
      constexpr int kEB = FP8 ? 1 : 2;  // bytes per element
      const int d = 32 * ks + 8 * g4 + ((ks & 1) ? -32 * kh : 32 * kh);
      const char* pa = ks < kDv / 32 ? sb + qr * F::kAStride + kEB * d
                                     : sb + F::kABytes + qr * F::kRStride + kEB * (d - kDv);
      return *(const KRaw*)pa;
    };
#pragma unroll
    for (int ks = 0; ks < kPre; ++ks) kr[ks] = kread(ks);
    bf16x8 ql[2][2];  // [step parity][ht]: Q fragments from LDS, read one step ahead
#pragma unroll
    for (int ks = 0; ks < kDqk / 32; ++ks) {
      if (ks + 1 >= kQR && ks + 1 < kNQ) {
#pragma unroll
        for (int ht = 0; ht < 2; ++ht)
          ql[(ks + 1) & 1][ht] =
              *(const bf16x8*)(((ks + 1) & 1 ? qxo : qxe) + (ht * kNQ + ks + 1) * 1024);
      }
      const KRaw cur = kr[ks % kPre];
      if (ks + kPre < kDqk / 32) kr[ks % kPre] = kread(ks + kPre);
      bf16x8 a;
      if constexpr (FP8) {
        const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cur[0], 1.f, false);
        const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cur[0], 1.f, true);
        const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cur[1], 1.f, false);
        const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cur[1], 1.f, true);
        a = __builtin_shufflevector(__builtin_shufflevector(p0, p1, 0, 1, 2, 3),
                                    __builtin_shufflevector(p2, p3, 0, 1, 2, 3), 0, 1, 2, 3, 4,
                                    5, 6, 7);
      } else {
        a = cur;
      }
#pragma unroll
      for (int ht = 0; ht < 2; ++ht)
        s[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            a, ks < kQR ? qf[ht][ks < kQR ? ks : 0] : ql[ks & 1][ht], s[ht], 0, 0, 0);
      // (unconditional: near the end of the split they re-load the last tile into the ring
      // slot that is not read again, and the queue keeps a fixed order for the counters)
      if ((ks & 1) == 0 && ks / 2 < F::kIssueW) {
        const int k = ks / 2;
        write_one(st + 1, jlo + k, stg[k]);
        stg[k] = load_one(trn, jlo + k);
      }
    }

    // ---- online softmax in log2 units: t = z - m_run with z = s * zsc (zsc = softmax scale *
    // log2 e, times the row scale for e4m3), p = 2^t.  The running max is raised only when
    // some t of the tile exceeds 8 (a lane-local test; the exact tile max across the four
    // 16-lane rows is formed only then), so p <= 2^8.  Masked keys (a split's last tile only)
    // get s = -inf, hence p = 0; m_run starts at a finite floor so this holds before the first
    // live key too.  (The mask applies to t, not to s: a masked e4m3 row has scale 0.)
    const uint32_t mk = (mask >> (4 * g4)) & 0xFu;
    f32x4 zsc = {c2, c2, c2, c2};
    if (FP8) {
      const f32x4 sc = *(const f32x4*)(scl + rbase + 4 * g4);
      zsc = sc * c2;
    }
    float tz[2][4];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
      for (int i = 0; i < 4; ++i) tz[ht][i] = fmaf(s[ht][i], zsc[i], -m_run[ht]);
    if (mask != 0xFFFFu) {  // wave-uniform
#pragma unroll
      for (int ht = 0; ht < 2; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) tz[ht][i] = ((mk >> i) & 1u) ? tz[ht][i] : -INFINITY;
    }
    const float tmax = fmaxf(fmaxf(fmaxf(tz[0][0], tz[0][1]), fmaxf(tz[0][2], tz[0][3])),
                             fmaxf(fmaxf(tz[1][0], tz[1][1]), fmaxf(tz[1][2], tz[1][3])));
    if (__any(tmax > 8.f)) {
      float alpha[2];
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        float zm = -INFINITY;  // (from z itself: t loses z next to the floor)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if ((mk >> i) & 1u) zm = fmaxf(zm, s[ht][i] * zsc[i]);
        const float m_new = fmaxf(m_run[ht], rows4_max(zm));
        alpha[ht] = __builtin_amdgcn_exp2f(m_run[ht] - m_new);
        l_run[ht] *= alpha[ht];
        le_run[ht] *= alpha[ht];
        m_run[ht] = m_new;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          tz[ht][i] = ((mk >> i) & 1u) ? fmaf(s[ht][i], zsc[i], -m_new) : -INFINITY;
      }
      const float a_sel = hsel ? alpha[1] : alpha[0];
#pragma unroll
      for (int mi = 0; mi < kDv / 32; ++mi) acc_scale(o[mi], a_sel);
    }
    float p[2][4];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[ht][i] = __builtin_amdgcn_exp2f(tz[ht][i]);
        le_run[ht] += p[ht][i];
      }

    // ---- P^T in the 32x32x16 B layout: lane l gets keys 8h2 + j of head c32
    uint32_t pk[2][2];  // [tile ht][pair]: packed 16-bit P of keys 4g4 + 2*pair + {0,1}
    if (FP8) {
      f32x4 rs = {0.f, 0.f, 0.f, 0.f}, sn = {0.f, 0.f, 0.f, 0.f};
      const f32x4 sc = *(const f32x4*)(scl + rbase + 4 * g4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sn[i] = sc[i] * inv_smax;
        rs[i] = sc[i] > 0.f ? smax / sc[i] : 0.f;
      }
#pragma unroll
      for (int ht = 0; ht < 2; ++ht)
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          const _Float16 v0 = (_Float16)(p[ht][2 * pr] * sn[2 * pr]);
          const _Float16 v1 = (_Float16)(p[ht][2 * pr + 1] * sn[2 * pr + 1]);
          l_run[ht] = fmaf((float)v0, rs[2 * pr], l_run[ht]);
          l_run[ht] = fmaf((float)v1, rs[2 * pr + 1], l_run[ht]);
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
              uint32_t, __builtin_convertvector(f32x2{p[ht][2 * pr], p[ht][2 * pr + 1]}, bf16x2));
    }
    // lanes of the low 16-row of each half keep tile 0 and take tile 0 of the row above;
    // lanes of the high 16-row take tile 1 of the row below and keep their tile 1
    i32x4 pb;
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      auto r = __builtin_amdgcn_permlane16_swap(pk[0][pr], pk[1][pr], false, false);
      pb[pr] = (int)r[0];      // keys 8h2 + 2pr + {0,1}
      pb[2 + pr] = (int)r[1];  // keys 8h2 + 4 + 2pr + {0,1}
    }

    // ---- O^T[32 dims][32 heads] += V^T[32 dims][16 keys] . P^T
    const int G = g4;
#pragma unroll
    for (int mi = 0; mi < kDv / 32; ++mi) {
      const int d0 = 32 * mi + 16 * (G & 1);
      if (FP8) {
        // lane k of the 16-row group: key j = k / 2 (row pi(8h + j)), bytes d0 + 8 (k % 2)
        const int kr = 8 * (G >> 1) + 2 * ((c16 >> 1) & 3) + (c16 >> 3);
        const i32x2 c8 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            LDS_PTR(i32x2, sb + kr * F::kAStride + d0 + 8 * (c16 & 1)));
        const f16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c8[0], 1.f, false);
        const f16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c8[0], 1.f, true);
        const f16x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c8[1], 1.f, false);
        const f16x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c8[1], 1.f, true);
        const f16x8 a = __builtin_shufflevector(__builtin_shufflevector(a0, a1, 0, 1, 2, 3),
                                                __builtin_shufflevector(a2, a3, 0, 1, 2, 3), 0,
                                                1, 2, 3, 4, 5, 6, 7);
        o[mi] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, __builtin_bit_cast(f16x8, pb), o[mi],
                                                       0, 0, 0);
      } else {
        // lane k of the 16-row group: keys j = k / 4 (row pi(8h + j) = 8h + 2j) and j + 4
        // (the next row), dims d0 + 4 (k % 4)
        const int kr = 8 * (G >> 1) + 2 * (c16 >> 2);
        // whole-vector moves only: element-wise assembly of this operand from the two
        // 64-bit halves was mistranslated by the compiler
        const char* base = sb + kr * F::kAStride + 2 * (d0 + 4 * (c16 & 3));
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, base));
        const bf16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, base + F::kAStride));
        const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, pb),
                                                        o[mi], 0, 0, 0);
      }
    }
  }
  }  // nst > 0

  // ---- merge the two key halves of each head (waves w and w ^ 2): M = max m, factors
  // 2^(m - M) (a wave that saw no live key has m at the floor and l = 0)
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    le_run[ht] = rows4_sum(le_run[ht]);
    l_run[ht] = FP8 ? rows4_sum(l_run[ht]) : le_run[ht];
  }
  if (g4 == 0) {
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      xm[(wave * 3 + 0) * kHB + 16 * ht + c16] = m_run[ht];
      xm[(wave * 3 + 1) * kHB + 16 * ht + c16] = l_run[ht];
      xm[(wave * 3 + 2) * kHB + 16 * ht + c16] = le_run[ht];
    }
  }
  __syncthreads();
  float fme;  // this wave's factor for head c32
  {
    const int pw = wave ^ 2;
    const float m0 = xm[(wave * 3 + 0) * kHB + c32], m1 = xm[(pw * 3 + 0) * kHB + c32];
    const float M = fmaxf(m0, m1);
    const float f0 = exp2f(m0 - M), f1 = exp2f(m1 - M);
    const float Ls = f0 * xm[(wave * 3 + 1) * kHB + c32] + f1 * xm[(pw * 3 + 1) * kHB + c32];
    const float LEs = f0 * xm[(wave * 3 + 2) * kHB + c32] + f1 * xm[(pw * 3 + 2) * kHB + c32];
    fme = f0;
    if (FP8) fme *= smax;  // O was accumulated relative to the largest row scale
    if (kh == 0 && h2 == 0) {
      xf[(hh * 3 + 0) * kHB + c32] = M;
      xf[(hh * 3 + 1) * kHB + c32] = Ls;
      xf[(hh * 3 + 2) * kHB + c32] = LEs;
      const int head = h0 + c32;
      if (nsplit == 1) {
        if (lse) lse[(int64_t)t * kH + head] = LEs > 0.f ? (M + log2f(LEs)) * kLn2 : -INFINITY;
      } else {
        const int64_t pr = ((int64_t)tl * nsplit + split) * kH + head;
        *(f32x4*)(part_ml + pr * 4) = f32x4{M, Ls, LEs, 0.f};
      }
    }
  }
  // four rounds of 128 dims: every wave stores its scaled O^T, then wave (hh, kh) sums dims
  // 64kh .. 64kh+63 of the round over the two key halves of head half hh and writes them out,
  // lane l taking dims 64kh + 8(l & 7) .. +7 of heads (l >> 3) + 8q, q < 4: eight lanes cover
  // the 64 dims of a head, so each store instruction writes whole 128-byte lines of fp16 /
  // bf16 (one straight-line copy of the rounds per kind of output)
  float* xo = (float*)tiles;  // [wave][head][kXPitch]
  const int sh = lane >> 3;   // summed head of q = 0
  const int sd = 64 * kh + 8 * (lane & 7);
  // (the normalisers of the summed heads are read after the first barrier of the rounds:
  // the merged sums in xf come from the kh = 0 waves)
  float inv[4];
  const int head = h0 + sh;
  const int64_t orow = ((int64_t)t * kH + head) * kDv;                         // output row
  const int64_t prow = (((int64_t)tl * nsplit + split) * kH + head) * kDv;    // partial row
  auto rounds = [&](auto&& emit) {
#pragma unroll
    for (int rd = 0; rd < 4; ++rd) {
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) {
        const int mi = 4 * rd + mm;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d = 32 * mm + 8 * q4 + 4 * h2;
          const f32x4 v = {acc_read_scaled(o[mi][4 * q4], fme),
                           acc_read_scaled(o[mi][4 * q4 + 1], fme),
                           acc_read_scaled(o[mi][4 * q4 + 2], fme),
                           acc_read_scaled(o[mi][4 * q4 + 3], fme)};
          *(f32x4*)(xo + (wave * kHB + c32) * kXPitch + d) = v;
        }
      }
      __syncthreads();
      if (rd == 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float L = xf[(hh * 3 + 1) * kHB + sh + 8 * q];
          inv[q] = L > 0.f ? 1.f / L : 0.f;
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float* a = xo + (hh * kHB + sh + 8 * q) * kXPitch + sd;
        const float* b = xo + ((hh + 2) * kHB + sh + 8 * q) * kXPitch + sd;
        const f32x4 lo = *(const f32x4*)a + *(const f32x4*)b;
        const f32x4 hi = *(const f32x4*)(a + 4) + *(const f32x4*)(b + 4);
        emit(q, (int64_t)8 * q * kDv + 128 * rd + sd, lo, hi);
      }
      if (rd < 3) __syncthreads();
    }
  };
  if (nsplit == 1) {
    rounds([&](int q, int64_t off, f32x4 lo, f32x4 hi) {
      store_out8<OUT_F32>(out, orow + off, lo * inv[q], hi * inv[q]);
    });
  } else if (OUT_F32) {
    rounds([&](int q, int64_t off, f32x4 lo, f32x4 hi) {
      (void)q;
      *(f32x4*)(part_o + prow + off) = lo;
      *(f32x4*)(part_o + prow + off + 4) = hi;
    });
  } else {  // bf16 output: the split's own normalised O as an fp16 partial
    rounds([&](int q, int64_t off, f32x4 lo, f32x4 hi) {
      store_part16x8(part_o, prow + off, lo * inv[q], hi * inv[q]);
    });
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
                           hipStream_t st) {
  const int kps = attn_keys_per_split(K, nsplit);
  const float c2 = softmax_scale * kLog2e;
  const size_t shm = attn_smem_bytes(fp8, kps);
  auto* fn = fp8 ? (out_f32 ? mla_attn_fp8_o32_kernel : mla_attn_fp8_kernel)
                 : (out_f32 ? mla_attn_bf16_o32_kernel : mla_attn_bf16_kernel);
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
