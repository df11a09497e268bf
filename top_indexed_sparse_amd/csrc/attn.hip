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
// Matrix-core kernel (128 heads, bf16 or e4m3 cache), one workgroup per (token, key split):
//   * the split's positions are translated through the page table once into LDS;
//   * 32-row tiles are gathered straight into LDS with 16-byte global->LDS loads, double
//     buffered; e4m3 rows stay e4m3 in LDS and are widened per fragment;
//   * wave w owns heads 32w..32w+31.  S^T = K_tile . Q^T on v_mfma_f32_32x32x16 with Q^T
//     resident in registers (36 fragments of 16 dims); the accumulator holds, per lane, one
//     head and 16 keys, so the online softmax is lane-local plus one permlane swap;
//   * O^T[vdim][head] += V^T . P^T: P is already in the MFMA B layout (the 16 keys of a lane
//     are reused as the k index, with V^T rows read in the same order), and V^T fragments
//     come from the row-major tile via ds_read_b64_tr_b16 (bf16) / ds_read_b64_tr_b8 (e4m3);
//   * the running max is raised lazily (only when a tile exceeds it by 2^8), so rescaling
//     the 256 accumulator registers is rare;
//   * e4m3: per-token scales go into the logits in fp32 and into P relative to the split's
//     largest scale; P then is fp16 (11-bit significand) so that heavy rows stay accurate,
//     and the normaliser is accumulated from the same rounded P values;
//   * with several splits per token, (m, l, unnormalised O) partials are merged by
//     mla_combine_kernel with log-sum-exp weights.
#include "common.h"
#include "launch.h"

#include <algorithm>

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
constexpr int kH = 128, kDqk = 576, kDv = 512, kTile = 32;

// One gather stage holds 32 bf16 rows or 64 e4m3 rows, each followed by a 16-byte pad chunk:
// 2336 or 2368 chunks of 16 bytes, stored in a 2368-chunk buffer.  Every wave issues ten
// 16-byte-per-lane global->LDS loads per stage: nine windows of its own (chunks
// 256i + 64w + lane) and a tenth window [2304, 2368) that all four waves load with identical
// bytes.  The count per wave is therefore always ten, which lets the waits use immediates.
// Lanes whose chunk is a pad (or beyond the rows) load row 0 into it; those bytes are never
// read.
template <bool FP8>
struct KvFmt {
  static constexpr int kRowBytes = FP8 ? kDqk : 2 * kDqk;  // 576 or 1152
  static constexpr int kCpr = kRowBytes / 16 + 1;           // chunks per LDS row incl. pad
  static constexpr int kRS = kCpr * 16;                     // LDS row stride
  static constexpr int kStageRows = FP8 ? 64 : 32;
  static constexpr int kStageChunks = 2368;
  static constexpr int kStageBytes = kStageChunks * 16;    // 37888
  static constexpr int kStages = FP8 ? 3 : 4;               // LDS ring depth
  static constexpr int kIssue = 10;
  static_assert(kStageRows * kCpr <= kStageChunks, "stage rows overflow the buffer");
};

struct AttnSmem {  // offsets into dynamic LDS
  int rows, masks, zs, scn, rsc, tiles, total;
};
template <bool FP8>
__host__ __device__ constexpr AttnSmem attn_smem(int kps) {
  AttnSmem s{};
  int o = 0;
  s.rows = o; o += kps * 4;
  s.masks = o; o += ((kps + kTile - 1) / kTile) * 4;
  o = (o + 15) & ~15;
  s.zs = o; o += FP8 ? kps * 4 : 0;
  s.scn = o; o += FP8 ? kps * 4 : 0;
  s.rsc = o; o += FP8 ? kps * 4 : 0;
  o = (o + 15) & ~15;
  s.tiles = o; o += KvFmt<FP8>::kStages * KvFmt<FP8>::kStageBytes;
  s.total = o;
  return s;
}

// Four consecutive outputs at element offset `off`: fp32, or bf16 (round to nearest even).
template <bool OUT_F32>
__device__ __forceinline__ void store_out4(void* out, int64_t off, f32x4 v) {
  if (OUT_F32) {
    *(f32x4*)((float*)out + off) = v;
  } else {
    const uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[0]) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[1]) << 16);
    const uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[2]) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[3]) << 16);
    *(i32x2*)((uint16_t*)out + off) = i32x2{(int)w0, (int)w1};
  }
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

// s_waitcnt with vmcnt <= n (n < 64), other counters untouched (gfx9 encoding).
#define TIS_WAIT_VM(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (0x7 << 4) | (0xf << 8))

__device__ __forceinline__ void wait_stages_after(int later) {
  // each stage issued after the awaited one contributes 10 outstanding loads per wave
  switch (later) {
    case 0: TIS_WAIT_VM(0); break;
    case 1: TIS_WAIT_VM(10); break;
    case 2: TIS_WAIT_VM(20); break;
    default: TIS_WAIT_VM(30); break;
  }
}

template <bool FP8, bool OUT_F32>
__device__ __forceinline__ void mla_attn_body(DevBatch bt, int t_begin, int t_count,
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv,
    const float* __restrict__ kvscale, const int32_t* __restrict__ idx, int K, float c2,
    int nsplit, int kps, void* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_ml) {
  using F = KvFmt<FP8>;
  extern __shared__ __attribute__((aligned(16))) char sm[];
  const AttnSmem L = attn_smem<FP8>(kps);
  int* rows = (int*)(sm + L.rows);
  uint32_t* masks = (uint32_t*)(sm + L.masks);
  float* zs = (float*)(sm + L.zs);
  float* scn = (float*)(sm + L.scn);
  float* rsc = (float*)(sm + L.rsc);
  char* tiles = sm + L.tiles;
  __shared__ float red[8];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, col = lane & 31;
  const int g = lane >> 4, gi = lane & 15;
  const int tl = blockIdx.x % t_count, split = blockIdx.x / t_count;
  const int t = t_begin + tl;

  // ---- this wave's 32 query heads as MFMA B fragments (dims 16ks + 8h .. +7); issued first
  //      so their latency overlaps the index translation
  bf16x8 qf[kDqk / 16];
  {
    const uint16_t* qr = q + ((int64_t)t * kH + wave * 32 + col) * kDqk + 8 * h;
#pragma unroll
    for (int ks = 0; ks < kDqk / 16; ++ks) qf[ks] = *(const bf16x8*)(qr + 16 * ks);
  }

  const TokLoc loc = locate(bt, t);
  const int b = loc.b;
  const int Lb = loc.L;
  const int kbeg = split * kps;
  const int nk = min(kps, K - kbeg);
  const int ntiles = (nk + kTile - 1) / kTile;
  const int nstage = (nk + F::kStageRows - 1) / F::kStageRows;
  const int nrows = nstage * F::kStageRows;

  // ---- positions -> physical slots (and per-key scale factors); masked keys read slot 0
  float smax = 0.f;
  for (int i = tid; i < nrows; i += 256) {
    int slot = -1;
    if (i < nk) {
      const int s = idx[(int64_t)t * K + kbeg + i];
      if (s >= 0 && s < Lb) slot = (int)slot_of(bt, b, s);
    }
    rows[i] = slot;
    if (FP8) {
      const float sc = slot >= 0 ? kvscale[slot] : 0.f;
      zs[i] = sc;
      smax = fmaxf(smax, sc);
    }
  }
  if (FP8) {
    for (int o = 32; o > 0; o >>= 1) smax = fmaxf(smax, __shfl_xor(smax, o));
    if (lane == 0) red[wave] = smax;
  }
  __syncthreads();
  if (FP8) {
    smax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float inv_smax = smax > 0.f ? 1.f / smax : 0.f;
    for (int i = tid; i < nrows; i += 256) {
      const float sc = zs[i];
      scn[i] = sc * inv_smax;
      rsc[i] = sc > 0.f ? smax / sc : 0.f;
      zs[i] = sc * c2;
    }
  }
  for (int it = tid; it < nrows / kTile; it += 256) {
    uint32_t m = 0u;
    for (int r = 0; r < kTile; ++r) m |= (rows[it * kTile + r] >= 0 ? 1u : 0u) << r;
    masks[it] = m;
  }
  __syncthreads();

  // ---- stage gather: ten 1 KB global->LDS loads per wave; slot lookups batched first
  auto issue_stage = [&](int st) {
    char* tb = tiles + (st % F::kStages) * F::kStageBytes;
    int slot[F::kIssue];
#pragma unroll
    for (int i = 0; i < F::kIssue; ++i) {
      const int c = (i < 9 ? 256 * i + 64 * wave : 2304) + lane;
      const int r = c / F::kCpr;
      slot[i] = (r < F::kStageRows) ? rows[st * F::kStageRows + r] : -1;
    }
#pragma unroll
    for (int i = 0; i < F::kIssue; ++i) {
      const int w0 = i < 9 ? 256 * i + 64 * wave : 2304;
      const int c = w0 + lane;
      const int r = c / F::kCpr;
      const int cl = c - r * F::kCpr;
      const bool data = r < F::kStageRows && cl < F::kCpr - 1 && slot[i] >= 0;
      const int64_t src = data ? (int64_t)slot[i] * F::kRowBytes + cl * 16 : 0;
      __builtin_amdgcn_global_load_lds(kv + src, LDS_PTR(void, tb + w0 * 16), 16, 0, 0);
    }
  };

  f32x16 o[kDv / 32];
#pragma unroll
  for (int mt = 0; mt < kDv / 32; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[mt][i] = 0.f;
  // l_run sums the P values as rounded for the matrix cores (normalises O, which then is an
  // exact convex combination of the rows); le_run sums them unrounded (for lse)
  float m_run = -INFINITY, l_run = 0.f, le_run = 0.f;

  constexpr int kTilesPerStage = F::kStageRows / kTile;
  for (int st = 0; st < min(nstage, F::kStages - 1); ++st) issue_stage(st);
  for (int it = 0; it < ntiles; ++it) {
    const int st = it / kTilesPerStage;
    if (it % kTilesPerStage == 0) {
      wait_stages_after(min(F::kStages - 2, nstage - 1 - st));
      __builtin_amdgcn_s_barrier();
      if (st + F::kStages - 1 < nstage) issue_stage(st + F::kStages - 1);
    }
    const char* sb = tiles + (st % F::kStages) * F::kStageBytes;
    {
      const int rb = (it % kTilesPerStage) * kTile;  // first row of this tile in the stage

      // S^T[key][head] over the 576 dims
      f32x16 s;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < kDqk / 16; ++ks) {
        bf16x8 a;
        if (FP8) {
          const i32x2 c8 = *(const i32x2*)(sb + (rb + col) * F::kRS + 16 * ks + 8 * h);
          const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c8[0], 1.f, false);
          const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c8[0], 1.f, true);
          const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c8[1], 1.f, false);
          const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c8[1], 1.f, true);
          a = __builtin_shufflevector(__builtin_shufflevector(p0, p1, 0, 1, 2, 3),
                                      __builtin_shufflevector(p2, p3, 0, 1, 2, 3), 0, 1, 2, 3,
                                      4, 5, 6, 7);
        } else {
          a = *(const bf16x8*)(sb + (rb + col) * F::kRS + 2 * (16 * ks + 8 * h));
        }
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s, 0, 0, 0);
      }

      // online softmax, lane = (head col, keys 8(i/4) + 4h + i%4)
      const uint32_t mask = masks[it];
      float z[16];
      float mt = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 8 * (i >> 2) + 4 * h + (i & 3);
        float f = c2;
        if (FP8) f = zs[it * kTile + r];
        z[i] = ((mask >> r) & 1u) ? s[i] * f : -INFINITY;
        mt = fmaxf(mt, z[i]);
      }
      mt = xor32_max(mt);
      if (__any(mt > m_run + 8.f)) {
        const float m_new = fmaxf(m_run, mt);
        const float alpha = (m_run == -INFINITY) ? 0.f : exp2f(m_run - m_new);
#pragma unroll
        for (int mi = 0; mi < kDv / 32; ++mi) acc_scale(o[mi], alpha);
        l_run *= alpha;
        le_run *= alpha;
        m_run = m_new;
      }
      const bool live = m_run != -INFINITY;
      float p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = live ? exp2f(z[i] - m_run) : 0.f;
        le_run += p[i];
      }

      if (FP8) {
        f16x8 pf[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = it * kTile + 8 * (i >> 2) + 4 * h + (i & 3);
          const _Float16 v = (_Float16)(p[i] * scn[r]);
          pf[i >> 3][i & 7] = v;
          l_run = fmaf((float)v, rsc[r], l_run);
        }
#pragma unroll
        for (int mi = 0; mi < kDv / 32; ++mi) {
          const int v0 = 32 * mi + 16 * (g & 1);
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const int jj = gi >> 1;
            const int krow = rb + 16 * ks + 8 * (jj >> 2) + 4 * (g >> 1) + (jj & 3);
            const i32x2 c8 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                LDS_PTR(i32x2, sb + krow * F::kRS + v0 + 8 * (gi & 1)));
            const f16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c8[0], 1.f, false);
            const f16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c8[0], 1.f, true);
            const f16x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c8[1], 1.f, false);
            const f16x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c8[1], 1.f, true);
            const f16x8 a = __builtin_shufflevector(__builtin_shufflevector(a0, a1, 0, 1, 2, 3),
                                                    __builtin_shufflevector(a2, a3, 0, 1, 2, 3),
                                                    0, 1, 2, 3, 4, 5, 6, 7);
            o[mi] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[ks], o[mi], 0, 0, 0);
          }
        }
      } else {
        bf16x8 pb[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const __bf16 v = (__bf16)p[i];
          pb[i >> 3][i & 7] = v;
          l_run += (float)v;
        }
#pragma unroll
        for (int mi = 0; mi < kDv / 32; ++mi) {
          const int v0 = 32 * mi + 16 * (g & 1);
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const int krow = rb + 16 * ks + 4 * (g >> 1) + (gi >> 2);
            // whole-vector moves only: element-wise assembly of this operand from the two
            // 64-bit halves was mistranslated by the compiler
            const char* base = sb + krow * F::kRS + 2 * (v0 + 4 * (gi & 3));
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, base));
            const bf16x4 hi =
                __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, base + 8 * F::kRS));
            const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            o[mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[ks], o[mi], 0, 0, 0);
          }
        }
      }
    }
  }

  // ---- epilogue: lane holds head 32w+col, vdims 32mi + 8(i/4) + 4h + i%4
  const float l_tot = xor32_sum(l_run);
  const float le_tot = xor32_sum(le_run);
  const int head = wave * 32 + col;
  const float oscale = FP8 ? smax : 1.f;
  if (nsplit == 1) {
    const float inv = l_tot > 0.f ? oscale / l_tot : 0.f;
    const int64_t obase = ((int64_t)t * kH + head) * kDv;
#pragma unroll
    for (int mi = 0; mi < kDv / 32; ++mi)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int vd = 32 * mi + 8 * q4 + 4 * h;
        const f32x4 v = {o[mi][4 * q4] * inv, o[mi][4 * q4 + 1] * inv, o[mi][4 * q4 + 2] * inv,
                         o[mi][4 * q4 + 3] * inv};
        store_out4<OUT_F32>(out, obase + vd, v);
      }
    if (lse && h == 0)
      lse[(int64_t)t * kH + head] = le_tot > 0.f ? (m_run + log2f(le_tot)) * kLn2 : -INFINITY;
  } else {
    const int64_t pr = ((int64_t)tl * nsplit + split) * kH + head;
    float* po = part_o + pr * kDv;
#pragma unroll
    for (int mi = 0; mi < kDv / 32; ++mi)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int vd = 32 * mi + 8 * q4 + 4 * h;
        *(f32x4*)(po + vd) = f32x4{o[mi][4 * q4] * oscale, o[mi][4 * q4 + 1] * oscale,
                                   o[mi][4 * q4 + 2] * oscale, o[mi][4 * q4 + 3] * oscale};
      }
    if (h == 0) *(f32x4*)(part_ml + pr * 4) = f32x4{m_run, l_tot, le_tot, 0.f};
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

// Merge split partials (m in log2 units; l = sum of the rounded P, le = unrounded sum):
// O = sum_j 2^(m_j - M) O_j / sum_j 2^(m_j - M) l_j,  lse = M + log2 sum_j 2^(m_j - M) le_j.
template <bool OUT_F32>
__global__ __launch_bounds__(128) void mla_combine_kernel(int t_begin, int t_count, int nsplit,
    const float* __restrict__ part_o, const float* __restrict__ part_ml,
    void* __restrict__ out, float* __restrict__ lse) {
  const int tl = blockIdx.x / kH, head = blockIdx.x % kH;
  const int t = t_begin + tl;
  const int tid = threadIdx.x;
  float M = -INFINITY;
  for (int j = 0; j < nsplit; ++j) {
    const int64_t pr = ((int64_t)tl * nsplit + j) * kH + head;
    if (part_ml[pr * 4 + 1] > 0.f) M = fmaxf(M, part_ml[pr * 4]);
  }
  float Lsum = 0.f, LEsum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < nsplit; ++j) {
    const int64_t pr = ((int64_t)tl * nsplit + j) * kH + head;
    const f32x4 ml = *(const f32x4*)(part_ml + pr * 4);
    if (!(ml[1] > 0.f)) continue;
    const float wgt = exp2f(ml[0] - M);
    Lsum = fmaf(wgt, ml[1], Lsum);
    LEsum = fmaf(wgt, ml[2], LEsum);
    const f32x4 v = *(const f32x4*)(part_o + pr * kDv + 4 * tid);
    acc += wgt * v;
  }
  const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
  store_out4<OUT_F32>(out, ((int64_t)t * kH + head) * kDv + 4 * tid, acc * inv);
  if (lse && tid == 0)
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
  return (kps + kTile - 1) / kTile * kTile;
}

int attn_split_count(int t_count, int K) {
  // enough workgroups to cover the 256 CUs, at least 64 keys per split, <= 2048 keys per
  // split; recomputed from the rounded split length so that no split is empty
  int s = (256 + t_count - 1) / t_count;
  s = std::max(1, std::min(s, (K + 63) / 64));
  s = std::max(s, (K + 2047) / 2048);
  const int kps = attn_keys_per_split(K, s);
  return (K + kps - 1) / kps;
}

size_t attn_smem_bytes(bool fp8, int kps) {
  return fp8 ? (size_t)attn_smem<true>(kps).total : (size_t)attn_smem<false>(kps).total;
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
  hipLaunchKernelGGL(fn, dim3(t_count * nsplit), dim3(256), shm, st, bt, t_begin, t_count, q, kv,
                     kvscale, idx, K, c2, nsplit, kps, out, lse, part_o, part_ml);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  auto* cfn = out_f32 ? mla_combine_kernel<true> : mla_combine_kernel<false>;
  hipLaunchKernelGGL(cfn, dim3(t_count * kH), dim3(128), 0, st, t_begin, t_count, nsplit, part_o,
                     part_ml, out, lse);
  return hipGetLastError();
}

}  // namespace tis
