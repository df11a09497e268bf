// Cache append: the rows of a batch's new tokens written into their slots of a paged cache, as
// e4m3 codes with one fp32 scale per token, as MXFP8 (e4m3 codes with one power-of-two scale
// byte per 32 elements, the indexer keys' format of Key Optimization 2 of the same page), or as
// bf16.
//
// Method: "Day 0 Support for New LLM Architectures", Key Optimization 2 (the FP8 cache whose
// scale factors are computed online; here one scale per token over the whole row, amax/448,
// so that the largest magnitude lands on the largest finite e4m3 value, and each code is the
// round-to-nearest-even of the fp32 quotient x/scale) and "Day-0 Support for Large Model
// Inference", Core Operator Optimization 1 (the selection index is kept on the device and
// updated incrementally, not rebuilt).  Slots follow the block table of "Achieving Day-0
// Readiness ... Million-Token Context", section 2.2.
//
// One wave per token: the row's 16-byte pieces are dealt to the lanes in order (coalesced
// loads and stores), the row maximum is a wave reduction, and each lane converts and writes
// its own pieces.  The work is bound by HBM: 4 (or 2) bytes read and 1 (or 2) written per
// element.
#include "common.h"
#include "launch.h"

namespace tis {

// e4m3 code of y, |y| <= 448, by round-to-nearest-even; the sign is kept (also for zero).
// Below 2^-6 the quantum is 2^-9 (subnormal codes 0..7; 8 quanta is the code of 2^-6); in the
// binade [2^e, 2^(e+1)) it is 2^(e-3), and the code is 8(e + 7) + m - 8 for m quanta (m = 16,
// a carry into the next binade, gives that binade's first code).  Both scalings by powers of
// two are exact, so rint (ties to even) is the only rounding.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  uint32_t mag;
  if (a < 0x1p-6f) {
    mag = (uint32_t)__builtin_rintf(a * 512.f);
  } else {
    const int e = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;
    mag = (uint32_t)(8 * (e + 7) - 8) + (uint32_t)__builtin_rintf(ldexpf(a, 3 - e));
  }
  return sign | mag;
}

// bf16 bits of x by round-to-nearest-even (finite x)
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

enum AppendFmt : int { kOutBf16 = 0, kOutE4m3 = 1, kOutMx = 2 };

template <bool IN_BF16, int OUT>
__global__ __launch_bounds__(256) void cache_append_kernel(DevBatch bt, const void* __restrict__ rows,
    int D, uint8_t* __restrict__ pool, void* __restrict__ pool_scale) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= bt.T) return;  // (uniform over the wave)
  // the token's position: the last q_len positions of its request are its new tokens
  const TokLoc loc = locate(bt, t);
  const int p = loc.n - 1;
  const int page = bt.page_table[(int64_t)loc.b * bt.pt_stride + (p >> 6)];
  if (page < 0 || page >= bt.n_pages) return;  // (no slot: nothing is written)
  const int64_t slot = (int64_t)page * kPage + (p & (kPage - 1));
  // pieces of 4 elements: piece i = lane + 64j; D is a multiple of 16, at most 2048 (the
  // row stays in registers between the maximum and the conversion)
  const int npc = D / 4;
  constexpr int kMaxJ = 2048 / 4 / 64;
  float4 v[kMaxJ];
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxJ; ++j) {
    const int i = lane + 64 * j;
    if (64 * j >= npc) break;  // (uniform)
    float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i < npc) {
      if (IN_BF16) {
        const uint2 h = ((const uint2*)rows)[(int64_t)t * npc + i];
        f = make_float4(__uint_as_float(h.x << 16), __uint_as_float(h.x & 0xffff0000u),
                        __uint_as_float(h.y << 16), __uint_as_float(h.y & 0xffff0000u));
      } else {
        f = ((const float4*)rows)[(int64_t)t * npc + i];
      }
    }
    v[j] = f;
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(f.x), fabsf(f.y)), fmaxf(fabsf(f.z), fabsf(f.w))));
  }
  if constexpr (OUT == kOutMx) {
    // group i / 8 of piece i = lane + 64j: the eight lanes 8k..8k+7 of step j hold one group
    // (D is a multiple of 32, so a group is wholly inside or wholly past the row)
    uint32_t* out = (uint32_t*)(pool + slot * D);
    uint8_t* sb = (uint8_t*)pool_scale + slot * (D / 32);
#pragma unroll
    for (int j = 0; j < kMaxJ; ++j) {
      if (64 * j >= npc) break;  // (uniform)
      const int i = lane + 64 * j;
      float gm = fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)), fmaxf(fabsf(v[j].z), fabsf(v[j].w)));
#pragma unroll
      for (int o = 4; o > 0; o >>= 1) gm = fmaxf(gm, __shfl_xor(gm, o));
      const int X = mx_exponent(gm);
      if (i < npc) {
        const float y[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
        uint32_t w = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w |= e4m3_code(fminf(fmaxf(ldexpf(y[e], -X), -448.f), 448.f)) << (8 * e);
        out[i] = w;
        if ((lane & 7) == 0) sb[i >> 3] = (uint8_t)(X + 127);
      }
    }
  } else if constexpr (OUT == kOutE4m3) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    float scale = __fdiv_rn(amax, 448.f);
    scale = scale == 0.f ? 1.f : scale;
    uint32_t* out = (uint32_t*)(pool + slot * D);
#pragma unroll
    for (int j = 0; j < kMaxJ; ++j) {
      const int i = lane + 64 * j;
      if (64 * j >= npc) break;
      if (i < npc) {
        const float y[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
        uint32_t w = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float q = fminf(fmaxf(__fdiv_rn(y[e], scale), -448.f), 448.f);
          w |= e4m3_code(q) << (8 * e);
        }
        out[i] = w;
      }
    }
    if (lane == 0) ((float*)pool_scale)[slot] = scale;
  } else {
    uint2* out = (uint2*)((uint16_t*)pool + slot * D);
#pragma unroll
    for (int j = 0; j < kMaxJ; ++j) {
      const int i = lane + 64 * j;
      if (64 * j >= npc) break;
      if (i < npc)
        out[i] = make_uint2(bf16_bits(v[j].x) | (bf16_bits(v[j].y) << 16),
                            bf16_bits(v[j].z) | (bf16_bits(v[j].w) << 16));
    }
  }
}

hipError_t launch_cache_append(const DevBatch& bt, const void* rows, bool rows_bf16, int D,
                               void* pool, int pool_fmt, void* pool_scale, hipStream_t st) {
  if (bt.T < 1) return hipSuccess;
  if (D < 16 || D % 16 || D > 2048) return hipErrorInvalidValue;
  if (pool_fmt == kOutMx && D % 32) return hipErrorInvalidValue;
  using Fn = void (*)(DevBatch, const void*, int, uint8_t*, void*);
  static const Fn fns[2][3] = {
      {cache_append_kernel<false, kOutBf16>, cache_append_kernel<false, kOutE4m3>,
       cache_append_kernel<false, kOutMx>},
      {cache_append_kernel<true, kOutBf16>, cache_append_kernel<true, kOutE4m3>,
       cache_append_kernel<true, kOutMx>}};
  if (pool_fmt < 0 || pool_fmt > 2) return hipErrorInvalidValue;
  const Fn fn = fns[rows_bf16 ? 1 : 0][pool_fmt];
  hipLaunchKernelGGL(fn, dim3((bt.T + 3) / 4), dim3(256), 0, st, bt, rows, D, (uint8_t*)pool,
                     pool_scale);
  return hipGetLastError();
}

}  // namespace tis
