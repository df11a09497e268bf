// Shared device-side definitions for the gfx950 kernels of libtopidx.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))
#define GLOBAL_PTR(T, a) ((__attribute__((address_space(1))) T*)(a))

namespace tis {

constexpr int kPage = 64;
// Word 3 of a raw buffer resource on gfx9-family chips (32-bit data format, no swizzle):
// accesses at byte offsets at or past the resource's record count are dropped (stores) or
// read as zero (loads).
constexpr int kBufDword3 = 0x00020000;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Device view of a ragged paged batch (launches take a token range on top of it).  row_shift:
// the selection kernels' rows hold one entry per 2^row_shift positions (0: token scores;
// 6: one score per 64-position page); no other kernel reads it.
struct DevBatch {
  const int32_t* seq_lens;
  const int32_t* cu_q;
  const int32_t* page_table;
  int32_t B, T, pt_stride, n_pages;
  int32_t row_shift;
};

// Where flattened token t sits: its request b (the largest b with cu_q[b] <= t, so empty
// requests are skipped), that request's length L = seq_lens[b] and the token's candidate
// count n = p_t + 1 (positions 0..p_t, p_t = L - (cu_q[b+1] - t)).
struct TokLoc {
  int b, L, n;
};

// One memory round trip for up to 64 requests (a kernel start waits on this before it can
// address anything else, so a binary search of dependent loads would stall every wave for
// several latencies): lane i holds cu_q[i+1] and seq_lens[i] of a 64-request window, and b is
// the number of i in [1, B-1] with cu_q[i] <= t, which cu_q being nondecreasing makes a prefix
// count.  Must be called by all 64 lanes of the wave with the same t.
__device__ __forceinline__ TokLoc locate(const DevBatch& bt, int t) {
  const int lane = threadIdx.x & 63;
  for (int base = 0;; base += 64) {
    const int i = base + lane;
    const int cq = i + 1 <= bt.B ? bt.cu_q[i + 1] : 0;
    const int sl = i < bt.B ? bt.seq_lens[i] : 0;
    const int c = __popcll(__ballot(i + 1 <= bt.B - 1 && cq <= t));
    if (c < 64) {  // always reached once base + 64 > B - 1
      TokLoc r;
      r.b = base + c;
      r.L = __builtin_amdgcn_readlane(sl, c);
      r.n = r.L - (__builtin_amdgcn_readlane(cq, c) - t) + 1;
      return r;
    }
  }
}

// The same lookup split in two, so that other loads can be issued between the loads of the
// first 64-request window and their use.
struct LocLoads {
  int cq, sl;
};
// (The loads are unconditional, from clamped indices, with the values masked after: a load
// under a branch makes the compiler wait for every load issued before the join.)
__device__ __forceinline__ LocLoads locate_issue(const DevBatch& bt) {
  const int lane = threadIdx.x & 63;
  LocLoads r;
  r.cq = bt.cu_q[min(lane + 1, bt.B)];
  r.sl = bt.seq_lens[min(lane, bt.B - 1)];
  r.cq = lane + 1 <= bt.B ? r.cq : 0;
  r.sl = lane < bt.B ? r.sl : 0;
  return r;
}
__device__ __forceinline__ TokLoc locate_finish(const DevBatch& bt, int t, LocLoads w0) {
  const int lane = threadIdx.x & 63;
  const int c = __popcll(__ballot(lane + 1 <= bt.B - 1 && w0.cq <= t));
  // (both values are read out before the branch: a load whose value is used only inside it
  // is sunk into it by the compiler, which costs a second memory round trip)
  TokLoc r;
  r.b = c;
  r.L = __builtin_amdgcn_readlane(w0.sl, min(c, 63));
  r.n = r.L - (__builtin_amdgcn_readlane(w0.cq, min(c, 63)) - t) + 1;
  if (c < 64) return r;
  for (int base = 64;; base += 64) {  // more than 64 requests: the remaining windows
    const int i = base + lane;
    const int cq = i + 1 <= bt.B ? bt.cu_q[i + 1] : 0;
    const int sl = i < bt.B ? bt.seq_lens[i] : 0;
    const int cc = __popcll(__ballot(i + 1 <= bt.B - 1 && cq <= t));
    if (cc < 64) {
      TokLoc r;
      r.b = base + cc;
      r.L = __builtin_amdgcn_readlane(sl, cc);
      r.n = r.L - (__builtin_amdgcn_readlane(cq, cc) - t) + 1;
      return r;
    }
  }
}

// Physical slot (page*64 + offset) of logical position s of request b, or -1 when the page
// table entry is outside [0, n_pages).
__device__ __forceinline__ int64_t slot_of(const DevBatch& bt, int b, int s) {
  int page = bt.page_table[(int64_t)b * bt.pt_stride + (s >> 6)];
  if (page < 0 || page >= bt.n_pages) return -1;
  return (int64_t)page * kPage + (s & (kPage - 1));
}

// Shared exponent of an MXFP8 group (one power-of-two scale 2^X per 32 elements, stored as the
// byte X + 127): X = floor(log2 amax) - 8, so that amax / 2^X lies in e4m3's top binade
// [256, 512); at least -127 (-127 for an all-zero group; a finite fp32 amax keeps X <= 119).
// frexp: amax = m 2^E with m in [0.5, 1), so floor(log2 amax) = E - 1.
__device__ __forceinline__ int mx_exponent(float amax) {
  int E;
  (void)frexpf(amax, &E);
  return amax > 0.f ? max(E - 9, -127) : -127;
}

// Lane-pair sums across wave halves / 16-lane rows using the gfx950 permlane swaps:
// permlane32_swap(a, b) -> {[a_lo32, b_lo32], [a_hi32, b_hi32]}; permlane16_swap does the
// same with the 16-lane halves of each 32-lane half.
__device__ __forceinline__ float xor32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Largest value over the 64 lanes of the wave (every lane gets it).
__device__ __forceinline__ float wave_max(float x) {
  x = xor32_max(x);
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
// Pairwise sums across the halves: lanes [0,32) get a[l] + a[l+32], lanes [32,64) get
// b[l-32] + b[l].  pair16_sum does the same within each 32-lane half, on 16-lane halves.
__device__ __forceinline__ float pair32_sum(float a, float b) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair16_sum(float a, float b) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace tis
