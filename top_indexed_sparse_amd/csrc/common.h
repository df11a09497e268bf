// Shared device-side definitions for the gfx950 kernels of libtopidx.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

namespace tis {

constexpr int kPage = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Device view of a ragged paged batch (launches take a token range on top of it).
struct DevBatch {
  const int32_t* seq_lens;
  const int32_t* cu_q;
  const int32_t* page_table;
  int32_t B, T, pt_stride, n_pages;
};

// Request of flattened token t: the largest b with cu_q[b] <= t (empty requests skipped).
__device__ __forceinline__ int find_request(const DevBatch& bt, int t) {
  int lo = 0, hi = bt.B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (bt.cu_q[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Absolute position of token t inside request b: its request's last q_len positions.
__device__ __forceinline__ int token_position(const DevBatch& bt, int b, int t) {
  return bt.seq_lens[b] - (bt.cu_q[b + 1] - t);
}

// Physical slot (page*64 + offset) of logical position s of request b, or -1 when the page
// table entry is outside [0, n_pages).
__device__ __forceinline__ int64_t slot_of(const DevBatch& bt, int b, int s) {
  int page = bt.page_table[(int64_t)b * bt.pt_stride + (s >> 6)];
  if (page < 0 || page >= bt.n_pages) return -1;
  return (int64_t)page * kPage + (s & (kPage - 1));
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
