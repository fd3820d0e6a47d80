// Device-side helpers shared by the HIP kernels of the encoder library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mt {

typedef uint16_t bf16_t;  // bf16 storage (upper half of an fp32)
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// fp32 -> bf16, round to nearest, ties to even (NaN kept quiet).
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// Exact erf-based GELU, 0.5 x (1 + erf(x / sqrt 2)), through the device math
// library's erff.
__device__ __forceinline__ float gelu_f(float x) {
  return 0.5f * x * (1.0f + erff(x * 0.70710678118654752440f));
}

__device__ __forceinline__ float silu_f(float x) { return x / (1.0f + expf(-x)); }

// Order-preserving map float -> int for atomicMax on floats of any sign.
__device__ __forceinline__ int float_key(float f) {
  int i = __float_as_int(f);
  return i >= 0 ? i : i ^ 0x7fffffff;
}
__device__ __forceinline__ float key_float(int k) {
  return __int_as_float(k >= 0 ? k : k ^ 0x7fffffff);
}

// Index of the sequence that holds row r, given prefix offsets cu[0..n]
// (cu[0] = 0, non-decreasing): the largest i with cu[i] <= r.
__device__ __forceinline__ int find_seq(const int32_t* __restrict__ cu, int n, int r) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <typename T> struct Elem;
template <> struct Elem<bf16_t> {
  static constexpr int per16 = 8;  // elements per 16-byte chunk
  __device__ static __forceinline__ bf16_t from_f(float f) { return f2bf(f); }
  __device__ static __forceinline__ float to_f(bf16_t v) { return bf2f(v); }
};
template <> struct Elem<float> {
  static constexpr int per16 = 4;
  __device__ static __forceinline__ float from_f(float f) { return f; }
  __device__ static __forceinline__ float to_f(float v) { return v; }
};

}  // namespace mt
