// Device-side helpers shared by the HIP kernels of the encoder library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mt {

// 16-bit matrix-operand types.  Conversions from fp32 round to nearest even
// (v_cvt_pk_bf16_f32 / v_cvt_f16_f32); fp16 saturates at +-65504.
typedef __bf16 bf16_t;
typedef _Float16 f16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16_t f2bf(float f) { return (bf16_t)f; }
__device__ __forceinline__ float bf2f(bf16_t h) { return (float)h; }
__device__ __forceinline__ f16_t f2h(float f) { return (f16_t)fminf(fmaxf(f, -65504.0f), 65504.0f); }

// Two 16-bit values packed into one 32-bit word (low half first).
template <typename T>
__device__ __forceinline__ uint32_t pack2(T a, T b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// pack2((T)a, (T)b) as one v_cvt_pk_{f16,bf16}_f32 (round to nearest even)
// instead of two conversions and a shift-or.
template <typename T>
__device__ __forceinline__ uint32_t pack2_cast(float a, float b) {
  typedef float f2v __attribute__((ext_vector_type(2)));
  typedef T t2v __attribute__((ext_vector_type(2)));
  const f2v v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, t2v));
}

// pack2(from_f(a), from_f(b)) in one packed conversion: fp16 saturates at
// +-65504 first, bf16 converts as is.
template <typename T>
__device__ __forceinline__ uint32_t pack2f(float a, float b) {
  if constexpr (__is_same(T, _Float16))
    return pack2_cast<T>(fminf(fmaxf(a, -65504.0f), 65504.0f), fminf(fmaxf(b, -65504.0f), 65504.0f));
  else
    return pack2_cast<T>(a, b);
}

// GELU with the erf form, x Phi(x), Phi(x) = (1 + erf(x / sqrt 2)) / 2.
// erfc after Abramowitz & Stegun, Handbook of Mathematical Functions, 7.1.26:
// erfc(z) = t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-z^2), t = 1 / (1 + p z),
// z >= 0, |error| <= 1.5e-7.  With z = |x| / sqrt 2 and the coefficients
// halved, q = erfc(z) / 2 is the tail mass of the normal law beyond |x|:
// Phi(x) = 1 - q for x >= 0 and q for x < 0, so GELU = x - x q or x q.
// Both signs in one expression: x Phi(x) = x / 2 + |x| (1/2 - q).  Written
// so for few instructions (every element of conv1-3 and fc1 runs it, in the
// gelu_h form below): one reciprocal, one exp2, ten other ops, no compare or
// select; |error| below 3.5e-7 (float32, measured against the exact erf form
// on [-12, 12]).  gelu_f is the reference form; the kernels call gelu_h.
__device__ __forceinline__ float gelu_f(float x) {
  const float t = __builtin_amdgcn_rcpf(fmaf(0.23164190f, fabsf(x), 1.0f));  // p / sqrt 2
  const float P =
      t * fmaf(fmaf(fmaf(fmaf(0.5307027145f, t, -0.726576013f), t, 0.7107068705f), t, -0.142248368f),
               t, 0.127414796f);
  const float r = fmaf(-P, __builtin_amdgcn_exp2f(x * x * -0.72134752044f), 0.5f);  // 1/2 - q
  return fmaf(fabsf(x), r, 0.5f * x);
}

// gelu_f(x) from h = x / 2, with the same bits and one instruction less.
// Every step of gelu_f is rescaled by a power of two, which commutes with
// rounding: p |x| = (2 p) |h|, x x c = (h h)(4 c), the polynomial with
// doubled coefficients is 2 P, fma(-2 P, e, 1) = 2 r, and fma(|h|, 2 r, h)
// rounds |x| r + x / 2 once, as gelu_f does.  h itself comes from the
// pre-activation in one instruction: fma(acc, 1/2, b / 2) = (acc + b) / 2
// (or a dot product whose weights and bias were halved).
__device__ __forceinline__ float gelu_h(float h) {
  const float t = __builtin_amdgcn_rcpf(fmaf(2.0f * 0.23164190f, fabsf(h), 1.0f));
  const float P = t * fmaf(fmaf(fmaf(fmaf(2.0f * 0.5307027145f, t, 2.0f * -0.726576013f), t, 2.0f * 0.7107068705f),
                                t, 2.0f * -0.142248368f),
                           t, 2.0f * 0.127414796f);
  const float r = fmaf(-P, __builtin_amdgcn_exp2f(h * h * (4.0f * -0.72134752044f)), 1.0f);  // 1 - 2 q
  return fmaf(fabsf(h), r, h);
}
// GELU(acc + b) given hb = b / 2.
__device__ __forceinline__ float gelu_ab(float acc, float hb) { return gelu_h(fmaf(acc, 0.5f, hb)); }

__device__ __forceinline__ float silu_f(float x) { return x / (1.0f + expf(-x)); }

// Reductions over the 64 lanes of a wavefront in the butterfly order (the
// partner of lane l is l ^ 32, then l ^ 16, 8, 4, 2, 1), every lane ending
// with the same bits, without the LDS: v_permlane32_swap / v_permlane16_swap
// of a register with itself hand each lane its xor-32 / xor-16 partner (as
// the pair (own, partner) or (partner, own); addition is commutative), and
// once the bits above m are reduced the values repeat with period 2m, so a
// DPP rotation by m within each 16-lane row reads the same value as the xor
// partner.  Same results as __shfl_xor butterflies, without the ds_bpermute
// round trips.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <bool MAX>
__device__ __forceinline__ float wave_reduce64(float v) {
  auto op = [](float x, float y) { return MAX ? fmaxf(x, y) : x + y; };
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = op(__uint_as_float(b[0]), __uint_as_float(b[1]));
  v = op(v, dpp_f<0x128>(v));  // row_ror:8
  v = op(v, dpp_f<0x124>(v));  // row_ror:4
  v = op(v, dpp_f<0x122>(v));  // row_ror:2
  v = op(v, dpp_f<0x121>(v));  // row_ror:1
  return v;
}
__device__ __forceinline__ float wave_sum64(float v) { return wave_reduce64<false>(v); }
__device__ __forceinline__ float wave_max64(float v) { return wave_reduce64<true>(v); }

// fp16 saturation report.  fp16 conversions clamp at +-65504; a kernel that
// converts to fp16 tracks, per lane, the largest |value| it converted and
// then calls this once with every lane of the wavefront that is still
// running: if any of them exceeded 65504, the first such lane sets `bit` in
// *sat (a stage mask the host reads back), so a clamp is reported instead of
// passing silently.  sat == nullptr (other operand types): nothing.
__device__ __forceinline__ void report_saturation(int* sat, int bit, float amax) {
  if (!sat) return;
  const uint64_t over = __ballot(amax > 65504.0f);
  if (over && (int)(threadIdx.x & 63) == __ffsll((unsigned long long)over) - 1) atomicOr(sat, bit);
}
// Largest magnitude so far.  Written as medians with +inf (max(x, m) =
// med3(x, m, inf)), which the compiler folds into two v_max3_f32 with
// absolute-value modifiers per four values; with fmaxf it first quietened
// every input that came from another block (up to seven instructions per
// four values in the GEMM epilogues).  NaNs are ignored, as with fmaxf.
__device__ __forceinline__ float absmax4(float m, float a, float b, float c, float d) {
  const float inf = __builtin_inff();
  m = __builtin_amdgcn_fmed3f(__builtin_fabsf(a), m, inf);
  m = __builtin_amdgcn_fmed3f(__builtin_fabsf(b), m, inf);
  m = __builtin_amdgcn_fmed3f(__builtin_fabsf(c), m, inf);
  return __builtin_amdgcn_fmed3f(__builtin_fabsf(d), m, inf);
}

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
template <> struct Elem<f16_t> {
  static constexpr int per16 = 8;
  __device__ static __forceinline__ f16_t from_f(float f) { return f2h(f); }
  __device__ static __forceinline__ float to_f(f16_t v) { return (float)v; }
};
template <> struct Elem<float> {
  static constexpr int per16 = 4;
  __device__ static __forceinline__ float from_f(float f) { return f; }
  __device__ static __forceinline__ float to_f(float v) { return v; }
};

// One 16 x 16 x 32 matrix-core step on 16-byte operand chunks (8 x 16-bit).
__device__ __forceinline__ void mma16(f32x4& acc, const uint4& a, const uint4& b, bf16_t) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                               __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x4& acc, const uint4& a, const uint4& b, f16_t) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                              __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
}
// Four 16 x 16 x 4 fp32 steps, element e of every lane's chunk in step e.
__device__ __forceinline__ void mma_f32x4(f32x4& acc, const uint4& a, const uint4& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

// s_waitcnt vmcnt(n) with expcnt / lgkmcnt left unconstrained (gfx9
// encoding: vmcnt bits 3:0 and 15:14); n beyond the listed cases waits for
// everything, which is always safe.
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
#define MT_WAITVM(N) case N: __builtin_amdgcn_s_waitcnt(((N) & 15) | (7 << 4) | (15 << 8) | (((N) >> 4) << 14)); break;
    MT_WAITVM(0) MT_WAITVM(1) MT_WAITVM(2) MT_WAITVM(3) MT_WAITVM(4) MT_WAITVM(5) MT_WAITVM(6)
    MT_WAITVM(7) MT_WAITVM(8) MT_WAITVM(9) MT_WAITVM(10) MT_WAITVM(11) MT_WAITVM(12)
    MT_WAITVM(13) MT_WAITVM(14) MT_WAITVM(15) MT_WAITVM(16) MT_WAITVM(17) MT_WAITVM(18) MT_WAITVM(19)
    MT_WAITVM(20) MT_WAITVM(21) MT_WAITVM(22) MT_WAITVM(23) MT_WAITVM(24) MT_WAITVM(28) MT_WAITVM(32)
#undef MT_WAITVM
    default: __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); break;
  }
}

}  // namespace mt
