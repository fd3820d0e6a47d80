// LayerNorm over the fp32 residual stream: one wavefront per row.
//
// Pre-LN layers and ln_post (model card "MOSS-Transcribe-preview-2B-GGUF",
// Architecture table, Audio encoder and Encoder head rows): y = (x - mean) /
// sqrt(var + eps) * g + b with the biased variance, statistics in fp32.
// A row of D = 256 * VEC floats is held in registers (VEC float4 per lane);
// mean and variance are two wavefront reductions over the register copy, so
// the row is read from memory once.
#include "common.h"
#include "kernels.h"

namespace mt {

namespace {

__device__ __forceinline__ float wave_sum(float v) { return wave_sum64(v); }

template <int VEC, typename T, bool SPLIT>
__global__ __launch_bounds__(256) void layernorm_kernel(const float* __restrict__ x,
                                                        const float* __restrict__ g,
                                                        const float* __restrict__ b,
                                                        void* __restrict__ out, int M, float eps,
                                                        int* sat, int sat_bit) {
  constexpr int D = 256 * VEC;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const float4* xr = (const float4*)(x + (int64_t)row * D);
  float4 v[VEC];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < VEC; ++i) {
    v[i] = xr[lane + 64 * i];
    s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  }
  const float mean = wave_sum(s) * (1.0f / D);
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < VEC; ++i) {
    const float a0 = v[i].x - mean, a1 = v[i].y - mean, a2 = v[i].z - mean, a3 = v[i].w - mean;
    q += (a0 * a0 + a1 * a1) + (a2 * a2 + a3 * a3);
  }
  const float rstd = 1.0f / sqrtf(wave_sum(q) * (1.0f / D) + eps);
  const float4* g4 = (const float4*)g;
  const float4* b4 = (const float4*)b;
  [[maybe_unused]] float amax = 0.f;
#pragma unroll
  for (int i = 0; i < VEC; ++i) {
    const int c4 = lane + 64 * i;
    const float4 gg = g4[c4], bb = b4[c4];
    float4 y;
    y.x = (v[i].x - mean) * rstd * gg.x + bb.x;
    y.y = (v[i].y - mean) * rstd * gg.y + bb.y;
    y.z = (v[i].z - mean) * rstd * gg.z + bb.z;
    y.w = (v[i].w - mean) * rstd * gg.w + bb.w;
    if constexpr (__is_same(T, f16_t)) amax = absmax4(amax, y.x, y.y, y.z, y.w);
    if constexpr (sizeof(T) == 4) {
      ((float4*)out)[(int64_t)row * (D / 4) + c4] = y;
    } else {
      const T h0 = Elem<T>::from_f(y.x), h1 = Elem<T>::from_f(y.y);
      const T h2 = Elem<T>::from_f(y.z), h3 = Elem<T>::from_f(y.w);
      const uint2 hi = make_uint2(pack2(h0, h1), pack2(h2, h3));
      if constexpr (!SPLIT) {
        ((uint2*)out)[(int64_t)row * (D / 4) + c4] = hi;
      } else {
        const T l0 = Elem<T>::from_f(y.x - Elem<T>::to_f(h0));
        const T l1 = Elem<T>::from_f(y.y - Elem<T>::to_f(h1));
        const T l2 = Elem<T>::from_f(y.z - Elem<T>::to_f(h2));
        const T l3 = Elem<T>::from_f(y.w - Elem<T>::to_f(h3));
        const uint2 lo = make_uint2(pack2(l0, l1), pack2(l2, l3));
        ((uint2*)out)[(int64_t)row * (D / 2) + c4] = hi;
        ((uint2*)out)[(int64_t)row * (D / 2) + D / 4 + c4] = lo;
      }
    }
  }
  if constexpr (__is_same(T, f16_t)) report_saturation(sat, sat_bit, amax);
}

template <int VEC, typename T, bool SPLIT>
hipError_t ln_run(const float* x, const float* g, const float* b, void* out, int M, float eps,
                  hipStream_t s, int* sat, int bit) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL((layernorm_kernel<VEC, T, SPLIT>), dim3((M + 3) / 4), dim3(256), 0, s, x, g, b,
                     out, M, eps, sat, bit);
  return hipGetLastError();
}

template <int VEC>
hipError_t ln_mode(const float* x, const float* g, const float* b, void* out, int M, float eps,
                   int dtype, bool split, hipStream_t s, int* sat, int bit) {
  if (dtype == DT_F32)
    return split ? hipErrorInvalidValue : ln_run<VEC, float, false>(x, g, b, out, M, eps, s, nullptr, 0);
  if (dtype == DT_BF16)
    return split ? ln_run<VEC, bf16_t, true>(x, g, b, out, M, eps, s, nullptr, 0)
                 : ln_run<VEC, bf16_t, false>(x, g, b, out, M, eps, s, nullptr, 0);
  return split ? ln_run<VEC, f16_t, true>(x, g, b, out, M, eps, s, sat, bit)
               : ln_run<VEC, f16_t, false>(x, g, b, out, M, eps, s, sat, bit);
}

}  // namespace

hipError_t launch_layernorm(const float* x, const float* g, const float* b, void* out, int M, int D,
                            float eps, int dtype, bool split, hipStream_t s, int* sat, int sat_bit) {
  switch (D / 256) {
    case 1: return ln_mode<1>(x, g, b, out, M, eps, dtype, split, s, sat, sat_bit);
    case 2: return ln_mode<2>(x, g, b, out, M, eps, dtype, split, s, sat, sat_bit);
    case 3: return ln_mode<3>(x, g, b, out, M, eps, dtype, split, s, sat, sat_bit);
    case 4: return ln_mode<4>(x, g, b, out, M, eps, dtype, split, s, sat, sat_bit);
    case 5: return ln_mode<5>(x, g, b, out, M, eps, dtype, split, s, sat, sat_bit);
    case 6: return ln_mode<6>(x, g, b, out, M, eps, dtype, split, s, sat, sat_bit);
    case 7: return ln_mode<7>(x, g, b, out, M, eps, dtype, split, s, sat, sat_bit);
    case 8: return ln_mode<8>(x, g, b, out, M, eps, dtype, split, s, sat, sat_bit);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mt
