// First front-end convolution: 1 -> C channels, 3x3, stride 2, padding 1,
// bias, GELU (model card "MOSS-Transcribe-preview-2B-GGUF", Architecture
// table, Conv front-end row).  The log-mel is an image of height 128 (mel
// bin) and width T (time); zero outside each sequence.
//
// One input channel and nine taps make this a VALU kernel (no contraction
// worth the matrix cores).  One workgroup per output time row t1 of the
// packed batch: the three mel rows 2 t1 - 1 .. 2 t1 + 1 are staged in LDS
// with a zero border, each thread keeps the weights of 8 output channels in
// registers and walks the 64 output frequencies assigned to its lane group.
// Output is channels-last [t1][f1][C], 16 bytes per store.
#include "common.h"
#include "kernels.h"

namespace mt {

namespace {

template <typename T>
__global__ __launch_bounds__(256) void conv1_kernel(Conv1Args a, int pl) {
  __shared__ float rows[3][130];  // mel rows with a zero column at f = -1 and f = 128
  const int r = blockIdx.x;       // packed conv1 output time row
  const int sq = find_seq(a.cu_T1, a.nseq, r);
  const int t1 = r - a.cu_T1[sq];
  const int Tm = a.cu_T[sq + 1] - a.cu_T[sq];
  const float* mel = a.mel + a.mel_row_off[sq] * 128;
  for (int i = threadIdx.x; i < 3 * 130; i += blockDim.x) {
    const int dt = i / 130, f = i - dt * 130 - 1;
    const int t = 2 * t1 + dt - 1;
    float v = 0.f;
    if (t >= 0 && t < Tm && f >= 0 && f < 128) v = mel[(int64_t)t * 128 + f];
    rows[dt][f + 1] = v;
  }
  __syncthreads();

  const int CG = a.C / 8;
  const int tid = threadIdx.x;
  if (tid >= CG * pl) return;
  const int cg = tid % CG, lane_pos = tid / CG;
  // weights and bias halved (exact): the sums below are then (acc + b) / 2,
  // bit for bit, the argument gelu_h takes
  float w[8][9], b[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    b[c] = 0.5f * a.b[cg * 8 + c];
#pragma unroll
    for (int k = 0; k < 9; ++k) w[c][k] = 0.5f * a.w[(cg * 8 + c) * 9 + k];
  }
  T* out = (T*)a.out + (int64_t)r * 64 * a.C + cg * 8;
  [[maybe_unused]] float amax = 0.f;
  for (int f1 = lane_pos; f1 < 64; f1 += pl) {
    float p[9];
#pragma unroll
    for (int df = 0; df < 3; ++df)
#pragma unroll
      for (int dt = 0; dt < 3; ++dt) p[df * 3 + dt] = rows[dt][2 * f1 + df];  // f = 2 f1 + df - 1
    float y[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float s = b[c];
#pragma unroll
      for (int k = 0; k < 9; ++k) s += w[c][k] * p[k];
      y[c] = gelu_h(s);
    }
    if constexpr (__is_same(T, f16_t))
      amax = absmax4(absmax4(amax, y[0], y[1], y[2], y[3]), y[4], y[5], y[6], y[7]);
    if constexpr (sizeof(T) == 2) {
      uint4 v;
      v.x = pack2f<T>(y[0], y[1]);
      v.y = pack2f<T>(y[2], y[3]);
      v.z = pack2f<T>(y[4], y[5]);
      v.w = pack2f<T>(y[6], y[7]);
      *(uint4*)(out + (int64_t)f1 * a.C) = v;
    } else {
      float4* o = (float4*)(out + (int64_t)f1 * a.C);
      o[0] = make_float4(y[0], y[1], y[2], y[3]);
      o[1] = make_float4(y[4], y[5], y[6], y[7]);
    }
  }
  if constexpr (__is_same(T, f16_t)) report_saturation(a.sat, SAT_FRONTEND, amax);
}

}  // namespace

hipError_t launch_conv1(const Conv1Args& a, hipStream_t s) {
  if (a.total_T1 == 0) return hipSuccess;
  const int CG = a.C / 8;
  int pl = 256 / CG;
  if (pl < 1) return hipErrorInvalidValue;
  if (pl > 64) pl = 64;
  const int threads = ((CG * pl + 63) / 64) * 64;
  const dim3 grid((unsigned)a.total_T1), block(threads);
  if (a.dtype == DT_BF16) hipLaunchKernelGGL(conv1_kernel<bf16_t>, grid, block, 0, s, a, pl);
  else if (a.dtype == DT_F16) hipLaunchKernelGGL(conv1_kernel<f16_t>, grid, block, 0, s, a, pl);
  else hipLaunchKernelGGL(conv1_kernel<float>, grid, block, 0, s, a, pl);
  return hipGetLastError();
}

}  // namespace mt
