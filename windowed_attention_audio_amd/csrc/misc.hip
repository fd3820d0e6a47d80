// Small kernels: table upload, fills, the log-mel clamp pass, row copies and
// the one-time weight repacking.
#include <climits>

#include "common.h"
#include "kernels.h"

namespace mt {

namespace {

constexpr int BLOB_WORDS = 960;
struct Blob {
  int32_t n;
  uint32_t w[BLOB_WORDS];
};

__global__ void words_kernel(uint32_t* __restrict__ dst, Blob b) {
  for (int i = threadIdx.x; i < b.n; i += blockDim.x) dst[i] = b.w[i];
}

__global__ void fill_i32_kernel(int* p, int v, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// Log-mel clamp.  The frame kernel wrote y = (L + 4) / 4; with g the
// clip's maximum (the largest of its slots) the result is (max(L, g - 8) +
// 4) / 4, i.e. y raised to (g - 8 + 4) / 4 where L < g - 8 ((x + 4) / 4 in
// fp32 is monotone, so comparing y decides the same entries and gives the
// same values).  A chunk with nothing below the floor is left as it is.
// Padded rows beyond a clip are set to 0.  A workgroup covers 8 rows, one
// float4 per thread; its first wavefront reduces each row's slots first (8
// lanes per row).
__global__ __launch_bounds__(256) void mel_norm_kernel(MelArgs a, int64_t tmax) {
  __shared__ float floor_s[8];
  __shared__ int valid_s[8];
  const int64_t row0 = (int64_t)blockIdx.x * 8;
  if (threadIdx.x < 64) {
    const int r = threadIdx.x >> 3, part = threadIdx.x & 7;
    const int64_t row = min(row0 + r, a.out_rows - 1);
    int sq;
    bool valid;
    if (a.padded) {
      sq = (int)(row / tmax);
      valid = row - sq * tmax < (int64_t)(a.cu_frames[sq + 1] - a.cu_frames[sq]);
    } else {
      sq = find_seq(a.cu_frames, a.nseq, (int)row);
      valid = true;
    }
    int key = INT_MIN;  // below every float's key
    for (int i = part; i < a.nslot; i += 8)  // keys order as the floats do
      key = max(key, a.gmax[(int64_t)(sq * a.nslot + i) * a.slot_stride]);
    key = max(key, __shfl_xor(key, 1));
    key = max(key, __shfl_xor(key, 2));
    key = max(key, __shfl_xor(key, 4));
    if (part == 0) {
      floor_s[r] = (key_float(key) - 8.0f + 4.0f) * 0.25f;
      valid_s[r] = valid;
    }
  }
  __syncthreads();
  const int64_t i4 = row0 * 32 + threadIdx.x;
  if (i4 >= a.out_rows * 32) return;
  const int r = threadIdx.x >> 5;
  float4* p = (float4*)a.mel + i4;
  if (!valid_s[r]) {
    *p = make_float4(0.f, 0.f, 0.f, 0.f);
    return;
  }
  const float lo = floor_s[r];
  const float4 v = *p;
  if (v.x < lo || v.y < lo || v.z < lo || v.w < lo)
    *p = make_float4(fmaxf(v.x, lo), fmaxf(v.y, lo), fmaxf(v.z, lo), fmaxf(v.w, lo));
}

// Rows >= N_i of each padded output sequence are set to 0.
__global__ void zero_pad_kernel(float* out, const int32_t* cu_rows, int64_t stride, int D) {
  const int sq = blockIdx.y;
  const int n = cu_rows[sq + 1] - cu_rows[sq];
  const int64_t cnt = (stride - n) * (int64_t)D;
  float* base = out + ((int64_t)sq * stride + n) * D;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < cnt;
       i += (int64_t)gridDim.x * blockDim.x)
    base[i] = 0.f;
}

// Copy packed rows [M][D] into packed or padded output rows.
__global__ void copy_rows_kernel(const float* __restrict__ x, float* __restrict__ out, int M, int D,
                                 const int32_t* cu_rows, int nseq, int64_t stride) {
  const int row = blockIdx.x;
  int64_t orow = row;
  if (stride > 0) {
    const int sq = find_seq(cu_rows, nseq, row);
    orow = (int64_t)sq * stride + (row - cu_rows[sq]);
  }
  for (int c = threadIdx.x; c < D; c += blockDim.x) out[orow * D + c] = x[(int64_t)row * D + c];
}

__device__ __forceinline__ void put(void* dst, int64_t i, float v, int dtype) {
  if (dtype == DT_BF16) ((bf16_t*)dst)[i] = f2bf(v);
  else if (dtype == DT_F16) ((f16_t*)dst)[i] = f2h(v);
  else ((float*)dst)[i] = v;
}

// dst[r * dst_ld + col0 + c] = src[r * cols + c]
__global__ void convert_kernel(const float* __restrict__ src, void* dst, int64_t rows, int64_t cols,
                               int64_t dst_ld, int64_t col0, int dtype) {
  const int64_t n = rows * cols;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / cols, c = i - r * cols;
    put(dst, r * dst_ld + col0 + c, src[i], dtype);
  }
}

// conv [C][C][3][3] -> [C][9C], column (df * 3 + dt) * C + ci
__global__ void pack_conv_kernel(const float* __restrict__ w, void* dst, int C, int dtype) {
  const int64_t n = (int64_t)C * C * 9;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t co = i / (9LL * C);
    const int64_t rem = i - co * 9LL * C;
    const int tap = (int)(rem / C), ci = (int)(rem - (int64_t)tap * C);
    put(dst, i, w[((co * C + ci) * 9) + tap], dtype);
  }
}

// Conv1d [Co][Ci][3] -> [Co][3 Ci], column dt * Ci + ci (tap-major, the
// order of the 1-D convolution gather).
__global__ void pack_conv1d_kernel(const float* __restrict__ w, void* dst, int Co, int Ci, int dtype) {
  const int64_t n = 3LL * Co * Ci;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t co = i / (3LL * Ci);
    const int rem = (int)(i - co * 3LL * Ci);
    const int dt = rem / Ci, ci = rem - dt * Ci;
    put(dst, i, w[(co * Ci + ci) * 3 + dt], dtype);
  }
}

// One workgroup per packed output row: the fp32 source row of sequence sq at
// time r - cu[sq], converted to 16 bits (round to nearest even).
__global__ void rows_to_half_kernel(const float* __restrict__ src, const int64_t* __restrict__ row_off,
                                    const int32_t* __restrict__ cu, int nseq, int W, void* dst,
                                    int dtype) {
  const int64_t r = blockIdx.x;
  const int sq = find_seq(cu, nseq, (int)r);
  const float* s = src + (row_off[sq] + (r - cu[sq])) * W;
  for (int c = threadIdx.x; c < W; c += blockDim.x) put(dst, r * W + c, s[c], dtype);
}

// conv_out [D][C*F] (column c*F + f) -> [D][F*C] (column f*C + c), matching the
// channels-last [t][f][c] output of the last convolution.
__global__ void pack_conv_out_kernel(const float* __restrict__ w, void* dst, int D, int C, int F,
                                     int dtype) {
  const int64_t n = (int64_t)D * C * F;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t d = i / ((int64_t)C * F);
    const int rem = (int)(i - d * C * F);
    const int f = rem / C, c = rem - f * C;
    put(dst, i, w[d * C * F + (int64_t)c * F + f], dtype);
  }
}

// gate/up [A][O] -> [2A][O], rows interleaved in blocks of 16 (16 gate rows,
// then the 16 up rows of the same features).
__global__ void pack_swiglu_kernel(const float* __restrict__ gate, const float* __restrict__ up,
                                   void* dst, int A, int O, int dtype) {
  const int64_t n = 2LL * A * O;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / O, c = i - r * O;
    const int64_t p = r >> 5, q = r & 31;
    const float v = q < 16 ? gate[(p * 16 + q) * O + c] : up[(p * 16 + q - 16) * O + c];
    put(dst, i, v, dtype);
  }
}

__global__ void copy_f32_kernel(const float* __restrict__ src, float* __restrict__ dst, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

inline dim3 grid_for(int64_t n) {
  int64_t b = (n + 255) / 256;
  if (b > 65536) b = 65536;
  if (b < 1) b = 1;
  return dim3((unsigned)b);
}


// Prompt embedding with the audio spliced in (model card "MOSS-Transcribe-
// preview-2B-GGUF", Architecture table, rows Prompt and Audio injection):
// output row i is table row map[i] (map[i] >= 0) or audio row -map[i] - 1.
// One workgroup per row, 16-byte stores.
__global__ void splice_kernel(const int64_t* __restrict__ map, const void* __restrict__ table,
                              int dtype, const float* __restrict__ audio, float* __restrict__ out,
                              int d) {
  const int64_t row = blockIdx.x;
  const int64_t src = map[row];
  float4* o = (float4*)(out + row * d);
  for (int c4 = threadIdx.x; c4 < d / 4; c4 += blockDim.x) {
    float4 v;
    if (src < 0) {
      v = ((const float4*)(audio + (-src - 1) * (int64_t)d))[c4];
    } else if (dtype == DT_F32) {
      v = ((const float4*)((const float*)table + src * d))[c4];
    } else {
      const uint2 u = ((const uint2*)((const char*)table + src * d * 2))[c4];
      const uint32_t w[4] = {u.x & 0xffffu, u.x >> 16, u.y & 0xffffu, u.y >> 16};
      float f[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (dtype == DT_BF16) f[e] = Elem<bf16_t>::to_f(__builtin_bit_cast(bf16_t, (uint16_t)w[e]));
        else f[e] = Elem<f16_t>::to_f(__builtin_bit_cast(f16_t, (uint16_t)w[e]));
      }
      v = make_float4(f[0], f[1], f[2], f[3]);
    }
    o[c4] = v;
  }
}

}  // namespace

hipError_t upload_words(uint32_t* dst, const uint32_t* src, int64_t n, hipStream_t s) {
  for (int64_t off = 0; off < n; off += BLOB_WORDS) {
    Blob b;
    b.n = (int32_t)((n - off) < BLOB_WORDS ? (n - off) : BLOB_WORDS);
    for (int i = 0; i < b.n; ++i) b.w[i] = src[off + i];
    hipLaunchKernelGGL(words_kernel, dim3(1), dim3(256), 0, s, dst + off, b);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_fill_i32(int* p, int v, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, grid_for(n), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

hipError_t launch_mel_norm(const MelArgs& a, int64_t tmax, hipStream_t s) {
  if (a.out_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(mel_norm_kernel, dim3((unsigned)((a.out_rows + 7) / 8)), dim3(256), 0, s, a, tmax);
  return hipGetLastError();
}

hipError_t launch_zero_pad_rows(float* out, const int32_t* cu_rows, int nseq, int64_t stride, int D,
                                hipStream_t s) {
  if (nseq == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_pad_kernel, dim3(64, nseq), dim3(256), 0, s, out, cu_rows, stride, D);
  return hipGetLastError();
}

hipError_t launch_copy_rows(const float* x, float* out, int M, int D, const int32_t* cu_rows,
                            int nseq, int64_t stride, hipStream_t s) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_rows_kernel, dim3(M), dim3(256), 0, s, x, out, M, D, cu_rows, nseq, stride);
  return hipGetLastError();
}

hipError_t launch_convert(const float* src, void* dst, int64_t rows, int64_t cols, int64_t dst_ld,
                          int64_t dst_col0, int dtype, hipStream_t s) {
  hipLaunchKernelGGL(convert_kernel, grid_for(rows * cols), dim3(256), 0, s, src, dst, rows, cols,
                     dst_ld, dst_col0, dtype);
  return hipGetLastError();
}

hipError_t launch_splice(const int64_t* map, int64_t rows, const void* table, int dtype,
                         const float* audio, float* out, int d, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(splice_kernel, dim3((unsigned)rows), dim3(256), 0, s, map, table, dtype, audio, out,
                     d);
  return hipGetLastError();
}

hipError_t launch_pack_conv(const float* w, void* dst, int C, int dtype, hipStream_t s) {
  hipLaunchKernelGGL(pack_conv_kernel, grid_for(9LL * C * C), dim3(256), 0, s, w, dst, C, dtype);
  return hipGetLastError();
}

hipError_t launch_pack_conv1d(const float* w, void* dst, int Co, int Ci, int dtype, hipStream_t s) {
  hipLaunchKernelGGL(pack_conv1d_kernel, grid_for(3LL * Co * Ci), dim3(256), 0, s, w, dst, Co, Ci,
                     dtype);
  return hipGetLastError();
}

hipError_t launch_rows_to_half(const float* src, const int64_t* row_off, const int32_t* cu, int nseq,
                               int64_t rows, int W, void* dst, int dtype, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (dtype != DT_BF16 && dtype != DT_F16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rows_to_half_kernel, dim3((unsigned)rows), dim3(128), 0, s, src, row_off, cu, nseq,
                     W, dst, dtype);
  return hipGetLastError();
}

hipError_t launch_pack_conv_out(const float* w, void* dst, int D, int C, int F, int dtype,
                                hipStream_t s) {
  hipLaunchKernelGGL(pack_conv_out_kernel, grid_for((int64_t)D * C * F), dim3(256), 0, s, w, dst, D,
                     C, F, dtype);
  return hipGetLastError();
}

hipError_t launch_pack_swiglu(const float* gate, const float* up, void* dst, int A, int O, int dtype,
                              hipStream_t s) {
  hipLaunchKernelGGL(pack_swiglu_kernel, grid_for(2LL * A * O), dim3(256), 0, s, gate, up, dst, A,
                     O, dtype);
  return hipGetLastError();
}

hipError_t launch_copy_f32(const float* src, float* dst, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_f32_kernel, grid_for(n), dim3(256), 0, s, src, dst, n);
  return hipGetLastError();
}

}  // namespace mt
