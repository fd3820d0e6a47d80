// Language-model decoder step over a KV cache (model card "MOSS-Transcribe-
// preview-2B-GGUF", Architecture table, row LLM: Qwen3-1.7B, hidden 2048,
// 16 query / 8 key-value heads of 128, SwiGLU 6144, RMSNorm, per-head Q/K-norm,
// NEOX rotary positions base 1e6, tied embeddings).
//
// A decode step reads every weight once for a handful of rows: the products
// are HBM-bound matrix-vector work.  The skinny product (at most 16 rows)
// runs on the matrix cores anyway -- one 16 x 16 x 32 step per 16 weight rows
// and 32 columns, the weight fragments loaded straight from memory -- so the
// vector units stay free and 16 rows cost what one does.  K is split across
// wavefronts so that each product keeps enough loads in flight; the partial
// sums land in fixed slots and their consumers add them in order (no
// atomics: results do not depend on timing).
//   * qkv partials -> qk_rope_kernel: sum, RMSNorm of each q / k head,
//     rotation, q kept in fp32, k and v written into the cache;
//   * attention: one workgroup per (row, key/value head, 256-key chunk), both
//     query heads of the group; chunk partials (max, sum, output) combined
//     by attn_combine_kernel;
//   * o and down partials -> add_rmsnorm_kernel: residual += sum, then the
//     next RMSNorm;
//   * gate/up (rows interleaved by 16) at full K with the SwiGLU epilogue;
//   * the head: the tied embedding table, then argmax_kernel.
#include "common.h"
#include "kernels.h"

namespace mt {

namespace {

constexpr int HD = 128;  // head_dim

__device__ __forceinline__ float wsum64(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ float wmax64(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// ---------------------------------------------------------------- skinny GEMV
// out[s][r][n] = sum_{k in split s} x[r][k] W[n][k] for r < rows (<= 16).
// One wavefront per (16 weight rows, K split); lane (g, l16) loads weight
// row n0 + l16, columns k + 8g .. k + 8g + 7 (16 bytes) and the same columns
// of x row l16.  The MFMA is issued as B = weights, A = x, so the lane holds
// out[x row l16][n0 + 4g .. n0 + 4g + 3].
// EPI 0: fp32 partials [S][rows][N]; EPI 1 (SwiGLU, S = 1): W rows
// interleaved in blocks of 16 (16 gate rows, then the 16 up rows of the same
// features), each wavefront takes 32 rows and writes SiLU(g) u as 16 bits
// to out[r][feature].
template <typename T, int EPI>
__global__ __launch_bounds__(256) void gemv16_kernel(const T* __restrict__ W, const T* __restrict__ x,
                                                     void* __restrict__ out, int rows, int N, int K,
                                                     int ksplit) {
  constexpr int TILES = EPI == 1 ? 2 : 1;  // 16-row weight tiles per wavefront
  const int lane = threadIdx.x & 63, g = lane >> 4, l16 = lane & 15;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nblk = N / (16 * TILES);
  const int s = wid / nblk, blk = wid - s * nblk;
  if (s >= ksplit) return;
  const int n0 = blk * 16 * TILES;
  const int kl = K / ksplit, k0 = s * kl;
  const bool xr = l16 < rows;
  const T* wp0 = W + (int64_t)(n0 + l16) * K + k0 + 8 * g;
  const T* wp1 = W + (int64_t)(n0 + 16 + l16) * K + k0 + 8 * g;
  const T* xp = x + (int64_t)(xr ? l16 : 0) * K + k0 + 8 * g;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  constexpr int U = 8;  // K steps in flight
  for (int k = 0; k < kl; k += 32 * U) {
    uint4 wa[U], wb[U], xa[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = k + 32 * u < kl;
      wa[u] = in ? *(const uint4*)(wp0 + k + 32 * u) : make_uint4(0, 0, 0, 0);
      if constexpr (TILES == 2) wb[u] = in ? *(const uint4*)(wp1 + k + 32 * u) : make_uint4(0, 0, 0, 0);
      xa[u] = (in && xr) ? *(const uint4*)(xp + k + 32 * u) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      mma16(acc0, wa[u], xa[u], T{});
      if constexpr (TILES == 2) mma16(acc1, wb[u], xa[u], T{});
    }
  }
  if (!xr) return;
  if constexpr (EPI == 0) {
    float* o = (float*)out + ((int64_t)s * rows + l16) * N + n0 + 4 * g;
    *(float4*)o = make_float4(acc0[0], acc0[1], acc0[2], acc0[3]);
  } else {
    // features blk * 16 + 4g .. + 3: gate in acc0, up in acc1
    T* o = (T*)out + (int64_t)l16 * (N / 2) + blk * 16 + 4 * g;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = silu_f(acc0[e]) * acc1[e];
    *(uint2*)o = make_uint2(pack2(Elem<T>::from_f(v[0]), Elem<T>::from_f(v[1])),
                            pack2(Elem<T>::from_f(v[2]), Elem<T>::from_f(v[3])));
  }
}

// --------------------------------------------------- residual add + RMSNorm
// One wavefront per row: x[r] += sum_s part[s][r] (S may be 0), then
// h[r] = x[r] / sqrt(mean(x^2) + eps) * w as T (or fp32 when T = float).
template <typename T>
__global__ __launch_bounds__(256) void add_rmsnorm_kernel(float* __restrict__ x, const float* __restrict__ part,
                                                          int S, const float* __restrict__ w, void* __restrict__ h,
                                                          int rows, int D, float eps) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  float* xr = x + (int64_t)r * D;
  float ss = 0.f;
  for (int c = lane * 4; c < D; c += 256) {
    float4 v = *(float4*)(xr + c);
    for (int s = 0; s < S; ++s) {
      const float4 p = *(const float4*)(part + ((int64_t)s * rows + r) * D + c);
      v.x += p.x;
      v.y += p.y;
      v.z += p.z;
      v.w += p.w;
    }
    if (S) *(float4*)(xr + c) = v;
    ss += (v.x * v.x + v.y * v.y) + (v.z * v.z + v.w * v.w);
  }
  const float rs = 1.0f / sqrtf(wsum64(ss) / D + eps);
  for (int c = lane * 4; c < D; c += 256) {
    const float4 v = *(const float4*)(xr + c);
    const float4 ww = *(const float4*)(w + c);
    const float y0 = v.x * rs * ww.x, y1 = v.y * rs * ww.y, y2 = v.z * rs * ww.z, y3 = v.w * rs * ww.w;
    if constexpr (sizeof(T) == 4) {
      *(float4*)((float*)h + (int64_t)r * D + c) = make_float4(y0, y1, y2, y3);
    } else {
      typedef Elem<T> E;
      *(uint2*)((T*)h + (int64_t)r * D + c) =
          make_uint2(pack2(E::from_f(y0), E::from_f(y1)), pack2(E::from_f(y2), E::from_f(y3)));
    }
  }
}

// ------------------------------------------- Q/K-norm, rotation, cache append
// One wavefront per (row, head of q | k | v): lane l holds values l and l + 64
// of the head (the rotation's pairs).  qkv: S partials [S][rows][(Hq + 2 Hkv)
// HD] (fp32).  q -> qf [rows][Hq][HD] fp32; k, v -> cache.
template <typename T>
__global__ __launch_bounds__(256) void qk_rope_kernel(DecArgs a, const float* __restrict__ qkv, int S) {
  const int lane = threadIdx.x & 63;
  const int nh = a.Hq + 2 * a.Hkv;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= a.rows * nh) return;
  const int r = item / nh, hh = item - r * nh;
  const int ld = nh * HD;
  float v0 = 0.f, v1 = 0.f;
  for (int s = 0; s < S; ++s) {
    const float* p = qkv + ((int64_t)s * a.rows + r) * ld + hh * HD;
    v0 += p[lane];
    v1 += p[lane + 64];
  }
  const int pos = a.pos[r], sq = a.seq[r];
  if (hh < a.Hq + a.Hkv) {
    const float* nw = hh < a.Hq ? a.q_norm : a.k_norm;
    const float rs = 1.0f / sqrtf(wsum64(v0 * v0 + v1 * v1) / HD + a.eps);
    const float a0 = v0 * rs * nw[lane], a1 = v1 * rs * nw[lane + 64];
    // angle pos * base^(-lane / 64), in double then reduced to [-pi, pi]
    double ang = (double)pos * exp(-(double)lane * a.log_base / 64.0);
    ang -= 6.283185307179586 * rint(ang * 0.15915494309189535);
    float sn, cs;
    sincosf((float)ang, &sn, &cs);
    v0 = a0 * cs - a1 * sn;
    v1 = a1 * cs + a0 * sn;
  }
  if (hh < a.Hq) {
    float* q = a.qf + ((int64_t)r * a.Hq + hh) * HD;
    q[lane] = v0;
    q[lane + 64] = v1;
  } else {
    const int isv = hh >= a.Hq + a.Hkv;
    const int kh = hh - a.Hq - isv * a.Hkv;
    T* c = (T*)a.cache + ((((int64_t)a.layer * a.max_seqs + sq) * 2 + isv) * a.Hkv + kh) * a.max_pos * HD +
           (int64_t)pos * HD;
    c[lane] = Elem<T>::from_f(v0);
    c[lane + 64] = Elem<T>::from_f(v1);
  }
}

// ------------------------------------------------------------ attention
// One workgroup per (chunk item, key/value head): item = (row, chunk of 256
// keys) from the host's table; both query heads 2 kh, 2 kh + 1 (groups of
// Hq / Hkv consecutive query heads; the kernel handles groups of 2).
//   scores: thread t takes key c0 + t (keys past the row's position drop
//   out), dot with both heads' q (fp32, LDS); chunk max / sum per head;
//   output: thread (head, d) sums p V over the chunk's keys.
template <typename T>
__global__ __launch_bounds__(256) void attn_dec_kernel(DecArgs a) {
  __shared__ float qs[2][HD];
  __shared__ float ps[2][256];
  __shared__ float red[2][8];
  const int it = blockIdx.x, kh = blockIdx.y, t = threadIdx.x;
  const int r = a.items[2 * it], c0 = a.items[2 * it + 1] * 256;
  const int pos = a.pos[r], sq = a.seq[r];
  const int nk = min(256, pos + 1 - c0);  // keys of this chunk (>= 1)
  const T* Kc = (const T*)a.cache + ((((int64_t)a.layer * a.max_seqs + sq) * 2 + 0) * a.Hkv + kh) * a.max_pos * HD;
  const T* Vc = Kc + (int64_t)a.Hkv * a.max_pos * HD;
  {
    const int h = t >> 7, d = t & 127;
    qs[h][d] = a.qf[((int64_t)r * a.Hq + 2 * kh + h) * HD + d];
  }
  __syncthreads();
  const float scale = 0.08838834764831845f;  // 1 / sqrt(128)
  float s0 = -INFINITY, s1 = -INFINITY;
  if (t < nk) {
    const uint4* kr = (const uint4*)(Kc + (int64_t)(c0 + t) * HD);
    float d0 = 0.f, d1 = 0.f;
#pragma unroll 4
    for (int c = 0; c < HD / 8; ++c) {
      const uint4 u = kr[c];
      const T* e = (const T*)&u;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float kv = Elem<T>::to_f(e[j]);
        d0 = fmaf(kv, qs[0][8 * c + j], d0);
        d1 = fmaf(kv, qs[1][8 * c + j], d1);
      }
    }
    s0 = d0 * scale;
    s1 = d1 * scale;
  }
  // chunk max per head
  const int wv = t >> 6;
  float m0 = wmax64(s0), m1 = wmax64(s1);
  if ((t & 63) == 0) {
    red[0][wv] = m0;
    red[1][wv] = m1;
  }
  __syncthreads();
  m0 = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  m1 = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
  const float p0 = t < nk ? __expf(s0 - m0) : 0.f, p1 = t < nk ? __expf(s1 - m1) : 0.f;
  ps[0][t] = p0;
  ps[1][t] = p1;
  const float l0 = wsum64(p0), l1 = wsum64(p1);
  __syncthreads();  // red (max) read by all before it is reused
  if ((t & 63) == 0) {
    red[0][4 + wv] = l0;
    red[1][4 + wv] = l1;
  }
  __syncthreads();
  // output: thread (h, d)
  const int h = t >> 7, d = t & 127;
  float o = 0.f;
  const T* vp = Vc + (int64_t)c0 * HD + d;
  const float* pp = ps[h];
  for (int k = 0; k < nk; ++k) o = fmaf(pp[k], Elem<T>::to_f(vp[(int64_t)k * HD]), o);
  // partial: [item][kh][h] -> (m, l) and o[HD]
  const int64_t slot = ((int64_t)it * a.Hkv + kh) * 2 + h;
  a.part_o[slot * HD + d] = o;
  if (d == 0) {
    a.part_ml[2 * slot] = h ? m1 : m0;
    a.part_ml[2 * slot + 1] = h ? (red[1][4] + red[1][5] + red[1][6] + red[1][7])
                                : (red[0][4] + red[0][5] + red[0][6] + red[0][7]);
  }
}

// One workgroup of 128 threads per (row, query head): combine the row's chunk
// partials (chunks first_item[r] .. first_item[r + 1] - 1) into o16.
template <typename T>
__global__ __launch_bounds__(128) void attn_combine_kernel(DecArgs a) {
  const int r = blockIdx.x, hq = blockIdx.y, d = threadIdx.x;
  const int kh = hq >> 1, h = hq & 1;
  const int i0 = a.first_item[r], i1 = a.first_item[r + 1];
  float M = -INFINITY;
  for (int i = i0; i < i1; ++i) M = fmaxf(M, a.part_ml[2 * (((int64_t)i * a.Hkv + kh) * 2 + h)]);
  float L = 0.f, o = 0.f;
  for (int i = i0; i < i1; ++i) {
    const int64_t slot = ((int64_t)i * a.Hkv + kh) * 2 + h;
    const float f = __expf(a.part_ml[2 * slot] - M);
    L += a.part_ml[2 * slot + 1] * f;
    o += a.part_o[slot * HD + d] * f;
  }
  ((T*)a.o16)[((int64_t)r * a.Hq + hq) * HD + d] = Elem<T>::from_f(o / L);
}

// ------------------------------------------------------------- argmax
// One workgroup per row: the first index of the largest logit.
__global__ __launch_bounds__(256) void argmax_kernel(const float* __restrict__ logits, int V, int32_t* next) {
  __shared__ float bv[4];
  __shared__ int bi[4];
  const int r = blockIdx.x, t = threadIdx.x;
  const float* l = logits + (int64_t)r * V;
  float best = -INFINITY;
  int idx = 0x7fffffff;
  for (int i = t; i < V; i += 256) {
    const float v = l[i];
    if (v > best) {  // increasing i: the first maximum of this thread's subset
      best = v;
      idx = i;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(best, off, 64);
    const int oi = __shfl_xor(idx, off, 64);
    if (ov > best || (ov == best && oi < idx)) {
      best = ov;
      idx = oi;
    }
  }
  if ((t & 63) == 0) {
    bv[t >> 6] = best;
    bi[t >> 6] = idx;
  }
  __syncthreads();
  if (t == 0) {
    for (int w = 1; w < 4; ++w)
      if (bv[w] > best || (bv[w] == best && bi[w] < idx)) {
        best = bv[w];
        idx = bi[w];
      }
    next[r] = idx;
  }
}

}  // namespace

hipError_t launch_gemv16(const void* W, const void* x, void* out, int rows, int N, int K, int ksplit, bool swiglu,
                         int dtype, hipStream_t s) {
  if (rows < 1 || rows > 16 || K % (32 * ksplit) || N % (swiglu ? 32 : 16) || (swiglu && ksplit != 1))
    return hipErrorInvalidValue;
  const int waves = (N / (swiglu ? 32 : 16)) * ksplit;
  const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
  if (dtype == DT_BF16) {
    if (swiglu) hipLaunchKernelGGL((gemv16_kernel<bf16_t, 1>), grid, block, 0, s, (const bf16_t*)W, (const bf16_t*)x, out, rows, N, K, 1);
    else hipLaunchKernelGGL((gemv16_kernel<bf16_t, 0>), grid, block, 0, s, (const bf16_t*)W, (const bf16_t*)x, out, rows, N, K, ksplit);
  } else if (dtype == DT_F16) {
    if (swiglu) hipLaunchKernelGGL((gemv16_kernel<f16_t, 1>), grid, block, 0, s, (const f16_t*)W, (const f16_t*)x, out, rows, N, K, 1);
    else hipLaunchKernelGGL((gemv16_kernel<f16_t, 0>), grid, block, 0, s, (const f16_t*)W, (const f16_t*)x, out, rows, N, K, ksplit);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_add_rmsnorm(float* x, const float* part, int S, const float* w, void* h, int rows, int D, float eps,
                              int dtype, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (D % 256) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  if (dtype == DT_BF16) hipLaunchKernelGGL(add_rmsnorm_kernel<bf16_t>, grid, block, 0, s, x, part, S, w, h, rows, D, eps);
  else if (dtype == DT_F16) hipLaunchKernelGGL(add_rmsnorm_kernel<f16_t>, grid, block, 0, s, x, part, S, w, h, rows, D, eps);
  else hipLaunchKernelGGL(add_rmsnorm_kernel<float>, grid, block, 0, s, x, part, S, w, h, rows, D, eps);
  return hipGetLastError();
}

hipError_t launch_qk_rope(const DecArgs& a, const float* qkv, int S, int dtype, hipStream_t s) {
  const int items = a.rows * (a.Hq + 2 * a.Hkv);
  const dim3 grid((unsigned)((items + 3) / 4)), block(256);
  if (dtype == DT_BF16) hipLaunchKernelGGL(qk_rope_kernel<bf16_t>, grid, block, 0, s, a, qkv, S);
  else if (dtype == DT_F16) hipLaunchKernelGGL(qk_rope_kernel<f16_t>, grid, block, 0, s, a, qkv, S);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_attn_dec(const DecArgs& a, int n_items, int dtype, hipStream_t s) {
  if (a.Hq != 2 * a.Hkv) return hipErrorInvalidValue;
  const dim3 grid((unsigned)n_items, (unsigned)a.Hkv);
  if (dtype == DT_BF16) {
    hipLaunchKernelGGL(attn_dec_kernel<bf16_t>, grid, dim3(256), 0, s, a);
    hipLaunchKernelGGL(attn_combine_kernel<bf16_t>, dim3((unsigned)a.rows, (unsigned)a.Hq), dim3(128), 0, s, a);
  } else if (dtype == DT_F16) {
    hipLaunchKernelGGL(attn_dec_kernel<f16_t>, grid, dim3(256), 0, s, a);
    hipLaunchKernelGGL(attn_combine_kernel<f16_t>, dim3((unsigned)a.rows, (unsigned)a.Hq), dim3(128), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_argmax(const float* logits, int rows, int V, int32_t* next, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(argmax_kernel, dim3((unsigned)rows), dim3(256), 0, s, logits, V, next);
  return hipGetLastError();
}

}  // namespace mt
