// Language-model decoder step over a KV cache (model card "MOSS-Transcribe-
// preview-2B-GGUF", Architecture table, row LLM: Qwen3-1.7B, hidden 2048,
// 16 query / 8 key-value heads of 128, SwiGLU 6144, RMSNorm, per-head Q/K-norm,
// NEOX rotary positions base 1e6, tied embeddings).
//
// A decode step reads every weight once for a handful of rows: the products
// are HBM-bound matrix-vector work.  The skinny product (at most 64 rows)
// runs on the matrix cores anyway -- one 16 x 16 x 32 step per 16 weight rows,
// 32 columns and 16 rows, the weight fragments loaded straight from memory
// once for up to four row tiles -- so the vector units stay free and 64 rows
// cost little more than one.  K is split across
// wavefronts so that each product keeps enough loads in flight; the partial
// sums land in fixed slots and their consumers add them in order (no
// atomics: results do not depend on timing).
//   * qkv partials -> qk_rope_kernel: sum, RMSNorm of each q / k head,
//     rotation, q kept in fp32, k and v written into the cache (calls with
//     one row per sequence do this inside the attention kernel instead);
//   * attention: one workgroup per (row, key/value head, 64-key chunk), both
//     query heads of the group; chunk partials (max, sum, output) combined
//     by attn_combine_kernel (at most GEMV_FUSE_ROWS rows: inside the output
//     projection, gemv16x_kernel);
//   * o and down partials -> add_rmsnorm_kernel: residual += sum, then the
//     next RMSNorm;
//   * gate/up partials (rows interleaved by 16) -> swiglu_kernel (at most
//     GEMV_FUSE_ROWS rows: inside the down projection);
//   * the head: the tied embedding table, then a two-pass argmax.
// Small kernels issue every load of their rows before the first use: at a
// few rows per step, memory latency rather than bandwidth sets their time.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace mt {

namespace {

constexpr int HD = 128;  // head_dim

__device__ __forceinline__ float wsum64(float v) { return wave_sum64(v); }
__device__ __forceinline__ float wmax64(float v) { return wave_max64(v); }

// ---------------------------------------------------------------- skinny GEMV
// out[s][r][n] = sum_{k in split s} x[r][k] W[n][k] for r < rows (<= 64).
// One wavefront per (16 weight rows, K split); lane (g, l16) loads weight
// row n0 + l16, columns k + 8g .. k + 8g + 7 (16 bytes) and the same columns
// of x rows 16 q + l16.  The MFMA is issued as B = weights, A = x, so the
// lane holds out[x row 16 q + l16][n0 + 4g .. n0 + 4g + 3].
// Output: fp32 partial sums [S][rows][N].  U K steps are loaded before the
// first MFMA: U covers a wavefront's whole K range (one round trip to
// memory) up to 32 steps.  RT tiles of 16 x rows (rows <= 16 RT) share each
// weight fragment: up to 64 rows cost about what 16 do.
template <typename T, int U, int RT>
__global__ __launch_bounds__(256) void gemv16_kernel(const T* __restrict__ W, const T* __restrict__ x,
                                                     float* __restrict__ out, int rows, int N, int K, int ksplit) {
  const int lane = threadIdx.x & 63, g = lane >> 4, l16 = lane & 15;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nblk = N / 16;
  const int s = wid / nblk, blk = wid - s * nblk;
  if (s >= ksplit) return;
  const int n0 = blk * 16;
  const int kl = K / ksplit, k0 = s * kl;
  const T* wp = W + (int64_t)(n0 + l16) * K + k0 + 8 * g;
  const T* xp[RT];
  bool xr[RT];
#pragma unroll
  for (int q = 0; q < RT; ++q) {
    xr[q] = 16 * q + l16 < rows;
    xp[q] = x + (int64_t)(xr[q] ? 16 * q + l16 : 0) * K + k0 + 8 * g;
  }
  f32x4 acc[RT];
#pragma unroll
  for (int q = 0; q < RT; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < kl; k += 32 * U) {
    uint4 wa[U], xa[RT][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = k + 32 * u < kl;
      wa[u] = in ? *(const uint4*)(wp + k + 32 * u) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int q = 0; q < RT; ++q)
        xa[q][u] = (in && xr[q]) ? *(const uint4*)(xp[q] + k + 32 * u) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int q = 0; q < RT; ++q) mma16(acc[q], wa[u], xa[q][u], T{});
  }
#pragma unroll
  for (int q = 0; q < RT; ++q) {
    if (!xr[q]) continue;
    float* o = out + ((int64_t)s * rows + 16 * q + l16) * N + n0 + 4 * g;
    *(float4*)o = make_float4(acc[q][0], acc[q][1], acc[q][2], acc[q][3]);
  }
}

// --------------------------------------------------- residual add + RMSNorm
// One workgroup per row: x[r] += sum_s part[s][r] (S <= 8, may be 0), then
// h[r] = x[r] / sqrt(mean(x^2) + eps) * w as T (fp32 when T = float).  A row
// is 8 KB: latency, not bandwidth, sets the time, so every load of the row
// (residual, partials, norm weight) is issued before the first use, from
// clamped addresses (chunks past the row's end reload chunk 0 and are
// ignored; S is a template parameter): guarded loads became branches that
// waited for each load.
constexpr int MAXS = 8;
template <typename T, int S>
__global__ __launch_bounds__(256) void add_rmsnorm_kernel(float* __restrict__ x, const float* __restrict__ part,
                                                          const float* __restrict__ w, void* __restrict__ h,
                                                          int rows, int D, float eps) {
  __shared__ float red[4];
  constexpr int MC = 4;  // float4 chunks per thread: D <= 4096
  const int r = blockIdx.x, t = threadIdx.x;
  float* xr = x + (int64_t)r * D;
  const int nc = D / 4;
  float4 v[MC], ww[MC], p[MC][S > 0 ? S : 1];
#pragma unroll
  for (int i = 0; i < MC; ++i) {
    const int c = t + 256 * i < nc ? t + 256 * i : 0;
    v[i] = ((const float4*)xr)[c];
#pragma unroll
    for (int s2 = 0; s2 < S; ++s2) p[i][s2] = ((const float4*)(part + ((int64_t)s2 * rows + r) * D))[c];
    ww[i] = ((const float4*)w)[c];
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < MC; ++i) {
    const int c = t + 256 * i;
    if (c < nc) {
#pragma unroll
      for (int s2 = 0; s2 < S; ++s2) {
        v[i].x += p[i][s2].x;
        v[i].y += p[i][s2].y;
        v[i].z += p[i][s2].z;
        v[i].w += p[i][s2].w;
      }
      if (S) ((float4*)xr)[c] = v[i];
      ss += (v[i].x * v[i].x + v[i].y * v[i].y) + (v[i].z * v[i].z + v[i].w * v[i].w);
    }
  }
  ss = wsum64(ss);
  if ((t & 63) == 0) red[t >> 6] = ss;
  __syncthreads();
  const float rs = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / D + eps);
#pragma unroll
  for (int i = 0; i < MC; ++i) {
    const int c = t + 256 * i;
    if (c < nc) {
      const float4 wv = ww[i];
      const float y0 = v[i].x * rs * wv.x, y1 = v[i].y * rs * wv.y, y2 = v[i].z * rs * wv.z, y3 = v[i].w * rs * wv.w;
      if constexpr (sizeof(T) == 4) {
        ((float4*)((float*)h + (int64_t)r * D))[c] = make_float4(y0, y1, y2, y3);
      } else {
        ((uint2*)((T*)h + (int64_t)r * D))[c] = make_uint2(pack2f<T>(y0, y1), pack2f<T>(y2, y3));
      }
    }
  }
}

// SwiGLU of the gate/up partial sums: act[r][f] = SiLU(sum g) * (sum u), gate
// row 32 (f / 16) + f % 16 and up row 32 (f / 16) + 16 + f % 16 of the [S][rows]
// [2F] partials.  One function for the standalone pass and for the fused
// load of the down projection, so that both give the same bits.
template <typename T>
__device__ __forceinline__ T swiglu_one(const float* __restrict__ part, int S, int rows, int F, int r, int f) {
  const int gi = 32 * (f >> 4) + (f & 15);
  float gp[MAXS], up[MAXS];
#pragma unroll
  for (int s2 = 0; s2 < MAXS; ++s2)
    if (s2 < S) {
      const float* p = part + ((int64_t)s2 * rows + r) * 2 * F;
      gp[s2] = p[gi];
      up[s2] = p[gi + 16];
    }
  float g = 0.f, u = 0.f;
#pragma unroll
  for (int s2 = 0; s2 < MAXS; ++s2)
    if (s2 < S) {
      g += gp[s2];
      u += up[s2];
    }
  return Elem<T>::from_f(silu_f(g) * u);
}

template <typename T>
__global__ __launch_bounds__(256) void swiglu_kernel(const float* __restrict__ part, int S, T* __restrict__ act,
                                                     int rows, int F) {
  const int r = blockIdx.y, f = blockIdx.x * 256 + threadIdx.x;
  if (f >= F) return;
  act[(int64_t)r * F + f] = swiglu_one<T>(part, S, rows, F, r, f);
}

// ------------------------------------------- Q/K-norm, rotation, cache append
// One wavefront per (row, head of q | k | v): lane l holds values l and l + 64
// of the head (the rotation's pairs).  qkv: S partials [S][rows][(Hq + 2 Hkv)
// HD] (fp32).  q -> qf [rows][Hq][HD] fp32; k, v -> cache.
// One head of one row from its S fp32 partials: lane l gets values l and
// l + 64.  q and k heads (rot): RMSNorm over the head with weights (w0, w1),
// then the rotation at position pos (value j paired with j + 64, angle
// pos * base^(-j / 64)).  Shared by the standalone pass and the attention
// kernel that computes its own queries, so both give the same bits.
template <int S>
__device__ __forceinline__ void qk_head(const DecArgs& a, const float (&p0)[S], const float (&p1)[S], float w0,
                                        float w1, bool rot, int pos, int lane, float& v0, float& v1) {
  v0 = 0.f;
  v1 = 0.f;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    v0 += p0[s];
    v1 += p1[s];
  }
  if (rot) {
    const float rs = 1.0f / sqrtf(wsum64(v0 * v0 + v1 * v1) / HD + a.eps);
    const float a0 = v0 * rs * w0, a1 = v1 * rs * w1;
    // angle pos * base^(-lane / 64), in double then reduced to [-pi, pi]
    double ang = (double)pos * exp(-(double)lane * a.log_base / 64.0);
    ang -= 6.283185307179586 * rint(ang * 0.15915494309189535);
    float sn, cs;
    sincosf((float)ang, &sn, &cs);
    v0 = a0 * cs - a1 * sn;
    v1 = a1 * cs + a0 * sn;
  }
}

template <typename T, int S>
__global__ __launch_bounds__(256) void qk_rope_kernel(DecArgs a, const float* __restrict__ qkv) {
  const int lane = threadIdx.x & 63;
  const int nh = a.Hq + 2 * a.Hkv;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= a.rows * nh) return;
  const int r = item / nh, hh = item - r * nh;
  const int ld = nh * HD;
  // every load first (S is a template parameter: no guarded loads)
  float p0[S], p1[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const float* p = qkv + ((int64_t)s * a.rows + r) * ld + hh * HD;
    p0[s] = p[lane];
    p1[s] = p[lane + 64];
  }
  const float* nw = hh < a.Hq ? a.q_norm : a.k_norm;
  const float w0 = nw[lane], w1 = nw[lane + 64];
  const int pos = a.pos[r], sq = a.seq[r];
  float v0, v1;
  qk_head<S>(a, p0, p1, w0, w1, hh < a.Hq + a.Hkv, pos, lane, v0, v1);
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
// One workgroup per (chunk item, key/value head): item = (row, chunk of 64
// keys) from the host's table; both query heads 2 kh, 2 kh + 1 of the group.
//   scores: four threads per key, 32 values each (four 16-byte loads),
//   reduced by shuffles; keys past the row's position drop out;
//   output: thread (key group kg, 8 values dg) sums p V over keys kg, kg +
//   16, kg + 32, kg + 48 with 16-byte loads, then the 16 key groups are
//   added through LDS.
constexpr int CHUNK = 64;
//
// S > 0: the calls with one row per sequence.  The workgroup computes its two
// query heads itself from the S qkv partials (qkv, the standalone pass's
// helper), and the workgroup whose chunk holds the row's own position also
// the new key and value: it writes them into the cache for later steps and
// uses a copy in LDS (the same 16-bit values) for that key, since the
// chunk's cache loads were issued before they were written.  No other row
// of the call reads this sequence's cache, so the standalone pass can go.
template <typename T, int S>
__global__ __launch_bounds__(256) void attn_dec_kernel(DecArgs a, const float* __restrict__ qkv) {
  __shared__ float qs[2][HD];
  __shared__ float ps[2][CHUNK];
  __shared__ float red[2][8];
  __shared__ float ro[16][2][HD];
  __shared__ __align__(16) T kvn[2][HD];  // S > 0: the new key and value (read as 16-byte vectors)
  const int it = blockIdx.x, kh = blockIdx.y, t = threadIdx.x;
  const int r = a.items[2 * it], c0 = a.items[2 * it + 1] * CHUNK;
  const int pos = a.pos[r], sq = a.seq[r];
  const int nk = min(CHUNK, pos + 1 - c0);  // keys of this chunk (>= 1)
  const bool own = pos - c0 < CHUNK;        // the chunk holds position pos
  const T* Kc = (const T*)a.cache + ((((int64_t)a.layer * a.max_seqs + sq) * 2 + 0) * a.Hkv + kh) * a.max_pos * HD;
  const T* Vc = Kc + (int64_t)a.Hkv * a.max_pos * HD;
  // Every global load of the workgroup -- the queries (or their partials),
  // then its K and V fragments, in the order of use (loads complete in
  // order) -- is issued before the first wait: three dependent round trips
  // to memory would otherwise set the time of this small kernel.
  const int kk = t >> 2, part = t & 3;
  const int kg = t >> 4, dg = t & 15;
  const int wv = t >> 6, lane = t & 63;
  [[maybe_unused]] float qv = 0.f;
  [[maybe_unused]] float pq0[S > 0 ? S : 1], pq1[S > 0 ? S : 1];
  [[maybe_unused]] float w0 = 0.f, w1 = 0.f;
  if constexpr (S == 0) {
    qv = a.qf[((int64_t)r * a.Hq + 2 * kh + (t >> 7)) * HD + (t & 127)];
  } else {
    // wavefronts 0, 1: query heads 2 kh, 2 kh + 1; 2: key head kh; 3: value
    // head kh (the last two only in the chunk that holds pos)
    const int nh = a.Hq + 2 * a.Hkv, ld = nh * HD;
    const int hh = wv < 2 ? 2 * kh + wv : a.Hq + (wv - 2) * a.Hkv + kh;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const float* pp = qkv + ((int64_t)s * a.rows + r) * ld + hh * HD;
      pq0[s] = pp[lane];
      pq1[s] = pp[lane + 64];
    }
    const float* nw = wv < 2 ? a.q_norm : a.k_norm;
    w0 = nw[lane];
    w1 = nw[lane + 64];
  }
  // Keys past the chunk's end load key c0 (always present) and are zeroed
  // afterwards: guarded loads became branches that waited for each load.
  uint4 u[4], vv[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) u[c] = ((const uint4*)(Kc + (int64_t)(c0 + (kk < nk ? kk : 0)) * HD + part * 32))[c];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = kg + 16 * i;
    vv[i] = *(const uint4*)(Vc + (int64_t)(c0 + (k < nk ? k : 0)) * HD + dg * 8);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (kk >= nk) u[i] = make_uint4(0, 0, 0, 0);
    if (kg + 16 * i >= nk) vv[i] = make_uint4(0, 0, 0, 0);
  }
  if constexpr (S == 0) {
    qs[t >> 7][t & 127] = qv;
  } else {
    if (wv < 2 || own) {
      float v0, v1;
      qk_head<S>(a, pq0, pq1, w0, w1, wv < 3, pos, lane, v0, v1);
      if (wv < 2) {
        qs[wv][lane] = v0;
        qs[wv][lane + 64] = v1;
      } else {
        const T e0 = Elem<T>::from_f(v0), e1 = Elem<T>::from_f(v1);
        kvn[wv - 2][lane] = e0;
        kvn[wv - 2][lane + 64] = e1;
        T* c = (T*)(wv == 2 ? Kc : Vc) + (int64_t)pos * HD;
        c[lane] = e0;
        c[lane + 64] = e1;
      }
    }
  }
  __syncthreads();
  if constexpr (S > 0) {
    // the new key and value replace what the chunk's loads found at pos
    if (own && c0 + kk == pos) {
#pragma unroll
      for (int c = 0; c < 4; ++c) u[c] = *(const uint4*)&kvn[0][part * 32 + 8 * c];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (own && c0 + kg + 16 * i == pos) vv[i] = *(const uint4*)&kvn[1][dg * 8];
  }
  float d0 = 0.f, d1 = 0.f;
  if (kk < nk) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const T* e = (const T*)&u[c];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float kv = Elem<T>::to_f(e[j]);
        d0 = fmaf(kv, qs[0][part * 32 + 8 * c + j], d0);
        d1 = fmaf(kv, qs[1][part * 32 + 8 * c + j], d1);
      }
    }
  }
  // sum over the key's four threads (a quad): DPP quad permutations
  // [1, 0, 3, 2] and [2, 3, 0, 1] give the xor-1 and xor-2 partners
  d0 += dpp_f<0xB1>(d0);
  d1 += dpp_f<0xB1>(d1);
  d0 += dpp_f<0x4E>(d0);
  d1 += dpp_f<0x4E>(d1);
  const float scale = 0.08838834764831845f;  // 1 / sqrt(128)
  const float s0 = kk < nk ? d0 * scale : -INFINITY, s1 = kk < nk ? d1 * scale : -INFINITY;
  float m0 = wmax64(s0), m1 = wmax64(s1);
  if ((t & 63) == 0) {
    red[0][wv] = m0;
    red[1][wv] = m1;
  }
  __syncthreads();
  m0 = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  m1 = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
  const float p0 = kk < nk ? __expf(s0 - m0) : 0.f, p1 = kk < nk ? __expf(s1 - m1) : 0.f;
  if (part == 0) {
    ps[0][kk] = p0;
    ps[1][kk] = p1;
  }
  // each key counted once (part 0 of its four threads)
  const float l0 = wsum64(part == 0 ? p0 : 0.f), l1 = wsum64(part == 0 ? p1 : 0.f);
  __syncthreads();
  if ((t & 63) == 0) {
    red[0][4 + wv] = l0;
    red[1][4 + wv] = l1;
  }
  float o0[8], o1[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o0[j] = o1[j] = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = kg + 16 * i;
    const float q0 = k < nk ? ps[0][k] : 0.f, q1 = k < nk ? ps[1][k] : 0.f;
    const T* e = (const T*)&vv[i];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v = Elem<T>::to_f(e[j]);
      o0[j] = fmaf(q0, v, o0[j]);
      o1[j] = fmaf(q1, v, o1[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    ro[kg][0][dg * 8 + j] = o0[j];
    ro[kg][1][dg * 8 + j] = o1[j];
  }
  __syncthreads();
  const int h = t >> 7, d = t & 127;
  float o = 0.f;
#pragma unroll
  for (int g2 = 0; g2 < 16; ++g2) o += ro[g2][h][d];
  // partial: [item][kh][h] -> (m, l) and o[HD]
  const int64_t slot = ((int64_t)it * a.Hkv + kh) * 2 + h;
  a.part_o[slot * HD + d] = o;
  if (d == 0) {
    a.part_ml[2 * slot] = h ? m1 : m0;
    a.part_ml[2 * slot + 1] = h ? (red[1][4] + red[1][5] + red[1][6] + red[1][7])
                                : (red[0][4] + red[0][5] + red[0][6] + red[0][7]);
  }
}

// Combining a row's chunk partials for query head hq (kv head hq / 2, head
// h = hq % 2 of the group; chunks first_item[r] .. first_item[r + 1] - 1):
// M = max m_i, f_i = exp(m_i - M), L = sum l_i f_i, o[d] = sum o_i[d] f_i,
// out = o / L.  These helpers are shared by the standalone combine and the
// fused load of the output projection, so that both give the same bits.
__device__ __forceinline__ int64_t combine_slot(const DecArgs& a, int i, int hq) {
  return ((int64_t)i * a.Hkv + (hq >> 1)) * 2 + (hq & 1);
}
__device__ __forceinline__ float combine_max(const DecArgs& a, int r, int hq) {
  float M = -INFINITY;
#pragma unroll 8
  for (int i = a.first_item[r]; i < a.first_item[r + 1]; ++i) M = fmaxf(M, a.part_ml[2 * combine_slot(a, i, hq)]);
  return M;
}
__device__ __forceinline__ float combine_f(const DecArgs& a, int i, int hq, float M) {
  return __expf(a.part_ml[2 * combine_slot(a, i, hq)] - M);
}

// One workgroup of 128 threads per (row, query head).
template <typename T>
__global__ __launch_bounds__(128) void attn_combine_kernel(DecArgs a) {
  const int r = blockIdx.x, hq = blockIdx.y, d = threadIdx.x;
  const float M = combine_max(a, r, hq);
  float L = 0.f, o = 0.f;
#pragma unroll 8
  for (int i = a.first_item[r]; i < a.first_item[r + 1]; ++i) {
    const int64_t slot = combine_slot(a, i, hq);
    const float f = combine_f(a, i, hq, M);
    L += a.part_ml[2 * slot + 1] * f;
    o += a.part_o[slot * HD + d] * f;
  }
  ((T*)a.o16)[((int64_t)r * a.Hq + hq) * HD + d] = Elem<T>::from_f(o / L);
}

// ------------------------------------------ skinny GEMV with a computed x
// The same product for at most GEMV_FUSE_ROWS rows whose x is computed from
// its producer's partials instead of being stored first: XM = 1, SwiGLU of
// the gate/up partials (src, S splits) for the down projection; XM = 2, the
// attention chunk partials combined for the output projection.  The four
// wavefronts of a workgroup share one K range (N is a multiple of 64): the
// workgroup computes x[rows][k0, k0 + kl) once into LDS with the standalone
// passes' helpers (so the bits are the same), then each wavefront reads its
// fragments from there.  This saves the producer's launch; the price, every
// workgroup of a split recomputing the same x, stays small at a few rows.
// The weight fragments of the whole K range (kl <= 32 U) are requested
// first, so their latency covers the x computation.
//   dynamic LDS: x [rows][kl] (16-bit), then for XM = 2 per (row, head) of
//   the range 2 + 3 cmax floats: L, unused, f_i and (m_i, l_i) of each chunk.
template <typename T, int U, int XM>
__global__ __launch_bounds__(256) void gemv16x_kernel(const T* __restrict__ W, const float* __restrict__ src, int S,
                                                      DecArgs a, int cmax, float* __restrict__ out, int rows, int N,
                                                      int K, int ksplit) {
  extern __shared__ uint4 smem_x[];
  const int lane = threadIdx.x & 63, g = lane >> 4, l16 = lane & 15;
  const int nblk = N / 16;
  const int s = blockIdx.x * 4 / nblk, blk = blockIdx.x * 4 + (threadIdx.x >> 6) - s * nblk;
  const int kl = K / ksplit, k0 = s * kl;
  const int n0 = blk * 16;
  const T* wp = W + (int64_t)(n0 + l16) * K + k0 + 8 * g;
  uint4 wa[U];
#pragma unroll
  for (int u = 0; u < U; ++u) wa[u] = 32 * u < kl ? *(const uint4*)(wp + 32 * u) : make_uint4(0, 0, 0, 0);

  T* xs = (T*)smem_x;
  if constexpr (XM == 1) {
    for (int i = threadIdx.x; i < rows * kl; i += 256) {
      const int r = i / kl;
      xs[i] = swiglu_one<T>(src, S, rows, K, r, k0 + i - r * kl);
    }
  } else {
    // Every chunk's (max, sum) of the workgroup's (row, head) pairs is
    // fetched at once (a loop per pair would wait for one load at a time),
    // then one thread per pair forms M, the weights f_i and L from LDS, in
    // the standalone combine's order.
    const int nhl = kl / HD, h0 = k0 / HD;  // query heads of this K range
    const int cs = 2 + 3 * cmax;            // floats per pair: L, -, f[cmax], (m, l)[cmax]
    float* cw = (float*)(xs + rows * kl);   // [rows][nhl][cs]
    for (int idx = threadIdx.x; idx < rows * nhl * cmax; idx += 256) {
      const int pair = idx / cmax, i = idx - pair * cmax, r = pair / nhl;
      const int i0 = a.first_item[r];
      if (i0 + i < a.first_item[r + 1]) {
        const int64_t slot = combine_slot(a, i0 + i, h0 + pair % nhl);
        float* c = cw + pair * cs + 2 + cmax + 2 * i;
        c[0] = a.part_ml[2 * slot];
        c[1] = a.part_ml[2 * slot + 1];
      }
    }
    __syncthreads();
    if (threadIdx.x < rows * nhl) {
      const int r = threadIdx.x / nhl;
      float* c = cw + threadIdx.x * cs;
      const float* ml = c + 2 + cmax;
      const int nch = a.first_item[r + 1] - a.first_item[r];
      float M = -INFINITY;
      for (int i = 0; i < nch; ++i) M = fmaxf(M, ml[2 * i]);
      float L = 0.f;
      for (int i = 0; i < nch; ++i) {
        const float f = __expf(ml[2 * i] - M);
        L += ml[2 * i + 1] * f;
        c[2 + i] = f;
      }
      c[0] = L;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < rows * kl; i += 256) {
      const int r = i / kl, k = k0 + i - r * kl, hq = k / HD, d = k % HD;
      const float* c = cw + (r * nhl + hq - h0) * cs;
      const int i0 = a.first_item[r], nch = a.first_item[r + 1] - i0;
      float o = 0.f;
#pragma unroll 8
      for (int j = 0; j < nch; ++j) o += a.part_o[combine_slot(a, i0 + j, hq) * HD + d] * c[2 + j];
      xs[i] = Elem<T>::from_f(o / c[0]);
    }
  }
  __syncthreads();

  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  const bool xr = l16 < rows;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint4 xa = (xr && 32 * u < kl) ? *(const uint4*)(xs + l16 * kl + 32 * u + 8 * g) : make_uint4(0, 0, 0, 0);
    mma16(acc, wa[u], xa, T{});
  }
  if (xr) *(float4*)(out + ((int64_t)s * rows + l16) * N + n0 + 4 * g) = make_float4(acc[0], acc[1], acc[2], acc[3]);
}

// ------------------------------------------------------------- argmax
// Two passes: workgroup (b, r) reduces slice b of row r's logits to (value,
// first index); then one wavefront per row reduces the AMB slices.  Ties go
// to the lower index in both passes: the result is the row's first maximum.
constexpr int AMB = 64;
__device__ __forceinline__ void better(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) {
    bv = v;
    bi = i;
  }
}
__global__ __launch_bounds__(256) void argmax_part_kernel(const float* __restrict__ logits, int V, float* pv,
                                                          int* pi) {
  __shared__ float bv[4];
  __shared__ int bi[4];
  const int b = blockIdx.x, r = blockIdx.y, t = threadIdx.x;
  const int len = (V + AMB - 1) / AMB, i0 = b * len, i1 = min(V, i0 + len);
  const float* l = logits + (int64_t)r * V;
  float best = -INFINITY;
  int idx = 0x7fffffff;
  for (int i = i0 + t; i < i1; i += 256) better(best, idx, l[i], i);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) better(best, idx, __shfl_xor(best, off, 64), __shfl_xor(idx, off, 64));
  if ((t & 63) == 0) {
    bv[t >> 6] = best;
    bi[t >> 6] = idx;
  }
  __syncthreads();
  if (t == 0) {
    for (int w = 1; w < 4; ++w) better(best, idx, bv[w], bi[w]);
    pv[r * AMB + b] = best;
    pi[r * AMB + b] = idx;
  }
}
__global__ __launch_bounds__(64) void argmax_final_kernel(const float* __restrict__ pv, const int* __restrict__ pi,
                                                          int32_t* next) {
  const int r = blockIdx.x, t = threadIdx.x;
  float best = pv[r * AMB + t];
  int idx = pi[r * AMB + t];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) better(best, idx, __shfl_xor(best, off, 64), __shfl_xor(idx, off, 64));
  if (t == 0) next[r] = idx;
}

}  // namespace

hipError_t launch_gemv16(const void* W, const void* x, float* out, int rows, int N, int K, int ksplit, int dtype,
                         hipStream_t s) {
  if (rows < 1 || rows > GEMV_MAX_ROWS || ksplit < 1 || K % (32 * ksplit) || N % 16) return hipErrorInvalidValue;
  if (dtype != DT_BF16 && dtype != DT_F16) return hipErrorInvalidValue;
  const int waves = (N / 16) * ksplit;
  const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
  const int steps = K / ksplit / 32;
  const int rt = (rows + 15) / 16;
  auto go = [&](auto u, auto r) {
    constexpr int U = decltype(u)::value, RT = decltype(r)::value;
    if (dtype == DT_BF16)
      hipLaunchKernelGGL((gemv16_kernel<bf16_t, U, RT>), grid, block, 0, s, (const bf16_t*)W, (const bf16_t*)x, out,
                         rows, N, K, ksplit);
    else
      hipLaunchKernelGGL((gemv16_kernel<f16_t, U, RT>), grid, block, 0, s, (const f16_t*)W, (const f16_t*)x, out,
                         rows, N, K, ksplit);
  };
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I4 = std::integral_constant<int, 4>;
  using U8 = std::integral_constant<int, 8>;
  using U16 = std::integral_constant<int, 16>;
  using U24 = std::integral_constant<int, 24>;
  using U32 = std::integral_constant<int, 32>;
  if (rt == 1) {  // one row tile: unroll to the wavefront's whole K range
    if (steps <= 8) go(U8{}, I1{});
    else if (steps <= 16) go(U16{}, I1{});
    else if (steps <= 24) go(U24{}, I1{});
    else if (steps <= 32) go(U32{}, I1{});
    else go(U8{}, I1{});
  } else if (rt == 2) {  // x fragments of two row tiles: at most 16 steps in registers
    if (steps <= 8) go(U8{}, I2{});
    else go(U16{}, I2{});
  } else {
    go(U8{}, I4{});
  }
  return hipGetLastError();
}

hipError_t launch_add_rmsnorm(float* x, const float* part, int S, const float* w, void* h, int rows, int D, float eps,
                              int dtype, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (D % 256 || D > 4096 || S < 0 || S > MAXS || (S > 0 && !part)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)rows), block(256);
  auto go = [&](auto sc) {
    constexpr int SC = decltype(sc)::value;
    if (dtype == DT_BF16)
      hipLaunchKernelGGL((add_rmsnorm_kernel<bf16_t, SC>), grid, block, 0, s, x, part, w, h, rows, D, eps);
    else if (dtype == DT_F16)
      hipLaunchKernelGGL((add_rmsnorm_kernel<f16_t, SC>), grid, block, 0, s, x, part, w, h, rows, D, eps);
    else
      hipLaunchKernelGGL((add_rmsnorm_kernel<float, SC>), grid, block, 0, s, x, part, w, h, rows, D, eps);
  };
  switch (S) {
    case 0: go(std::integral_constant<int, 0>{}); break;
    case 1: go(std::integral_constant<int, 1>{}); break;
    case 2: go(std::integral_constant<int, 2>{}); break;
    case 3: go(std::integral_constant<int, 3>{}); break;
    case 4: go(std::integral_constant<int, 4>{}); break;
    case 5: go(std::integral_constant<int, 5>{}); break;
    case 6: go(std::integral_constant<int, 6>{}); break;
    case 7: go(std::integral_constant<int, 7>{}); break;
    default: go(std::integral_constant<int, 8>{}); break;
  }
  return hipGetLastError();
}

hipError_t launch_qk_rope(const DecArgs& a, const float* qkv, int S, int dtype, hipStream_t s) {
  if (S < 1 || S > MAXS || (dtype != DT_BF16 && dtype != DT_F16)) return hipErrorInvalidValue;
  const int items = a.rows * (a.Hq + 2 * a.Hkv);
  const dim3 grid((unsigned)((items + 3) / 4)), block(256);
  auto go = [&](auto sc) {
    constexpr int SC = decltype(sc)::value;
    if (dtype == DT_BF16) hipLaunchKernelGGL((qk_rope_kernel<bf16_t, SC>), grid, block, 0, s, a, qkv);
    else hipLaunchKernelGGL((qk_rope_kernel<f16_t, SC>), grid, block, 0, s, a, qkv);
  };
  switch (S) {
    case 1: go(std::integral_constant<int, 1>{}); break;
    case 2: go(std::integral_constant<int, 2>{}); break;
    case 3: go(std::integral_constant<int, 3>{}); break;
    case 4: go(std::integral_constant<int, 4>{}); break;
    case 5: go(std::integral_constant<int, 5>{}); break;
    case 6: go(std::integral_constant<int, 6>{}); break;
    case 7: go(std::integral_constant<int, 7>{}); break;
    default: go(std::integral_constant<int, 8>{}); break;
  }
  return hipGetLastError();
}

hipError_t launch_attn_dec(const DecArgs& a, int n_items, bool combine, const float* qkv, int S, int dtype,
                           hipStream_t s) {
  if (a.Hq != 2 * a.Hkv) return hipErrorInvalidValue;
  if (dtype != DT_BF16 && dtype != DT_F16) return hipErrorInvalidValue;
  if (S != 0 && S != 1 && S != 2 && S != 4 && S != 8) return hipErrorInvalidValue;
  if (S && !qkv) return hipErrorInvalidValue;
  const dim3 grid((unsigned)n_items, (unsigned)a.Hkv);
  const dim3 cgrid((unsigned)a.rows, (unsigned)a.Hq);
  auto go = [&](auto tt, auto sc) {
    using T = decltype(tt);
    constexpr int SC = decltype(sc)::value;
    hipLaunchKernelGGL((attn_dec_kernel<T, SC>), grid, dim3(256), 0, s, a, qkv);
    if (combine) hipLaunchKernelGGL(attn_combine_kernel<T>, cgrid, dim3(128), 0, s, a);
  };
  auto by_s = [&](auto tt) {
    switch (S) {
      case 0: go(tt, std::integral_constant<int, 0>{}); break;
      case 1: go(tt, std::integral_constant<int, 1>{}); break;
      case 2: go(tt, std::integral_constant<int, 2>{}); break;
      case 4: go(tt, std::integral_constant<int, 4>{}); break;
      default: go(tt, std::integral_constant<int, 8>{}); break;
    }
  };
  if (dtype == DT_BF16) by_s(bf16_t{});
  else by_s(f16_t{});
  return hipGetLastError();
}

hipError_t launch_gemv16x(const void* W, int xm, const float* src, int S, const DecArgs& a, int cmax, float* out,
                          int rows, int N, int K, int ksplit, int dtype, hipStream_t s) {
  if (rows < 1 || rows > GEMV_FUSE_ROWS || ksplit < 1 || N % 64 || K % ksplit) return hipErrorInvalidValue;
  const int kl = K / ksplit, steps = kl / 32;
  if (kl % 32 || steps > 32) return hipErrorInvalidValue;
  size_t lds = (size_t)rows * kl * 2;
  if (xm == 1) {
    if (S < 1 || S > MAXS) return hipErrorInvalidValue;
  } else if (xm == 2) {
    if (kl % HD || cmax < 1 || a.Hq != 2 * a.Hkv || K != a.Hq * HD) return hipErrorInvalidValue;
    lds += (size_t)rows * (kl / HD) * (2 + 3 * cmax) * sizeof(float);
  } else {
    return hipErrorInvalidValue;
  }
  if (lds > 65536) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(N / 16 * ksplit / 4)), block(256);
  auto go = [&](auto u, auto m) {
    constexpr int U = decltype(u)::value, XM = decltype(m)::value;
    if (dtype == DT_BF16)
      hipLaunchKernelGGL((gemv16x_kernel<bf16_t, U, XM>), grid, block, lds, s, (const bf16_t*)W, src, S, a, cmax,
                         out, rows, N, K, ksplit);
    else
      hipLaunchKernelGGL((gemv16x_kernel<f16_t, U, XM>), grid, block, lds, s, (const f16_t*)W, src, S, a, cmax,
                         out, rows, N, K, ksplit);
  };
  auto by_u = [&](auto m) {
    if (steps <= 8) go(std::integral_constant<int, 8>{}, m);
    else if (steps <= 16) go(std::integral_constant<int, 16>{}, m);
    else if (steps <= 24) go(std::integral_constant<int, 24>{}, m);
    else go(std::integral_constant<int, 32>{}, m);
  };
  if (dtype != DT_BF16 && dtype != DT_F16) return hipErrorInvalidValue;
  if (xm == 1) by_u(std::integral_constant<int, 1>{});
  else by_u(std::integral_constant<int, 2>{});
  return hipGetLastError();
}

hipError_t launch_argmax(const float* logits, int rows, int V, float* pv, int* pi, int32_t* next, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(argmax_part_kernel, dim3(AMB, (unsigned)rows), dim3(256), 0, s, logits, V, pv, pi);
  hipLaunchKernelGGL(argmax_final_kernel, dim3((unsigned)rows), dim3(64), 0, s, pv, pi, next);
  return hipGetLastError();
}

hipError_t launch_swiglu(const float* part, int S, void* act, int rows, int F, int dtype, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (S < 1 || S > MAXS || F % 16) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((F + 255) / 256), (unsigned)rows), block(256);
  if (dtype == DT_BF16) hipLaunchKernelGGL(swiglu_kernel<bf16_t>, grid, block, 0, s, part, S, (bf16_t*)act, rows, F);
  else if (dtype == DT_F16) hipLaunchKernelGGL(swiglu_kernel<f16_t>, grid, block, 0, s, part, S, (f16_t*)act, rows, F);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace mt
