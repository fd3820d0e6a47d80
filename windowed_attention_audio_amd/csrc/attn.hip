// Block-diagonal (windowed) self-attention on the matrix cores.
//
// Model card "MOSS-Transcribe-preview-2B-GGUF", Architecture table, Audio
// encoder row: 20 heads of 64 with windowed, block-diagonal attention.  The
// encoder frames [kW, min((k+1)W, N)) of each sequence form window k; a row
// attends only to the rows of its own window: o = softmax(q k^T / 8) v.
//
// One workgroup per (window, head), or for windows longer than 256 keys per
// (window, 128 queries, head) with the keys streamed through LDS (each
// wavefront two interleaved groups of 16 queries that share every K and V
// fragment read).  Each wavefront takes groups of 16 query rows and walks the
// keys in chunks of
// 64 with an online softmax (running maximum and output in fp32 registers;
// probabilities enter the second product in the operand type).  Scores are computed
// transposed, S^T = K Q^T, so that every lane owns one query row (its lane
// index mod 16): the row statistics need only two cross-lane steps, and the
// probabilities already sit where the next product, O^T = V^T P^T, wants its
// second operand.  For 16-bit operands the keys of each 32-wide step are stored in V^T
// in the order in which a lane holds its probabilities, so each operand
// fragment is one 16-byte LDS read.
#include "common.h"
#include "kernels.h"

namespace mt {

namespace {

// K rows: chunk c of key row r at chunk slot c ^ (r & 7) (conflict-free reads of
// 16 consecutive rows at one chunk)
__device__ __forceinline__ int swz(int r) { return r & 7; }

// position of key kv inside a V^T row (bf16: permuted within 32-key blocks)
template <typename T>
__device__ __forceinline__ int vt_pos(int kv) {
  if constexpr (sizeof(T) == 2) {
    const int u = kv >> 5, h = (kv >> 4) & 1, g = (kv >> 2) & 3, j = kv & 3;
    return (u << 5) | (g << 3) | (h << 2) | j;
  } else {
    return kv;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void wattn_kernel(AttnArgs a) {
  constexpr int HD = 64;
  constexpr int EPC = Elem<T>::per16;      // elements per 16-byte chunk
  constexpr int CPR = HD / EPC;            // chunks per K row
  extern __shared__ uint4 smem[];
  const int wpad = a.wpad;
  uint4* Ks = smem;                                   // [wpad][CPR] chunks
  T* Vt = (T*)(smem + wpad * CPR);                    // [HD][vstride]
  const int vstride = wpad + 16 / (int)sizeof(T);     // +16 bytes per row

  const int win = blockIdx.x;
  const int head = blockIdx.y;
  const int sq = find_seq(a.cu_win, a.nseq, win);
  const int kwin = win - a.cu_win[sq];
  const int N = a.cu_rows[sq + 1] - a.cu_rows[sq];
  const int s0 = a.cu_rows[sq] + kwin * a.window;
  const int w = min(a.window, N - kwin * a.window);
  const int64_t ld = 3 * (int64_t)a.D;
  const T* qkv = (const T*)a.qkv;
  const T* Qg = qkv + (int64_t)s0 * ld + head * HD;
  const T* Kg = Qg + a.D;
  const T* Vg = Qg + 2 * a.D;

  // ---- stage K and V^T (rows >= w are zero)
  for (int idx = threadIdx.x; idx < wpad * CPR; idx += 256) {
    const int kv = idx / CPR, c = idx - kv * CPR;
    uint4 kvec = make_uint4(0, 0, 0, 0), vvec = make_uint4(0, 0, 0, 0);
    if (kv < w) {
      kvec = *(const uint4*)(Kg + (int64_t)kv * ld + c * EPC);
      vvec = *(const uint4*)(Vg + (int64_t)kv * ld + c * EPC);
    }
    Ks[kv * CPR + (c ^ swz(kv))] = kvec;
    const T* ve = (const T*)&vvec;
    const int p = vt_pos<T>(kv);
#pragma unroll
    for (int e = 0; e < EPC; ++e) Vt[(c * EPC + e) * vstride + p] = ve[e];
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const float sl2 = 0.125f * 1.4426950408889634f;  // 1/sqrt(64) * log2(e)
  const int nqg = (w + 15) >> 4;
  const int nkc = (w + 63) >> 6;

  for (int qg = wave; qg < nqg; qg += 4) {
    const int q = qg * 16 + l16;  // this lane's query row (window-local)
    // Q fragments: k-chunks (4s + g) of row q
    constexpr int QS = CPR / 4;
    uint4 qf[QS];
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      qf[s] = make_uint4(0, 0, 0, 0);
      if (q < w) qf[s] = *(const uint4*)(Qg + (int64_t)q * ld + (4 * s + g) * EPC);
    }
    float m_run = -INFINITY, l_part = 0.f;
    f32x4 o[4];
#pragma unroll
    for (int nd = 0; nd < 4; ++nd) o[nd] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int kc = 0; kc < nkc; ++kc) {
      f32x4 st[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        st[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int kvr = kc * 64 + t * 16 + l16;
#pragma unroll
        for (int s = 0; s < QS; ++s) {
          const int cc = 4 * s + g;
          const uint4 kf = Ks[kvr * CPR + (cc ^ swz(kvr))];
          if constexpr (sizeof(T) == 2) mma16(st[t], kf, qf[s], T{});
          else mma_f32x4(st[t], kf, qf[s]);
        }
      }
      // lane holds S^T[kv = kc*64 + 16t + 4g + e][q]; scale, mask, row max
      float cmax = -INFINITY;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int kv = kc * 64 + t * 16 + 4 * g + e;
          const float v = kv < w ? st[t][e] * sl2 : -INFINITY;
          st[t][e] = v;
          cmax = fmaxf(cmax, v);
        }
      cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
      cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
      const float m_new = fmaxf(m_run, cmax);
      const float alpha = exp2f(m_run - m_new);
      m_run = m_new;
      float psum = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = exp2f(st[t][e] - m_new);
          st[t][e] = p;
          psum += p;
        }
      l_part = l_part * alpha + psum;
#pragma unroll
      for (int nd = 0; nd < 4; ++nd) o[nd] *= alpha;

      // O^T[d][q] += sum_kv V^T[d][kv] P^T[kv][q]
#pragma unroll
      for (int nd = 0; nd < 4; ++nd) {
        const T* vrow = Vt + (nd * 16 + l16) * vstride + kc * 64;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const uint4 vf = *(const uint4*)(vrow + 32 * u + 8 * g);
            uint4 pf;
            pf.x = pack2f<T>(st[2 * u][0], st[2 * u][1]);
            pf.y = pack2f<T>(st[2 * u][2], st[2 * u][3]);
            pf.z = pack2f<T>(st[2 * u + 1][0], st[2 * u + 1][1]);
            pf.w = pack2f<T>(st[2 * u + 1][2], st[2 * u + 1][3]);
            mma16(o[nd], vf, pf, T{});
          }
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float4 vf = *(const float4*)(vrow + 16 * t + 4 * g);
            o[nd] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf.x, st[t][0], o[nd], 0, 0, 0);
            o[nd] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf.y, st[t][1], o[nd], 0, 0, 0);
            o[nd] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf.z, st[t][2], o[nd], 0, 0, 0);
            o[nd] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf.w, st[t][3], o[nd], 0, 0, 0);
          }
        }
      }
    }
    float l_tot = l_part + __shfl_xor(l_part, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    const float inv = 1.0f / l_tot;
    if (q < w) {
      T* orow = (T*)a.out + (int64_t)(s0 + q) * a.D + head * HD;
#pragma unroll
      for (int nd = 0; nd < 4; ++nd) {
        const int d0 = nd * 16 + 4 * g;  // lane holds O^T[d0 + e][q]
        if constexpr (sizeof(T) == 2) {
          uint2 pk;
          pk.x = pack2f<T>(o[nd][0] * inv, o[nd][1] * inv);
          pk.y = pack2f<T>(o[nd][2] * inv, o[nd][3] * inv);
          *(uint2*)(orow + d0) = pk;
        } else {
          *(float4*)(orow + d0) =
              make_float4(o[nd][0] * inv, o[nd][1] * inv, o[nd][2] * inv, o[nd][3] * inv);
        }
      }
    }
  }
}

// 16-bit operands, same algorithm with a different staging:
//  * K and V of the (window, head) go to LDS by buffer loads straight into
//    LDS (no trip through registers, no transposing stores).  The buffer
//    descriptor spans exactly the window's w rows, so rows >= w read as
//    zeros.  Both are kept row-major (128 bytes per key), 16-byte chunk c of
//    key row r at chunk slot c ^ (r & 7).
//  * V^T fragments for O^T = V^T P^T come from transposing LDS reads
//    (ds_read_b64_tr_b16).  Within each 16-lane group G, element j of lane i
//    of that read is element i & 3 of the 8-byte vector addressed by lane
//    4 j + (i >> 2) of the same group.  So to give lane (d, g) the keys
//    32 u + 4 g + e (and + 16) of dimension d -- the order in which the P
//    fragment holds its probabilities -- lane (g, s) addresses key row
//    kc 64 + 32 u + 4 g + (s >> 2) (+ 16), columns 16 nd + 4 (s & 3) .. + 3.
//  * each wavefront's Q fragments are read from global memory before the
//    wait for the staging, one query group ahead.
typedef short tr4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) tr4_t* tr_ptr_t;
typedef __attribute__((address_space(3))) void* lds_vptr_t;

// Maximum over lanes l, l ^ 16, l ^ 32 and l ^ 48 (the four lanes holding
// one query's scores).  v_permlane16_swap of a register with itself gives
// each lane the value of lane l ^ 16, v_permlane32_swap that of lane l ^ 32:
// two VALU swaps instead of two LDS permutes, which waited on the LDS.
// Scores are finite or -inf, so a plain comparison serves as the maximum.
__device__ __forceinline__ float max4_lanes(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float a0 = __uint_as_float(a[0]), a1 = __uint_as_float(a[1]);
  v = a0 > a1 ? a0 : a1;
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float b0 = __uint_as_float(b[0]), b1 = __uint_as_float(b[1]);
  return b0 > b1 ? b0 : b1;
}

// One chunk of 64 keys for one 16-query group: S^T = K Q^T (lane = query
// l16), scale, mask keys >= w, online-softmax update, O^T += V^T P^T.  K and
// V rows r0 .. r0 + 63 of the LDS arrays hold keys kv0 .. kv0 + 63; 16-byte
// chunk c of a row sits at slot c ^ (row & 7) (r0 is a multiple of 64).
// The running sum of the probabilities is a matrix product too: lsum +=
// 1 P^T with an all-ones first operand, so every lane gets its query's sum
// of exactly the 16-bit probabilities that weight V, and the vector units
// (which bound this kernel) skip an add per score.
template <typename T, int NG>
__device__ __forceinline__ void attn_chunkN(const uint4* Ks, const uint4* Vs, int r0, int kv0, int w,
                                            const uint4 (&qf)[NG][2], float (&m_run)[NG], f32x4 (&lsum)[NG],
                                            f32x4 (&o)[NG][4], int g, int l16) {
  constexpr int CPR = 8;
  const float sl2 = 0.125f * 1.4426950408889634f;  // 1/sqrt(64) * log2(e)
  f32x4 st[NG][4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int G = 0; G < NG; ++G) st[G][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int kvr = r0 + t * 16 + l16;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint4 kf = Ks[kvr * CPR + ((4 * s + g) ^ (kvr & 7))];
#pragma unroll
      for (int G = 0; G < NG; ++G) mma16(st[G][t], kf, qf[G][s], T{});
    }
  }
#pragma unroll
  for (int G = 0; G < NG; ++G) {
    // lane holds S^T[kv = kv0 + 16t + 4g + e][q] (unscaled); mask, row max.
    // m_run is kept in raw-score units: p = 2^((s - m) sl2) is one fma and
    // one v_exp_f32 (its argument is never positive: no range handling).
    float cmax = -INFINITY;
    if (kv0 + 64 <= w) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) cmax = fmaxf(cmax, st[G][t][e]);
    } else {  // last, partial chunk: keys >= w drop out
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int kv = kv0 + t * 16 + 4 * g + e;
          const float v = kv < w ? st[G][t][e] : -INFINITY;
          st[G][t][e] = v;
          cmax = fmaxf(cmax, v);
        }
    }
    cmax = max4_lanes(cmax);
    // Lazy rescaling: the reference maximum m_run moves (and the running
    // sum and the output accumulators are scaled down to it) only when some
    // query of the group has gained more than a factor 2^8 over it --
    // always in the first chunk (m_run = -inf), rarely after.  Otherwise
    // the probabilities stay relative to the old reference, below 2^8,
    // which the 16-bit operand types hold at the same relative precision as
    // values below 1; the final division by the sum cancels the reference.
    // The decision is per group of 16 queries (all lanes of the wavefront),
    // so the branch is uniform.
    const float m_new = fmaxf(m_run[G], cmax);
    if (__any((m_new - m_run[G]) * sl2 > 8.0f)) {
      const float alpha = __builtin_amdgcn_exp2f((m_run[G] - m_new) * sl2);
      m_run[G] = m_new;
      lsum[G] *= alpha;
#pragma unroll
      for (int nd = 0; nd < 4; ++nd) o[G][nd] *= alpha;
    }
    const float mb = -m_run[G] * sl2;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) st[G][t][e] = __builtin_amdgcn_exp2f(fmaf(st[G][t][e], sl2, mb));
  }

  // O^T[d][q] += sum_kv V^T[d][kv] P^T[kv][q]; probabilities lie in
  // [0, 2^8]: plain round-to-nearest-even conversions, no clamp.  Each V
  // fragment read feeds the NG groups' products.
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    uint4 pf[NG];
    const uint32_t one2 = pack2_cast<T>(1.0f, 1.0f);
#pragma unroll
    for (int G = 0; G < NG; ++G) {
      pf[G].x = pack2_cast<T>(st[G][2 * u][0], st[G][2 * u][1]);
      pf[G].y = pack2_cast<T>(st[G][2 * u][2], st[G][2 * u][3]);
      pf[G].z = pack2_cast<T>(st[G][2 * u + 1][0], st[G][2 * u + 1][1]);
      pf[G].w = pack2_cast<T>(st[G][2 * u + 1][2], st[G][2 * u + 1][3]);
      mma16(lsum[G], make_uint4(one2, one2, one2, one2), pf[G], T{});
    }
    const int r1 = r0 + 32 * u + 4 * g + (l16 >> 2), r2 = r1 + 16;
#pragma unroll
    for (int nd = 0; nd < 4; ++nd) {
      const int c = 2 * nd + ((l16 & 3) >> 1), half = (l16 & 1) * 8;  // bytes within chunk
      const tr4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (tr_ptr_t)((char*)(Vs + r1 * CPR + (c ^ (r1 & 7))) + half));
      const tr4_t v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (tr_ptr_t)((char*)(Vs + r2 * CPR + (c ^ (r2 & 7))) + half));
      const uint2 w1 = __builtin_bit_cast(uint2, v1), w2 = __builtin_bit_cast(uint2, v2);
#pragma unroll
      for (int G = 0; G < NG; ++G) mma16(o[G][nd], make_uint4(w1.x, w1.y, w2.x, w2.y), pf[G], T{});
    }
  }
}

// One query group (the on-chip kernel).
template <typename T>
__device__ __forceinline__ void attn_chunk16(const uint4* Ks, const uint4* Vs, int r0, int kv0, int w,
                                             const uint4 (&qf)[2], float& m_run, f32x4& lsum,
                                             f32x4 (&o)[4], int g, int l16) {
  uint4 q1[1][2] = {{qf[0], qf[1]}};
  float m1[1] = {m_run};
  f32x4 l1[1] = {lsum};
  f32x4 o1[1][4] = {{o[0], o[1], o[2], o[3]}};
  attn_chunkN<T, 1>(Ks, Vs, r0, kv0, w, q1, m1, l1, o1, g, l16);
  m_run = m1[0];
  lsum = l1[0];
#pragma unroll
  for (int nd = 0; nd < 4; ++nd) o[nd] = o1[0][nd];
}

template <typename T>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5))) void wattn16_kernel(AttnArgs a) {
  static_assert(sizeof(T) == 2, "16-bit operands");
  constexpr int HD = 64, CPR = 8;  // 8 chunks of 8 elements per 128-byte row
  extern __shared__ uint4 smem[];
  const int wpad = a.wpad;
  uint4* Ks = smem;               // [wpad][8] chunks
  uint4* Vs = smem + wpad * CPR;  // [wpad][8] chunks

  const int win = blockIdx.x;
  const int head = blockIdx.y;
  const int sq = find_seq(a.cu_win, a.nseq, win);
  const int kwin = win - a.cu_win[sq];
  const int N = a.cu_rows[sq + 1] - a.cu_rows[sq];
  const int s0 = a.cu_rows[sq] + kwin * a.window;
  const int w = min(a.window, N - kwin * a.window);
  const int ldb = 3 * a.D * (int)sizeof(T);  // bytes per qkv row
  const char* base = (const char*)a.qkv + (int64_t)s0 * ldb;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;

  // ---- DMA: 1 KB blocks of 8 rows; blocks [0, wpad/8) are K, the rest V
  {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, w * ldb, 0x00020000);
    const int nb = wpad / 8;
    const int r8 = lane >> 3, slot = lane & 7;
    for (int b = wave; b < 2 * nb; b += 4) {
      const bool isv = b >= nb;
      const int r = 8 * (isv ? b - nb : b) + r8;
      const int c = slot ^ (r & 7);
      const int col = (isv ? 2 : 1) * a.D + head * HD + c * 8;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_vptr_t)(smem + b * 64), 16,
                                               r * ldb + col * (int)sizeof(T), 0, 0, 0);
    }
  }

  const int nqg = (w + 15) >> 4;
  const int nkc = (w + 63) >> 6;
  const T* Qg = (const T*)base + head * HD;
  const int ldq = 3 * a.D;

  auto load_q = [&](int qg, uint4 (&qf)[2]) {
    const int q = qg * 16 + l16;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      qf[s] = make_uint4(0, 0, 0, 0);
      if (qg < nqg && q < w) qf[s] = *(const uint4*)(Qg + (int64_t)q * ldq + (4 * s + g) * 8);
    }
  };
  uint4 qn[2];
  load_q(wave, qn);

  __builtin_amdgcn_s_waitcnt(0);  // this wavefront's DMA and Q loads
  __syncthreads();

  for (int qg = wave; qg < nqg; qg += 4) {
    const int q = qg * 16 + l16;  // this lane's query row (window-local)
    uint4 qf[2] = {qn[0], qn[1]};
    load_q(qg + 4, qn);  // next group, in flight during this one
    float m_run = -INFINITY;
    f32x4 lsum = f32x4{0.f, 0.f, 0.f, 0.f}, o[4];
#pragma unroll
    for (int nd = 0; nd < 4; ++nd) o[nd] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int kc = 0; kc < nkc; ++kc) attn_chunk16<T>(Ks, Vs, kc * 64, kc * 64, w, qf, m_run, lsum, o, g, l16);
    const float inv = 1.0f / lsum[0];
    if (q < w) {
      T* orow = (T*)a.out + (int64_t)(s0 + q) * a.D + head * HD;
#pragma unroll
      for (int nd = 0; nd < 4; ++nd) {
        const int d0 = nd * 16 + 4 * g;  // lane holds O^T[d0 + e][q]
        uint2 pk;
        pk.x = pack2f<T>(o[nd][0] * inv, o[nd][1] * inv);
        pk.y = pack2f<T>(o[nd][2] * inv, o[nd][3] * inv);
        *(uint2*)(orow + d0) = pk;
      }
    }
  }
}

template <typename T>
hipError_t run_attn16(const AttnArgs& a, hipStream_t s) {
  if (a.n_windows == 0) return hipSuccess;
  const size_t lds = (size_t)a.wpad * 2 * 128;  // K and V, 128 bytes per key each
  hipError_t e = hipFuncSetAttribute((const void*)wattn16_kernel<T>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(wattn16_kernel<T>, dim3(a.n_windows, a.n_heads), dim3(256), lds, s, a);
  return hipGetLastError();
}

// Windows longer than the on-chip maximum (any W; W >= N is full attention
// over each sequence): one workgroup per (window, block of 128 queries,
// head), two groups of 16 queries per wavefront, and the window's keys
// stream through LDS in tiles of 64 (K and V, 16 KB per stage, four stages:
// each tile's DMA is issued three tiles ahead; tiles past the window read
// zeros, so every wavefront issues the same loads).  Same per-chunk math as
// above; each K and V fragment read from LDS feeds both groups, and the two
// groups' softmax chains interleave (one group per wavefront left the
// matrix cores waiting on each chunk's max -> exp -> product chain).
template <typename T>
__global__ __launch_bounds__(256) void wattn16s_kernel(AttnArgs a, int qblocks) {
  static_assert(sizeof(T) == 2, "16-bit operands");
  constexpr int HD = 64, CPR = 8;
  constexpr int NG = 2, QB = 64 * NG;  // query groups per wavefront, queries per workgroup
  __shared__ uint4 k0[64 * CPR], k1[64 * CPR], k2[64 * CPR], k3[64 * CPR];
  __shared__ uint4 v0[64 * CPR], v1[64 * CPR], v2[64 * CPR], v3[64 * CPR];

  const int win = blockIdx.x / qblocks, qb = blockIdx.x - win * qblocks;
  const int head = blockIdx.y;
  const int sq = find_seq(a.cu_win, a.nseq, win);
  const int kwin = win - a.cu_win[sq];
  const int N = a.cu_rows[sq + 1] - a.cu_rows[sq];
  const int s0 = a.cu_rows[sq] + kwin * a.window;
  const int w = min(a.window, N - kwin * a.window);
  if (qb * QB >= w) return;  // the whole workgroup: before any barrier

  const int ldb = 3 * a.D * (int)sizeof(T);  // bytes per qkv row
  const char* base = (const char*)a.qkv + (int64_t)s0 * ldb;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, w * ldb, 0x00020000);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const int nkt = (w + 63) >> 6;

  // query groups of this wavefront: rows qb QB + 64 G + 16 wave + l16 (the
  // second may lie past w, then it is computed and not stored)
  int q[NG];
  uint4 qf[NG][2];
  {
    const T* Qg = (const T*)base + head * HD;
#pragma unroll
    for (int G = 0; G < NG; ++G) {
      q[G] = qb * QB + 64 * G + wave * 16 + l16;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        qf[G][s] = make_uint4(0, 0, 0, 0);
        if (q[G] < w) qf[G][s] = *(const uint4*)(Qg + (int64_t)q[G] * (3 * a.D) + (4 * s + g) * 8);
      }
    }
  }
  const bool active = qb * QB + wave * 16 < w;

  // tile kt into (K, V): 16 blocks of 8 rows, four per wavefront
  auto issue = [&](int kt, uint4* K, uint4* V) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = wave + 4 * i;
      const bool isv = b >= 8;
      const int r = 8 * (isv ? b - 8 : b) + (lane >> 3);
      const int c = (lane & 7) ^ (r & 7);
      const int col = (isv ? 2 : 1) * a.D + head * HD + c * 8;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_vptr_t)((isv ? V + (b - 8) * 64 : K + b * 64)), 16,
                                               (kt * 64 + r) * ldb + col * (int)sizeof(T), 0, 0, 0);
    }
  };

  float m_run[NG];
  f32x4 lsum[NG], o[NG][4];
#pragma unroll
  for (int G = 0; G < NG; ++G) {
    m_run[G] = -INFINITY;
    lsum[G] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nd = 0; nd < 4; ++nd) o[G][nd] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  issue(0, k0, v0);
  issue(1, k1, v1);
  issue(2, k2, v2);
  // Step kt: this wavefront's DMA of tile kt has landed (the 8 loads of the
  // next two tiles may be in flight), everyone's has (barrier), and no one
  // reads the stage of tile kt - 1 any more: it takes tile kt + 3.
  auto step = [&](int kt, uint4* K, uint4* V, uint4* FK, uint4* FV) {
    __builtin_amdgcn_s_waitcnt((8 & 15) | (7 << 4) | (15 << 8) | ((8 >> 4) << 14));  // vmcnt(8)
    __syncthreads();
    issue(kt + 3, FK, FV);
    if (active) attn_chunkN<T, NG>(K, V, 0, kt * 64, w, qf, m_run, lsum, o, g, l16);
  };
  for (int kt = 0; kt < nkt; kt += 4) {
    step(kt, k0, v0, k3, v3);
    if (kt + 1 < nkt) step(kt + 1, k1, v1, k0, v0);
    if (kt + 2 < nkt) step(kt + 2, k2, v2, k1, v1);
    if (kt + 3 < nkt) step(kt + 3, k3, v3, k2, v2);
  }
  __builtin_amdgcn_s_waitcnt(0);  // drain the loads of tiles past the window

#pragma unroll
  for (int G = 0; G < NG; ++G) {
    if (active && q[G] < w) {
      const float inv = 1.0f / lsum[G][0];
      T* orow = (T*)a.out + (int64_t)(s0 + q[G]) * a.D + head * HD;
#pragma unroll
      for (int nd = 0; nd < 4; ++nd) {
        const int d0 = nd * 16 + 4 * g;  // lane holds O^T[d0 + e][q]
        uint2 pk;
        pk.x = pack2f<T>(o[G][nd][0] * inv, o[G][nd][1] * inv);
        pk.y = pack2f<T>(o[G][nd][2] * inv, o[G][nd][3] * inv);
        *(uint2*)(orow + d0) = pk;
      }
    }
  }
}

template <typename T>
hipError_t run_attn16s(const AttnArgs& a, hipStream_t s) {
  if (a.n_windows == 0) return hipSuccess;
  const int qblocks = (a.wpad + 127) / 128;  // 128 queries per workgroup
  hipLaunchKernelGGL(wattn16s_kernel<T>, dim3(a.n_windows * qblocks, a.n_heads), dim3(256), 0, s, a,
                     qblocks);
  return hipGetLastError();
}

template <typename T>
hipError_t run_attn(const AttnArgs& a, hipStream_t s) {
  if (a.n_windows == 0) return hipSuccess;
  const size_t lds = (size_t)a.wpad * 64 * sizeof(T) + (size_t)64 * (a.wpad * sizeof(T) + 16);
  hipError_t e = hipFuncSetAttribute((const void*)wattn_kernel<T>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(wattn_kernel<T>, dim3(a.n_windows, a.n_heads), dim3(256), lds, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, int dtype, hipStream_t s) {
  // keys of a window stay on chip up to 256 (LDS per workgroup 2 x 32 KB);
  // longer windows stream them
  if (dtype == DT_BF16) return a.wpad <= 256 ? run_attn16<bf16_t>(a, s) : run_attn16s<bf16_t>(a, s);
  if (dtype == DT_F16) return a.wpad <= 256 ? run_attn16<f16_t>(a, s) : run_attn16s<f16_t>(a, s);
  if (a.wpad > 256) return hipErrorInvalidValue;  // fp32: on-chip windows only
  return run_attn<float>(a, s);
}

}  // namespace mt
