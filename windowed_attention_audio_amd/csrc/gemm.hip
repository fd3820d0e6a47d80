// Tiled matrix products on the gfx950 matrix cores, with fused epilogues.
//
// C[M, N] = A[M, K] * B[N, K]^T, both operands K-contiguous.  A is either a
// plain row-major activation or, for the stride-2 3x3 convolutions of the
// front-end (model card "MOSS-Transcribe-preview-2B-GGUF", Architecture
// table, Conv front-end row), gathered on the fly from a channels-last
// activation (implicit GEMM: K index = tap * C + input channel, tap =
// 3 * freq offset + time offset, zero outside each sequence).
//
// Kernels (pick_tile at the end chooses by shape, epilogue and dtype):
//   gemm_w8_kernel   256 x BN tiles, eight wavefronts, two LDS stages of
//                    64-wide K slices loaded by DMA straight into LDS (wide
//                    outputs: qkv, fc1; narrow ones at M >= 2048 when the
//                    tiles fill the CUs);
//   gemm_w8q_kernel  the same with four stages of 32-wide slices (narrow
//                    outputs at M = 6000, the convolutions with the tap
//                    gather);
//   gemm_lds_kernel  128 x 128 / 64 x 64 tiles, four wavefronts, four LDS
//                    stages (few rows);
//   gemm_kernel      register-staged tiles for fp32 operands (K split over
//                    workgroups when the tiles are few).
// Every 16-bit kernel accumulates each output over K in 32-wide steps in
// the same order, so a row's result does not depend on the kernel, the tile
// or the batch it was computed in.  Within LDS each row's 16-byte chunks are XOR-
// swizzled by the row index so that 16 lanes reading 16 rows at one chunk
// hit distinct banks.
//
// Operand fragments: one 16-byte chunk per lane and operand.  For bf16 and
// fp16 this is one v_mfma_f32_16x16x32_{bf16,f16} (lane l supplies row l%16,
// k = 8*(l/16)..+7 of the 32-wide step).  For fp32 it is four v_mfma_f32_16x16x4_f32, the e-th
// one taking element e of every lane's chunk; as both operands use the same
// assignment of k to (lane group, element), the sum over k is unchanged.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace mt {

namespace {

// Chunk swizzle: chunk c of row r is stored at chunk slot c ^ (r & 7).  A
// 16-byte fragment read (16 consecutive rows at one chunk, four chunk
// groups) then runs at the LDS's full 256 bytes per clock; measured with the
// LDS bank-conflict counter, the unswizzled layout costs 4x and a swizzle
// that also folds in bit 3 of the row still 2x.  It depends only on r % 8,
// so fragments of 16-row tiles are a base address plus constant offsets.
__device__ __forceinline__ int swz(int r) { return r & 7; }

template <typename T>
__device__ __forceinline__ void mma_chunk(f32x4& acc, const uint4& a, const uint4& b) {
  if constexpr (sizeof(T) == 4) mma_f32x4(acc, a, b);
  else mma16(acc, a, b, T{});
}

// Per-row state of the convolution gather.
struct ConvRow {
  const char* base;  // first byte of the sequence's input activation
  int t0;            // 2 * t_out - 1
  int f0;            // 2 * f_out - 1
  int Tin;           // input time rows of the sequence
};

// Fused epilogue for accumulators of C^T tiles (the products are issued as
// B * A^T): acc[i][j][e] holds C[rbase + 16 i][cbase + 16 j + e], i.e. four
// consecutive columns of one row, so every store is 8 (16-bit) or 16 (fp32)
// bytes.  rbase = first row of the lane, cbase = its first column.
template <typename T>
__device__ __forceinline__ void store4(T* p, float v0, float v1, float v2, float v3) {
  if constexpr (sizeof(T) == 4) {
    *(float4*)p = make_float4(v0, v1, v2, v3);
  } else {
    *(uint2*)p = make_uint2(pack2f<T>(v0, v1), pack2f<T>(v2, v3));
  }
}

// The bias vectors of a lane's NI column fragments (cbase + 16 j .. + 3),
// all requested before the first is used: a guarded load per fragment
// compiled to a branch and a wait each, one L2 round trip after another at
// the end of every tile.  Columns past N read the last four (never stored;
// N is a multiple of 4); without a bias, zeros (a uniform branch).
template <int NI>
__device__ __forceinline__ void load_bias(const GemmArgs& a, const int cbase, float4 (&b)[NI]) {
  if (!a.bias) {
#pragma unroll
    for (int j = 0; j < NI; ++j) b[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    return;
  }
#pragma unroll
  for (int j = 0; j < NI; ++j) b[j] = *(const float4*)(a.bias + min(cbase + 16 * j, a.N - 4));
}

// GELU epilogues take the halved bias (gelu_ab: same bits as gelu_f(acc + b)).
template <int EPI, int NI>
__device__ __forceinline__ void halve_bias_for_gelu(float4 (&b)[NI]) {
  if constexpr (EPI == EPI_GELU || EPI == EPI_GELU_SPLIT || EPI == EPI_GELU_PE) {
#pragma unroll
    for (int j = 0; j < NI; ++j) b[j] = make_float4(0.5f * b[j].x, 0.5f * b[j].y, 0.5f * b[j].z, 0.5f * b[j].w);
  }
}

template <typename T, int EPI, int MI, int NI>
__device__ __forceinline__ void epilogue4(const GemmArgs& a, f32x4 (&acc)[MI][NI], const int rbase,
                                          const int cbase) {
  float4 bias[NI];
  load_bias<NI>(a, cbase, bias);
  halve_bias_for_gelu<EPI, NI>(bias);
  constexpr bool PE = EPI == EPI_PE || EPI == EPI_GELU_PE;
  double tau[PE ? NI * 4 : 1];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int col = cbase + 16 * j;
    if constexpr (PE) {
      const int half = a.N / 2;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = col + e;
        const int jj = c < half ? c : c - half;
        // timescale 10000^(-jj / (half - 1)), in revolutions per position
        tau[4 * j + e] = exp(-(double)jj * 9.2103403719761836 / (double)(half - 1)) * 0.15915494309189535;
      }
    }
  }
  if constexpr (EPI == EPI_RESID) {
    // C += acc + bias on the fp32 residual stream.  A guarded read per
    // fragment compiled to a branch and a wait each (MI x NI round trips in a
    // row); instead the NI vectors of fragment row i + 1 are requested,
    // from clamped addresses, before row i is added and stored.
    auto read_row = [&](int i, float4 (&R)[NI]) {
      const int row = min(rbase + 16 * i, a.M - 1);
#pragma unroll
      for (int j = 0; j < NI; ++j)
        R[j] = *(const float4*)((const float*)a.C + (int64_t)row * a.ldc + min(cbase + 16 * j, a.N - 4));
    };
    float4 Rn[NI];
    read_row(0, Rn);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      float4 R[NI];
#pragma unroll
      for (int j = 0; j < NI; ++j) R[j] = Rn[j];
      if (i + 1 < MI) read_row(i + 1, Rn);
      const int row = rbase + 16 * i;
      if (row >= a.M) continue;
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int col = cbase + 16 * j;
        if (col >= a.N) continue;
        const float v0 = acc[i][j][0] + bias[j].x, v1 = acc[i][j][1] + bias[j].y;
        const float v2 = acc[i][j][2] + bias[j].z, v3 = acc[i][j][3] + bias[j].w;
        float4 r = R[j];
        r.x += v0;
        r.y += v1;
        r.z += v2;
        r.w += v3;
        *(float4*)((float*)a.C + (int64_t)row * a.ldc + col) = r;
      }
    }
    return;
  }
  // Sequence of the lane's rows (PE, padded EPI_OUT): one search for its
  // first row, then a step forward whenever a row passes the sequence's end
  // (rows rbase + 16 i increase; a search per row waited on its chain of
  // dependent loads for every row).  Same result as find_seq for each row.
  [[maybe_unused]] int sq_c = 0, sq_lo = 0, sq_hi = 0;
  [[maybe_unused]] float amax = 0.f;  // fp16: largest |value| converted (saturation report)
  constexpr bool SEQ = PE || EPI == EPI_OUT;
  if constexpr (SEQ) {
    if (PE || a.out_seq_stride > 0) {
      sq_c = find_seq(a.cu_rows, a.nseq, min(rbase, a.M - 1));
      sq_lo = a.cu_rows[sq_c];
      sq_hi = a.cu_rows[sq_c + 1];
    }
  }
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int row = rbase + 16 * i;
    if (row >= a.M) continue;
    int64_t orow = row;
    int pos = 0;
    if constexpr (SEQ) {
      if (PE || a.out_seq_stride > 0) {
        while (row >= sq_hi && sq_c + 1 < a.nseq) {
          ++sq_c;
          sq_lo = sq_hi;
          sq_hi = a.cu_rows[sq_c + 1];
        }
        pos = row - sq_lo + (PE ? a.pos_offset : 0);
        if (EPI == EPI_OUT) orow = (int64_t)sq_c * a.out_seq_stride + pos;
      }
    }
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int col = cbase + 16 * j;
      if (col >= a.N) continue;
      if constexpr (EPI == EPI_SWIGLU) {
        if (j & 1) continue;  // tile j holds gate, tile j + 1 up, of the same 16 features
        const int feat = (col - (col & 15)) / 2 + (col & 15);
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = silu_f(acc[i][j][e]) * acc[i][j + 1][e];
        if constexpr (__is_same(T, f16_t)) amax = absmax4(amax, o[0], o[1], o[2], o[3]);
        store4((T*)a.C + (int64_t)row * a.ldc + feat, o[0], o[1], o[2], o[3]);
        continue;
      } else {
        const float v0 = acc[i][j][0] + bias[j].x, v1 = acc[i][j][1] + bias[j].y;
        const float v2 = acc[i][j][2] + bias[j].z, v3 = acc[i][j][3] + bias[j].w;
        if constexpr (EPI == EPI_F32) {
          store4((float*)a.C + (int64_t)row * a.ldc + col, v0, v1, v2, v3);
        } else if constexpr (EPI == EPI_ACT) {
          if constexpr (__is_same(T, f16_t)) amax = absmax4(amax, v0, v1, v2, v3);
          store4((T*)a.C + (int64_t)row * a.ldc + col, v0, v1, v2, v3);
        } else if constexpr (EPI == EPI_GELU) {
          const float g0 = gelu_ab(acc[i][j][0], bias[j].x), g1 = gelu_ab(acc[i][j][1], bias[j].y);
          const float g2 = gelu_ab(acc[i][j][2], bias[j].z), g3 = gelu_ab(acc[i][j][3], bias[j].w);
          if constexpr (__is_same(T, f16_t)) amax = absmax4(amax, g0, g1, g2, g3);
          store4((T*)a.C + (int64_t)row * a.ldc + col, g0, g1, g2, g3);
        } else if constexpr (EPI == EPI_GELU_SPLIT) {
          const float g4[4] = {gelu_ab(acc[i][j][0], bias[j].x), gelu_ab(acc[i][j][1], bias[j].y),
                               gelu_ab(acc[i][j][2], bias[j].z), gelu_ab(acc[i][j][3], bias[j].w)};
          if constexpr (__is_same(T, f16_t)) amax = absmax4(amax, g4[0], g4[1], g4[2], g4[3]);
          float lo[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) lo[e] = g4[e] - Elem<T>::to_f(Elem<T>::from_f(g4[e]));
          T* C = (T*)a.C + (int64_t)row * a.ldc;
          store4(C + col, g4[0], g4[1], g4[2], g4[3]);
          store4(C + a.N + col, lo[0], lo[1], lo[2], lo[3]);
        } else if constexpr (EPI == EPI_RESID) {
          float4* R = (float4*)((float*)a.C + (int64_t)row * a.ldc + col);
          float4 r = *R;
          r.x += v0;
          r.y += v1;
          r.z += v2;
          r.w += v3;
          *R = r;
        } else if constexpr (PE) {
          // EPI_PE: the bias-free conv_out plus sinusoids; EPI_GELU_PE: the
          // last convolution's GELU(acc + bias) plus sinusoids
          const int half = a.N / 2;
          const float hb[4] = {bias[j].x, bias[j].y, bias[j].z, bias[j].w};  // halved (GELU) or bias-free
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // angle in revolutions, reduced to [-1/2, 1/2] in double; the
            // hardware sine / cosine take revolutions (max error 1.2e-7 on
            // this range, as for sinf of the angle rounded to float)
            double rev = (double)pos * tau[4 * j + e];
            rev -= rint(rev);
            const float fr = (float)rev;
            o[e] = (EPI == EPI_GELU_PE ? gelu_ab(acc[i][j][e], hb[e]) : acc[i][j][e]) +
                   (col + e < half ? __builtin_amdgcn_sinf(fr) : __builtin_amdgcn_cosf(fr));
          }
          store4((float*)a.C + (int64_t)row * a.ldc + col, o[0], o[1], o[2], o[3]);
        } else if constexpr (EPI == EPI_OUT) {
          store4((float*)a.C + orow * a.ldc + col, v0, v1, v2, v3);
        }
      }
    }
  }
  if constexpr (__is_same(T, f16_t) &&
                (EPI == EPI_ACT || EPI == EPI_GELU || EPI == EPI_GELU_SPLIT || EPI == EPI_SWIGLU))
    report_saturation(a.sat, a.sat_bit, amax);
}

// EPI_RESID with the residual tile already in registers (R[i][j] = C at the
// accumulator's place, read before the main loop): C = R + (acc + bias), the
// same arithmetic as epilogue4.
template <int MI, int NI>
__device__ __forceinline__ void epilogue_resid_pre(const GemmArgs& a, f32x4 (&acc)[MI][NI],
                                                   const float4 (&R)[MI][NI], const int rbase, const int cbase) {
  float4 bias[NI];
  load_bias<NI>(a, cbase, bias);
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int row = rbase + 16 * i;
    if (row >= a.M) continue;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int col = cbase + 16 * j;
      if (col >= a.N) continue;
      float4 r = R[i][j];
      r.x += acc[i][j][0] + bias[j].x;
      r.y += acc[i][j][1] + bias[j].y;
      r.z += acc[i][j][2] + bias[j].z;
      r.w += acc[i][j][3] + bias[j].w;
      *(float4*)((float*)a.C + (int64_t)row * a.ldc + col) = r;
    }
  }
}

template <typename T, int BM, int BN, int EPI, bool CONV>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a) {
  constexpr int NT = 256;
  constexpr int WTM = BM / 2, WTN = BN / 2;
  constexpr int MI = WTM / 16, NI = WTN / 16;
  constexpr int EPC = Elem<T>::per16;
  constexpr int BK = 8 * EPC;  // elements per 128-byte slice
  constexpr int RPP = NT / 8;  // rows covered per load pass
  constexpr int AP = BM / RPP, BP = BN / RPP;
  static_assert(BM % RPP == 0 && BN % RPP == 0, "tile rows must be multiples of 32");
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be 16-aligned");
  static_assert(EPI != EPI_SWIGLU || (WTN % 32) == 0, "SwiGLU pairs need 32-column wave tiles");

  __shared__ uint4 lds[2][(BM + BN) * 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_n = (a.N + BN - 1) / BN;
  const int bm = blockIdx.x / tiles_n, bn = blockIdx.x % tiles_n;
  const int m0 = bm * BM, n0 = bn * BN;
  const int c = tid & 7;
  const int r0 = tid >> 3;

  const char* Ab = (const char*)a.A;
  const char* Bb = (const char*)a.B;
  const int64_t ldab = a.lda * (int64_t)sizeof(T);
  const int64_t ldbb = a.ldb * (int64_t)sizeof(T);

  // ---- per-row load state
  ConvRow cr[CONV ? AP : 1];
  bool arow_ok[AP];
#pragma unroll
  for (int i = 0; i < AP; ++i) {
    const int m = m0 + r0 + i * RPP;
    arow_ok[i] = m < a.M;
    if constexpr (CONV) {
      const int mm = arow_ok[i] ? m : 0;
      const int t_glob = mm / a.conv_Fout;
      const int fo = mm - t_glob * a.conv_Fout;
      const int sq = find_seq(a.cu_out, a.nseq, t_glob);
      const int tl = t_glob - a.cu_out[sq];
      const int tin_base = a.cu_in[sq];
      cr[i].base = Ab + (int64_t)tin_base * a.conv_Fin * a.conv_C * (int64_t)sizeof(T);
      cr[i].t0 = 2 * tl - 1;
      cr[i].f0 = 2 * fo - 1;
      cr[i].Tin = a.cu_in[sq + 1] - tin_base;
    }
  }
  bool brow_ok[BP];
#pragma unroll
  for (int j = 0; j < BP; ++j) brow_ok[j] = (n0 + r0 + j * RPP) < a.N;

  // K split (fp32 products with few output tiles): this workgroup sums the
  // K steps [kb0, kb1) of its tile and leaves the partial sums to
  // gemm_split_sum_kernel.
  const int nkb_all = (a.K + BK - 1) / BK;
  const int nz = gridDim.y, kz = blockIdx.y;
  const int kb0 = (int)((int64_t)nkb_all * kz / nz), kb1 = (int)((int64_t)nkb_all * (kz + 1) / nz);

  // convolution: track (tap, channel) of this thread's chunk incrementally
  int ctap = 0, cch = 0;
  if constexpr (CONV) {
    const int k0 = kb0 * BK + c * EPC;
    ctap = k0 / a.conv_C;
    cch = k0 - ctap * a.conv_C;
  }

  uint4 ra[AP], rb[BP];
  auto gload = [&](int kb) {
    const int k = kb * BK + c * EPC;
    const bool kok = k < a.K;
#pragma unroll
    for (int i = 0; i < AP; ++i) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if constexpr (CONV) {
        const int df = ctap / 3, dt = ctap - 3 * (ctap / 3);
        const int t = cr[i].t0 + dt, f = cr[i].f0 + df;
        if (kok && arow_ok[i] && t >= 0 && t < cr[i].Tin && f >= 0 && f < a.conv_Fin) {
          const int64_t off = (((int64_t)t * a.conv_Fin + f) * a.conv_C + cch) * (int64_t)sizeof(T);
          v = *(const uint4*)(cr[i].base + off);
        }
      } else {
        if (kok && arow_ok[i]) {
          const int m = m0 + r0 + i * RPP;
          v = *(const uint4*)(Ab + (int64_t)m * ldab + (int64_t)k * sizeof(T));
        }
      }
      ra[i] = v;
    }
#pragma unroll
    for (int j = 0; j < BP; ++j) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (kok && brow_ok[j]) {
        const int n = n0 + r0 + j * RPP;
        v = *(const uint4*)(Bb + (int64_t)n * ldbb + (int64_t)k * sizeof(T));
      }
      rb[j] = v;
    }
    if constexpr (CONV) {
      cch += BK;
      while (cch >= a.conv_C) { cch -= a.conv_C; ++ctap; }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < AP; ++i) {
      const int r = r0 + i * RPP;
      lds[buf][r * 8 + (c ^ swz(r))] = ra[i];
    }
#pragma unroll
    for (int j = 0; j < BP; ++j) {
      const int r = r0 + j * RPP;
      lds[buf][(BM + r) * 8 + (c ^ swz(r))] = rb[j];
    }
  };

  f32x4 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  gload(kb0);
  sstore(0);
  __syncthreads();

  const int g = lane >> 4;
  const int l16 = lane & 15;
  for (int kb = kb0; kb < kb1; ++kb) {
    const int buf = (kb - kb0) & 1;
    if (kb + 1 < kb1) gload(kb + 1);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int cc = 4 * s + g;
      uint4 af[MI], bfr[NI];
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int r = wm * WTM + i * 16 + l16;
        af[i] = lds[buf][r * 8 + (cc ^ swz(r))];
      }
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int r = wn * WTN + j * 16 + l16;
        bfr[j] = lds[buf][(BM + r) * 8 + (cc ^ swz(r))];
      }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) mma_chunk<T>(acc[i][j], bfr[j], af[i]);  // C^T tile
    }
    if (kb + 1 < kb1) sstore(buf ^ 1);
    __syncthreads();
  }

  if (nz > 1) {
    // partial sums as [split][tile][wavefront][i][j][lane] float4, added up
    // in split order by gemm_split_sum_kernel
    constexpr int PER = MI * NI * 64;  // float4 per wavefront and split
    float4* mine = (float4*)a.part + (((int64_t)kz * gridDim.x + blockIdx.x) * 4 + wave) * PER + lane;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
        mine[(i * NI + j) * 64] = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
    return;
  }

  // ---- epilogue: lane holds C[l16][4g + e] of every 16 x 16 tile
  epilogue4<T, EPI, MI, NI>(a, acc, m0 + wm * WTM + l16, n0 + wn * WTN + 4 * g);
}

// The second half of a K-split product (gemm_kernel with gridDim.y = nz >
// 1): per output tile, the nz partial sums added in split order (the same
// order every time), then the product's epilogue.
template <typename T, int BM, int BN, int EPI>
__global__ __launch_bounds__(256) void gemm_split_sum_kernel(GemmArgs a, int nz) {
  constexpr int WTM = BM / 2, WTN = BN / 2;
  constexpr int MI = WTM / 16, NI = WTN / 16;
  constexpr int PER = MI * NI * 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_n = (a.N + BN - 1) / BN;
  const int bm = blockIdx.x / tiles_n, bn = blockIdx.x % tiles_n;
  const int m0 = bm * BM, n0 = bn * BN;
  const int g = lane >> 4, l16 = lane & 15;
  f32x4 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int z = 0; z < nz; ++z) {
    const float4* pz = (const float4*)a.part + (((int64_t)z * gridDim.x + blockIdx.x) * 4 + wave) * PER + lane;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const float4 v = pz[(i * NI + j) * 64];
        acc[i][j][0] += v.x;
        acc[i][j][1] += v.y;
        acc[i][j][2] += v.z;
        acc[i][j][3] += v.w;
      }
  }
  epilogue4<T, EPI, MI, NI>(a, acc, m0 + wm * WTM + l16, n0 + wn * WTN + 4 * g);
}


// ---------------------------------------------------------------------------
// 16-bit operands: WM x WN wavefronts, BM x BN tile, K slices of 64 copied
// global -> LDS by the matrix-load DMA (global_load_lds_dwordx4: lane j of a
// wavefront writes bytes [16 j, 16 j + 16) of a 1 KB LDS block), two or
// four LDS stages.  The next slices are in flight while slice kb feeds the
// matrix cores; each wavefront waits only for its own earlier loads (vmcnt)
// before the barrier that publishes a stage.  Loads that fall outside the matrices
// (row or K tails, convolution padding) read a 16-byte block of zeros.
// Rows of a stage: A rows [0, BM), then B rows [BM, BM + BN); 128 bytes each,
// chunk c of row r stored at chunk slot c ^ swz(r).

typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <typename T, int BM, int BN, int WM, int WN, int NST, int EPI, bool CONV>
__global__ __launch_bounds__(WM * WN * 64, 1) void gemm_lds_kernel(GemmArgs a) {
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MI = WTM / 16, NI = WTN / 16;
  constexpr int ROWS = BM + BN;
  constexpr int NBLK = ROWS / 8;               // 1 KB blocks per stage
  constexpr int BPW = (NBLK + NW - 1) / NW;    // blocks per wavefront (the last may be idle)
  static_assert(sizeof(T) == 2, "16-bit operands only");
  static_assert(BM % 16 == 0 && BN % 16 == 0 && ROWS % 8 == 0, "tile shape");
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be 16-aligned");
  static_assert(EPI != EPI_SWIGLU || (WTN % 32) == 0, "SwiGLU pairs need 32-column wave tiles");
  static_assert(BPW <= 16, "too many loads per wavefront");
  static_assert(NST == 2 || NST == 4, "two or four LDS stages");

  __shared__ uint4 st0[ROWS * 8];
  __shared__ uint4 st1[ROWS * 8];
  __shared__ uint4 st2[NST == 4 ? ROWS * 8 : 1];
  __shared__ uint4 st3[NST == 4 ? ROWS * 8 : 1];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int tiles_n = (a.N + BN - 1) / BN;
  const int bm = blockIdx.x / tiles_n, bn = blockIdx.x % tiles_n;
  const int m0 = bm * BM, n0 = bn * BN;
  const char* zeros = (const char*)a.zeros;

  // ---- load plan.  Block blk (8 rows x 8 chunks) is loaded by wavefront
  // blk % NW; lane j of it fills LDS row 8 blk + j / 8, chunk slot j % 8.  So
  // this lane's rows are r0 + RPI * i (i = 0 .. BPW-1), and since swz depends
  // only on r % 16 it loads the same logical chunk c in all of them.
  constexpr int RPI = NW * 8;                  // rows per load round
  constexpr int AI = BM / RPI;                 // rounds that fill A rows
  static_assert(BM % RPI == 0, "A rows must fill whole load rounds");
  const int r0 = wave * 8 + (lane >> 3);
  const int c = (lane & 7) ^ swz(r0);
  const int64_t ldab = a.lda * (int64_t)sizeof(T), ldbb = a.ldb * (int64_t)sizeof(T);
  const char* a_base = (const char*)a.A + (int64_t)(m0 + r0) * ldab + c * 16;
  const char* b_base = (const char*)a.B + (int64_t)(n0 + r0) * ldbb + c * 16;
  const int64_t a_step = RPI * ldab, b_step = RPI * ldbb;
  uint32_t a_ok = 0, b_ok = 0;  // bit i: row of load round i inside the matrix
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    if (m0 + r0 + RPI * i < a.M) a_ok |= 1u << i;
    if (n0 + r0 + RPI * i < a.N) b_ok |= 1u << i;
  }
  int nblk = 0;
#pragma unroll
  for (int i = 0; i < BPW; ++i) nblk += (wave + i * NW < NBLK) ? 1 : 0;

  ConvRow cr[CONV ? AI : 1];
  int ctap = 0, cch = c * 8;  // (tap, channel) of this lane's chunk in the current slice
  if constexpr (CONV) {
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      const int m = m0 + r0 + RPI * i;
      const bool ok = m < a.M;
      const int mm = ok ? m : 0;
      const int t_glob = mm / a.conv_Fout;
      const int fo = mm - t_glob * a.conv_Fout;
      const int sq = find_seq(a.cu_out, a.nseq, t_glob);
      const int tl = t_glob - a.cu_out[sq];
      const int tin_base = a.cu_in[sq];
      cr[i].base = (const char*)a.A + (int64_t)tin_base * a.conv_Fin * a.conv_C * (int64_t)sizeof(T);
      cr[i].t0 = ok ? 2 * tl - 1 : -(1 << 28);  // rows past M never pass the time test
      cr[i].f0 = 2 * fo - 1;
      cr[i].Tin = a.cu_in[sq + 1] - tin_base;
    }
  }

  auto issue = [&](uint4* stage, int kb) {
    const bool kok = kb * 64 + c * 8 < a.K;
    int df = 0, dt = 0;
    if constexpr (CONV) {
      df = ctap / 3;
      dt = ctap - 3 * df;
    }
    const char* pa = a_base + kb * 128;
    const char* pb = b_base + kb * 128;
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int blk = wave + i * NW;
      if (i * NW >= NBLK) break;  // no wavefront has this round
      const char* p = zeros;
      if (i < AI) {
        if constexpr (CONV) {
          const int t = cr[i].t0 + dt, f = cr[i].f0 + df;
          if (kok && t >= 0 && t < cr[i].Tin && f >= 0 && f < a.conv_Fin)
            p = cr[i].base + (((int64_t)t * a.conv_Fin + f) * a.conv_C + cch) * (int64_t)sizeof(T);
        } else {
          p = (kok && ((a_ok >> i) & 1)) ? pa : zeros;
          pa += a_step;
        }
      } else {
        p = (kok && ((b_ok >> (i - AI)) & 1)) ? pb : zeros;
        pb += b_step;
      }
      if (blk < NBLK)
        __builtin_amdgcn_global_load_lds((const void*)p, (lds_ptr_t)(stage + blk * 64), 16, 0, 0);
    }
    if constexpr (CONV) {
      cch += 64;
      while (cch >= a.conv_C) { cch -= a.conv_C; ++ctap; }
    }
  };

  f32x4 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- main loop.  A 64-wide K slice is two 32-wide MFMA steps; their
  // operand fragments alternate between two register sets so that the LDS
  // reads of one step overlap the matrix-core work of the other.  One barrier
  // per slice publishes the next slice (all wavefronts' DMA landed) and
  // retires the slice whose stage is refilled next.
  const int g = lane >> 4, l16 = lane & 15;
  uint4 fa0[MI], fb0[NI], fa1[MI], fb1[NI];
  auto ldfrag = [&](const uint4* stage, int s2, uint4 (&fa)[MI], uint4 (&fb)[NI]) {
    const int cc = 4 * s2 + g;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int r = wm * WTM + i * 16 + l16;
      fa[i] = stage[r * 8 + (cc ^ swz(r))];
    }
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int r = BM + wn * WTN + j * 16 + l16;
      fb[j] = stage[r * 8 + (cc ^ swz(r))];
    }
  };
  // MFMAs of rows [i0, i1) of the wave tile
  auto mma = [&](const uint4 (&fa)[MI], const uint4 (&fb)[NI], int i0, int i1) {
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      if (i < i0 || i >= i1) continue;
#pragma unroll
      for (int j = 0; j < NI; ++j) mma16(acc[i][j], fb[j], fa[i], T{});  // C^T tile
    }
  };

  // NST LDS stages: slice kb lives in stage kb % NST, and once its stage is
  // free slice kb + NST is requested, NST - 1 slices ahead of its use (four
  // stages for few rows: their workgroups walk K with little matrix-core
  // work per slice to cover the loads).  The slice count is padded to a
  // multiple of NST (a slice past K loads zeros and adds nothing) and the
  // last slice is peeled off, so the loop body has no branch that touches
  // the accumulators (the register allocator keeps them in place).  Phases
  // are pinned with sched_barrier: the compiler would otherwise wait for all
  // outstanding LDS reads before the first MFMA of a phase and hoist the DMA
  // address arithmetic in front of the matrix-core work.
  constexpr int MH = MI / 2;
  const int nkb = (a.K + 64 * NST - 1) / (64 * NST) * NST;
  auto step = [&](int kb, const uint4* CUR, const uint4* NXT) {  // kb + 1 < nkb
    mma(fa0, fb0, 0, MH);              // k-step 0 of slice kb (read during the last phase)
    __builtin_amdgcn_sched_barrier(0);
    ldfrag(CUR, 1, fa1, fb1);          // k-step 1 of slice kb, behind the MFMAs
    __builtin_amdgcn_sched_barrier(0);
    mma(fa0, fb0, MH, MI);
    __builtin_amdgcn_sched_barrier(0);
    // this wavefront's DMA of slice kb+1 has landed (slices kb+2 .. kb+NST-1
    // may still be in flight)
    wait_vm(nblk * max(0, min(nkb - kb - 2, NST - 2)));
    __builtin_amdgcn_s_waitcnt((0 << 8) | (7 << 4) | 15 | (3 << 14));  // lgkmcnt(0): reads of CUR done
    __builtin_amdgcn_s_barrier();      // every wavefront's has; CUR is no longer read
    __builtin_amdgcn_sched_barrier(0);
    ldfrag(NXT, 0, fa0, fb0);          // k-step 0 of slice kb+1
    __builtin_amdgcn_sched_barrier(0);
    mma(fa1, fb1, 0, MH);
    __builtin_amdgcn_sched_barrier(0);
    if (kb + NST < nkb) issue((uint4*)CUR, kb + NST);
    __builtin_amdgcn_sched_barrier(0);
    mma(fa1, fb1, MH, MI);
    __builtin_amdgcn_sched_barrier(0);
  };

  issue(st0, 0);
  issue(st1, 1);
  if constexpr (NST == 4) {
    issue(st2, 2);
    issue(st3, 3);
  }
  wait_vm(nblk * (NST - 1));
  __builtin_amdgcn_s_barrier();
  ldfrag(st0, 0, fa0, fb0);
  // unrolled by NST so that every LDS access names its stage array: the
  // compiler then sees that reads of one stage do not alias DMA into another
  if constexpr (NST == 2) {
    for (int kb = 0; kb < nkb - 2; kb += 2) {
      step(kb, st0, st1);
      step(kb + 1, st1, st0);
    }
    step(nkb - 2, st0, st1);
    ldfrag(st1, 1, fa1, fb1);            // last slice
  } else {
    for (int kb = 0; kb < nkb - 4; kb += 4) {
      step(kb, st0, st1);
      step(kb + 1, st1, st2);
      step(kb + 2, st2, st3);
      step(kb + 3, st3, st0);
    }
    step(nkb - 4, st0, st1);
    step(nkb - 3, st1, st2);
    step(nkb - 2, st2, st3);
    ldfrag(st3, 1, fa1, fb1);            // last slice
  }
  mma(fa0, fb0, 0, MI);
  mma(fa1, fb1, 0, MI);

  epilogue4<T, EPI, MI, NI>(a, acc, m0 + wm * WTM + l16, n0 + wn * WTN + 4 * g);
}

template <typename T, int BM, int BN, int WM, int WN, int NST, int EPI, bool CONV>
hipError_t run_lds(const GemmArgs& a, hipStream_t s) {
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_lds_kernel<T, BM, BN, WM, WN, NST, EPI, CONV>), dim3(tiles),
                     dim3(WM * WN * 64), 0, s, a);
  return hipGetLastError();
}


// Epilogue through LDS for 16-bit outputs (bias, optional GELU).  Written
// straight from the MFMA layout, each store instruction of a wavefront
// touches 16 rows x 32 bytes, and with every CU in its epilogue at once the
// partial-line writes, not the math, set the pace (measured ~7.7 us per
// 256 x 256 tile).  Instead each wavefront parks its converted fragments in
// LDS -- rows 64 q .. 64 q + 63 of the tile in stage q, 16-byte chunks
// XOR-swizzled by row -- and the workgroup then writes whole rows, 16 bytes
// per lane, so each instruction covers full 128-byte lines.
template <typename T, int EPI, int BN, int MI, int NI>
__device__ __forceinline__ void epilogue_staged4(const GemmArgs& a, f32x4 (&acc)[MI][NI], uint4* st0,
                                                uint4* st1, uint4* st2, uint4* st3, int m0, int n0,
                                                int wm, int wn) {
  auto stage = [&](int q) { return q == 0 ? st0 : q == 1 ? st1 : q == 2 ? st2 : st3; };
  static_assert(EPI == EPI_ACT || EPI == EPI_GELU, "16-bit outputs");
  static_assert(MI == 8 || MI == 4, "wave tiles of 128 or 64 rows");
  constexpr int WTM = MI * 16, WTN = NI * 16;
  constexpr int CPR = BN / 8;  // 16-byte chunks per output row
  static_assert(CPR % 4 == 0, "swizzle groups");
  constexpr int SWM = CPR % 8 == 0 ? 7 : 3;  // chunks are swizzled within aligned groups
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, l16 = lane & 15;
  float4 bias[NI];
  load_bias<NI>(a, n0 + wn * WTN + 4 * g, bias);
  halve_bias_for_gelu<EPI, NI>(bias);
  [[maybe_unused]] float amax = 0.f;  // fp16: largest |value| converted (saturation report)
  __syncthreads();  // every wavefront is done reading operand fragments
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int R = wm * WTM + 16 * i;  // first tile row of fragment row i
    char* qb = (char*)stage(R >> 6);
    const int r = (R & 63) + l16;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const float4 b = bias[j];
      const int q = (wn * WTN + 16 * j + 4 * g) >> 3;  // chunk of the 4 values
      float v0, v1, v2, v3;
      if constexpr (EPI == EPI_GELU) {
        v0 = gelu_ab(acc[i][j][0], b.x);
        v1 = gelu_ab(acc[i][j][1], b.y);
        v2 = gelu_ab(acc[i][j][2], b.z);
        v3 = gelu_ab(acc[i][j][3], b.w);
      } else {
        v0 = acc[i][j][0] + b.x;
        v1 = acc[i][j][1] + b.y;
        v2 = acc[i][j][2] + b.z;
        v3 = acc[i][j][3] + b.w;
      }
      if constexpr (__is_same(T, f16_t)) amax = absmax4(amax, v0, v1, v2, v3);
      const uint2 w = make_uint2(pack2f<T>(v0, v1), pack2f<T>(v2, v3));
      *(uint2*)(qb + r * (BN * 2) + ((q ^ (r & SWM)) << 4) + ((g & 1) << 3)) = w;
    }
  }
  if constexpr (__is_same(T, f16_t)) report_saturation(a.sat, a.sat_bit, amax);
  __syncthreads();
  // 64 rows x CPR chunks per stage, 512 threads
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const char* src = (const char*)stage(h);
#pragma unroll
    for (int it = 0; it < (64 * CPR + 511) / 512; ++it) {
      const int t = it * 512 + threadIdx.x;
      if (t < 64 * CPR) {
        const int r = t / CPR, q = t % CPR;
        const int row = m0 + 64 * h + r, col = n0 + 8 * q;
        const uint4 v = *(const uint4*)(src + r * (BN * 2) + ((q ^ (r & SWM)) << 4));
        if (row < a.M && col < a.N) *(uint4*)((T*)a.C + (int64_t)row * a.ldc + col) = v;
      }
    }
  }
}

// Epilogue through LDS for 16-bit outputs (bias, optional GELU), two-stage
// variant (rows 0-127 of the tile in stage 0, 128-255 in stage 1).  Written
// straight from the MFMA layout, each store instruction of a wavefront
// touches 16 rows x 32 bytes, and with every CU in its epilogue at once the
// partial-line writes, not the math, set the pace (measured ~7.7 us per
// 256 x 256 tile).  Instead each wavefront parks its converted fragments in
// LDS (rows 0-127 of the tile in stage 0, 128-255 in stage 1; 16-byte
// chunks XOR-swizzled by row), and the workgroup then writes whole rows,
// 16 bytes per lane, so each instruction covers full 128-byte lines.
template <typename T, int EPI, int BN, int MI, int NI>
__device__ __forceinline__ void epilogue_staged2(const GemmArgs& a, f32x4 (&acc)[MI][NI], uint4* st0,
                                                uint4* st1, int m0, int n0, int wm, int wn) {
  static_assert(EPI == EPI_ACT || EPI == EPI_GELU, "16-bit outputs");
  static_assert(MI == 8 || MI == 4, "wave tiles of 128 or 64 rows");
  constexpr int WTM = MI * 16, WTN = NI * 16;
  constexpr int WPS = 128 / WTM;  // wavefront rows per LDS stage
  constexpr int CPR = BN / 8;  // 16-byte chunks per output row
  static_assert(CPR % 4 == 0, "swizzle groups");
  constexpr int SWM = CPR % 8 == 0 ? 7 : 3;  // chunks are swizzled within aligned groups
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, l16 = lane & 15;
  uint4* half = wm / WPS ? st1 : st0;
  char* hb = (char*)half;
  const int rw = (wm % WPS) * WTM;  // first row of this wavefront inside its stage
  float4 bias[NI];
  load_bias<NI>(a, n0 + wn * WTN + 4 * g, bias);
  halve_bias_for_gelu<EPI, NI>(bias);
  [[maybe_unused]] float amax = 0.f;  // fp16: largest |value| converted (saturation report)
  __syncthreads();  // every wavefront is done reading operand fragments
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const float4 b = bias[j];
    const int q = (wn * WTN + 16 * j + 4 * g) >> 3;  // chunk of the 4 values
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int r = rw + 16 * i + l16;
      float v0, v1, v2, v3;
      if constexpr (EPI == EPI_GELU) {
        v0 = gelu_ab(acc[i][j][0], b.x);
        v1 = gelu_ab(acc[i][j][1], b.y);
        v2 = gelu_ab(acc[i][j][2], b.z);
        v3 = gelu_ab(acc[i][j][3], b.w);
      } else {
        v0 = acc[i][j][0] + b.x;
        v1 = acc[i][j][1] + b.y;
        v2 = acc[i][j][2] + b.z;
        v3 = acc[i][j][3] + b.w;
      }
      if constexpr (__is_same(T, f16_t)) amax = absmax4(amax, v0, v1, v2, v3);
      const uint2 w = make_uint2(pack2f<T>(v0, v1), pack2f<T>(v2, v3));
      *(uint2*)(hb + r * (BN * 2) + ((q ^ (r & SWM)) << 4) + ((g & 1) << 3)) = w;
    }
  }
  if constexpr (__is_same(T, f16_t)) report_saturation(a.sat, a.sat_bit, amax);
  __syncthreads();
  // 128 rows x CPR chunks per stage, 512 threads
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const char* src = (const char*)(h ? st1 : st0);
#pragma unroll
    for (int it = 0; it < 128 * CPR / 512; ++it) {
      const int t = it * 512 + threadIdx.x;
      const int r = t / CPR, q = t % CPR;
      const int row = m0 + 128 * h + r, col = n0 + 8 * q;
      const uint4 v = *(const uint4*)(src + r * (BN * 2) + ((q ^ (r & SWM)) << 4));
      if (row < a.M && col < a.N) *(uint4*)((T*)a.C + (int64_t)row * a.ldc + col) = v;
    }
  }
}

// ---------------------------------------------------------------------------
// Large tiles: 256 x BN (BN = 256, 192 or 128), eight wavefronts of
// 128 x BN/4, one workgroup per CU (two wavefronts per SIMD).
//
// Why: with 128 x 128 tiles the per-CU vector-memory path that feeds the
// LDS (one 1 KB global_load_lds per 16-plus cycles) is busy for ~1.75 cycles
// per matrix-core cycle, so the tile, not the matrix cores, sets the pace.
// A 256 x 256 tile moves half the bytes per FLOP.  The accumulators
// (128 per lane at BN = 256) stay in AGPRs; A fragments are single-buffered
// and refilled row by row right behind the MFMAs that last read them, B
// fragments are double-buffered across K steps, and the second wavefront on
// each SIMD covers the LDS latency the first one waits on.
template <typename T, int BN, int WM, int EPI, bool CONV>
__global__ __launch_bounds__(512, 1) void gemm_w8_kernel(GemmArgs a) {
  constexpr int BM = 256, NW = 8, WN = NW / WM;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MI = WTM / 16, NI = WTN / 16;
  constexpr int RPI = NW * 8;     // rows per load round
  constexpr int BNP = (BN + RPI - 1) / RPI * RPI;  // B rows loaded (the rest of the
                                                   // last round: next tile's, unused)
  constexpr int ROWS = BM + BNP;
  constexpr int NBLK = ROWS / 8;  // 1 KB blocks per stage
  constexpr int BPW = NBLK / NW;  // blocks per wavefront
  constexpr int AI = BM / RPI;    // rounds that load A rows
  static_assert(sizeof(T) == 2, "16-bit operands");
  static_assert(MI == 8 || MI == 4, "128- or 64-row wave tiles");
  static_assert(NBLK % NW == 0 && BM % RPI == 0, "load plan");
  static_assert(WTN % 16 == 0, "wave tile");
  static_assert(EPI != EPI_SWIGLU || (WTN % 32) == 0, "SwiGLU pairs need 32-column wave tiles");

  __shared__ uint4 st0[ROWS * 8];
  __shared__ uint4 st1[ROWS * 8];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int tiles_n = (a.N + BN - 1) / BN;
  // Workgroups are dealt to the 8 XCDs (each with its own L2) round-robin.
  // Renumber so that each XCD runs a contiguous range of tiles, ordered in
  // groups of 4 rows of A: the ~32 tiles an XCD runs at once then cover
  // about 4 A rows x 8 B columns of tiles, whose K slices its L2 shares,
  // instead of ~13 x 5 (fc1, counters: 197 MB fetched from the fabric per
  // launch before, for 28.5 MB of operands).
  int tile = blockIdx.x;
  {
    const int nt = gridDim.x, q = nt / 8, r = nt % 8, x = tile % 8, idx = tile / 8;
    tile = (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + idx;
  }
  constexpr int GM = 4;
  const int tiles_m = (a.M + BM - 1) / BM;
  const int grp = tile / (GM * tiles_n), gw = tile - grp * (GM * tiles_n);
  const int grows = min(GM, tiles_m - grp * GM);
  const int bm = grp * GM + gw % grows, bn = gw / grows;
  const int m0 = bm * BM, n0 = bn * BN;

  // DMA plan: block (wave + NW i) holds LDS rows r0 + RPI i; rows < BM are
  // A rows, the rest B rows.  Lane j fills chunk slot j % 8 of its row with
  // logical chunk c (the slot XOR the row's swizzle, the same for all i).
  // Loads go through buffer descriptors, one per round i, based at row
  // RPI i of the operand and sized to the rows that remain, so rows past M
  // or N read as zeros and a single offset register serves every round.  K
  // is a multiple of 128 (checked by the caller): no slice runs past a row's
  // end.  32-bit offsets: the caller also checks that each operand spans
  // less than 2 GiB.
  const int r0 = wave * 8 + (lane >> 3);
  const int c = (lane & 7) ^ swz(r0);
  const int ldab = a.lda * (int)sizeof(T), ldbb = a.ldb * (int)sizeof(T);
  const int va = (m0 + r0) * ldab + c * 16;
  const int vb = (n0 + r0) * ldbb + c * 16;

  // Implicit-GEMM convolution (3x3, stride 2, padding 1, channels-last
  // input [t][f][C]): A row m is output position (t, f) = (m / Fout, m %
  // Fout) of its sequence and A column k is tap k / C (= 3 df + dt), channel
  // k % C.  C is a multiple of 8, so each lane's 16-byte chunk lies inside one
  // tap; lanes of one K slice may straddle two.  One descriptor per
  // workgroup, based at the first input time row the tile can touch and
  // ending at the end of the input; a tap outside the sequence or the
  // frequency range, and k >= K in the last slice, get an offset past the
  // end and read zeros.
  int cv_off[CONV ? AI : 1];        // input position (2t, 2f) of the row, bytes from the base
  uint32_t cv_ok[CONV ? AI : 1];    // bit dt: time tap dt inside; bit 3 + df: frequency tap df inside
  const char* cv_base = nullptr;
  int cv_bytes = 0;
  if constexpr (CONV) {
    const int pos_b = a.conv_C * (int)sizeof(T);  // bytes per input position
    const int tg0 = m0 / a.conv_Fout;
    const int sq0 = find_seq(a.cu_out, a.nseq, tg0);
    const int t_base = a.cu_in[sq0] + max(2 * (tg0 - a.cu_out[sq0]) - 1, 0);
    const int64_t row_b = (int64_t)a.conv_Fin * pos_b;
    cv_base = (const char*)a.A + t_base * row_b;
    const int64_t left = ((int64_t)a.cu_in[a.nseq] - t_base) * row_b;
    cv_bytes = (int)min(left, (int64_t)0x7fffffff);
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      const int m = m0 + r0 + RPI * i;
      cv_off[i] = 0;
      cv_ok[i] = 0;
      if (m < a.M) {
        const int tg = m / a.conv_Fout, f2 = m - tg * a.conv_Fout;
        const int sq = find_seq(a.cu_out, a.nseq, tg);
        const int t2 = tg - a.cu_out[sq], Tin = a.cu_in[sq + 1] - a.cu_in[sq];
        cv_off[i] = (int)((((int64_t)a.cu_in[sq] + 2 * t2 - t_base) * a.conv_Fin + 2 * f2) * pos_b);
#pragma unroll
        for (int d = 0; d < 3; ++d) {
          if (2 * t2 + d - 1 >= 0 && 2 * t2 + d - 1 < Tin) cv_ok[i] |= 1u << d;
          if (2 * f2 + d - 1 >= 0 && 2 * f2 + d - 1 < a.conv_Fin) cv_ok[i] |= 8u << d;
        }
      }
    }
  }

  auto issue = [&](uint4* stage, int kb) {
    int cdelta = 0;
    uint32_t need = 0;
    if constexpr (CONV) {
      const int k = kb * 64 + c * 8;  // first column of this lane's chunk
      const int tap = k / a.conv_C, ch = k - tap * a.conv_C;
      const int df = tap / 3, dt = tap - 3 * df;
      cdelta = ((dt - 1) * a.conv_Fin + (df - 1)) * a.conv_C * (int)sizeof(T) + ch * (int)sizeof(T);
      need = k < a.K ? (1u << dt) | (8u << df) : 0xffffffffu;  // past K: never satisfied
    }
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const bool isa = i < AI;
      if (CONV && isa) {
        const uint32_t voff = (cv_ok[CONV ? i : 0] & need) == need ? (uint32_t)(cv_off[CONV ? i : 0] + cdelta)
                                                                   : 0x80000000u;  // past any descriptor
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            __builtin_amdgcn_make_buffer_rsrc((void*)cv_base, (short)0, cv_bytes, 0x00020000),
            (lds_ptr_t)(stage + (wave + i * NW) * 64), 16, (int)voff, 0, 0, 0);
        continue;
      }
      const int row = (isa ? i : i - AI) * RPI;
      const int rows = (isa ? a.M : a.N) - row;
      const int ld = isa ? ldab : ldbb;
      const char* base = (const char*)(isa ? a.A : a.B) + (int64_t)row * ld;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, rows > 0 ? rows * ld : 0, 0x00020000),
          (lds_ptr_t)(stage + (wave + i * NW) * 64), 16, isa ? va : vb, kb * 128, 0, 0);
    }
  };

  f32x4 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int g = lane >> 4, l16 = lane & 15;
  const int sw = swz(l16);
  // fragment of K step s (chunk 4 s + g) of tile row r: r % 8 == l16 % 8
  auto a_idx = [&](int i, int s) { return (wm * WTM + i * 16 + l16) * 8 + ((4 * s + g) ^ sw); };
  auto b_idx = [&](int j, int s) { return (BM + wn * WTN + j * 16 + l16) * 8 + ((4 * s + g) ^ sw); };

  uint4 fa[MI];
  uint4 fb0[NI], fb1[NI];

  // K step s of the slice in S with B fragments FB: MFMAs row by row, each
  // row's A fragment reloaded from (SN, sn) right after its last use, and
  // the next step's B fragments read into FBN halfway through.
  auto kstep = [&](const uint4 (&FB)[NI], uint4 (&FBN)[NI], const uint4* SN, int sn, bool more) {
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int j = 0; j < NI; ++j) mma16(acc[i][j], FB[j], fa[i], T{});  // C^T tile
      if (more) {
        fa[i] = SN[a_idx(i, sn)];
        if (i == MI / 2 - 1) {
#pragma unroll
          for (int j = 0; j < NI; ++j) FBN[j] = SN[b_idx(j, sn)];
        }
      }
    }
    // Interleave: each row's MFMAs, then that row's reload (left alone, the
    // scheduler batches every read after every MFMA, all wavefronts of the
    // workgroup do so in step, and the LDS reads stop overlapping the MFMAs).
    if (more) {
#define MT_ROW(NREAD)                                    \
  __builtin_amdgcn_sched_group_barrier(0x008, NI, 0);    \
  __builtin_amdgcn_sched_group_barrier(0x100, NREAD, 0);
      if constexpr (MI == 8) {
        MT_ROW(1) MT_ROW(1) MT_ROW(1) MT_ROW(1 + NI) MT_ROW(1) MT_ROW(1) MT_ROW(1) MT_ROW(1)
      } else {
        MT_ROW(1) MT_ROW(1 + NI) MT_ROW(1) MT_ROW(1)
      }
#undef MT_ROW
    }
  };
  // The barrier that hands slice kb+1 over and frees the stage of slice kb
  // for slice kb+2: every read of that stage has been issued by now.
  auto handover = [&](uint4* CUR, bool refill, int kb) {
    wait_vm(0);  // this wavefront's DMA of slice kb+1 has landed
    __builtin_amdgcn_s_waitcnt((0 << 8) | (7 << 4) | 15 | (3 << 14));  // lgkmcnt(0): reads done
    __builtin_amdgcn_s_barrier();
    if (refill) issue(CUR, kb + 2);
  };

  const int nkb = CONV ? (a.K + 127) / 128 * 2 : a.K / 64;  // even; conv pads with zero slices
  issue(st0, 0);
  issue(st1, 1);
  wait_vm(BPW);
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int i = 0; i < MI; ++i) fa[i] = st0[a_idx(i, 0)];
#pragma unroll
  for (int j = 0; j < NI; ++j) fb0[j] = st0[b_idx(j, 0)];

  // Slices kb (stage 0) and kb+1 (stage 1) per iteration; inside the loop
  // slices kb+2 and kb+3 exist, so the body has no branch.  The last two
  // slices are peeled.
  for (int kb = 0; kb < nkb - 2; kb += 2) {
    kstep(fb0, fb1, st0, 1, true);
    handover(st0, true, kb);
    kstep(fb1, fb0, st1, 0, true);
    kstep(fb0, fb1, st1, 1, true);
    handover(st1, true, kb + 1);
    kstep(fb1, fb0, st0, 0, true);
  }
  kstep(fb0, fb1, st0, 1, true);
  handover(st0, false, nkb - 2);
  kstep(fb1, fb0, st1, 0, true);
  kstep(fb0, fb1, st1, 1, true);
  kstep(fb1, fb0, st1, 0, false);

  static_assert(128 * BN * 2 <= ROWS * 128, "staged output fits a stage");
  if constexpr (EPI == EPI_ACT || EPI == EPI_GELU)
    epilogue_staged2<T, EPI, BN, MI, NI>(a, acc, st0, st1, m0, n0, wm, wn);
  else
    epilogue4<T, EPI, MI, NI>(a, acc, m0 + wm * WTM + l16, n0 + wn * WTN + 4 * g);
}

template <typename T, int BN, int EPI, int WM = 2, bool CONV = false>
hipError_t run_w8(const GemmArgs& a, hipStream_t s) {
  const int tiles = ((a.M + 255) / 256) * ((a.N + BN - 1) / BN);
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_w8_kernel<T, BN, WM, EPI, CONV>), dim3(tiles), dim3(512), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The same 256-row eight-wavefront design with K in slices of 32 (one MFMA
// K step) through four LDS stages, for the narrow outputs (N tiles of 128
// or 160: o-proj, fc2, the convolutions).  A slice's DMA is issued three
// steps before its fragments are read (global loads under full load take
// ~2 us, more than the ~1.5 us the two-stage pipeline of 64-wide slices
// gives them); the price is a barrier every K step instead of every two,
// which the wide tiles (32 MFMAs per wavefront per step) did not recover:
// measured per 16 x 30 s step, conv2 2.19 -> 1.98 ms, fc2 3.27 -> 3.08 ms,
// but fc1 3.09 -> 3.34 and qkv 2.05 -> 2.37, so those keep two stages.
// Rows are 64 bytes (4 chunks, chunk slot c ^ ((r >> 2) & 3)), so a
// slice's DMA is issued three steps before its fragments are read: global
// loads under full load take ~2 us, more than the 1.5 us that a two-stage
// pipeline of 64-wide slices left them.
template <typename T, int BN, int WM, int EPI, bool CONV>
__global__ __launch_bounds__(512, 1) void gemm_w8q_kernel(GemmArgs a) {
  constexpr int BM = 256, NW = 8, WN = NW / WM;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MI = WTM / 16, NI = WTN / 16;
  constexpr int RPB = 16;                          // rows per 1 KB block (64-byte rows)
  constexpr int RPI = NW * RPB;                    // rows per load round
  constexpr int AI = BM / RPI;                     // rounds that load A rows
  constexpr int BNP = (BN + RPB - 1) / RPB * RPB;  // B rows loaded
  constexpr int NBLK = (BM + BNP) / RPB;           // 1 KB blocks of operands per stage
  constexpr int BPW = (NBLK + NW - 1) / NW;        // blocks per wavefront (the last
                                                   // round's spare ones load zeros)
  constexpr int SROWS = BPW * NW * RPB;            // rows per stage
  static_assert(sizeof(T) == 2, "16-bit operands");
  static_assert(MI == 8 || MI == 4, "128- or 64-row wave tiles");
  static_assert(BM % RPI == 0, "load plan");
  static_assert(WTN % 16 == 0, "wave tile");
  static_assert(EPI != EPI_SWIGLU || (WTN % 32) == 0, "SwiGLU pairs need 32-column wave tiles");
  static_assert(64 * BN * 2 <= SROWS * 64, "a quarter of the staged output fits a stage");

  __shared__ uint4 st0[SROWS * 4];
  __shared__ uint4 st1[SROWS * 4];
  __shared__ uint4 st2[SROWS * 4];
  __shared__ uint4 st3[SROWS * 4];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar registers
  const int wm = wave / WN, wn = wave % WN;
  const int tiles_n = (a.N + BN - 1) / BN;
  // Workgroups are dealt to the 8 XCDs (each with its own L2) round-robin;
  // for narrow outputs (few N tiles per row of A) and the convolutions,
  // renumber so that each XCD runs a contiguous range of tiles (row-major:
  // the N tiles of one row of A, then the next row) and the A rows -- and,
  // for the convolution, the overlapping input rows -- stay in one L2
  // (measured: conv2 2.31 -> 2.19 ms, fc2 3.46 -> 3.30, o 1.21 -> 1.16 per
  // 16 x 30 s step; the wide GEMMs did not gain).
  int tile = blockIdx.x;
  if (CONV || BN < 192) {
    const int nt = gridDim.x, q = nt / 8, r = nt % 8, x = tile % 8, idx = tile / 8;
    tile = (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + idx;
  }
  const int bm = tile / tiles_n, bn = tile % tiles_n;
  const int m0 = bm * BM, n0 = bn * BN;

  // DMA plan: block (wave + NW i) of a stage holds LDS rows r0 + RPI i
  // (64-byte rows, 4 chunks of 8 elements); rows < BM are A rows, the next
  // BNP are B rows, the rest (spare blocks) receive zeros.  Lane j fills chunk
  // slot j % 4 of its row with logical chunk c = slot ^ swz(row), swz(r) =
  // (r >> 2) & 3, the same for all i; a 16-row fragment read of one chunk is
  // then conflict-free.  Loads go through buffer descriptors, one per round,
  // based at row RPI i of the operand and sized to the rows that remain, so
  // rows past M or N read as zeros and one offset register serves every
  // round.  K is a multiple of 128 (checked by the caller): no slice runs
  // past a row's end.  32-bit offsets: the caller also checks that each
  // operand spans less than 2 GiB.
  const int r0 = wave * RPB + (lane >> 2);
  const int c = (lane & 3) ^ ((r0 >> 2) & 3);
  const int ldab = a.lda * (int)sizeof(T), ldbb = a.ldb * (int)sizeof(T);
  const int va = (m0 + r0) * ldab + c * 16;
  const int vb = (n0 + r0) * ldbb + c * 16;

  // Implicit-GEMM convolution, channels-last input [t][f][C], padding 1.
  // CONV_2D_S2 (3x3, stride 2): A row m is output position (t, f) = (m /
  // Fout, m % Fout) of its sequence and A column k is tap k / C (= 3 df +
  // dt), channel k % C.  CONV_1D_S1 / CONV_1D_S2 (3 taps over time, stride 1
  // or 2, Fin = Fout = 1): tap k / C is dt and df is the centre.  C is a
  // multiple of 8, so each lane's 16-byte chunk lies inside one tap; lanes of
  // one K slice may straddle two.  One descriptor per workgroup, based at the
  // first input time row the tile can touch and ending at the end of the
  // input; a tap outside the sequence or the frequency range, and k >= K in
  // the last slices, get an offset past the end and read zeros.
  [[maybe_unused]] const bool one_d = a.conv_kind != CONV_2D_S2;
  [[maybe_unused]] const int tstride = a.conv_kind == CONV_1D_S1 ? 1 : 2;
  int cv_off[CONV ? AI : 1];        // input position (s t, 2f) of the row, bytes from the base
  uint32_t cv_ok[CONV ? AI : 1];    // bit dt: time tap dt inside; bit 3 + df: frequency tap df inside
  const char* cv_base = nullptr;
  int cv_bytes = 0;
  if constexpr (CONV) {
    const int pos_b = a.conv_C * (int)sizeof(T);  // bytes per input position
    const int tg0 = m0 / a.conv_Fout;
    const int sq0 = find_seq(a.cu_out, a.nseq, tg0);
    const int t_base = a.cu_in[sq0] + max(tstride * (tg0 - a.cu_out[sq0]) - 1, 0);
    const int64_t row_b = (int64_t)a.conv_Fin * pos_b;
    cv_base = (const char*)a.A + t_base * row_b;
    const int64_t left = ((int64_t)a.cu_in[a.nseq] - t_base) * row_b;
    cv_bytes = (int)min(left, (int64_t)0x7fffffff);
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      const int m = m0 + r0 + RPI * i;
      cv_off[i] = 0;
      cv_ok[i] = 0;
      if (m < a.M) {
        const int tg = m / a.conv_Fout, f2 = m - tg * a.conv_Fout;
        const int sq = find_seq(a.cu_out, a.nseq, tg);
        const int t2 = tg - a.cu_out[sq], Tin = a.cu_in[sq + 1] - a.cu_in[sq];
        cv_off[i] = (int)((((int64_t)a.cu_in[sq] + tstride * t2 - t_base) * a.conv_Fin + 2 * f2) * pos_b);
#pragma unroll
        for (int d = 0; d < 3; ++d) {
          if (tstride * t2 + d - 1 >= 0 && tstride * t2 + d - 1 < Tin) cv_ok[i] |= 1u << d;
          if (2 * f2 + d - 1 >= 0 && 2 * f2 + d - 1 < a.conv_Fin) cv_ok[i] |= 8u << d;
        }
      }
    }
  }

  // This lane's K column k = kb * 32 + c * 8 as (tap, channel): slices are
  // issued in order (kb = 0, 1, 2, ...), so the pair is carried forward by
  // 32 columns per call (C >= 32: one wrap at most) instead of divided out.
  [[maybe_unused]] int cv_k = c * 8, cv_tap = 0, cv_ch = c * 8;
  if constexpr (CONV) {
    cv_tap = cv_k / a.conv_C;
    cv_ch = cv_k - cv_tap * a.conv_C;
  }
  auto issue = [&](uint4* stage, int kb) {
    (void)kb;
    int cdelta = 0;
    uint32_t need = 0;
    if constexpr (CONV) {
      const int tap = cv_tap, ch = cv_ch;
      const int df = one_d ? 1 : (tap * 11) >> 5, dt = one_d ? tap : tap - 3 * df;  // tap / 3 for tap < 9
      cdelta = ((dt - 1) * a.conv_Fin + (df - 1)) * a.conv_C * (int)sizeof(T) + ch * (int)sizeof(T);
      need = cv_k < a.K ? (1u << dt) | (8u << df) : 0xffffffffu;  // past K: never satisfied
      cv_k += 32;
      cv_ch += 32;
      if (cv_ch >= a.conv_C) {
        cv_ch -= a.conv_C;
        ++cv_tap;
      }
    }
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const lds_ptr_t dst = (lds_ptr_t)(stage + (wave + i * NW) * 64);
      if (i < AI) {
        if constexpr (CONV) {
          const uint32_t voff = (cv_ok[i] & need) == need ? (uint32_t)(cv_off[i] + cdelta)
                                                          : 0x80000000u;  // past any descriptor
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              __builtin_amdgcn_make_buffer_rsrc((void*)cv_base, (short)0, cv_bytes, 0x00020000), dst, 16,
              (int)voff, 0, 0, 0);
        } else {
          const int rows = a.M - i * RPI;
          const char* base = (const char*)a.A + (int64_t)(i * RPI) * ldab;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, rows > 0 ? rows * ldab : 0, 0x00020000),
              dst, 16, va, kb * 64, 0, 0);
        }
      } else {
        // B rounds; blocks past the B rows (spare ones of the last round)
        // get an empty descriptor and load zeros
        const int row = (i - AI) * RPI;
        const int rows = (wave + i * NW) * RPB < BM + BNP ? a.N - row : 0;
        const char* base = (const char*)a.B + (int64_t)row * ldbb;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, rows > 0 ? rows * ldbb : 0, 0x00020000),
            dst, 16, vb, kb * 64, 0, 0);
      }
    }
  };

  f32x4 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int g = lane >> 4, l16 = lane & 15;
  const int sw = (l16 >> 2) & 3;
  // fragment of chunk g of tile row r (r % 16 == l16): index r * 4 + (g ^ swz(r))
  auto a_idx = [&](int i) { return (wm * WTM + i * 16 + l16) * 4 + (g ^ sw); };
  auto b_idx = [&](int j) { return (BM + wn * WTN + j * 16 + l16) * 4 + (g ^ sw); };

  uint4 fa[MI];
  uint4 fb0[NI], fb1[NI];

  // One K step with B fragments FB: MFMAs row by row, each row's A fragment
  // reloaded from SN (the next slice's stage) right after its last use, and
  // the next step's B fragments read into FBN halfway through.
  auto kstep = [&](const uint4 (&FB)[NI], uint4 (&FBN)[NI], const uint4* SN, bool more) {
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int j = 0; j < NI; ++j) mma16(acc[i][j], FB[j], fa[i], T{});  // C^T tile
      if (more) {
        fa[i] = SN[a_idx(i)];
        if (i == MI / 2 - 1) {
#pragma unroll
          for (int j = 0; j < NI; ++j) FBN[j] = SN[b_idx(j)];
        }
      }
    }
    // Interleave: each row's MFMAs, then that row's reload (left alone, the
    // scheduler batches every read after every MFMA, all wavefronts of the
    // workgroup do so in step, and the LDS reads stop overlapping the MFMAs).
    if (more) {
#define MT_ROW(NREAD)                                    \
  __builtin_amdgcn_sched_group_barrier(0x008, NI, 0);    \
  __builtin_amdgcn_sched_group_barrier(0x100, NREAD, 0);
      if constexpr (MI == 8) {
        MT_ROW(1) MT_ROW(1) MT_ROW(1) MT_ROW(1 + NI) MT_ROW(1) MT_ROW(1) MT_ROW(1) MT_ROW(1)
      } else {
        MT_ROW(1) MT_ROW(1 + NI) MT_ROW(1) MT_ROW(1)
      }
#undef MT_ROW
    }
  };
  // Before step s (slice s in stage s % 4): slice s + 1 has landed for every
  // wavefront (own DMA: at most the BPW loads of slice s + 2 still in flight;
  // everyone's: the barrier), and every wavefront is past step s - 1, so no
  // one still reads the stage of slice s - 1: it takes slice s + 3.
  auto handover = [&](uint4* FREE, bool refill, int s, int newer) {
    wait_vm(newer);
    __builtin_amdgcn_s_barrier();
    if (refill) issue(FREE, s + 3);
  };

  // Residual epilogue: this wavefront's part of the fp32 residual tile is
  // requested before the first DMA, so its read overlaps the main loop
  // instead of following it (with one round of tiles every CU would read
  // and write the residual stream at the same moment).  Rows past M read
  // row M - 1 and are not stored.
  constexpr bool PRE = EPI == EPI_RESID && !CONV;
  float4 rpre[PRE ? MI : 1][PRE ? NI : 1];
  if constexpr (PRE) {
    const int rb = m0 + wm * WTM + (lane & 15), cb = n0 + wn * WTN + 4 * (lane >> 4);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int row = min(rb + 16 * i, a.M - 1), col = min(cb + 16 * j, a.N - 4);
        rpre[i][j] = *(const float4*)((const float*)a.C + (int64_t)row * a.ldc + col);
      }
  }
  const int nkb = CONV ? (a.K + 127) / 128 * 4 : a.K / 32;  // a multiple of 4; conv: zero slices
  issue(st0, 0);
  issue(st1, 1);
  issue(st2, 2);
  wait_vm(2 * BPW);
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int i = 0; i < MI; ++i) fa[i] = st0[a_idx(i)];
#pragma unroll
  for (int j = 0; j < NI; ++j) fb0[j] = st0[b_idx(j)];

  // Four steps per iteration (stages 0-3); inside the loop slices s + 3 all
  // exist, so the body has no branch.  The last four steps are peeled.
  for (int s = 0; s < nkb - 4; s += 4) {
    handover(st3, true, s, BPW);
    kstep(fb0, fb1, st1, true);
    handover(st0, true, s + 1, BPW);
    kstep(fb1, fb0, st2, true);
    handover(st1, true, s + 2, BPW);
    kstep(fb0, fb1, st3, true);
    handover(st2, true, s + 3, BPW);
    kstep(fb1, fb0, st0, true);
  }
  handover(st3, true, nkb - 4, BPW);
  kstep(fb0, fb1, st1, true);
  handover(st0, false, nkb - 3, BPW);
  kstep(fb1, fb0, st2, true);
  handover(st1, false, nkb - 2, 0);
  kstep(fb0, fb1, st3, true);
  kstep(fb1, fb0, st0, false);

  if constexpr (EPI == EPI_ACT || EPI == EPI_GELU) {
    epilogue_staged4<T, EPI, BN, MI, NI>(a, acc, st0, st1, st2, st3, m0, n0, wm, wn);
  } else if constexpr (PRE) {
    epilogue_resid_pre<MI, NI>(a, acc, rpre, m0 + wm * WTM + l16, n0 + wn * WTN + 4 * g);
  } else {
    epilogue4<T, EPI, MI, NI>(a, acc, m0 + wm * WTM + l16, n0 + wn * WTN + 4 * g);
  }
}

template <typename T, int BN, int EPI, int WM = 2, bool CONV = false>
hipError_t run_w8q(const GemmArgs& a, hipStream_t s) {
  const int tiles = ((a.M + 255) / 256) * ((a.N + BN - 1) / BN);
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_w8q_kernel<T, BN, WM, EPI, CONV>), dim3(tiles), dim3(512), 0, s, a);
  return hipGetLastError();
}

// Register-staged kernel.  With a partial-sum workspace (fp32 products),
// K is split when the output tiles alone would leave most CUs idle: up to
// GEMM_SPLIT_MAX splits of at least four 32-wide K steps, about 512
// workgroups in all, as many as the workspace holds; a second kernel adds
// the partial sums (the kernel boundary orders them, no fences or counters).
template <typename T, int BM, int BN, int EPI, bool CONV>
hipError_t run(const GemmArgs& a, hipStream_t s) {
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  if (tiles == 0) return hipSuccess;
  int nz = 1;
  if (a.part && tiles < 256) {
    constexpr int BK = 8 * Elem<T>::per16;
    const int nkb = (a.K + BK - 1) / BK;
    nz = std::min(std::min(GEMM_SPLIT_MAX, nkb / 4), (511 + tiles) / tiles);
    while (nz > 1 && (int64_t)nz * tiles * BM * BN > a.part_floats) --nz;
    nz = std::max(nz, 1);
  }
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, EPI, CONV>), dim3(tiles, nz), dim3(256), 0, s, a);
  if (nz > 1) hipLaunchKernelGGL((gemm_split_sum_kernel<T, BM, BN, EPI>), dim3(tiles), dim3(256), 0, s, a, nz);
  return hipGetLastError();
}

template <typename T, int EPI, bool CONV>
hipError_t pick_tile(const GemmArgs& a, hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    // Convolutions: the four-stage eight-wavefront kernel with the tap
    // gather.  Bias + GELU: 256 x 256 tiles of 128 x 64 wavefronts (480
    // output channels = 2 tiles, 6 % of the MFMA work on padding, but 17 %
    // fewer operand bytes per MFMA than 256 x 160 tiles of 64 x 80: in the
    // 16 x 30 s step conv2 1.86 -> 1.57 ms, conv3 0.53 -> 0.40 ms); with the
    // sinusoids added (more epilogue state) the 256 x 160 tiles stay.  The
    // two-stage 256 x 256 kernel spills with the gather's per-row state.
    if constexpr (CONV) {
      if (a.conv_C % 8 == 0 && a.conv_C >= 32 && (int64_t)a.N * a.ldb * 2 < (1ll << 31)) {
        if constexpr (EPI == EPI_GELU) return run_w8q<T, 256, EPI, 2, true>(a, s);
        return run_w8q<T, 160, EPI, 4, true>(a, s);
      }
    }
    if (CONV && a.conv_kind != CONV_2D_S2) return hipErrorInvalidValue;  // 1-D: that kernel only
    if constexpr (!CONV) {
      // Wide outputs: 256-row tiles where K allows them (whole 128-wide K
      // pairs, operands addressable with 32-bit offsets), 256 or 192 wide by
      // how full the last round of tiles leaves the CUs (measured at
      // M = 6000: N = 5120 -> 256 x 256, 855 TFLOP/s; N = 3840 -> 256 x 192,
      // 793 TFLOP/s; 128 x 128: 670 / 651).  Narrow outputs (N = 1280: too
      // few wide tiles to fill 256 CUs): the four-stage kernel with 256 x 128
      // tiles of eight 64 x 64 wavefronts (two-stage variant, standalone:
      // K = 5120: 847 TFLOP/s with a 16-bit epilogue, 730 with the fp32
      // residual add, against 752 / 622 for 128 x 128; K = 1280: 740 / 595
      // against 617 / 541; four stages gained another ~6 % on fc2).
      const bool w8 = a.K % 128 == 0 && (int64_t)a.M * a.lda * 2 < (1ll << 31) &&
                      (int64_t)a.N * a.ldb * 2 < (1ll << 31);
      // With fewer than 128 such tiles (a single clip, a stream chunk) most
      // CUs would idle: the smaller tiles below (same K order, same results).
      const int t256 = ((a.M + 255) / 256) * ((a.N + 255) / 256);
      if (w8 && a.N >= 2048 && t256 >= 128) {
        if constexpr (EPI != EPI_SWIGLU) {
          const int t192 = ((a.M + 255) / 256) * ((a.N + 191) / 192);
          const double e256 = t256 / (256.0 * ((t256 + 255) / 256));
          const double e192 = t192 / (256.0 * ((t192 + 255) / 256));
          if (e192 > 1.15 * e256) return run_w8<T, 192, EPI>(a, s);
        }
        return run_w8<T, 256, EPI>(a, s);
      }
      // Narrow outputs (N < 2048) with many rows: 256 x 256 tiles once they
      // fill 1.5 rounds of CUs (N = 1280, M = 24000, fp32 residual epilogue:
      // K = 5120 360 us against 489 for the four-stage 256 x 128 kernel,
      // K = 1280 106 against 129; in the encoder step, fc2 15.0 -> 10.6 ms
      // and o 5.0 -> 4.1).  At M = 6000 the four-stage kernel stays (in
      // the encoder step 256 x 128 tiles of 128 x 32 wavefronts measured
      // fc2 3.25 ms against 2.97, although alone they ran 8 % faster).
      if (w8 && a.M >= 2048 && ((a.M + 255) / 256) * ((a.N + 255) / 256) >= 384)
        return run_w8<T, 256, EPI>(a, s);
      if (w8 && a.M >= 2048) return run_w8q<T, 128, EPI, 4>(a, s);
      if (a.M >= 2048) return run_lds<T, 256, 128, 4, 2, 2, EPI, CONV>(a, s);
      // Few rows (a single clip, a stream chunk, a decoder prompt): 128 x 128
      // tiles only when there are enough of them for the CUs, else 64 x 64
      // (measured: M = 375, N = 1280, K = 1280 17.7 -> 8.9 us; M = 832,
      // N = 1280, K = 5120 67.3 -> 42.0 us; M = 832, N = 5120: 128 x 128
      // stays ahead with 280 tiles).
      if (((a.M + 127) / 128) * ((a.N + 127) / 128) >= 256) return run_lds<T, 128, 128, 2, 2, 4, EPI, CONV>(a, s);
      return run_lds<T, 64, 64, 2, 2, 4, EPI, CONV>(a, s);
    }
  }
  if constexpr (CONV) {
    if (a.conv_kind != CONV_2D_S2) return hipErrorInvalidValue;  // 1-D: 16-bit operands only
    // output channels 480 = 3 x 160
    if (a.N % 160 == 0) return run<T, 128, 160, EPI, CONV>(a, s);
    return run<T, 128, 128, EPI, CONV>(a, s);
  } else {
    // few rows (a short clip): 32 x 64 tiles, not 128 x 128 of which most
    // rows would be padding
    if (a.M <= 32) return run<T, 32, 64, EPI, CONV>(a, s);
    return run<T, 128, 128, EPI, CONV>(a, s);
  }
}

template <typename T, bool CONV>
hipError_t by_epi(const GemmArgs& a, int epi, hipStream_t s) {
  switch (epi) {
    case EPI_F32: return pick_tile<T, EPI_F32, CONV>(a, s);
    case EPI_ACT: return pick_tile<T, EPI_ACT, CONV>(a, s);
    case EPI_GELU: return pick_tile<T, EPI_GELU, CONV>(a, s);
    case EPI_RESID: return pick_tile<T, EPI_RESID, CONV>(a, s);
    case EPI_PE: return pick_tile<T, EPI_PE, CONV>(a, s);
    case EPI_SWIGLU: return pick_tile<T, EPI_SWIGLU, CONV>(a, s);
    case EPI_OUT: return pick_tile<T, EPI_OUT, CONV>(a, s);
    case EPI_GELU_SPLIT:
      if constexpr (sizeof(T) == 2) return pick_tile<T, EPI_GELU_SPLIT, CONV>(a, s);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, int epi, int dtype, bool conv, hipStream_t s) {
  if (a.N < 4 || a.N % 4) return hipErrorInvalidValue;  // epilogues write 4 columns at a time
  // the convolutions always end in bias + GELU (then the sinusoids for the
  // last 1-D one); no other product takes EPI_GELU_PE
  if (conv && epi != EPI_GELU && epi != EPI_GELU_PE) return hipErrorInvalidValue;
  if (!conv && epi == EPI_GELU_PE) return hipErrorInvalidValue;
  if (dtype == DT_BF16) {
    if (conv) return epi == EPI_GELU ? pick_tile<bf16_t, EPI_GELU, true>(a, s)
                                     : pick_tile<bf16_t, EPI_GELU_PE, true>(a, s);
    return by_epi<bf16_t, false>(a, epi, s);
  }
  if (dtype == DT_F16) {
    if (conv) return epi == EPI_GELU ? pick_tile<f16_t, EPI_GELU, true>(a, s)
                                     : pick_tile<f16_t, EPI_GELU_PE, true>(a, s);
    return by_epi<f16_t, false>(a, epi, s);
  }
  if (conv) return epi == EPI_GELU ? pick_tile<float, EPI_GELU, true>(a, s) : hipErrorInvalidValue;
  return by_epi<float, false>(a, epi, s);
}

}  // namespace mt
