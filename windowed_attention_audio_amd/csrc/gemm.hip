// Tiled matrix products on the gfx950 matrix cores, with fused epilogues.
//
// C[M, N] = A[M, K] * B[N, K]^T, both operands K-contiguous.  A is either a
// plain row-major activation or, for the stride-2 3x3 convolutions of the
// front-end (model card "MOSS-Transcribe-preview-2B-GGUF", Architecture
// table, Conv front-end row), gathered on the fly from a channels-last
// activation (implicit GEMM: K index = tap * C + input channel, tap =
// 3 * freq offset + time offset, zero outside each sequence).
//
// Block: 256 threads = 4 wavefronts in a 2 x 2 grid; each wavefront owns a
// (BM/2) x (BN/2) tile made of 16 x 16 MFMA tiles.  K advances in slices of
// 128 bytes per row (64 bf16 or 32 fp32).  Slices are double-buffered in
// LDS; the next slice is fetched into registers while the current one feeds
// the matrix cores.  Within LDS each row's eight 16-byte chunks are XOR-
// swizzled by the row index so that 16 lanes reading 16 rows at one chunk
// hit distinct banks.
//
// Operand fragments: one 16-byte chunk per lane and operand.  For bf16 and
// fp16 this is one v_mfma_f32_16x16x32_{bf16,f16} (lane l supplies row l%16,
// k = 8*(l/16)..+7 of the 32-wide step).  For fp32 it is four v_mfma_f32_16x16x4_f32, the e-th
// one taking element e of every lane's chunk; as both operands use the same
// assignment of k to (lane group, element), the sum over k is unchanged.
#include "common.h"
#include "kernels.h"

namespace mt {

namespace {

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

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

  // convolution: track (tap, channel) of this thread's chunk incrementally
  int ctap = 0, cch = c * EPC;
  if constexpr (CONV) {
    while (cch >= a.conv_C) { cch -= a.conv_C; ++ctap; }
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

  const int nkb = (a.K + BK - 1) / BK;
  gload(0);
  sstore(0);
  __syncthreads();

  const int g = lane >> 4;
  const int l16 = lane & 15;
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nkb) gload(kb + 1);
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
        for (int j = 0; j < NI; ++j) mma_chunk<T>(acc[i][j], af[i], bfr[j]);
    }
    if (kb + 1 < nkb) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds C[4g + e][l16] of every 16 x 16 tile
  const int rbase = m0 + wm * WTM + 4 * g;
  const int cbase = n0 + wn * WTN + l16;
  if constexpr (EPI == EPI_SWIGLU) {
    T* C = (T*)a.C;
#pragma unroll
    for (int j = 0; j < NI; j += 2) {
      const int colg = cbase + j * 16;  // gate column (its pair: + 16)
      if (colg >= a.N) continue;
      const int feat = (colg - l16) / 2 + l16;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = rbase + i * 16 + e;
          if (row < a.M) {
            const float gv = acc[i][j][e], uv = acc[i][j + 1][e];
            C[(int64_t)row * a.ldc + feat] = Elem<T>::from_f(silu_f(gv) * uv);
          }
        }
    }
  } else {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int col = cbase + j * 16;
      if (col >= a.N) continue;
      const float bias = a.bias ? a.bias[col] : 0.f;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = rbase + i * 16 + e;
          if (row >= a.M) continue;
          const float v = acc[i][j][e] + bias;
          if constexpr (EPI == EPI_F32) {
            ((float*)a.C)[(int64_t)row * a.ldc + col] = v;
          } else if constexpr (EPI == EPI_ACT) {
            ((T*)a.C)[(int64_t)row * a.ldc + col] = Elem<T>::from_f(v);
          } else if constexpr (EPI == EPI_GELU) {
            ((T*)a.C)[(int64_t)row * a.ldc + col] = Elem<T>::from_f(gelu_f(v));
          } else if constexpr (EPI == EPI_GELU_SPLIT) {
            const float gv = gelu_f(v);
            const T hi = Elem<T>::from_f(gv);
            const T lo = Elem<T>::from_f(gv - Elem<T>::to_f(hi));
            T* C = (T*)a.C;
            C[(int64_t)row * a.ldc + col] = hi;
            C[(int64_t)row * a.ldc + a.N + col] = lo;
          } else if constexpr (EPI == EPI_RESID) {
            float* R = (float*)a.C;
            R[(int64_t)row * a.ldc + col] += v;
          } else if constexpr (EPI == EPI_PE) {
            const int sq = find_seq(a.cu_rows, a.nseq, row);
            const int pos = row - a.cu_rows[sq];
            const int half = a.N / 2;
            const int jj = col < half ? col : col - half;
            // timescale 10000^(-jj/(half-1)); angle reduced mod 2 pi in double
            const double ts = exp(-(double)jj * 9.2103403719761836 / (double)(half - 1));
            double ang = (double)pos * ts;
            ang -= 6.283185307179586 * rint(ang * 0.15915494309189535);
            const float fa = (float)ang;
            const float pe = col < half ? sinf(fa) : cosf(fa);
            ((float*)a.C)[(int64_t)row * a.ldc + col] = acc[i][j][e] + pe;
          } else if constexpr (EPI == EPI_OUT) {
            int64_t orow = row;
            if (a.out_seq_stride > 0) {
              const int sq = find_seq(a.cu_rows, a.nseq, row);
              orow = (int64_t)sq * a.out_seq_stride + (row - a.cu_rows[sq]);
            }
            ((float*)a.C)[orow * a.ldc + col] = v;
          }
        }
    }
  }
}

template <typename T, int BM, int BN, int EPI, bool CONV>
hipError_t run(const GemmArgs& a, hipStream_t s) {
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, EPI, CONV>), dim3(tiles), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, int EPI, bool CONV>
hipError_t pick_tile(const GemmArgs& a, hipStream_t s) {
  if constexpr (CONV) {
    // output channels 480 = 3 x 160
    if (a.N % 160 == 0) return run<T, 128, 160, EPI, CONV>(a, s);
    return run<T, 128, 128, EPI, CONV>(a, s);
  } else {
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
  // the convolutions always end in bias + GELU
  if (conv && epi != EPI_GELU) return hipErrorInvalidValue;
  if (dtype == DT_BF16) {
    if (conv) return pick_tile<bf16_t, EPI_GELU, true>(a, s);
    return by_epi<bf16_t, false>(a, epi, s);
  }
  if (dtype == DT_F16) {
    if (conv) return pick_tile<f16_t, EPI_GELU, true>(a, s);
    return by_epi<f16_t, false>(a, epi, s);
  }
  if (conv) return pick_tile<float, EPI_GELU, true>(a, s);
  return by_epi<float, false>(a, epi, s);
}

}  // namespace mt
