// Waveform -> log-mel frames (model card "MOSS-Transcribe-preview-2B-GGUF",
// Architecture table, Audio row; gotcha list: the trailing STFT frame is
// dropped, so a clip of n samples gives floor(n / 160) frames).
//
// Pass 1 (mel_frames_kernel): one workgroup of 128 threads per 8 consecutive
// frames (31 KB of LDS: five workgroups per CU).
//   load    each frame is 400 samples centred on 160 t, the clip mirrored at
//           both ends (reflect padding by 200, edge sample not repeated),
//           times a periodic Hann window; reads of neighbouring frames are
//           contiguous and coalesced.  The sequence tables (up to 128
//           sequences) are staged in LDS first, so a frame's sequence is found
//           without a chain of dependent memory reads.
//   DFT     400 = 16 x 25.  With n = 25 n1 + n2 and k = k1 + 16 k2,
//           X[k] = sum_n2 W400^(n2 k1) W25^(n2 k2) sum_n1 x[25 n1 + n2] W16^(n1 k1).
//           Step A: 25 real 16-point DFTs per frame (outputs k1 = 0..8; the
//           rest follow by conjugate symmetry), halved twice (even / odd
//           indices).  Step B: per k1, the W400^(n2 k1) factors and the 25-point
//           DFT as 5 x 5, with 5-point DFTs that pair the terms sharing a
//           cosine; bins k = k1 + 16 k2 <= 200 are kept.  Window, twiddles and
//           sums are in double: bins that sit 8 decades below the clip's
//           loudest bin (the clamp floor) carry rounding of the whole frame,
//           which in fp32 costs about 1e-4 of the normalised output.
//   mel     |X[k]|^2 (rounded to fp32) through the sparse Slaney filterbank
//           (about 2 non-zeros per bin); log10(max(., 1e-10)) in fp32 (a few
//           units in the last place of values up to ~10, far below the 1e-4
//           bar after the / 4 of pass 2), the floor itself giving -10 exactly.  The per-frame maxima are reduced in
//           LDS and folded into each clip's maximum with one atomicMax per
//           clip present in the workgroup.
// Pass 2 (mel_norm_kernel, misc.hip): y = (max(x, g_clip - 8) + 4) / 4.
#include "common.h"
#include "kernels.h"
#include "mel_tables.inc"

namespace mt {

namespace {

constexpr int FPB = 8;   // frames per workgroup
constexpr int NTH = 128; // threads per workgroup (FPB x 16 in step B)
constexpr int TBL = NTH; // sequences whose tables are staged in LDS

__device__ __forceinline__ double2 cmul(double2 a, double2 b) {
  return make_double2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}

// 5-point DFT Z[c] = sum_a u[a] w^(a c), w = exp(-2 pi i / 5) = (C1, -S1),
// w^2 = (C2, -S2): the terms of a and 5 - a share their cosines, so with
// t1 = u1 + u4, t2 = u2 + u3, t3 = u1 - u4, t4 = u2 - u3,
//   Z0 = u0 + t1 + t2,
//   Z1, Z4 = u0 + C1 t1 + C2 t2 -/+ i (S1 t3 + S2 t4),
//   Z2, Z3 = u0 + C2 t1 + C1 t2 -/+ i (S2 t3 - S1 t4).
__device__ __forceinline__ void dft5(double2 u0, double2 u1, double2 u2, double2 u3, double2 u4, double C1,
                                     double S1, double C2, double S2, double2 (&z)[5]) {
  const double2 t1 = make_double2(u1.x + u4.x, u1.y + u4.y), t2 = make_double2(u2.x + u3.x, u2.y + u3.y);
  const double2 t3 = make_double2(u1.x - u4.x, u1.y - u4.y), t4 = make_double2(u2.x - u3.x, u2.y - u3.y);
  z[0] = make_double2(u0.x + t1.x + t2.x, u0.y + t1.y + t2.y);
  const double2 A1 = make_double2(fma(C2, t2.x, fma(C1, t1.x, u0.x)), fma(C2, t2.y, fma(C1, t1.y, u0.y)));
  const double2 A2 = make_double2(fma(C1, t2.x, fma(C2, t1.x, u0.x)), fma(C1, t2.y, fma(C2, t1.y, u0.y)));
  const double2 B1 = make_double2(fma(S2, t4.x, S1 * t3.x), fma(S2, t4.y, S1 * t3.y));
  const double2 B2 = make_double2(fma(-S1, t4.x, S2 * t3.x), fma(-S1, t4.y, S2 * t3.y));
  // -i B = (B.y, -B.x)
  z[1] = make_double2(A1.x + B1.y, A1.y - B1.x);
  z[4] = make_double2(A1.x - B1.y, A1.y + B1.x);
  z[2] = make_double2(A2.x + B2.y, A2.y - B2.x);
  z[3] = make_double2(A2.x - B2.y, A2.y + B2.x);
}

__global__ __launch_bounds__(NTH) void mel_frames_kernel(MelArgs a) {
  // ys (the step-A output) and xs (raw frame samples, later |X|^2 [FPB][201])
  // share the LDS: each phase reads what it needs into registers before the
  // barrier after which the next phase overwrites it (29 KB: five workgroups
  // per CU instead of three).
  __shared__ double2 ys[FPB][25][9];   // step-A output, k1 = 0..8
  float(*xs)[400] = (float(*)[400])&ys[0][0][0];
  __shared__ float fmax_s[FPB];
  __shared__ int fseq_s[FPB], ft_s[FPB], fn_s[FPB];
  __shared__ int64_t foff_s[FPB];
  __shared__ int32_t cu_s[TBL + 1], len_s[TBL];
  __shared__ int64_t soff_s[TBL];

  const int tid = threadIdx.x;
  const int64_t f0 = (int64_t)blockIdx.x * FPB;

  // frame -> sequence, its frame index in the stream and the sequence's
  // samples.  Up to TBL sequences the tables are staged in LDS first (one
  // round trip to memory instead of one per step of the search).
  const bool staged = a.nseq <= TBL;
  if (staged) {
    if (tid <= a.nseq) cu_s[tid] = a.cu_frames[tid];
    if (tid < a.nseq) {
      len_s[tid] = a.seq_len[tid];
      soff_s[tid] = a.seq_sample_off[tid];
    }
    __syncthreads();
  }
  if (tid < FPB) {
    const int64_t gf = f0 + tid;
    const int32_t* cu = staged ? cu_s : a.cu_frames;
    const int sq = gf < a.total_frames ? find_seq(cu, a.nseq, (int)gf) : -1;
    fseq_s[tid] = sq;
    ft_s[tid] = sq >= 0 ? (int)gf - cu[sq] + (int)a.frame_off : 0;
    fn_s[tid] = sq >= 0 ? (staged ? len_s[sq] : a.seq_len[sq]) : 1;
    foff_s[tid] = sq >= 0 ? (staged ? soff_s[sq] : a.seq_sample_off[sq]) : 0;
  }
  __syncthreads();

  // ---- load (the window is applied in double in step A).  All 25 samples
  // of a thread are requested before the first is stored: a guarded load
  // per iteration waited for each one in turn.  Frames past the end read
  // sample 0 and store zeros.
  {
    constexpr int PER = FPB * 400 / NTH;
    static_assert(FPB * 400 % NTH == 0, "load plan");
    float v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int idx = tid + NTH * u;
      const int f = idx / 400, j = idx - f * 400;
      int64_t src = 0;
      if (fseq_s[f] >= 0) {
        const int n = fn_s[f];
        int q = 160 * ft_s[f] + j - 200;
        q = q < 0 ? -q : q;
        q = q >= n ? 2 * (n - 1) - q : q;
        src = foff_s[f] + q;
      }
      v[u] = a.wav[src];
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int idx = tid + NTH * u;
      const int f = idx / 400;
      xs[f][idx - f * 400] = fseq_s[f] >= 0 ? v[u] : 0.f;
    }
  }
  __syncthreads();

  // ---- step A: (frame, n2) -> 16-point real DFT over n1 of the windowed
  // frame, outputs k1 = 0..8.  Halving twice: with s = x[n] + x[n+8],
  // d = x[n] - x[n+8] (n < 8), the odd k1 are sum_n d[n] W16^(n k1); with
  // s2 = s[n] + s[n+4], d2 = s[n] - s[n+4] (n < 4), k1 = 0, 4, 8 are sums of
  // s2 times powers of -i and k1 = 2, 6 are sum_n d2[n] W8^(n k1 / 2).  Both
  // tasks' samples are read before the barrier: ys overwrites xs.
  constexpr int TA = (FPB * 25 + NTH - 1) / NTH;  // tasks per thread
  float xa[TA][16];
#pragma unroll
  for (int q = 0; q < TA; ++q) {
    const int task = min(tid + NTH * q, FPB * 25 - 1);
    const int f = task / 25, n2 = task - f * 25;
#pragma unroll
    for (int n1 = 0; n1 < 16; ++n1) xa[q][n1] = xs[f][25 * n1 + n2];
  }
  __syncthreads();
  {
    const double r8 = c_tw[50].x;  // cos(pi / 4)
#pragma unroll
    for (int q = 0; q < TA; ++q) {
      const int task = tid + NTH * q;
      if (task >= FPB * 25) break;
      const int f = task / 25, n2 = task - f * 25;
      double x[16];
#pragma unroll
      for (int n1 = 0; n1 < 16; ++n1) x[n1] = (double)xa[q][n1] * c_hann[25 * n1 + n2];
      double s[8], d[8], s2[4], d2[4];
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        s[n] = x[n] + x[n + 8];
        d[n] = x[n] - x[n + 8];
      }
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        s2[n] = s[n] + s[n + 4];
        d2[n] = s[n] - s[n + 4];
      }
      double2* out = ys[f][n2];
      out[0] = make_double2((s2[0] + s2[2]) + (s2[1] + s2[3]), 0.0);
      out[4] = make_double2(s2[0] - s2[2], s2[3] - s2[1]);
      out[8] = make_double2((s2[0] + s2[2]) - (s2[1] + s2[3]), 0.0);
      const double dp = r8 * (d2[1] - d2[3]), dq = r8 * (d2[1] + d2[3]);
      out[2] = make_double2(d2[0] + dp, -d2[2] - dq);
      out[6] = make_double2(d2[0] - dp, d2[2] - dq);
#pragma unroll
      for (int k1 = 1; k1 < 8; k1 += 2) {
        // n = 0: W16^0 = 1; n = 4: W16^(4 k1) = -i (k1 % 4 == 1) or i
        double re = d[0], im = (k1 & 2) ? d[4] : -d[4];
#pragma unroll
        for (int n = 1; n < 8; ++n) {
          if (n == 4) continue;
          const double2 w = c_tw[(25 * n * k1) % 400];
          re = fma(d[n], w.x, re);
          im = fma(d[n], w.y, im);
        }
        out[k1] = make_double2(re, im);
      }
    }
  }
  __syncthreads();

  // ---- step B: (frame, k1) -> W400^(n2 k1), then the 25-point DFT over n2
  // as 5 x 5 (n2 = 5 a + b, k2 = c + 5 d): five 5-point DFTs over a, the
  // W25^(b c) factors, five 5-point DFTs over b; bins k = k1 + 16 k2 <= 200
  // are kept.  The inputs are read before the barrier: xs overwrites ys.
  {
    const int f = tid >> 4, k1 = tid & 15;
    double2 y[25];
#pragma unroll
    for (int n2 = 0; n2 < 25; ++n2) {
      double2 v = k1 <= 8 ? ys[f][n2][k1] : ys[f][n2][16 - k1];
      if (k1 > 8) v.y = -v.y;  // real input: Y[16 - k1] = conj(Y[k1])
      y[n2] = cmul(v, c_tw[n2 * k1]);
    }
    __syncthreads();
    const double C1 = c_tw[80].x, S1 = -c_tw[80].y, C2 = c_tw[160].x, S2 = -c_tw[160].y;
    double2 z[5][5];  // z[b][c]
#pragma unroll
    for (int b = 0; b < 5; ++b) dft5(y[b], y[5 + b], y[10 + b], y[15 + b], y[20 + b], C1, S1, C2, S2, z[b]);
#pragma unroll
    for (int b = 1; b < 5; ++b)
#pragma unroll
      for (int c = 1; c < 5; ++c) z[b][c] = cmul(z[b][c], c_tw[16 * b * c]);  // W25^(b c)
#pragma unroll
    for (int c = 0; c < 5; ++c) {
      double2 o[5];  // o[d] = X[k1 + 16 (c + 5 d)]
      dft5(z[0][c], z[1][c], z[2][c], z[3][c], z[4][c], C1, S1, C2, S2, o);
#pragma unroll
      for (int dd = 0; dd < 3; ++dd) {
        const int k = k1 + 16 * (c + 5 * dd);
        if (k <= 200) xs[f][k] = (float)(o[dd].x * o[dd].x + o[dd].y * o[dd].y);
      }
    }
  }
  __syncthreads();

  // ---- mel + log10; thread (frame = tid/16, part = tid%16) does 8 mel bins
  {
    const int f = tid >> 4, part = tid & 15;
    const int sq = fseq_s[f];
    float lmax = -INFINITY;
    float L[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int m = part + 16 * r;
      const int first = c_mel_first[m], cnt = c_mel_count[m], off = c_mel_off[m];
      float e = 0.f;
      for (int b = 0; b < cnt; ++b) e += c_mel_w[off + b] * xs[f][first + b];
      L[r] = e > 1e-10f ? log10f(e) : -10.0f;  // the floor: log10(1e-10) = -10 exactly
      lmax = fmaxf(lmax, L[r]);
    }
    if (sq >= 0) {
      const int t = (int)(f0 + f) - (staged ? cu_s[sq] : a.cu_frames[sq]);
      float* out = a.mel + (a.seq_row_off[sq] + t) * 128;
#pragma unroll
      for (int r = 0; r < 8; ++r) out[part + 16 * r] = L[r];
    }
    // maximum over the 16 lanes of the frame: DPP row rotations (the maximum
    // does not depend on the order)
    lmax = fmaxf(lmax, dpp_f<0x128>(lmax));
    lmax = fmaxf(lmax, dpp_f<0x124>(lmax));
    lmax = fmaxf(lmax, dpp_f<0x122>(lmax));
    lmax = fmaxf(lmax, dpp_f<0x121>(lmax));
    if (part == 0) fmax_s[f] = lmax;
  }
  __syncthreads();
  if (tid == 0) {
    int cur = fseq_s[0];
    float m = -INFINITY;
    for (int f = 0; f < FPB; ++f) {
      const int sq = fseq_s[f];
      if (sq != cur) {
        if (cur >= 0) atomicMax(a.gmax + cur, float_key(m));
        cur = sq;
        m = -INFINITY;
      }
      m = fmaxf(m, fmax_s[f]);
    }
    if (cur >= 0) atomicMax(a.gmax + cur, float_key(m));
  }
}

}  // namespace

hipError_t launch_mel(const MelArgs& a, hipStream_t s) {
  if (a.total_frames == 0) return hipSuccess;
  const int64_t blocks = (a.total_frames + FPB - 1) / FPB;
  hipLaunchKernelGGL(mel_frames_kernel, dim3((unsigned)blocks), dim3(NTH), 0, s, a);
  return hipGetLastError();
}

}  // namespace mt
