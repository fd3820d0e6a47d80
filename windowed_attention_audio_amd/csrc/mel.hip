// Waveform -> log-mel frames (model card "MOSS-Transcribe-preview-2B-GGUF",
// Architecture table, Audio row; gotcha list: the trailing STFT frame is
// dropped, so a clip of n samples gives floor(n / 160) frames).
//
// Pass 1 (mel_frames_kernel): one workgroup of 128 threads per 8 consecutive
// frames (42 KB of LDS: three workgroups per CU).
//   load    each frame is 400 samples centred on 160 t, the clip mirrored at
//           both ends (reflect padding by 200, edge sample not repeated),
//           times a periodic Hann window; reads of neighbouring frames are
//           contiguous and coalesced.
//   DFT     400 = 16 x 25.  With n = 25 n1 + n2 and k = k1 + 16 k2,
//           X[k] = sum_n2 W400^(n2 k1) W25^(n2 k2) sum_n1 x[25 n1 + n2] W16^(n1 k1).
//           Step A: 25 real 16-point DFTs per frame (outputs k1 = 0..8; the
//           rest follow by conjugate symmetry).  Step B: per k1, the
//           W400^(n2 k1) factors and a 25-point DFT evaluated only for
//           k = k1 + 16 k2 <= 200.  Window, twiddles and sums are in double:
//           bins that sit 8 decades below the clip's loudest bin (the clamp
//           floor) carry rounding of the whole frame, which in fp32 costs
//           about 1e-4 of the normalised output.
//   mel     |X[k]|^2 (rounded to fp32) through the sparse Slaney filterbank
//           (about 2 non-zeros per bin); log10(max(., 1e-10)) in double.  The
//           per-frame maxima are reduced in LDS and folded into each clip's
//           maximum with one atomicMax per clip present in the workgroup.
// Pass 2 (mel_norm_kernel, misc.hip): y = (max(x, g_clip - 8) + 4) / 4.
#include "common.h"
#include "kernels.h"
#include "mel_tables.inc"

namespace mt {

namespace {

constexpr int FPB = 8;   // frames per workgroup
constexpr int NTH = 128; // threads per workgroup (FPB x 16 in step B)

__device__ __forceinline__ double2 cmul(double2 a, double2 b) {
  return make_double2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}

__global__ __launch_bounds__(NTH) void mel_frames_kernel(MelArgs a) {
  __shared__ float xs[FPB][400];       // raw frame samples, later |X|^2 [FPB][201]
  __shared__ double2 ys[FPB][25][9];   // step-A output, k1 = 0..8
  __shared__ float fmax_s[FPB];
  __shared__ int fseq_s[FPB], ft_s[FPB], fn_s[FPB];
  __shared__ int64_t foff_s[FPB];

  const int tid = threadIdx.x;
  const int64_t f0 = (int64_t)blockIdx.x * FPB;

  // frame -> sequence, its frame index in the stream and the sequence's
  // samples (one lookup per frame, kept in LDS for the load below)
  if (tid < FPB) {
    const int64_t gf = f0 + tid;
    const int sq = gf < a.total_frames ? find_seq(a.cu_frames, a.nseq, (int)gf) : -1;
    fseq_s[tid] = sq;
    ft_s[tid] = sq >= 0 ? (int)gf - a.cu_frames[sq] + (int)a.frame_off : 0;
    fn_s[tid] = sq >= 0 ? a.seq_len[sq] : 1;
    foff_s[tid] = sq >= 0 ? a.seq_sample_off[sq] : 0;
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

  // ---- step A: (frame, n2) -> 16-point real DFT over n1 of the windowed frame
  for (int task = tid; task < FPB * 25; task += NTH) {
    const int f = task / 25, n2 = task - f * 25;
    double x[16];
#pragma unroll
    for (int n1 = 0; n1 < 16; ++n1) x[n1] = (double)xs[f][25 * n1 + n2] * c_hann[25 * n1 + n2];
#pragma unroll
    for (int k1 = 0; k1 <= 8; ++k1) {
      double re = 0.0, im = 0.0;
#pragma unroll
      for (int n1 = 0; n1 < 16; ++n1) {
        const double2 w = c_tw[(25 * n1 * k1) % 400];
        re = fma(x[n1], w.x, re);
        im = fma(x[n1], w.y, im);
      }
      ys[f][n2][k1] = make_double2(re, im);
    }
  }
  __syncthreads();

  // ---- step B: (frame, k1) -> W400^(n2 k1), then a 25-point DFT over n2 for
  // k = k1 + 16 k2 <= 200
  {
    const int f = tid >> 4, k1 = tid & 15;
    double2 y[25];
#pragma unroll
    for (int n2 = 0; n2 < 25; ++n2) {
      double2 v = k1 <= 8 ? ys[f][n2][k1] : ys[f][n2][16 - k1];
      if (k1 > 8) v.y = -v.y;  // real input: Y[16 - k1] = conj(Y[k1])
      y[n2] = cmul(v, c_tw[n2 * k1]);
    }
    // all 13 outputs at once (13 independent accumulator pairs, compile-time
    // twiddles); k1 > 8 has only 12 bins <= 200
    double re[13], im[13];
#pragma unroll
    for (int k2 = 0; k2 < 13; ++k2) re[k2] = im[k2] = 0.0;
#pragma unroll
    for (int n2 = 0; n2 < 25; ++n2) {
#pragma unroll
      for (int k2 = 0; k2 < 13; ++k2) {
        const double2 w = c_tw[(16 * n2 * k2) % 400];
        re[k2] = fma(y[n2].x, w.x, fma(-y[n2].y, w.y, re[k2]));
        im[k2] = fma(y[n2].x, w.y, fma(y[n2].y, w.x, im[k2]));
      }
    }
#pragma unroll
    for (int k2 = 0; k2 < 13; ++k2)
      if (k1 + 16 * k2 <= 200) xs[f][k1 + 16 * k2] = (float)(re[k2] * re[k2] + im[k2] * im[k2]);
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
      L[r] = (float)log10(fmax((double)e, 1e-10));
      lmax = fmaxf(lmax, L[r]);
    }
    if (sq >= 0) {
      const int t = (int)(f0 + f) - a.cu_frames[sq];
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
