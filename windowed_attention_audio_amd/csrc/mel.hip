// Waveform -> log-mel frames (model card "MOSS-Transcribe-preview-2B-GGUF",
// Architecture table, Audio row; gotcha list: the trailing STFT frame is
// dropped, so a clip of n samples gives floor(n / 160) frames).
//
// Pass 1 (mel_frames_kernel): one wavefront per workgroup, one group of up to
// FPW = 7 consecutive frames of one sequence per wavefront (the host numbers
// each sequence's groups, so a group never spans two sequences).  The phases
// hand over through the wavefront's own LDS region (no workgroup barrier:
// the wavefront's LDS operations complete in order, a wait on them and a
// wave barrier separate the phases).
//   load    the group's samples as one span of 160 (FPW - 1) + 400 samples
//           (reflect padding by 200 at the sequence's ends, the edge sample
//           not repeated), coalesced, 22 loads per lane issued together.
//   DFT     400 = 16 x 25.  With n = 25 n1 + n2 and k = k1 + 16 k2,
//           X[k] = sum_n2 W400^(n2 k1) W25^(n2 k2) sum_n1 x[25 n1 + n2] W16^(n1 k1).
//           Step A: 25 real 16-point DFTs per frame (outputs k1 = 0..8; the
//           others follow by conjugate symmetry), halved twice (even / odd
//           indices), 175 tasks in three rounds of the 64 lanes.  Step B:
//           lane (frame, k1) for k1 = 0..8 only -- 63 lanes -- the
//           W400^(n2 k1) factors and the 25-point DFT as 5 x 5 with 5-point
//           DFTs that pair the terms sharing a cosine.  A real frame has
//           X[400 - k] = conj(X[k]), and 400 - (k1 + 16 k2) = (16 - k1) +
//           16 (24 - k2): lane k1 in 1..7 hands out its 25 outputs as bins
//           k1 + 16 k2 <= 200 and 400 - (k1 + 16 k2) < 200, lanes 0 and 8
//           their 13 bins up to 200, so the 201 bins come once each and no
//           lane computes k1 = 9..15.  Window, twiddles and sums in double:
//           bins 8 decades below the clip's loudest bin (the clamp floor)
//           carry rounding of the whole frame, which in fp32 costs about 1e-4
//           of the normalised output.
//   mel     |X[k]|^2 (rounded to fp32) through the Slaney filterbank (at
//           most nine taps per mel bin), lane (frame, j) doing the mel bins
//           j, j + 9, ...; log10(max(., 1e-10)) in fp32 from the hardware
//           log2, the floor giving -10 exactly; rows written as (L + 4) / 4,
//           staged in LDS and stored as whole 512-byte rows.
//   max     the wavefront's maximum goes to one of the sequence's `nslot`
//           slots (chosen by the group index; a cache line each when there
//           are several) with one atomicMax: few wavefronts meet on one line.
// Pass 2 (mel_norm_kernel, misc.hip): with g the largest of the sequence's
// slots, the entries below (g - 8 + 4) / 4 are raised to it -- the same
// values as (max(L, g - 8) + 4) / 4, since (x + 4) / 4 rounds monotonically
// -- and only the 16-byte chunks holding such an entry are written back.
#include "common.h"
#include "kernels.h"
#include "mel_tables.inc"

namespace mt {

namespace {

constexpr int SPAN = 160 * (MEL_FPW - 1) + 400;  // samples of one group
constexpr int SPAN_ITERS = (SPAN + 63) / 64;

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

// Every LDS access of this wavefront issued so far has completed; the
// wavefront's lanes may now overwrite what the others read.
__device__ __forceinline__ void lds_handover() {
  __builtin_amdgcn_s_waitcnt((0 << 8) | (7 << 4) | 15 | (3 << 14));  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
}

__global__ __launch_bounds__(64) void mel_frames_kernel(MelArgs a) {
  // One region, four uses in turn: the sample span (floats), the step-A
  // output Y[frame][n2][k1] (k1 = 0..8; a stride of 144 bytes per n2 keeps
  // the frames' rows on different LDS banks), the powers P[frame][201]
  // (floats), and from byte 8192 the log-mel rows L[frame][128] (floats).
  __shared__ double2 buf[MEL_FPW * 25 * 9];
  float* S = (float*)buf;
  float* P = (float*)buf;
  float* Lr = (float*)((char*)buf + 8192);
  // dump slots for stores a lane makes without effect: P_DUMP after P (below
  // byte 8192), L_DUMP after the last row of L (relative to any row of L)
  constexpr int P_DUMP = MEL_FPW * 201;
  constexpr int L_DUMP = MEL_FPW * 128;
  static_assert((P_DUMP + 1) * 4 <= 8192 && 8192 + 2 * MEL_FPW * 512 <= (int)sizeof(buf), "LDS plan");

  const int lane = threadIdx.x;
  const int g = blockIdx.x;

  // ---- the group's sequence: a 64-ary search over the group prefix
  // (cu_groups[0] = 0, strictly increasing): each step probes 64 evenly
  // spaced entries of [lo, hi) and keeps the last one <= g.
  int lo = 0, hi = a.nseq;
  while (hi - lo > 1) {
    const int step = (hi - lo + 63) / 64;
    const int p = min(lo + lane * step, hi - 1);
    const uint64_t le = __ballot(a.cu_groups[p] <= g);
    const int last = 63 - __clzll((unsigned long long)le);  // the last probe <= g (probe 0 always is)
    const int nlo = min(lo + last * step, hi - 1);
    hi = min(lo + (last + 1) * step, hi);
    lo = nlo;
  }
  const int sq = __builtin_amdgcn_readfirstlane(lo);
  const int T = a.cu_frames[sq + 1] - a.cu_frames[sq];
  const int t0 = (g - a.cu_groups[sq]) * MEL_FPW;  // the group's first frame in the sequence
  const int nf = min(MEL_FPW, T - t0);
  const int n = a.seq_len[sq];
  const int64_t soff = a.seq_sample_off[sq];
  const int64_t row0 = a.seq_row_off[sq] + t0;
  const int q0 = 160 * (t0 + (int)a.frame_off) - 200;  // stream sample of span element 0

  // ---- load the span (reflected at the sequence's ends); all loads first.
  // Interior spans (the usual case, uniform over the wavefront) need no
  // reflection.
  {
    float v[SPAN_ITERS];
    if (q0 >= 0 && q0 + SPAN <= n) {
      const float* src = a.wav + soff + q0;
#pragma unroll
      for (int i = 0; i < SPAN_ITERS; ++i) v[i] = src[min(lane + 64 * i, SPAN - 1)];
    } else {
#pragma unroll
      for (int i = 0; i < SPAN_ITERS; ++i) {
        int q = q0 + min(lane + 64 * i, SPAN - 1);
        q = q < 0 ? -q : q;
        q = q >= n ? 2 * (n - 1) - q : q;
        // the frames' own samples land in [0, n) (n > 200); span positions
        // past a partial group's last frame are only kept in bounds
        q = min(max(q, 0), n - 1);
        v[i] = a.wav[soff + q];
      }
    }
#pragma unroll
    for (int i = 0; i < SPAN_ITERS; ++i)
      if (lane + 64 * i < SPAN) S[lane + 64 * i] = v[i];
  }
  lds_handover();

  // ---- step A: task (frame, n2) -> 16-point real DFT over n1 of the
  // windowed frame, outputs k1 = 0..8.  Halving twice: with s = x[n] +
  // x[n+8], d = x[n] - x[n+8] (n < 8), the odd k1 are sum_n d[n] W16^(n k1);
  // with s2 = s[n] + s[n+4], d2 = s[n] - s[n+4] (n < 4), k1 = 0, 4, 8 are sums
  // of s2 times powers of -i and k1 = 2, 6 are sum_n d2[n] W8^(n k1 / 2).
  // Every task's samples are read before any output is written (Y overlays
  // the span).
  constexpr int NT = MEL_FPW * 25;
  constexpr int TA = (NT + 63) / 64;
  float xa[TA][16];
#pragma unroll
  for (int r = 0; r < TA; ++r) {
    const int task = min(lane + 64 * r, NT - 1);
    const int f = task / 25, n2 = task - f * 25;
#pragma unroll
    for (int n1 = 0; n1 < 16; ++n1) xa[r][n1] = S[160 * f + 25 * n1 + n2];
  }
  lds_handover();
  {
    const double r8 = c_tw[50].x;  // cos(pi / 4)
#pragma unroll
    for (int r = 0; r < TA; ++r) {
      const int task = lane + 64 * r;
      if (task >= NT) break;
      const int f = task / 25, n2 = task - f * 25;
      double x[16];
#pragma unroll
      for (int n1 = 0; n1 < 16; ++n1) x[n1] = (double)xa[r][n1] * c_hann[25 * n1 + n2];
      double s[8], d[8], s2[4], d2[4];
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        s[m] = x[m] + x[m + 8];
        d[m] = x[m] - x[m + 8];
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        s2[m] = s[m] + s[m + 4];
        d2[m] = s[m] - s[m + 4];
      }
      double2* out = buf + (f * 25 + n2) * 9;
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
        for (int m = 1; m < 8; ++m) {
          if (m == 4) continue;
          const double2 w = c_tw[(25 * m * k1) % 400];
          re = fma(d[m], w.x, re);
          im = fma(d[m], w.y, im);
        }
        out[k1] = make_double2(re, im);
      }
    }
  }
  lds_handover();

  // ---- step B: lane (frame, k1), k1 = 0..8 -> W400^(n2 k1), then the
  // 25-point DFT over n2 as 5 x 5 (n2 = 5 a + b, k2 = c + 5 d): five 5-point
  // DFTs over a, the W25^(b c) factors, five 5-point DFTs over b.  Powers of
  // the bins this lane hands out into P (over Y, once every lane has read it).
  const int fB = lane / 9, k1 = lane - 9 * fB;
  const bool laneB = lane < MEL_FPW * 9;
  {
    double2 y[25];
#pragma unroll
    for (int n2 = 0; n2 < 25; ++n2) y[n2] = buf[(min(fB, MEL_FPW - 1) * 25 + n2) * 9 + k1];
    lds_handover();
#pragma unroll
    for (int n2 = 1; n2 < 25; ++n2) y[n2] = cmul(y[n2], c_tw[n2 * k1]);
    const double C1 = c_tw[80].x, S1 = -c_tw[80].y, C2 = c_tw[160].x, S2 = -c_tw[160].y;
    double2 z[5][5];  // z[b][c]
#pragma unroll
    for (int b = 0; b < 5; ++b) dft5(y[b], y[5 + b], y[10 + b], y[15 + b], y[20 + b], C1, S1, C2, S2, z[b]);
#pragma unroll
    for (int b = 1; b < 5; ++b)
#pragma unroll
      for (int c = 1; c < 5; ++c) z[b][c] = cmul(z[b][c], c_tw[16 * b * c]);  // W25^(b c)
    // outputs this lane does not hand out (lane 63; k > 200 for k1 = 0, 8)
    // go to a dump slot past P, so the stores need no branch
    float* Pf = P + min(fB, MEL_FPW - 1) * 201;
    const int dump = P_DUMP - min(fB, MEL_FPW - 1) * 201;
    const bool mirror = laneB && k1 != 0 && k1 != 8;
#pragma unroll
    for (int c = 0; c < 5; ++c) {
      double2 o[5];  // o[d] = X[k1 + 16 (c + 5 d)]
      dft5(z[0][c], z[1][c], z[2][c], z[3][c], z[4][c], C1, S1, C2, S2, o);
#pragma unroll
      for (int dd = 0; dd < 5; ++dd) {
        const int k = k1 + 16 * (c + 5 * dd);
        const float pw = (float)(o[dd].x * o[dd].x + o[dd].y * o[dd].y);
        // bin k, or 400 - k (|X[400 - k]|^2 = |X[k]|^2) for k > 200
        Pf[k <= 200 ? (laneB ? k : dump) : (mirror ? 400 - k : dump)] = pw;
      }
    }
  }
  lds_handover();

  // ---- mel + log10; lane (frame, j) does the mel bins j, j + 9, ... with
  // the dense filter rows (nine weights from the filter's first bin, zero
  // past its end: the same sums as over the non-zero taps), every row's
  // three 16-byte loads issued before the first product.  log10 as the
  // hardware log2 times log10(2) (error ~1e-6 on values up to ~10, below the
  // 1e-4 bar by far after the / 4), the floor giving -10 exactly.  Rows are
  // written as (L + 4) / 4: the clamp pass then only raises the entries below
  // the floor.
  constexpr int MI = (128 + 8) / 9;  // 15 bins for lanes j < 2, 14 for the rest
  float lmax = -INFINITY;
  {
    float4 w[MI][3];
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int m = min(k1 + 9 * i, 127);
      const float4* row = (const float4*)(c_mel_pad + MEL_PAD * m);
      w[i][0] = row[0];
      w[i][1] = row[1];
      w[i][2] = row[2];
    }
    const float* Pf = P + min(fB, MEL_FPW - 1) * 201;
    float* Lf = Lr + min(fB, MEL_FPW - 1) * 128;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int m = k1 + 9 * i;
      const float* p = Pf + (int)w[i][2].y;
      float e = w[i][0].x * p[0];
      e += w[i][0].y * p[1];
      e += w[i][0].z * p[2];
      e += w[i][0].w * p[3];
      e += w[i][1].x * p[4];
      e += w[i][1].y * p[5];
      e += w[i][1].z * p[6];
      e += w[i][1].w * p[7];
      e += w[i][2].x * p[8];
      const float L = e > 1e-10f ? __builtin_amdgcn_logf(e) * 0.30102999566398120f : -10.0f;
      const bool keep = laneB && m < 128;
      Lf[keep ? m : L_DUMP] = (L + 4.0f) * 0.25f;  // Lf[L_DUMP]: past the rows, unused
      lmax = fmaxf(lmax, keep && fB < nf ? L : -INFINITY);
    }
  }
  lds_handover();

  // ---- whole rows out: nf x 32 float4
  float* out = a.mel + row0 * 128;
  for (int i = lane; i < nf * 32; i += 64) ((float4*)out)[i] = ((const float4*)Lr)[i];

  // ---- the wavefront's maximum into one of the sequence's slots
  lmax = wave_max64(lmax);
  if (lane == 0) atomicMax(a.gmax + (int64_t)(sq * a.nslot + g % a.nslot) * a.slot_stride, float_key(lmax));
}

}  // namespace

hipError_t launch_mel(const MelArgs& a, hipStream_t s) {
  if (a.total_groups == 0) return hipSuccess;
  hipLaunchKernelGGL(mel_frames_kernel, dim3((unsigned)a.total_groups), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace mt
