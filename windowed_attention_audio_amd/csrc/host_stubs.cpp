// Host-only stand-ins for the kernel launchers and the few HIP runtime calls
// of api.cpp, for the sanitizer build of the C ABI (g++ with AddressSanitizer
// and UndefinedBehaviorSanitizer, no GPU).  In that build every "device"
// pointer is host memory.  Each launcher runs no arithmetic; it reads (and,
// for outputs, writes) the first and last byte of every buffer range its
// kernel would access, computed from the same arguments, so that a workspace
// region carved too small, an output sized wrongly or a table uploaded to the
// wrong place shows up as an out-of-bounds access under AddressSanitizer.
// Tables that the kernels read from device memory (prefix sums, row maps)
// are read here the same way, after upload_words has copied them.
#include <stdio.h>
#include <string.h>

#include <algorithm>

#include "kernels.h"

namespace {

volatile unsigned char g_sink;

void rd(const void* p, size_t bytes) {
  if (!bytes) return;
  const unsigned char* c = (const unsigned char*)p;
  g_sink = c[0];
  g_sink = c[bytes - 1];
}

void wr(void* p, size_t bytes) {
  if (!bytes) return;
  unsigned char* c = (unsigned char*)p;
  c[0] = 0;
  c[bytes - 1] = 0;
}

size_t esize(int dtype) { return dtype == mt::DT_F32 ? 4 : 2; }

}  // namespace

extern "C" {

const char* hipGetErrorString(hipError_t) { return "host stub"; }
hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}
hipError_t hipGetSymbolAddress(void** ptr, const void* symbol) {
  *ptr = (void*)symbol;  // host build: the array itself
  return hipSuccess;
}
hipError_t hipEventCreate(hipEvent_t* e) {
  static char dummy[64];
  *e = (hipEvent_t)dummy;
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) {
  *ms = 0.f;
  return hipSuccess;
}

}  // extern "C"

namespace mt {

hipError_t upload_words(uint32_t* dst, const uint32_t* src, int64_t n, hipStream_t) {
  memcpy(dst, src, 4 * (size_t)n);
  return hipSuccess;
}

hipError_t launch_mel(const MelArgs& a, hipStream_t) {
  if (a.total_groups == 0) return hipSuccess;
  if (a.cu_groups[a.nseq] != a.total_groups) return hipErrorInvalidValue;
  for (int i = 0; i < a.nseq; ++i) {
    const int64_t T = a.cu_frames[i + 1] - a.cu_frames[i];
    if (a.cu_groups[i + 1] - a.cu_groups[i] != (T + MEL_FPW - 1) / MEL_FPW) return hipErrorInvalidValue;
  }
  wr(a.gmax, 4 * ((size_t)(a.nseq * a.nslot - 1) * a.slot_stride + 1));
  for (int i = 0; i < a.nseq; ++i) {
    const int64_t T = a.cu_frames[i + 1] - a.cu_frames[i];
    // frames [frame_off, frame_off + T) of a sequence of seq_len samples read
    // samples [160 frame_off - 200, 160 (frame_off + T - 1) + 200), reflected
    // into [0, seq_len)
    if (T > 0) {
      const int64_t lo = std::max<int64_t>(0, 160 * a.frame_off - 200);
      const int64_t hi = std::min<int64_t>(a.seq_len[i], 160 * (a.frame_off + T - 1) + 200);
      rd(a.wav + a.seq_sample_off[i] + lo, 4 * (size_t)(hi - lo));
    }
    wr(a.mel + a.seq_row_off[i] * 128, 4 * 128 * (size_t)T);
  }
  if (a.cu_frames[a.nseq] != a.total_frames) return hipErrorInvalidValue;
  return hipSuccess;
}

hipError_t launch_mel_norm(const MelArgs& a, int64_t, hipStream_t) {
  wr(a.mel, 4 * 128 * (size_t)a.out_rows);
  rd(a.gmax, 4 * ((size_t)(a.nseq * a.nslot - 1) * a.slot_stride + 1));
  return hipSuccess;
}

hipError_t launch_fill_i32(int* p, int v, int64_t n, hipStream_t) {
  for (int64_t i = 0; i < n; ++i) p[i] = v;
  return hipSuccess;
}

hipError_t launch_conv1(const Conv1Args& a, hipStream_t) {
  for (int i = 0; i < a.nseq; ++i)
    rd(a.mel + a.mel_row_off[i] * 128, 4 * 128 * (size_t)(a.cu_T[i + 1] - a.cu_T[i]));
  if (a.cu_T1[a.nseq] != a.total_T1) return hipErrorInvalidValue;
  wr(a.out, (size_t)a.total_T1 * 64 * a.C * esize(a.dtype));
  if (a.sat) wr(a.sat, 4);
  rd(a.w, 4 * 9 * (size_t)a.C);
  rd(a.b, 4 * (size_t)a.C);
  return hipSuccess;
}

hipError_t launch_gemm(const GemmArgs& a, int epi, int dtype, bool conv, hipStream_t) {
  if (a.N < 4 || a.N % 4) return hipErrorInvalidValue;
  if (a.M == 0) return hipSuccess;
  const size_t es = esize(dtype);
  if (conv) {
    // the gather reads the channels-last input rows of every sequence
    rd(a.A, (size_t)a.cu_in[a.nseq] * a.conv_Fin * a.conv_C * es);
    if ((int64_t)a.cu_out[a.nseq] * a.conv_Fout != a.M) return hipErrorInvalidValue;
  } else {
    rd(a.A, ((size_t)(a.M - 1) * a.lda + a.K) * es);
  }
  rd(a.B, ((size_t)(a.N - 1) * a.ldb + a.K) * es);
  if (a.bias) rd(a.bias, 4 * (size_t)a.N);
  if (a.zeros) rd(a.zeros, 16);
  if (a.sat) wr(a.sat, 4);
  size_t cols = a.N, ces = 4;
  int64_t rows = a.M;
  switch (epi) {
    case EPI_ACT: case EPI_GELU: ces = es; break;
    case EPI_GELU_SPLIT: ces = es; cols = 2 * (size_t)a.N; break;
    case EPI_SWIGLU: ces = es; cols = a.N / 2; break;
    case EPI_OUT:
      if (a.out_seq_stride > 0) {
        const int last = a.nseq - 1;
        rows = (int64_t)last * a.out_seq_stride + (a.cu_rows[last + 1] - a.cu_rows[last]);
      }
      break;
    default: break;
  }
  if (epi == EPI_PE || epi == EPI_GELU_PE || epi == EPI_OUT)
    if (a.cu_rows && a.cu_rows[a.nseq] != a.M) return hipErrorInvalidValue;
  wr(a.C, ((size_t)(rows - 1) * a.ldc + cols) * ces);
  return hipSuccess;
}

hipError_t launch_layernorm(const float* x, const float* g, const float* b, void* out, int M, int D, float,
                            int dtype, bool split, hipStream_t, int* sat, int) {
  if (sat) wr(sat, 4);
  rd(x, 4 * (size_t)M * D);
  rd(g, 4 * (size_t)D);
  rd(b, 4 * (size_t)D);
  wr(out, (size_t)M * D * (split ? 2 : 1) * esize(dtype));
  return hipSuccess;
}

hipError_t launch_attention(const AttnArgs& a, int dtype, hipStream_t) {
  const int64_t M = a.cu_rows[a.nseq];
  if (a.cu_win[a.nseq] != a.n_windows) return hipErrorInvalidValue;
  rd(a.qkv, (size_t)M * 3 * a.D * esize(dtype));
  wr(a.out, (size_t)M * a.D * esize(dtype));
  return hipSuccess;
}

hipError_t launch_copy_rows(const float* x, float* out, int M, int D, const int32_t* cu_rows, int nseq,
                            int64_t stride, hipStream_t) {
  rd(x, 4 * (size_t)M * D);
  if (cu_rows[nseq] != M) return hipErrorInvalidValue;
  const int64_t rows = stride > 0 ? (int64_t)(nseq - 1) * stride + (cu_rows[nseq] - cu_rows[nseq - 1]) : M;
  wr(out, 4 * (size_t)rows * D);
  return hipSuccess;
}

hipError_t launch_zero_pad_rows(float* out, const int32_t* cu_rows, int nseq, int64_t stride, int D,
                                hipStream_t) {
  rd(cu_rows, 4 * (size_t)(nseq + 1));
  wr(out, 4 * (size_t)nseq * stride * D);
  return hipSuccess;
}

hipError_t launch_rows_to_half(const float* src, const int64_t* row_off, const int32_t* cu, int nseq,
                               int64_t rows, int W, void* dst, int dtype, hipStream_t) {
  for (int i = 0; i < nseq; ++i) rd(src + row_off[i] * W, 4 * (size_t)(cu[i + 1] - cu[i]) * W);
  if (cu[nseq] != rows) return hipErrorInvalidValue;
  wr(dst, (size_t)rows * W * esize(dtype));
  return hipSuccess;
}

hipError_t launch_convert(const float* src, void* dst, int64_t rows, int64_t cols, int64_t dst_ld,
                          int64_t dst_col0, int dtype, hipStream_t) {
  rd(src, 4 * (size_t)rows * cols);
  const size_t es = esize(dtype);
  wr((char*)dst + dst_col0 * es, ((size_t)(rows - 1) * dst_ld + cols) * es);
  return hipSuccess;
}

hipError_t launch_copy_f32(const float* src, float* dst, int64_t n, hipStream_t) {
  rd(src, 4 * (size_t)n);
  wr(dst, 4 * (size_t)n);
  return hipSuccess;
}

hipError_t launch_pack_conv(const float* w, void* dst, int C, int dtype, hipStream_t) {
  rd(w, 4 * (size_t)C * C * 9);
  wr(dst, (size_t)C * 9 * C * esize(dtype));
  return hipSuccess;
}

hipError_t launch_pack_conv1d(const float* w, void* dst, int Co, int Ci, int dtype, hipStream_t) {
  rd(w, 4 * (size_t)Co * Ci * 3);
  wr(dst, (size_t)Co * 3 * Ci * esize(dtype));
  return hipSuccess;
}

hipError_t launch_pack_conv_out(const float* w, void* dst, int D, int C, int F, int dtype, hipStream_t) {
  rd(w, 4 * (size_t)D * C * F);
  wr(dst, (size_t)D * C * F * esize(dtype));
  return hipSuccess;
}

hipError_t launch_pack_swiglu(const float* gate, const float* up, void* dst, int A, int O, int dtype,
                              hipStream_t) {
  rd(gate, 4 * (size_t)A * O);
  rd(up, 4 * (size_t)A * O);
  wr(dst, 2 * (size_t)A * O * esize(dtype));
  return hipSuccess;
}

hipError_t launch_splice(const int64_t* map, int64_t rows, const void* table, int dtype, const float* audio,
                         float* out, int d, hipStream_t) {
  const size_t es = esize(dtype);
  for (int64_t i = 0; i < rows; ++i) {
    if (map[i] >= 0) rd((const char*)table + (size_t)map[i] * d * es, (size_t)d * es);
    else rd(audio + (size_t)(-map[i] - 1) * d, 4 * (size_t)d);
  }
  wr(out, 4 * (size_t)rows * d);
  return hipSuccess;
}

hipError_t launch_gemv16(const void* W, const void* x, float* out, int rows, int N, int K, int ksplit, int,
                         hipStream_t) {
  rd(W, 2 * (size_t)N * K);
  rd(x, 2 * (size_t)rows * K);
  wr(out, 4 * (size_t)ksplit * rows * N);
  return hipSuccess;
}

hipError_t launch_swiglu(const float* part, int S, void* act, int rows, int F, int, hipStream_t) {
  rd(part, 4 * (size_t)S * rows * 2 * F);
  wr(act, 2 * (size_t)rows * F);
  return hipSuccess;
}

hipError_t launch_add_rmsnorm(float* x, const float* part, int S, const float* w, void* h, int rows, int D,
                              float, int, hipStream_t) {
  wr(x, 4 * (size_t)rows * D);
  if (part) rd(part, 4 * (size_t)S * rows * D);
  rd(w, 4 * (size_t)D);
  wr(h, 2 * (size_t)rows * D);
  return hipSuccess;
}

hipError_t launch_qk_rope(const DecArgs& a, const float* qkv, int S, int, hipStream_t) {
  rd(qkv, 4 * (size_t)S * a.rows * (a.Hq + 2 * a.Hkv) * 128);
  wr(a.qf, 4 * (size_t)a.rows * a.Hq * 128);
  rd(a.seq, 4 * (size_t)a.rows);
  rd(a.pos, 4 * (size_t)a.rows);
  return hipSuccess;
}

hipError_t launch_attn_dec(const DecArgs& a, int n_items, bool combine, const float* qkv, int S, int,
                           hipStream_t) {
  rd(a.items, 8 * (size_t)n_items);
  rd(a.first_item, 4 * (size_t)(a.rows + 1));
  if (a.first_item[a.rows] != n_items) return hipErrorInvalidValue;
  wr(a.part_o, 4 * (size_t)n_items * a.Hkv * 2 * 128);
  wr(a.part_ml, 4 * (size_t)n_items * a.Hkv * 2 * 2);
  if (combine) wr(a.o16, 2 * (size_t)a.rows * a.Hq * 128);
  if (qkv) rd(qkv, 4 * (size_t)S * a.rows * (a.Hq + 2 * a.Hkv) * 128);
  else rd(a.qf, 4 * (size_t)a.rows * a.Hq * 128);
  return hipSuccess;
}

hipError_t launch_gemv16x(const void* W, int xm, const float* src, int S, const DecArgs& a, int, float* out,
                          int rows, int N, int K, int ksplit, int, hipStream_t) {
  rd(W, 2 * (size_t)N * K);
  if (xm == 1) rd(src, 4 * (size_t)S * rows * 2 * K);
  if (xm == 2) rd(a.part_o, 4);
  wr(out, 4 * (size_t)ksplit * rows * N);
  return hipSuccess;
}

hipError_t launch_argmax(const float* logits, int rows, int V, float* pv, int* pi, int32_t* next, hipStream_t) {
  rd(logits, 4 * (size_t)rows * V);
  wr(pv, 4 * (size_t)rows * 64);
  wr(pi, 4 * (size_t)rows * 64);
  wr(next, 4 * (size_t)rows);
  return hipSuccess;
}

}  // namespace mt
