// Host-side launchers of the HIP kernels.  Every launcher enqueues work on
// `s` and returns hipGetLastError() of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mt {

// Element type of matrix operands (same codes as mt_dtype).
enum Dt : int { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };

// ---------------------------------------------------------------- tables
// Copies n 32-bit words from host memory into device memory through kernel
// arguments (graph-capturable, no host buffer needs to outlive the call).
hipError_t upload_words(uint32_t* dst, const uint32_t* src, int64_t n, hipStream_t s);

// Stages whose fp16 conversions clamped a value at +-65504 (the encode
// workspace's saturation mask; the values are part of the C ABI, mt.h).
enum : int { SAT_FRONTEND = 1, SAT_LN = 2, SAT_QKV = 4, SAT_FFN = 8, SAT_HEAD = 16, SAT_ADAPTER = 32 };

// ---------------------------------------------------------------- log-mel
// Frames per group of the log-mel kernel (one wavefront each; a group never
// spans two sequences): sequence i has ceil(T_i / MEL_FPW) groups.
constexpr int MEL_FPW = 7;

struct MelArgs {
  const float* wav;
  float* mel;
  const int64_t* seq_sample_off;  // [B]  first sample of sequence i in wav
  const int32_t* seq_len;         // [B]  samples n_i
  const int32_t* cu_frames;       // [B+1] prefix of T_i (packed frame numbering)
  const int32_t* cu_groups;       // [B+1] prefix of ceil(T_i / MEL_FPW)
  const int64_t* seq_row_off;     // [B]  output row of frame 0 of sequence i
  int* gmax;                      // ordered-int keys: each clip's max is the largest
                                  // of its nslot slots; slot j of sequence i at
                                  // (i * nslot + j) * slot_stride
  int nslot;
  int slot_stride;
  int nseq;
  int64_t total_groups;
  int64_t total_frames;
  int64_t out_rows;               // rows of the mel output (padded: B * Tmax)
  int padded;
  int64_t frame_off;              // frame t of a sequence is its frame t + frame_off
                                  // (a window of a longer stream: reflection at the
                                  // stream's own ends, n_i = the stream's length)
};
hipError_t launch_mel(const MelArgs& a, hipStream_t s);

// ---------------------------------------------------------------- conv1
struct Conv1Args {
  const float* mel;          // normalised log-mel rows
  const int64_t* mel_row_off;  // [B] row of frame 0 of sequence i
  const int32_t* cu_T;       // [B+1] mel frames prefix
  const int32_t* cu_T1;      // [B+1] conv1 output rows prefix
  int nseq;
  int64_t total_T1;
  const float* w;            // [C][9] (tap = df*3 + dt)
  const float* b;            // [C]
  void* out;                 // [sum T1][64][C] channels-last, element type dtype
  int C;
  int dtype;
  int* sat;                  // fp16: saturation mask (SAT_* bits), else nullptr
};
hipError_t launch_conv1(const Conv1Args& a, hipStream_t s);

// ---------------------------------------------------------------- GEMM
enum Epi : int {
  EPI_F32 = 0,         // C (fp32) = acc (+ bias)
  EPI_ACT = 1,         // C (T) = acc + bias
  EPI_GELU = 2,        // C (T) = GELU(acc + bias)
  EPI_GELU_SPLIT = 3,  // C (16-bit) [row][col] = hi, [row][N + col] = lo of GELU(acc + bias)
  EPI_RESID = 4,       // C (fp32) += acc + bias
  EPI_PE = 5,          // C (fp32) = acc + sinusoid(position of row, col)
  EPI_SWIGLU = 6,      // C (T) [row][f] = SiLU(gate) * up (gate/up interleaved by 16)
  EPI_OUT = 7,         // C (fp32) [mapped row][col] = acc (+ bias)
  EPI_GELU_PE = 8,     // C (fp32) = GELU(acc + bias) + sinusoid(position of row, col)
};

// Convolution gathers (GemmArgs.conv_kind).
enum {
  CONV_2D_S2 = 0,  // 3x3, stride 2 in time and frequency: K index = (3 df + dt) C + channel
  CONV_1D_S1 = 1,  // 3 taps over time, stride 1 (Fin = Fout = 1): K index = dt C + channel
  CONV_1D_S2 = 2,  // 3 taps over time, stride 2
};

struct GemmArgs {
  const void* A;
  int64_t lda;  // elements
  const void* B;
  int64_t ldb;  // elements; B is [N][K] row-major
  int M, N, K;
  const float* bias;
  void* C;
  int64_t ldc;
  // implicit-GEMM convolution (A gathered from a channels-last activation)
  int conv_C, conv_Fin, conv_Fout;
  int conv_kind;          // CONV_*
  const int32_t* cu_in;   // [nseq+1] input time rows prefix
  const int32_t* cu_out;  // [nseq+1] output time rows prefix
  int nseq;
  // row -> sequence position (EPI_PE, EPI_OUT)
  const int32_t* cu_rows;  // [nseq+1]
  int pos_offset;          // EPI_PE: position of a sequence's row 0
  int64_t out_seq_stride;  // EPI_OUT padded: rows per sequence (0 = packed)
  const void* zeros;       // >= 16 bytes of zeros (device), read by out-of-range loads
  int* sat;                // fp16 16-bit outputs: saturation mask, bit sat_bit (nullptr: off)
  int sat_bit;
  // fp32 operands: when part is set and the product has too few output
  // tiles to fill the GPU, K is split over up to GEMM_SPLIT_MAX workgroups
  // per tile (as many as part_floats floats of partial sums allow) and a
  // second launch adds the partial sums.
  float* part;
  int64_t part_floats;
};

constexpr int GEMM_SPLIT_MAX = 16;

// dtype: DT_F32, DT_BF16 or DT_F16 operands (fp32 accumulation in every
// case).  conv: gather A as a 3x3 stride-2 convolution input.
hipError_t launch_gemm(const GemmArgs& a, int epi, int dtype, bool conv, hipStream_t s);

// ---------------------------------------------------------------- LayerNorm
// out = LN(x) * g + b per row of D fp32 values, written as dtype (DT_*);
// split: 16-bit hi/lo pair written as [row][2D] (hi | lo).
// sat / sat_bit: fp16 saturation report (nullptr: off).
hipError_t launch_layernorm(const float* x, const float* g, const float* b, void* out, int M, int D,
                            float eps, int dtype, bool split, hipStream_t s, int* sat = nullptr,
                            int sat_bit = 0);

// ---------------------------------------------------------------- attention
struct AttnArgs {
  const void* qkv;  // [M][3D] (q | k | v), head h at columns h*64 .. h*64+63
  void* out;        // [M][D]
  const int32_t* cu_rows;  // [nseq+1]
  const int32_t* cu_win;   // [nseq+1] prefix of window counts
  int nseq;
  int n_windows;
  int window;
  int n_heads;
  int D;
  int wpad;  // longest window rounded up to 64 (K/V rows held on chip, zero-filled)
};
hipError_t launch_attention(const AttnArgs& a, int dtype, hipStream_t s);

// ---------------------------------------------------------------- misc
// Second log-mel pass: clamp at each clip's maximum - 8, then (x + 4) / 4;
// padded rows beyond a clip are zeroed.  tmax = padded rows per sequence.
hipError_t launch_mel_norm(const MelArgs& a, int64_t tmax, hipStream_t s);
hipError_t launch_fill_i32(int* p, int v, int64_t n, hipStream_t s);
hipError_t launch_zero_pad_rows(float* out, const int32_t* cu_rows, int nseq, int64_t seq_stride,
                                int D, hipStream_t s);
hipError_t launch_copy_rows(const float* x, float* out, int M, int D, const int32_t* cu_rows,
                            int nseq, int64_t stride, hipStream_t s);
// Packed 16-bit rows from fp32 rows: dst[r] = src[row_off[sq] + r - cu[sq]]
// (r in sequence sq), W values per row, dtype DT_BF16 or DT_F16.
hipError_t launch_rows_to_half(const float* src, const int64_t* row_off, const int32_t* cu, int nseq,
                               int64_t rows, int W, void* dst, int dtype, hipStream_t s);
// ------------------------------------------------------------------ decoder
// Language-model decoder step (decoder.hip).  head_dim 128; the KV cache is
// [layers][max_seqs][2 (K, V)][Hkv][max_pos][128] of the 16-bit type.
struct DecArgs {
  int rows, Hq, Hkv, layer, max_seqs, max_pos;
  float eps;             // RMSNorm epsilon (Q/K-norm)
  double log_base;       // ln(rotary base)
  const int32_t* seq;    // [rows] cache slot of each row's sequence
  const int32_t* pos;    // [rows] position of each row
  const float* q_norm;   // [128] this layer's Q-norm weight
  const float* k_norm;   // [128]
  float* qf;             // [rows][Hq][128] rotated queries (fp32)
  void* cache;
  const int32_t* items;       // [n_items][2] (row, 64-key chunk), ordered by row
  const int32_t* first_item;  // [rows + 1]
  float* part_o;         // [n_items][Hkv][2][128]
  float* part_ml;        // [n_items][Hkv][2][2] (chunk max, chunk sum)
  void* o16;             // [rows][Hq][128] attention output (16-bit)
};
// out = x W^T for at most GEMV_MAX_ROWS rows of x (16-bit [rows][K]), W 16-bit
// [N][K]: fp32 partial sums [ksplit][rows][N].
constexpr int GEMV_MAX_ROWS = 64;
hipError_t launch_gemv16(const void* W, const void* x, float* out, int rows, int N, int K, int ksplit, int dtype,
                         hipStream_t s);
// act [rows][F] (dtype) = SiLU(gate) * up from S <= 8 fp32 partials
// [S][rows][2F] of rows interleaved in blocks of 16 (16 gate, 16 up).
hipError_t launch_swiglu(const float* part, int S, void* act, int rows, int F, int dtype, hipStream_t s);
// x += sum of S <= 8 fp32 partials [S][rows][D]; h = RMSNorm(x) * w as dtype.
hipError_t launch_add_rmsnorm(float* x, const float* part, int S, const float* w, void* h, int rows, int D, float eps,
                              int dtype, hipStream_t s);
hipError_t launch_qk_rope(const DecArgs& a, const float* qkv, int S, int dtype, hipStream_t s);
// attention over the chunk items -> part_o / part_ml; with combine, then
// o16 = the combined output (else the output projection combines them).
// S = 0: queries from qf (after launch_qk_rope).  S = 1, 2, 4 or 8, for calls
// with one row per sequence: the kernel computes the queries and the new
// key / value (cache append) itself from the S qkv partials.
hipError_t launch_attn_dec(const DecArgs& a, int n_items, bool combine, const float* qkv, int S, int dtype,
                           hipStream_t s);
// The skinny product for at most GEMV_FUSE_ROWS rows with x computed from
// its producer's partials: xm = 1, x = SwiGLU of the gate/up partials src
// (S splits, K = F); xm = 2, x = the attention chunk partials of a combined
// (K = Hq * 128, cmax >= chunks of any row).  Same partial-sum output.
constexpr int GEMV_FUSE_ROWS = 4;
hipError_t launch_gemv16x(const void* W, int xm, const float* src, int S, const DecArgs& a, int cmax, float* out,
                          int rows, int N, int K, int ksplit, int dtype, hipStream_t s);
// next[r] = first index of the largest logit; pv / pi: [rows][64] scratch.
hipError_t launch_argmax(const float* logits, int rows, int V, float* pv, int* pi, int32_t* next, hipStream_t s);

// Weight repacking (fp32 masters -> kernel layouts); dtype selects the
// destination element type (DT_*).
hipError_t launch_convert(const float* src, void* dst, int64_t rows, int64_t cols, int64_t dst_ld,
                          int64_t dst_col0, int dtype, hipStream_t s);
// Prompt embedding: out[i] = table[map[i]] (map[i] >= 0, table rows of d
// elements of dtype) or audio[-map[i] - 1] (fp32 rows); out fp32 [rows][d].
hipError_t launch_splice(const int64_t* map, int64_t rows, const void* table, int dtype,
                         const float* audio, float* out, int d, hipStream_t s);
hipError_t launch_pack_conv(const float* w, void* dst, int C, int dtype, hipStream_t s);
// Conv1d [Co][Ci][3] -> [Co][3 Ci], column dt * Ci + ci.
hipError_t launch_pack_conv1d(const float* w, void* dst, int Co, int Ci, int dtype, hipStream_t s);
hipError_t launch_pack_conv_out(const float* w, void* dst, int D, int C, int F, int dtype,
                                hipStream_t s);
hipError_t launch_pack_swiglu(const float* gate, const float* up, void* dst, int A, int O, int dtype,
                              hipStream_t s);
hipError_t launch_copy_f32(const float* src, float* dst, int64_t n, hipStream_t s);

}  // namespace mt
