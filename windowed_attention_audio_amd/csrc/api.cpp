// C ABI of the encoder library: argument validation, length planning,
// workspace carving and the launch sequence.  All validation happens on the
// host before the first launch, so a failing call enqueues nothing.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <cmath>
#include <string>
#include <vector>

#include "kernels.h"
#include "mt.h"

using namespace mt;

namespace {

thread_local std::string g_err;

mt_status fail(mt_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

mt_status hip_fail(hipError_t e, const char* where) {
  return fail(MT_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

#define HIP_TRY(call, where)                     \
  do {                                           \
    hipError_t e_ = (call);                      \
    if (e_ != hipSuccess) return hip_fail(e_, where); \
  } while (0)

// A launch of a named stage (timed when that stage is armed).
#define STAGE(call, stage)                       \
  do {                                           \
    TraceScope ts_(stage, s);                    \
    HIP_TRY(call, stage);                        \
  } while (0)

constexpr int64_t HOP = 160;
constexpr int TABLE_HEAD_WORDS = 64;
// fp32 encoders: partial sums of the K-split products (see GemmArgs::part)
constexpr int64_t SPLIT_PART_FLOATS = 4 << 20;  // the encode workspace's first 256 bytes: the saturation mask
constexpr int MAX_WINDOW = 256;
constexpr int64_t MAX_SEQS = 1 << 20;
constexpr size_t ALIGN = 256;

inline size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

// ---- stage timer (diagnostics): brackets launches of one named stage with
// hipEvents recorded on the launch stream.
struct Tracer {
  std::string stage;
  std::vector<hipEvent_t> ev;  // pairs
  int used = 0;
} g_trace;

struct TraceScope {
  hipEvent_t stop = nullptr;
  hipStream_t s;
  TraceScope(const char* stage, hipStream_t st) : s(st) {
    if (g_trace.stage.empty() || g_trace.stage != stage) return;
    if (2 * (g_trace.used + 1) > (int)g_trace.ev.size()) return;
    hipEvent_t start = g_trace.ev[2 * g_trace.used];
    stop = g_trace.ev[2 * g_trace.used + 1];
    ++g_trace.used;
    (void)hipEventRecord(start, s);
  }
  ~TraceScope() {
    if (stop) (void)hipEventRecord(stop, s);
  }
};
inline int64_t half_up(int64_t x) { return (x + 1) / 2; }
// Encoder frames of T mel frames: three stride-2 convs (8x) or one (2x).
inline int64_t frames_of(int frontend, int64_t T) {
  return frontend == MT_FRONTEND_CONV1D_2X ? half_up(T) : half_up(half_up(half_up(T)));
}

// Carves named regions out of one buffer.
struct Carver {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  }
};

mt_status check_batch(const mt_batch* b, const char* what) {
  if (!b) return fail(MT_ERR_INVALID_ARG, "%s: batch is NULL", what);
  if (b->layout != MT_PACKED && b->layout != MT_PADDED)
    return fail(MT_ERR_INVALID_ARG, "%s: layout %d is neither MT_PACKED nor MT_PADDED", what,
                b->layout);
  if (b->n_seqs < 1 || b->n_seqs > MAX_SEQS)
    return fail(MT_ERR_INVALID_ARG, "%s: n_seqs %d out of range [1, %lld]", what, b->n_seqs,
                (long long)MAX_SEQS);
  if (!b->len) return fail(MT_ERR_INVALID_ARG, "%s: len is NULL", what);
  for (int i = 0; i < b->n_seqs; ++i) {
    if (b->len[i] < 0) return fail(MT_ERR_INVALID_ARG, "%s: len[%d] < 0", what, i);
    if (b->layout == MT_PADDED && b->len[i] > b->max_len)
      return fail(MT_ERR_INVALID_ARG, "%s: len[%d] = %lld exceeds max_len %lld", what, i,
                  (long long)b->len[i], (long long)b->max_len);
  }
  return MT_OK;
}

// ------------------------------------------------------------------ log-mel plan
struct MelPlan {
  int B = 0;
  int nslot = 1;        // slots per sequence for its log-mel maximum
  int slot_stride = 1;  // ints from one slot to the next
  std::vector<int64_t> sample_off, row_off;
  std::vector<int32_t> seq_len, cu_frames, cu_groups;
  int64_t total_frames = 0, total_groups = 0, out_rows = 0, tmax = 0;
  size_t off_sample = 0, off_row = 0, off_len = 0, off_cu = 0, off_cug = 0, off_gmax = 0, bytes = 0;
};

// Slots per sequence for the log-mel maximum, each its own cache line for
// the frame kernel's atomics: 512 lines over the batch while it is small (a
// single long stream would otherwise put one atomic of every wavefront on a
// few lines), one per sequence once the sequences spread them.
int mel_slots(int B) {
  int n = 1;
  while (n < 64 && n * 2 * B <= 512) n *= 2;
  return n;
}

mt_status plan_mel(const mt_batch* wb, MelPlan& p) {
  mt_status st = check_batch(wb, "mt_logmel");
  if (st != MT_OK) return st;
  const int B = wb->n_seqs;
  p.B = B;
  p.sample_off.resize(B);
  p.row_off.resize(B);
  p.seq_len.resize(B);
  p.cu_frames.assign(B + 1, 0);
  p.cu_groups.assign(B + 1, 0);
  p.nslot = mel_slots(B);
  p.tmax = wb->layout == MT_PADDED ? wb->max_len / HOP : 0;
  int64_t s_acc = 0, t_acc = 0, g_acc = 0;
  for (int i = 0; i < B; ++i) {
    const int64_t n = wb->len[i];
    if (n <= 200)
      return fail(MT_ERR_INVALID_ARG,
                  "mt_logmel: len[%d] = %lld samples; reflect padding by 200 needs more than 200",
                  i, (long long)n);
    if (n > INT32_MAX) return fail(MT_ERR_UNSUPPORTED, "mt_logmel: len[%d] too long", i);
    const int64_t T = n / HOP;
    p.seq_len[i] = (int32_t)n;
    p.sample_off[i] = wb->layout == MT_PADDED ? (int64_t)i * wb->max_len : s_acc;
    p.row_off[i] = wb->layout == MT_PADDED ? (int64_t)i * p.tmax : t_acc;
    s_acc += n;
    t_acc += T;
    if (t_acc > INT32_MAX / 2) return fail(MT_ERR_UNSUPPORTED, "mt_logmel: batch too long");
    p.cu_frames[i + 1] = (int32_t)t_acc;
    g_acc += (T + MEL_FPW - 1) / MEL_FPW;
    p.cu_groups[i + 1] = (int32_t)g_acc;
  }
  p.total_frames = t_acc;
  p.total_groups = g_acc;
  p.out_rows = wb->layout == MT_PADDED ? (int64_t)B * p.tmax : t_acc;
  Carver c;
  p.off_sample = c.take(8 * (size_t)B);
  p.off_row = c.take(8 * (size_t)B);
  p.off_len = c.take(4 * (size_t)B);
  p.off_cu = c.take(4 * (size_t)(B + 1));
  p.off_cug = c.take(4 * (size_t)(B + 1));
  p.slot_stride = p.nslot > 1 ? 32 : 1;  // several slots: a 128-byte line each
  p.off_gmax = c.take(4 * (size_t)B * p.nslot * p.slot_stride);
  p.bytes = c.off;
  return MT_OK;
}

// ------------------------------------------------------------------ encoder
struct Layer {
  const float *ln1_g, *ln1_b;
  const void* wqkv;
  const float* bqkv;
  const void* wo;
  const float* bo;
  const float *ln2_g, *ln2_b;
  const void* w1;
  const float* b1;
  const void* w2;
  const float* b2;
};

struct PackedLayout {
  size_t conv1_w, conv1_b, conv2_w, conv2_b, conv3_w, conv3_b, conv_out_w;
  struct L {
    size_t ln1_g, ln1_b, wqkv, bqkv, wo, bo, ln2_g, ln2_b, w1, b1, w2, b2;
  };
  std::vector<L> layers;
  size_t lnp_g, lnp_b, wp1, bp1, wp2, bp2, wgu, wd;
  size_t zeros;  // 256 bytes of zeros read by out-of-range matrix loads
  size_t bytes;
};

mt_status check_config(const mt_encoder_config* c) {
  if (!c) return fail(MT_ERR_INVALID_ARG, "config is NULL");
  if (c->dtype != MT_F32 && c->dtype != MT_BF16 && c->dtype != MT_F16)
    return fail(MT_ERR_INVALID_ARG, "dtype %d is not MT_F32, MT_BF16 or MT_F16", c->dtype);
  if (c->n_layers < 0 || c->n_heads < 1 || c->head_dim < 1 || c->conv_ch < 1 || c->d_model < 1 ||
      c->d_ffn < 1 || c->d_out < 1 || c->adapter_hidden < 0 || c->n_mels < 1)
    return fail(MT_ERR_INVALID_ARG, "non-positive size in config");
  if (!(c->ln_eps > 0.f)) return fail(MT_ERR_INVALID_ARG, "ln_eps must be > 0");
  if (c->with_head != 0 && c->with_head != 1)
    return fail(MT_ERR_INVALID_ARG, "with_head must be 0 or 1");
  if (c->frontend != MT_FRONTEND_CONV2D_8X && c->frontend != MT_FRONTEND_CONV1D_2X)
    return fail(MT_ERR_INVALID_ARG, "frontend %d is not an mt_frontend", c->frontend);
  if (c->n_mels != 128) return fail(MT_ERR_UNSUPPORTED, "n_mels must be 128");
  if (c->head_dim != 64) return fail(MT_ERR_UNSUPPORTED, "head_dim must be 64");
  if (c->n_heads * c->head_dim != c->d_model)
    return fail(MT_ERR_UNSUPPORTED, "n_heads * head_dim must equal d_model");
  if (c->d_model % 256 || c->d_model > 2048)
    return fail(MT_ERR_UNSUPPORTED, "d_model must be a multiple of 256, at most 2048");
  if (c->d_ffn % 64 || c->d_out % 64 || c->adapter_hidden % 64)
    return fail(MT_ERR_UNSUPPORTED, "d_ffn, d_out, adapter_hidden must be multiples of 64");
  if (c->frontend == MT_FRONTEND_CONV1D_2X) {
    // 1-D convolutions and a ln_post-only head; the convolutions run on the
    // 16-bit matrix-core path only
    if (c->dtype == MT_F32)
      return fail(MT_ERR_UNSUPPORTED, "the 2x front-end needs MT_BF16 or MT_F16");
    if (c->adapter_hidden) return fail(MT_ERR_INVALID_ARG, "the 2x front-end has no adapter");
    if (c->d_out != c->d_model)
      return fail(MT_ERR_INVALID_ARG, "the 2x front-end's output is d_model wide (d_out = d_model)");
    return MT_OK;
  }
  if (c->conv_ch % 32) return fail(MT_ERR_UNSUPPORTED, "conv_ch must be a multiple of 32");
  if (c->conv_ch > 2048) return fail(MT_ERR_UNSUPPORTED, "conv_ch must be at most 2048");
  if (c->adapter_hidden && !c->with_head)
    return fail(MT_ERR_INVALID_ARG, "the adapter needs with_head = 1");
  return MT_OK;
}

PackedLayout packed_layout(const mt_encoder_config& c) {
  const bool half = c.dtype != MT_F32;
  const size_t es = half ? 2 : 4;
  const size_t C = c.conv_ch, D = c.d_model, F = c.d_ffn, O = c.d_out, A = c.adapter_hidden;
  const size_t KD = half ? 2 * D : D;  // hi/lo split head input
  const bool two_x = c.frontend == MT_FRONTEND_CONV1D_2X;
  PackedLayout p;
  Carver k;
  if (two_x) {  // conv1 [D][3 n_mels], conv2 [D][3 D], 16-bit
    p.conv1_w = k.take(D * 3 * (size_t)c.n_mels * es);
    p.conv1_b = k.take(D * 4);
    p.conv2_w = k.take(D * 3 * D * es);
    p.conv2_b = k.take(D * 4);
    p.conv3_w = p.conv3_b = p.conv_out_w = 0;
  } else {
    p.conv1_w = k.take(C * 9 * 4);
    p.conv1_b = k.take(C * 4);
    p.conv2_w = k.take(C * 9 * C * es);
    p.conv2_b = k.take(C * 4);
    p.conv3_w = k.take(C * 9 * C * es);
    p.conv3_b = k.take(C * 4);
    p.conv_out_w = k.take(D * 16 * C * es);
  }
  p.layers.resize(c.n_layers);
  for (auto& L : p.layers) {
    L.ln1_g = k.take(D * 4);
    L.ln1_b = k.take(D * 4);
    L.wqkv = k.take(3 * D * D * es);
    L.bqkv = k.take(3 * D * 4);
    L.wo = k.take(D * D * es);
    L.bo = k.take(D * 4);
    L.ln2_g = k.take(D * 4);
    L.ln2_b = k.take(D * 4);
    L.w1 = k.take(F * D * es);
    L.b1 = k.take(F * 4);
    L.w2 = k.take(D * F * es);
    L.b2 = k.take(D * 4);
  }
  p.lnp_g = k.take(D * 4);
  p.lnp_b = k.take(D * 4);
  p.wp1 = two_x ? 0 : k.take(D * KD * es);
  p.bp1 = two_x ? 0 : k.take(D * 4);
  p.wp2 = two_x ? 0 : k.take(O * KD * es);
  p.bp2 = two_x ? 0 : k.take(O * 4);
  p.wgu = A ? k.take(2 * A * O * es) : 0;
  p.wd = A ? k.take(O * A * es) : 0;
  p.zeros = k.take(256);
  p.bytes = k.off;
  return p;
}

int n_weights_of(const mt_encoder_config& c) {
  if (c.frontend == MT_FRONTEND_CONV1D_2X) return 4 + 16 * c.n_layers + 2;
  return 7 + 16 * c.n_layers + 6 + (c.adapter_hidden ? 3 : 0);
}

struct EncPlan {
  int B = 0;
  std::vector<int32_t> words;  // cu_T, cu_T1, cu_T2, cu_N, cu_win (B+1 each)
  std::vector<int64_t> mel_row_off;
  int64_t sumT = 0, sumT1 = 0, sumT2 = 0, M = 0, maxN = 0, n_windows = 0, out_stride = 0;
  int wpad = 0;
  // workspace offsets
  size_t o_words, o_rowoff, o_twords, o_act1, o_act2, o_act3, o_x, o_h, o_qkv, o_att, o_ffn, o_y, o_ahid,
      o_part, bytes;
};

// One chunk of a stream (mt_encode_stream): the batch is one sequence, a
// window of mel frames of the stream; its first `drop` encoder frames are the
// halo (their receptive field leaves the window) and the next `keep` are
// encoded; `pos` is the stream position of the sequence's encoder frame 0.
struct StreamChunk {
  int pos = 0, drop = 0, keep = 0;
};

}  // namespace

struct mt_encoder {
  mt_encoder_config cfg;
  int dt;     // element type of matrix operands (DT_F32, DT_BF16, DT_F16)
  size_t es;  // element bytes of matrix operands
  const float *conv1_w, *conv1_b, *conv2_b, *conv3_b;
  const void *conv2_w, *conv3_w, *conv_out_w;
  std::vector<Layer> layers;
  const float *lnp_g, *lnp_b, *bp1, *bp2;
  const void *wp1, *wp2, *wgu, *wd;
  const void* zeros;
};

struct mt_stream {
  const mt_encoder* enc = nullptr;
  int window = 0;
  int64_t max_push = 0;
  char* state = nullptr;
  int cur = 0;          // buffer holding the recent samples
  int64_t base = 0;     // stream index of that buffer's first sample
  int64_t have = 0;     // samples pushed so far
  int64_t next = 0;     // next window to encode
  bool finished = false;
};

namespace {

mt_status plan_encode(const mt_encoder* enc, const mt_batch* mb, int32_t window, EncPlan& p) {
  mt_status st = check_batch(mb, "mt_encode");
  if (st != MT_OK) return st;
  if (window < 1) return fail(MT_ERR_INVALID_ARG, "window must be >= 1 (got %d)", window);
  const mt_encoder_config& c = enc->cfg;
  const int B = mb->n_seqs;
  p.B = B;
  // word 0: the fp16 saturation mask (reset to 0 by the table upload), then
  // padding to 256 bytes, then cu_T | cu_T1 | cu_T2 | cu_N | cu_win
  p.words.assign(TABLE_HEAD_WORDS + 5 * (size_t)(B + 1), 0);
  int32_t* cuT = p.words.data() + TABLE_HEAD_WORDS;
  int32_t* cuT1 = cuT + (B + 1);
  int32_t* cuT2 = cuT1 + (B + 1);
  int32_t* cuN = cuT2 + (B + 1);
  int32_t* cuW = cuN + (B + 1);
  p.mel_row_off.resize(B);
  for (int i = 0; i < B; ++i) {
    const int64_t T = mb->len[i];
    if (T < 1) return fail(MT_ERR_INVALID_ARG, "mt_encode: len[%d] must be >= 1 mel frame", i);
    const bool two_x = c.frontend == MT_FRONTEND_CONV1D_2X;
    // 2x: T1 is conv1's output (stride 1), T2 unused
    const int64_t T1 = two_x ? T : half_up(T), T2 = two_x ? 0 : half_up(T1), N = frames_of(c.frontend, T);
    p.mel_row_off[i] = mb->layout == MT_PADDED ? (int64_t)i * mb->max_len : p.sumT;
    p.sumT += T;
    p.sumT1 += T1;
    p.sumT2 += T2;
    p.M += N;
    p.maxN = std::max(p.maxN, N);
    p.n_windows += (N + window - 1) / window;
    if (p.sumT1 * 64 > INT32_MAX)
      return fail(MT_ERR_UNSUPPORTED, "mt_encode: batch too long (%lld mel frames)", (long long)p.sumT);
    cuT[i + 1] = (int32_t)p.sumT;
    cuT1[i + 1] = (int32_t)p.sumT1;
    cuT2[i + 1] = (int32_t)p.sumT2;
    cuN[i + 1] = (int32_t)p.M;
    cuW[i + 1] = (int32_t)p.n_windows;
  }
  const int64_t weff = std::min<int64_t>(window, p.maxN);
  if (weff > MAX_WINDOW && enc->dt == DT_F32)
    return fail(MT_ERR_UNSUPPORTED, "mt_encode: window %d over sequences of up to %lld frames "
                "exceeds the fp32 on-chip maximum %d", window, (long long)p.maxN, MAX_WINDOW);
  // Windows longer than MAX_WINDOW stream their keys: that kernel addresses a
  // window's rows of the qkv buffer (3 d_model values each) with 32-bit byte
  // offsets, reaching up to four 64-row tiles past the window's end.
  const int64_t w_rows = (weff + 63) / 64 * 64 + 256;
  if (enc->dt != DT_F32 && weff > MAX_WINDOW && w_rows * 3 * (int64_t)c.d_model * (int64_t)enc->es > INT32_MAX)
    return fail(MT_ERR_UNSUPPORTED, "mt_encode: a window of %lld frames is too long for 32-bit offsets "
                "(at most %lld frames at d_model %d)", (long long)weff,
                (long long)(INT32_MAX / (3 * (int64_t)c.d_model * (int64_t)enc->es) - 256) / 64 * 64,
                c.d_model);
  p.wpad = (int)((weff + 63) / 64 * 64);  // whole key chunks of 64 (on chip up to MAX_WINDOW)
  p.out_stride = mb->layout == MT_PADDED ? frames_of(c.frontend, mb->max_len) : 0;

  const size_t es = enc->es;
  const size_t C = c.conv_ch, D = c.d_model, F = c.d_ffn, O = c.d_out, A = c.adapter_hidden;
  const size_t M = (size_t)p.M;
  Carver k;
  p.o_words = k.take(4 * p.words.size());
  p.o_rowoff = k.take(8 * (size_t)B);
  p.o_twords = k.take(16);
  if (c.frontend == MT_FRONTEND_CONV1D_2X) {
    p.o_act1 = k.take((size_t)p.sumT * D * es);                  // conv1 output [T][D]
    p.o_act2 = k.take((size_t)p.sumT * (size_t)c.n_mels * es);  // 16-bit log-mel [T][n_mels]
    p.o_act3 = k.take(0);
  } else {
    p.o_act1 = k.take((size_t)p.sumT1 * 64 * C * es);
    p.o_act2 = k.take((size_t)p.sumT2 * 32 * C * es);
    p.o_act3 = k.take(M * 16 * C * es);
  }
  p.o_x = k.take(M * D * 4);
  size_t hb = M * D * es;
  if (c.with_head && enc->dt != DT_F32) hb = std::max(hb, M * 2 * D * 2);  // hi/lo, or fp32 ln_post
  p.o_h = k.take(hb);
  p.o_qkv = k.take(M * 3 * D * es);
  p.o_att = k.take(M * D * es);
  size_t fb = M * F * es;
  if (c.with_head) fb = std::max(fb, enc->dt != DT_F32 ? M * 2 * D * 2 : M * D * 4);
  p.o_ffn = k.take(fb);
  p.o_y = k.take(A ? M * O * es : 0);
  p.o_ahid = k.take(A ? M * A * es : 0);
  // fp32 operands: partial sums and tile counters of the K-split products
  p.o_part = k.take(enc->dt == DT_F32 ? SPLIT_PART_FLOATS * 4 : 0);
  p.bytes = k.off;
  return MT_OK;
}

GemmArgs gemm(const void* A, int64_t lda, const void* B, int64_t ldb, int M, int N, int K,
              const float* bias, void* C, int64_t ldc) {
  GemmArgs g;
  memset(&g, 0, sizeof g);
  g.A = A;
  g.lda = lda;
  g.B = B;
  g.ldb = ldb;
  g.M = M;
  g.N = N;
  g.K = K;
  g.bias = bias;
  g.C = C;
  g.ldc = ldc;
  return g;
}

}  // namespace

// ====================================================================== C ABI

namespace {

// Launches the whole encoder for a planned batch (validated by the caller).
mt_status run_encode(const mt_encoder* enc, const EncPlan& p, const float* mel, int32_t window,
                     float* out, char* w, hipStream_t s, const StreamChunk* ch, int* sat_word) {
  const mt_encoder_config& c = enc->cfg;
  const int dt = enc->dt;
  const int B = p.B;
  int M = (int)p.M;
  const int C = c.conv_ch, D = c.d_model, F = c.d_ffn, O = c.d_out, A = c.adapter_hidden;

  // tables: the saturation mask word (zeroed here) and padding, words (cu_T |
  // cu_T1 | cu_T2 | cu_N | cu_win), then mel row offsets
  HIP_TRY(upload_words((uint32_t*)(w + p.o_words), (const uint32_t*)p.words.data(),
                       (int64_t)p.words.size(), s), "upload tables");
  HIP_TRY(upload_words((uint32_t*)(w + p.o_rowoff), (const uint32_t*)p.mel_row_off.data(),
                       2 * (int64_t)B, s), "upload tables");
  // fp16 conversions report clamps at +-65504 into the mask (a stream's
  // chunks share the one word of the stream's workspace)
  int* sat = dt == DT_F16 ? (sat_word ? sat_word : (int*)(w + p.o_words)) : nullptr;
  const int32_t* cuT = (const int32_t*)(w + p.o_words) + TABLE_HEAD_WORDS;
  const int32_t* cuT1 = cuT + (B + 1);
  const int32_t* cuT2 = cuT1 + (B + 1);
  const int32_t* cuN = cuT2 + (B + 1);
  const int32_t* cuW = cuN + (B + 1);
  void* act1 = w + p.o_act1;
  void* act2 = w + p.o_act2;
  void* act3 = w + p.o_act3;
  float* x = (float*)(w + p.o_x);
  void* h = w + p.o_h;
  void* qkv = w + p.o_qkv;
  void* att = w + p.o_att;
  void* ffn = w + p.o_ffn;
  void* ybuf = w + p.o_y;
  void* ahid = w + p.o_ahid;

  // fp32: partial sums of the K-split products
  float* part = dt == DT_F32 ? (float*)(w + p.o_part) : nullptr;
  auto gemm = [&](const void* A_, int64_t lda, const void* B_, int64_t ldb, int M_, int N_, int K_,
                  const float* bias, void* C_, int64_t ldc, int sat_bit = 0) {
    GemmArgs g_ = ::gemm(A_, lda, B_, ldb, M_, N_, K_, bias, C_, ldc);
    g_.zeros = enc->zeros;
    g_.sat = sat_bit ? sat : nullptr;
    g_.sat_bit = sat_bit;
    g_.part = part;
    g_.part_floats = part ? SPLIT_PART_FLOATS : 0;
    return g_;
  };

  // ---- front-end
  if (c.frontend == MT_FRONTEND_CONV1D_2X) {
    // 16-bit log-mel rows, packed; conv1 (stride 1) -> GELU; conv2 (stride
    // 2) -> GELU -> + sinusoids into the fp32 residual stream
    STAGE(launch_rows_to_half(mel, (const int64_t*)(w + p.o_rowoff), cuT, B, p.sumT, c.n_mels, act2, dt,
                              s), "mel16");
    GemmArgs g = gemm(act2, 0, enc->conv1_w, 3 * c.n_mels, (int)p.sumT, D, 3 * c.n_mels, enc->conv1_b,
                      act1, D, SAT_FRONTEND);
    g.conv_C = c.n_mels;
    g.conv_Fin = 1;
    g.conv_Fout = 1;
    g.conv_kind = CONV_1D_S1;
    g.cu_in = cuT;
    g.cu_out = cuT;
    g.nseq = B;
    STAGE(launch_gemm(g, EPI_GELU, dt, true, s), "conv1");
    g = gemm(act1, 0, enc->conv2_w, 3 * D, M, D, 3 * D, enc->conv2_b, x, D);
    g.conv_C = D;
    g.conv_Fin = 1;
    g.conv_Fout = 1;
    g.conv_kind = CONV_1D_S2;
    g.cu_in = cuT;
    g.cu_out = cuN;
    g.nseq = B;
    g.cu_rows = cuN;
    g.pos_offset = 0;
    STAGE(launch_gemm(g, EPI_GELU_PE, dt, true, s), "conv2");
  } else {
  Conv1Args c1;
  c1.mel = mel;
  c1.mel_row_off = (const int64_t*)(w + p.o_rowoff);
  c1.cu_T = cuT;
  c1.cu_T1 = cuT1;
  c1.nseq = B;
  c1.total_T1 = p.sumT1;
  c1.w = enc->conv1_w;
  c1.b = enc->conv1_b;
  c1.out = act1;
  c1.C = C;
  c1.dtype = dt;
  c1.sat = sat;
  STAGE(launch_conv1(c1, s), "conv1");

  GemmArgs g = gemm(act1, 0, enc->conv2_w, 9 * C, (int)(p.sumT2 * 32), C, 9 * C, enc->conv2_b, act2, C,
                    SAT_FRONTEND);
  g.conv_C = C;
  g.conv_Fin = 64;
  g.conv_Fout = 32;
  g.cu_in = cuT1;
  g.cu_out = cuT2;
  g.nseq = B;
  STAGE(launch_gemm(g, EPI_GELU, dt, true, s), "conv2");
  g = gemm(act2, 0, enc->conv3_w, 9 * C, (int)(p.M * 16), C, 9 * C, enc->conv3_b, act3, C, SAT_FRONTEND);
  g.conv_C = C;
  g.conv_Fin = 32;
  g.conv_Fout = 16;
  g.cu_in = cuT2;
  g.cu_out = cuN;
  g.nseq = B;
  STAGE(launch_gemm(g, EPI_GELU, dt, true, s), "conv3");
  g = gemm(act3, 16 * C, enc->conv_out_w, 16 * C, M, D, 16 * C, nullptr, x, D);
  g.cu_rows = cuN;
  g.nseq = B;
  g.pos_offset = ch ? ch->pos : 0;
  STAGE(launch_gemm(g, EPI_PE, dt, false, s), "conv_out");
  }

  // ---- tower (a stream chunk: its kept rows only, as one sequence)
  int64_t n_windows = p.n_windows;
  if (ch) {
    n_windows = (ch->keep + window - 1) / window;
    const int32_t tw[4] = {0, ch->keep, 0, (int32_t)n_windows};
    HIP_TRY(upload_words((uint32_t*)(w + p.o_twords), (const uint32_t*)tw, 4, s), "upload tables");
    cuN = (const int32_t*)(w + p.o_twords);
    cuW = cuN + 2;
    x += (size_t)ch->drop * D;
    M = ch->keep;
  }
  AttnArgs aa;
  aa.qkv = qkv;
  aa.out = att;
  aa.cu_rows = cuN;
  aa.cu_win = cuW;
  aa.nseq = ch ? 1 : B;
  aa.n_windows = (int)n_windows;
  aa.window = window;
  aa.n_heads = c.n_heads;
  aa.D = D;
  aa.wpad = p.wpad;
  const bool half = dt != DT_F32;
  for (int l = 0; l < c.n_layers; ++l) {
    const Layer& L = enc->layers[l];
    STAGE(launch_layernorm(x, L.ln1_g, L.ln1_b, h, M, D, c.ln_eps, dt, false, s, sat, SAT_LN), "ln1");
    STAGE(launch_gemm(gemm(h, D, L.wqkv, D, M, 3 * D, D, L.bqkv, qkv, 3 * D, SAT_QKV), EPI_ACT, dt, false, s),
          "qkv");
    STAGE(launch_attention(aa, dt, s), "attn");
    STAGE(launch_gemm(gemm(att, D, L.wo, D, M, D, D, L.bo, x, D), EPI_RESID, dt, false, s), "o");
    STAGE(launch_layernorm(x, L.ln2_g, L.ln2_b, h, M, D, c.ln_eps, dt, false, s, sat, SAT_LN), "ln2");
    STAGE(launch_gemm(gemm(h, D, L.w1, D, M, F, D, L.b1, ffn, F, SAT_FFN), EPI_GELU, dt, false, s), "fc1");
    STAGE(launch_gemm(gemm(ffn, F, L.w2, F, M, D, F, L.b2, x, D), EPI_RESID, dt, false, s), "fc2");
  }

  // ---- head / output
  const int64_t stride = p.out_stride;
  int out_d = D;
  if (!c.with_head) {
    STAGE(launch_copy_rows(x, out, M, D, cuN, ch ? 1 : B, stride, s), "copy_rows");
  } else if (c.frontend == MT_FRONTEND_CONV1D_2X) {
    float* y = (float*)h;  // ln_post in fp32, then into the output layout
    STAGE(launch_layernorm(x, enc->lnp_g, enc->lnp_b, y, M, D, c.ln_eps, DT_F32, false, s), "ln_post");
    STAGE(launch_copy_rows(y, out, M, D, cuN, B, stride, s), "copy_rows");
  } else {
    out_d = O;
    // 16-bit operands: the head's activations enter as hi/lo pairs (K doubled)
    const int KD = half ? 2 * D : D;
    STAGE(launch_layernorm(x, enc->lnp_g, enc->lnp_b, h, M, D, c.ln_eps, dt, half, s, sat, SAT_HEAD),
          "ln_post");
    STAGE(launch_gemm(gemm(h, KD, enc->wp1, KD, M, D, KD, enc->bp1, ffn, KD, SAT_HEAD),
                        half ? EPI_GELU_SPLIT : EPI_GELU, dt, false, s), "proj1");
    GemmArgs g2 = gemm(ffn, KD, enc->wp2, KD, M, O, KD, enc->bp2, A ? ybuf : (void*)out, O,
                       A ? SAT_ADAPTER : 0);
    g2.cu_rows = cuN;
    g2.nseq = ch ? 1 : B;
    g2.out_seq_stride = A ? 0 : stride;
    STAGE(launch_gemm(g2, A ? EPI_ACT : EPI_OUT, dt, false, s), "proj2");
    if (A) {
      STAGE(launch_gemm(gemm(ybuf, O, enc->wgu, O, M, 2 * A, O, nullptr, ahid, A, SAT_ADAPTER), EPI_SWIGLU,
                        dt, false, s), "adapter_gu");
      GemmArgs g3 = gemm(ahid, A, enc->wd, A, M, O, A, nullptr, out, O);
      g3.cu_rows = cuN;
      g3.nseq = ch ? 1 : B;
      g3.out_seq_stride = stride;
      STAGE(launch_gemm(g3, EPI_OUT, dt, false, s), "adapter_down");
    }
  }
  if (stride > 0) STAGE(launch_zero_pad_rows(out, cuN, ch ? 1 : B, stride, out_d, s), "zero_pad");
  return MT_OK;
}


// ------------------------------------------------------------- stream plan
// mt_encode_stream: encoder frames in chunks of chunk_windows windows.  Chunk
// [e0, e1) needs mel frames [8 e0 - 7, 8 e1) (the receptive field of encoder
// frame t is mel frames 8t - 7 .. 8t + 7); it is encoded from mel frames
// [max(0, 8 e0 - 8), min(T, 8 e1)): starting on a multiple of 8 keeps the
// stride-2 convolutions aligned with the stream's, and the one encoder frame
// before e0 that this range yields (its receptive field leaves the range) is
// dropped before the tower.  Every kept frame then goes through the same
// arithmetic as in mt_logmel + mt_encode over the whole stream.
struct StreamPlan {
  int64_t n = 0, T = 0, N = 0, Fc = 0, Tc = 0;  // samples, mel frames, encoder frames,
                                                // frames per chunk, largest chunk's mel frames
  size_t off_sat = 0, off_tab = 0, off_gmax = 0, off_mel = 0, off_enc = 0, bytes = 0;
  EncPlan enc;  // plan of the largest chunk (sizes the workspace)
};

mt_status plan_stream(const mt_encoder* enc, int64_t n_samples, int32_t window, int32_t chunk_windows,
                      StreamPlan& sp) {
  if (!enc) return fail(MT_ERR_INVALID_ARG, "encoder is NULL");
  if (enc->cfg.frontend != MT_FRONTEND_CONV2D_8X)
    return fail(MT_ERR_UNSUPPORTED, "mt_encode_stream: only the 8x (Conv2D) front-end streams");
  if (n_samples < 201 || n_samples > INT32_MAX)
    return fail(MT_ERR_INVALID_ARG, "mt_encode_stream: n_samples %lld out of range [201, %d]",
                (long long)n_samples, INT32_MAX);
  if (window < 1) return fail(MT_ERR_INVALID_ARG, "window must be >= 1 (got %d)", window);
  if (chunk_windows < 1)
    return fail(MT_ERR_INVALID_ARG, "chunk_windows must be >= 1 (got %d)", chunk_windows);
  sp.n = n_samples;
  sp.T = n_samples / 160;
  sp.N = half_up(half_up(half_up(sp.T)));
  sp.Fc = std::min<int64_t>((int64_t)chunk_windows * window, sp.N);
  sp.Tc = std::min<int64_t>(sp.T, 8 * sp.Fc + 8);
  int64_t lens[1] = {sp.Tc};
  mt_batch b;
  b.layout = MT_PACKED;
  b.n_seqs = 1;
  b.len = lens;
  b.max_len = 0;
  mt_status st = plan_encode(enc, &b, window, sp.enc);
  if (st != MT_OK) return st;
  Carver k;
  sp.off_sat = k.take(4);  // the fp16 saturation mask of the whole stream
  sp.off_tab = k.take(64);  // stream_mel_at's tables (36 bytes)
  sp.off_gmax = k.take(4);
  sp.off_mel = k.take((size_t)sp.Tc * 128 * 4);
  sp.off_enc = k.take(sp.enc.bytes);
  sp.bytes = k.off;
  return MT_OK;
}

// Mel frames [m0, m0 + nf) of one stream of n samples into mel (rows 0 ..
// nf - 1): sample q of the stream is wav[q + sample_off] (a live stream keeps
// only its recent samples), the reflection at the stream's ends uses n, the
// frames' maximum goes into *gmax; tables in `tab` (36 bytes).
mt_status stream_mel_at(const float* wav, int64_t sample_off, int64_t n, int64_t m0, int64_t nf, float* mel,
                        char* tab, int* gmax, bool normalise, hipStream_t s) {
  // sample_off (8) | row_off (8) | seq_len (4) | cu_frames (8) | cu_groups (8)
  const int64_t ng = (nf + MEL_FPW - 1) / MEL_FPW;
  uint32_t words[9] = {(uint32_t)(uint64_t)sample_off, (uint32_t)((uint64_t)sample_off >> 32), 0, 0,
                       (uint32_t)n, 0, (uint32_t)nf, 0, (uint32_t)ng};
  HIP_TRY(upload_words((uint32_t*)tab, words, 9, s), "upload tables");
  MelArgs a;
  a.wav = wav;
  a.mel = mel;
  a.seq_sample_off = (const int64_t*)tab;
  a.seq_row_off = (const int64_t*)(tab + 8);
  a.seq_len = (const int32_t*)(tab + 16);
  a.cu_frames = (const int32_t*)(tab + 20);
  a.cu_groups = (const int32_t*)(tab + 28);
  a.gmax = gmax;
  a.nslot = 1;
  a.slot_stride = 1;
  a.nseq = 1;
  a.total_groups = ng;
  a.total_frames = nf;
  a.out_rows = nf;
  a.padded = 0;
  a.frame_off = m0;
  STAGE(launch_mel(a, s), "mel");
  if (normalise) STAGE(launch_mel_norm(a, nf, s), "mel_norm");
  return MT_OK;
}

mt_status stream_mel(const float* wav, int64_t n, int64_t m0, int64_t nf, float* mel, char* w,
                     const StreamPlan& sp, bool normalise, hipStream_t s) {
  return stream_mel_at(wav, 0, n, m0, nf, mel, w + sp.off_tab, (int*)(w + sp.off_gmax), normalise, s);
}

// ------------------------------------------------------------- live stream
// Windows are encoded as their audio arrives.  Window k (encoder frames
// [kW, (k+1)W)) needs mel frames up to 8 (k+1) W - 1, i.e. samples up to
// 1280 (k+1) W + 39: once those are in, it is encoded from mel frames
// [max(0, 8 kW - 8), 8 (k+1) W) with the log clamp at the running maximum
// over every mel frame computed so far (frames [0, 8 (k+1) W)), the same
// chunk arithmetic as mt_encode_stream.  At the end of the stream the rest
// (with the reflection and zero padding of the stream's real end) follows.
// The state keeps the recent samples in two buffers used in turn: before an
// append that would overflow, the samples the next window still needs move to
// the other buffer.
struct LivePlan {
  int64_t cap = 0;  // samples per buffer
  int64_t Tc = 0;   // mel frames of a window's chunk
  size_t off_sat = 0, off_gmax = 0, off_tab = 0, off_buf[2] = {0, 0}, off_mel = 0, off_enc = 0, bytes = 0;
  EncPlan enc;      // plan of a full window's chunk (sizes the workspace)
};

constexpr int64_t LIVE_MAX_SAMPLES = INT32_MAX;  // sample indices of a stream fit 32 bits

mt_status plan_live(const mt_encoder* enc, int32_t window, int64_t max_push, LivePlan& lp) {
  if (!enc) return fail(MT_ERR_INVALID_ARG, "encoder is NULL");
  if (enc->cfg.frontend != MT_FRONTEND_CONV2D_8X)
    return fail(MT_ERR_UNSUPPORTED, "live streams: only the 8x (Conv2D) front-end streams");
  if (window < 1) return fail(MT_ERR_INVALID_ARG, "window must be >= 1 (got %d)", window);
  if (max_push < 1 || max_push > LIVE_MAX_SAMPLES)
    return fail(MT_ERR_INVALID_ARG, "max_push %lld out of range [1, %lld]", (long long)max_push,
                (long long)LIVE_MAX_SAMPLES);
  lp.Tc = 8 * (int64_t)window + 8;
  lp.cap = 1280 * (int64_t)window + 1680 + max_push;
  if (lp.cap > LIVE_MAX_SAMPLES)
    return fail(MT_ERR_UNSUPPORTED, "live streams: window %d with pushes of %lld samples is too large", window,
                (long long)max_push);
  int64_t lens[1] = {lp.Tc};
  mt_batch b;
  b.layout = MT_PACKED;
  b.n_seqs = 1;
  b.len = lens;
  b.max_len = 0;
  mt_status st = plan_encode(enc, &b, window, lp.enc);
  if (st != MT_OK) return st;
  Carver k;
  lp.off_sat = k.take(4);  // the fp16 saturation mask of the whole stream
  lp.off_gmax = k.take(4);
  lp.off_tab = k.take(64);  // stream_mel_at's tables (36 bytes)
  lp.off_buf[0] = k.take((size_t)lp.cap * 4);
  lp.off_buf[1] = k.take((size_t)lp.cap * 4);
  lp.off_mel = k.take((size_t)lp.Tc * 128 * 4);
  lp.off_enc = k.take(lp.enc.bytes);
  lp.bytes = k.off;
  return MT_OK;
}

// Windows whose samples are all in once `have` samples have arrived (before
// the end of the stream is known): k + 1 <= (have - 40) / (1280 W).
int64_t live_complete(int window, int64_t have) {
  return have >= 40 ? (have - 40) / (1280 * (int64_t)window) : 0;
}

// First stream sample that window k (or a later one) can still read.
int64_t live_keep_from(int window, int64_t k) {
  return std::max<int64_t>(0, 160 * std::max<int64_t>(0, 8 * k * window - 8) - 200);
}

// Encodes window k of a live stream into out (its rows only).  final: the
// stream has ended at st->have samples (its real end: reflection, zero
// padding, a last partial window).
mt_status live_encode_window(mt_stream* st, const LivePlan& lp, int64_t k, bool final, float* out, hipStream_t s) {
  const int W = st->window;
  char* w = st->state;
  int64_t e1 = (k + 1) * W, m1 = 8 * e1, n_len = LIVE_MAX_SAMPLES;
  if (final) {
    const int64_t T = st->have / HOP, N = half_up(half_up(half_up(T)));
    e1 = std::min(e1, N);
    m1 = std::min(m1, T);
    n_len = st->have;
  }
  const int64_t e0 = k * W, drop = e0 > 0 ? 1 : 0;
  const int64_t m0 = std::max<int64_t>(0, 8 * e0 - 8);
  if (half_up(half_up(half_up(m1 - m0))) != e1 - e0 + drop || m1 - m0 > lp.Tc)
    return fail(MT_ERR_INVALID_ARG, "live stream: internal window geometry error");
  float* mel = (float*)(w + lp.off_mel);
  // the buffer holds stream samples [base, base + cap): sample q at q - base
  mt_status st_ = stream_mel_at((const float*)(w + lp.off_buf[st->cur]), -st->base, n_len, m0, m1 - m0, mel,
                                w + lp.off_tab, (int*)(w + lp.off_gmax), true, s);
  if (st_ != MT_OK) return st_;
  int64_t lens[1] = {m1 - m0};
  mt_batch b;
  b.layout = MT_PACKED;
  b.n_seqs = 1;
  b.len = lens;
  b.max_len = 0;
  EncPlan ep;
  st_ = plan_encode(st->enc, &b, W, ep);
  if (st_ != MT_OK) return st_;
  StreamChunk ch;
  ch.pos = (int)(e0 - drop);
  ch.drop = (int)drop;
  ch.keep = (int)(e1 - e0);
  return run_encode(st->enc, ep, mel, W, out, w + lp.off_enc, s, &ch, (int*)(w + lp.off_sat));
}

// ------------------------------------------------------------- log-mel launch
// The launch sequence of mt_logmel on a planned batch, with its tables and
// per-clip maxima in `w` (the caller's workspace, or the fixed scratch array
// of mt_logmel_noalloc): table upload, the maxima set to -inf, the frame
// kernel, the clamp pass.
mt_status run_logmel(const float* wav, const mt_batch* wav_b, const MelPlan& p, float* mel, char* w,
                     hipStream_t s) {
  // one upload: sample_off | row_off | seq_len | cu_frames | cu_groups
  // (contiguous regions), then the maxima's slots set to -inf
  std::vector<uint32_t> words(p.off_gmax / 4, 0);
  memcpy((char*)words.data() + p.off_sample, p.sample_off.data(), 8 * (size_t)p.B);
  memcpy((char*)words.data() + p.off_row, p.row_off.data(), 8 * (size_t)p.B);
  memcpy((char*)words.data() + p.off_len, p.seq_len.data(), 4 * (size_t)p.B);
  memcpy((char*)words.data() + p.off_cu, p.cu_frames.data(), 4 * (size_t)(p.B + 1));
  memcpy((char*)words.data() + p.off_cug, p.cu_groups.data(), 4 * (size_t)(p.B + 1));
  HIP_TRY(upload_words((uint32_t*)w, words.data(), (int64_t)words.size(), s), "upload tables");
  int* gmax = (int*)(w + p.off_gmax);
  const float ninf = -INFINITY;
  int key;
  memcpy(&key, &ninf, 4);
  key = key >= 0 ? key : key ^ 0x7fffffff;
  HIP_TRY(launch_fill_i32(gmax, key, (int64_t)p.B * p.nslot * p.slot_stride, s), "fill");
  MelArgs a;
  a.wav = wav;
  a.mel = mel;
  a.seq_sample_off = (const int64_t*)(w + p.off_sample);
  a.seq_len = (const int32_t*)(w + p.off_len);
  a.cu_frames = (const int32_t*)(w + p.off_cu);
  a.cu_groups = (const int32_t*)(w + p.off_cug);
  a.seq_row_off = (const int64_t*)(w + p.off_row);
  a.gmax = gmax;
  a.nslot = p.nslot;
  a.slot_stride = p.slot_stride;
  a.nseq = p.B;
  a.total_groups = p.total_groups;
  a.total_frames = p.total_frames;
  a.out_rows = p.out_rows;
  a.padded = wav_b->layout == MT_PADDED;
  a.frame_off = 0;
  STAGE(launch_mel(a, s), "mel");
  STAGE(launch_mel_norm(a, p.tmax, s), "mel_norm");
  return MT_OK;
}

// ------------------------------------------------------------- fixed scratch
// mt_logmel_noalloc's tables and per-clip maxima: a fixed device array, one
// copy per device, kept until the process ends.  Host code uses the address
// hipGetSymbolAddress returns for the current device (taken once per device,
// with that device current), never the array's name, which in host code is
// only a stand-in for the symbol.
constexpr size_t NOALLOC_SCRATCH_BYTES = 256 << 10;
static __device__ __align__(256) char scratch[NOALLOC_SCRATCH_BYTES];
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

mt_status scratch_for_current_device(char** out) {
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= MAX_DEVICES) return fail(MT_ERR_UNSUPPORTED, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    HIP_TRY(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (!ptr || (uintptr_t)ptr % ALIGN)
      return fail(MT_ERR_HIP, "hipGetSymbolAddress(scratch) gave an unusable address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = (char*)g_scratch_ptr[dev];
  return MT_OK;
}

}  // namespace

// ================================================================== decoder
namespace {

struct DecLayer {
  const float *in_norm, *q_norm, *k_norm, *post_norm;
  const void *wqkv, *wo, *wgu, *wd;
};

struct DecLayout {
  size_t embed, norm, zeros, bytes;
  struct L {
    size_t in_norm, wqkv, q_norm, k_norm, wo, post_norm, wgu, wd;
  };
  std::vector<L> layers;
};

mt_status check_decoder_config(const mt_decoder_config* c) {
  if (!c) return fail(MT_ERR_INVALID_ARG, "decoder config is NULL");
  if (c->dtype != MT_BF16 && c->dtype != MT_F16)
    return fail(MT_ERR_UNSUPPORTED, "decoder dtype must be MT_BF16 or MT_F16 (got %d)", c->dtype);
  if (c->vocab < 1 || c->d_model < 1 || c->n_layers < 0 || c->n_heads < 1 || c->n_kv_heads < 1 ||
      c->head_dim < 1 || c->d_ffn < 1)
    return fail(MT_ERR_INVALID_ARG, "non-positive size in decoder config");
  if (!(c->rms_eps > 0.f) || !(c->rope_base > 1.f))
    return fail(MT_ERR_INVALID_ARG, "rms_eps must be > 0 and rope_base > 1");
  if (c->head_dim != 128) return fail(MT_ERR_UNSUPPORTED, "decoder head_dim must be 128");
  if (c->n_heads != 2 * c->n_kv_heads)
    return fail(MT_ERR_UNSUPPORTED, "decoder needs two query heads per key/value head");
  if (c->d_model % 256 || c->d_ffn % 256 || c->vocab % 16)
    return fail(MT_ERR_UNSUPPORTED, "decoder d_model and d_ffn must be multiples of 256, vocab of 16");
  return MT_OK;
}

DecLayout decoder_layout(const mt_decoder_config& c) {
  const size_t V = c.vocab, D = c.d_model, F = c.d_ffn, hd = c.head_dim;
  const size_t NQKV = (size_t)(c.n_heads + 2 * c.n_kv_heads) * hd, NQ = (size_t)c.n_heads * hd;
  DecLayout p;
  Carver k;
  p.embed = k.take(V * D * 2);
  p.layers.resize(c.n_layers);
  for (auto& L : p.layers) {
    L.in_norm = k.take(D * 4);
    L.wqkv = k.take(NQKV * D * 2);
    L.q_norm = k.take(hd * 4);
    L.k_norm = k.take(hd * 4);
    L.wo = k.take(D * NQ * 2);
    L.post_norm = k.take(D * 4);
    L.wgu = k.take(2 * F * D * 2);
    L.wd = k.take(D * F * 2);
  }
  p.norm = k.take(D * 4);
  p.zeros = k.take(256);
  p.bytes = k.off;
  return p;
}

// K splits of the skinny product: enough wavefronts in flight (~2048) for
// the weight stream, whole 32-wide K steps per split
int gemv_split(int N, int K) {
  int s = 1;
  while (s < 8 && (N / 16) * s < 2048 && K % (64 * s) == 0) s *= 2;
  return s;
}

struct DecPlan {
  int n = 0, n_items = 0, s_qkv = 1, s_o = 1, s_gu = 1, s_d = 1;
  bool gemv = true;
  // at most GEMV_FUSE_ROWS rows: the down projection computes its SwiGLU
  // input, the output projection combines the attention chunks itself
  bool fuse_d = false, fuse_o = false;
  int cmax = 0;  // most chunks of any row
  // one row per sequence: the attention kernel computes its queries and the
  // new keys / values itself (no row of the call reads another's new entry)
  bool fuse_qk = false;
  std::vector<int32_t> words;  // seq | pos | items | first_item
  size_t o_words, o_x, o_h, o_qkv, o_qf, o_po, o_pml, o_o16, o_opart, o_gu, o_act, o_dpart, o_amv, o_ami, bytes;
};

}  // namespace

struct mt_decoder {
  mt_decoder_config cfg;
  int dt;
  const void* embed;
  const float* norm;
  std::vector<DecLayer> layers;
  const void* zeros;
};

namespace {

mt_status plan_decode(const mt_decoder* dec, int32_t n, const int32_t* seq, const int32_t* pos, int32_t max_seqs,
                      int32_t max_pos, DecPlan& p) {
  if (!dec) return fail(MT_ERR_INVALID_ARG, "decoder is NULL");
  if (n < 1 || n > (1 << 20)) return fail(MT_ERR_INVALID_ARG, "mt_decode: n_rows %d out of range [1, 2^20]", n);
  if (!seq || !pos) return fail(MT_ERR_INVALID_ARG, "mt_decode: seq or pos is NULL");
  if (max_seqs < 1 || max_pos < 1)
    return fail(MT_ERR_INVALID_ARG, "mt_decode: max_seqs and max_pos must be >= 1");
  const mt_decoder_config& c = dec->cfg;
  std::vector<int64_t> keys(n);
  p.n = n;
  p.words.assign(2 * (size_t)n, 0);
  std::vector<int32_t> items, first(n + 1, 0);
  for (int i = 0; i < n; ++i) {
    if (seq[i] < 0 || seq[i] >= max_seqs)
      return fail(MT_ERR_INVALID_ARG, "mt_decode: seq[%d] = %d outside [0, %d)", i, seq[i], max_seqs);
    if (pos[i] < 0 || pos[i] >= max_pos)
      return fail(MT_ERR_INVALID_ARG, "mt_decode: pos[%d] = %d outside [0, %d)", i, pos[i], max_pos);
    keys[i] = (int64_t)seq[i] * max_pos + pos[i];
    p.words[i] = seq[i];
    p.words[n + i] = pos[i];
    first[i] = (int32_t)(items.size() / 2);
    for (int ch = 0; ch * 64 <= pos[i]; ++ch) {  // 64-key attention chunks
      items.push_back(i);
      items.push_back(ch);
    }
  }
  first[n] = (int32_t)(items.size() / 2);
  std::sort(keys.begin(), keys.end());
  for (int i = 1; i < n; ++i)
    if (keys[i] == keys[i - 1]) return fail(MT_ERR_INVALID_ARG, "mt_decode: two rows at the same (seq, pos)");
  p.n_items = first[n];
  p.words.insert(p.words.end(), items.begin(), items.end());
  p.words.insert(p.words.end(), first.begin(), first.end());
  const size_t D = c.d_model, F = c.d_ffn, hd = c.head_dim, Hq = c.n_heads, Hkv = c.n_kv_heads;
  const size_t NQKV = (Hq + 2 * Hkv) * hd, NQ = Hq * hd;
  p.gemv = n <= GEMV_MAX_ROWS;
  if (p.gemv) {
    p.s_qkv = gemv_split((int)NQKV, (int)D);
    p.s_o = gemv_split((int)D, (int)NQ);
    p.s_gu = gemv_split(2 * (int)F, (int)D);
    p.s_d = gemv_split((int)D, (int)F);
  } else {
    p.s_qkv = 1;
    p.s_gu = 0;
    p.s_o = p.s_d = 0;  // the matrix kernels add into the residual stream
  }
  {
    std::vector<int32_t> sq(seq, seq + n);
    std::sort(sq.begin(), sq.end());
    const bool distinct = std::adjacent_find(sq.begin(), sq.end()) == sq.end();
    const int S = p.s_qkv;
    p.fuse_qk = distinct && (S == 1 || S == 2 || S == 4 || S == 8);
  }
  if (p.gemv && n <= GEMV_FUSE_ROWS && D % 64 == 0) {
    for (int i = 0; i < n; ++i) p.cmax = std::max(p.cmax, first[i + 1] - first[i]);
    const size_t kld = F / p.s_d, klo = NQ / p.s_o;
    p.fuse_d = kld % 32 == 0 && kld <= 1024 && n * kld * 2 <= 65536;
    p.fuse_o = klo % hd == 0 && klo <= 1024 && p.cmax <= 64 &&
               n * klo * 2 + n * (klo / hd) * (2 + 3 * p.cmax) * 4 <= 65536;
  }
  Carver k;
  p.o_words = k.take(4 * p.words.size());
  p.o_x = k.take((size_t)n * D * 4);
  p.o_h = k.take((size_t)n * std::max(D, NQ) * 2);
  p.o_qkv = k.take((size_t)p.s_qkv * n * NQKV * 4);
  p.o_qf = k.take((size_t)n * NQ * 4);
  p.o_po = k.take((size_t)p.n_items * Hkv * 2 * hd * 4);
  p.o_pml = k.take((size_t)p.n_items * Hkv * 2 * 2 * 4);
  p.o_o16 = k.take((size_t)n * NQ * 2);
  p.o_opart = k.take((size_t)p.s_o * n * D * 4);
  p.o_gu = k.take((size_t)p.s_gu * n * 2 * F * 4);
  p.o_act = k.take((size_t)n * F * 2);
  p.o_dpart = k.take((size_t)p.s_d * n * D * 4);
  p.o_amv = k.take((size_t)n * 64 * 4);
  p.o_ami = k.take((size_t)n * 64 * 4);
  p.bytes = k.off;
  return MT_OK;
}

}  // namespace

extern "C" {

int32_t mt_decoder_n_weights(const mt_decoder_config* cfg) {
  if (check_decoder_config(cfg) != MT_OK) return -1;
  return 1 + 11 * cfg->n_layers + 1;
}

mt_status mt_decoder_packed_bytes(const mt_decoder_config* cfg, size_t* bytes) {
  mt_status st = check_decoder_config(cfg);
  if (st != MT_OK) return st;
  if (!bytes) return fail(MT_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = decoder_layout(*cfg).bytes;
  return MT_OK;
}

mt_status mt_decoder_create(const mt_decoder_config* cfg, const float* const* wts, int32_t n_weights, void* packed,
                            size_t packed_bytes, void* stream, mt_decoder** out) {
  mt_status st = check_decoder_config(cfg);
  if (st != MT_OK) return st;
  if (!out) return fail(MT_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  const mt_decoder_config c = *cfg;
  const int nw = 1 + 11 * c.n_layers + 1;
  if (!wts) return fail(MT_ERR_INVALID_ARG, "weights is NULL");
  if (n_weights != nw) return fail(MT_ERR_INVALID_ARG, "expected %d weight tensors, got %d", nw, n_weights);
  for (int i = 0; i < n_weights; ++i)
    if (!wts[i]) return fail(MT_ERR_INVALID_ARG, "weights[%d] is NULL", i);
  const DecLayout L = decoder_layout(c);
  if (!packed) return fail(MT_ERR_INVALID_ARG, "packed is NULL");
  if ((uintptr_t)packed % ALIGN) return fail(MT_ERR_INVALID_ARG, "packed must be 256-byte aligned");
  if (packed_bytes < L.bytes)
    return fail(MT_ERR_WORKSPACE, "packed buffer %zu bytes < required %zu", packed_bytes, L.bytes);
  hipStream_t s = (hipStream_t)stream;
  const int dt = c.dtype == MT_BF16 ? DT_BF16 : DT_F16;
  char* P = (char*)packed;
  const int64_t V = c.vocab, D = c.d_model, F = c.d_ffn, hd = c.head_dim;
  const int64_t NQ = (int64_t)c.n_heads * hd, NKV = (int64_t)c.n_kv_heads * hd;
  int wi = 0;
  auto next = [&]() { return wts[wi++]; };
  HIP_TRY(launch_convert(next(), P + L.embed, V, D, D, 0, dt, s), "pack embed");
  for (int l = 0; l < c.n_layers; ++l) {
    const auto& Ll = L.layers[l];
    HIP_TRY(launch_copy_f32(next(), (float*)(P + Ll.in_norm), D, s), "pack input_norm");
    HIP_TRY(launch_convert(next(), P + Ll.wqkv, NQ, D, D, 0, dt, s), "pack q");  // rows 0 .. NQ-1
    HIP_TRY(launch_convert(next(), P + Ll.wqkv + (size_t)NQ * D * 2, NKV, D, D, 0, dt, s), "pack k");
    HIP_TRY(launch_convert(next(), P + Ll.wqkv + (size_t)(NQ + NKV) * D * 2, NKV, D, D, 0, dt, s), "pack v");
    HIP_TRY(launch_copy_f32(next(), (float*)(P + Ll.q_norm), hd, s), "pack q_norm");
    HIP_TRY(launch_copy_f32(next(), (float*)(P + Ll.k_norm), hd, s), "pack k_norm");
    HIP_TRY(launch_convert(next(), P + Ll.wo, D, NQ, NQ, 0, dt, s), "pack o");
    HIP_TRY(launch_copy_f32(next(), (float*)(P + Ll.post_norm), D, s), "pack post_norm");
    const float* g = next();
    const float* u = next();
    HIP_TRY(launch_pack_swiglu(g, u, P + Ll.wgu, (int)F, (int)D, dt, s), "pack gate/up");
    HIP_TRY(launch_convert(next(), P + Ll.wd, D, F, F, 0, dt, s), "pack down");
  }
  HIP_TRY(launch_copy_f32(next(), (float*)(P + L.norm), D, s), "pack norm");
  HIP_TRY(launch_fill_i32((int*)(P + L.zeros), 0, 64, s), "zero block");
  mt_decoder* d = new mt_decoder();
  d->cfg = c;
  d->dt = dt;
  d->embed = P + L.embed;
  d->norm = (const float*)(P + L.norm);
  d->zeros = P + L.zeros;
  d->layers.resize(c.n_layers);
  for (int l = 0; l < c.n_layers; ++l) {
    const auto& Ll = L.layers[l];
    DecLayer& y = d->layers[l];
    y.in_norm = (const float*)(P + Ll.in_norm);
    y.q_norm = (const float*)(P + Ll.q_norm);
    y.k_norm = (const float*)(P + Ll.k_norm);
    y.post_norm = (const float*)(P + Ll.post_norm);
    y.wqkv = P + Ll.wqkv;
    y.wo = P + Ll.wo;
    y.wgu = P + Ll.wgu;
    y.wd = P + Ll.wd;
  }
  *out = d;
  return MT_OK;
}

void mt_decoder_destroy(mt_decoder* dec) { delete dec; }

const void* mt_decoder_embedding(const mt_decoder* dec) { return dec ? dec->embed : nullptr; }

mt_status mt_decoder_cache_bytes(const mt_decoder* dec, int32_t max_seqs, int32_t max_pos, size_t* bytes) {
  if (!dec || !bytes) return fail(MT_ERR_INVALID_ARG, "decoder or bytes is NULL");
  if (max_seqs < 1 || max_pos < 1) return fail(MT_ERR_INVALID_ARG, "max_seqs and max_pos must be >= 1");
  const mt_decoder_config& c = dec->cfg;
  *bytes = (size_t)c.n_layers * max_seqs * 2 * c.n_kv_heads * (size_t)max_pos * c.head_dim * 2;
  return MT_OK;
}

mt_status mt_decode_workspace_size(const mt_decoder* dec, int32_t n_rows, const int32_t* seq, const int32_t* pos,
                                   int32_t max_seqs, int32_t max_pos, size_t* bytes) {
  if (!bytes) return fail(MT_ERR_INVALID_ARG, "bytes is NULL");
  DecPlan p;
  mt_status st = plan_decode(dec, n_rows, seq, pos, max_seqs, max_pos, p);
  if (st != MT_OK) return st;
  *bytes = p.bytes;
  return MT_OK;
}

mt_status mt_decode(const mt_decoder* dec, const float* x_in, int32_t n_rows, const int32_t* seq, const int32_t* pos,
                    void* cache, int32_t max_seqs, int32_t max_pos, float* logits, int32_t* next, void* ws,
                    size_t ws_bytes, void* stream) {
  DecPlan p;
  mt_status st = plan_decode(dec, n_rows, seq, pos, max_seqs, max_pos, p);
  if (st != MT_OK) return st;
  if (!x_in || (!cache && dec->cfg.n_layers > 0) || !logits || !ws)
    return fail(MT_ERR_INVALID_ARG, "mt_decode: NULL device pointer");
  if ((uintptr_t)ws % ALIGN || (uintptr_t)x_in % 16 || (uintptr_t)logits % 16 || (uintptr_t)cache % 16 ||
      (uintptr_t)next % 4)
    return fail(MT_ERR_INVALID_ARG, "mt_decode: misaligned pointer");
  if (ws_bytes < p.bytes)
    return fail(MT_ERR_WORKSPACE, "mt_decode: workspace %zu bytes < required %zu", ws_bytes, p.bytes);
  const mt_decoder_config& c = dec->cfg;
  const int dt = dec->dt, n = p.n;
  const int D = c.d_model, F = c.d_ffn, hd = c.head_dim, Hq = c.n_heads, Hkv = c.n_kv_heads;
  const int NQKV = (Hq + 2 * Hkv) * hd, NQ = Hq * hd;
  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  HIP_TRY(upload_words((uint32_t*)(w + p.o_words), (const uint32_t*)p.words.data(), (int64_t)p.words.size(), s),
          "upload tables");
  const int32_t* wd = (const int32_t*)(w + p.o_words);
  float* x = (float*)(w + p.o_x);
  void* h = w + p.o_h;
  float* qkv = (float*)(w + p.o_qkv);
  float* opart = (float*)(w + p.o_opart);
  float* dpart = (float*)(w + p.o_dpart);
  void* act = w + p.o_act;
  DecArgs a;
  a.rows = n;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.max_seqs = max_seqs;
  a.max_pos = max_pos;
  a.eps = c.rms_eps;
  a.log_base = std::log((double)c.rope_base);
  a.seq = wd;
  a.pos = wd + n;
  a.items = wd + 2 * n;
  a.first_item = wd + 2 * n + 2 * p.n_items;
  a.qf = (float*)(w + p.o_qf);
  a.cache = cache;
  a.part_o = (float*)(w + p.o_po);
  a.part_ml = (float*)(w + p.o_pml);
  a.o16 = w + p.o_o16;
  auto gemm_ = [&](const void* A_, int64_t lda, const void* B_, int M_, int N_, int K_, void* C_, int64_t ldc) {
    GemmArgs g_ = ::gemm(A_, lda, B_, K_, M_, N_, K_, nullptr, C_, ldc);
    g_.zeros = dec->zeros;
    return g_;
  };

  HIP_TRY(launch_copy_f32(x_in, x, (int64_t)n * D, s), "copy input rows");
  STAGE(launch_add_rmsnorm(x, nullptr, 0, c.n_layers ? dec->layers[0].in_norm : dec->norm, h, n, D, c.rms_eps, dt, s),
        "rmsnorm");
  for (int l = 0; l < c.n_layers; ++l) {
    const DecLayer& L = dec->layers[l];
    a.layer = l;
    a.q_norm = L.q_norm;
    a.k_norm = L.k_norm;
    if (p.gemv) {
      STAGE(launch_gemv16(L.wqkv, h, qkv, n, NQKV, D, p.s_qkv, dt, s), "dec_qkv");
    } else {
      STAGE(launch_gemm(gemm_(h, D, L.wqkv, n, NQKV, D, qkv, NQKV), EPI_F32, dt, false, s), "dec_qkv");
    }
    if (!p.fuse_qk) STAGE(launch_qk_rope(a, qkv, p.s_qkv, dt, s), "dec_qk_rope");
    STAGE(launch_attn_dec(a, p.n_items, !p.fuse_o, p.fuse_qk ? qkv : nullptr, p.fuse_qk ? p.s_qkv : 0, dt, s),
          "dec_attn");
    if (p.fuse_o) {
      STAGE(launch_gemv16x(L.wo, 2, nullptr, 0, a, p.cmax, opart, n, D, NQ, p.s_o, dt, s), "dec_o");
    } else if (p.gemv) {
      STAGE(launch_gemv16(L.wo, a.o16, opart, n, D, NQ, p.s_o, dt, s), "dec_o");
    } else {
      STAGE(launch_gemm(gemm_(a.o16, NQ, L.wo, n, D, NQ, x, D), EPI_RESID, dt, false, s), "dec_o");
    }
    STAGE(launch_add_rmsnorm(x, opart, p.s_o, L.post_norm, h, n, D, c.rms_eps, dt, s), "rmsnorm");
    if (p.gemv) {
      STAGE(launch_gemv16(L.wgu, h, (float*)(w + p.o_gu), n, 2 * F, D, p.s_gu, dt, s), "dec_gate_up");
      if (p.fuse_d) {
        STAGE(launch_gemv16x(L.wd, 1, (const float*)(w + p.o_gu), p.s_gu, a, 0, dpart, n, D, F, p.s_d, dt, s),
              "dec_down");
      } else {
        STAGE(launch_swiglu((const float*)(w + p.o_gu), p.s_gu, act, n, F, dt, s), "dec_swiglu");
        STAGE(launch_gemv16(L.wd, act, dpart, n, D, F, p.s_d, dt, s), "dec_down");
      }
    } else {
      STAGE(launch_gemm(gemm_(h, D, L.wgu, n, 2 * F, D, act, F), EPI_SWIGLU, dt, false, s), "dec_gate_up");
      STAGE(launch_gemm(gemm_(act, F, L.wd, n, D, F, x, D), EPI_RESID, dt, false, s), "dec_down");
    }
    const float* nw = l + 1 < c.n_layers ? dec->layers[l + 1].in_norm : dec->norm;
    STAGE(launch_add_rmsnorm(x, dpart, p.s_d, nw, h, n, D, c.rms_eps, dt, s), "rmsnorm");
  }
  if (p.gemv) {
    STAGE(launch_gemv16(dec->embed, h, logits, n, c.vocab, D, 1, dt, s), "dec_head");
  } else {
    STAGE(launch_gemm(gemm_(h, D, dec->embed, n, c.vocab, D, logits, c.vocab), EPI_F32, dt, false, s), "dec_head");
  }
  if (next)
    STAGE(launch_argmax(logits, n, c.vocab, (float*)(w + p.o_amv), (int*)(w + p.o_ami), next, s), "argmax");
  return MT_OK;
}


int64_t mt_mel_frames(int64_t n) { return n < 0 ? -1 : n / HOP; }

int64_t mt_encoder_frames(int64_t T) { return T < 0 ? -1 : half_up(half_up(half_up(T))); }

int64_t mt_encoder_frames_for(int32_t frontend, int64_t T) {
  if (T < 0 || (frontend != MT_FRONTEND_CONV2D_8X && frontend != MT_FRONTEND_CONV1D_2X)) return -1;
  return frames_of(frontend, T);
}

int32_t mt_max_window(void) { return MAX_WINDOW; }

const char* mt_status_string(mt_status s) {
  switch (s) {
    case MT_OK: return "MT_OK";
    case MT_ERR_INVALID_ARG: return "MT_ERR_INVALID_ARG";
    case MT_ERR_UNSUPPORTED: return "MT_ERR_UNSUPPORTED";
    case MT_ERR_WORKSPACE: return "MT_ERR_WORKSPACE";
    case MT_ERR_HIP: return "MT_ERR_HIP";
  }
  return "unknown mt_status";
}

const char* mt_last_error(void) { return g_err.c_str(); }

mt_status mt_logmel_workspace_size(const mt_batch* wav, size_t* bytes) {
  if (!bytes) return fail(MT_ERR_INVALID_ARG, "bytes is NULL");
  MelPlan p;
  mt_status st = plan_mel(wav, p);
  if (st != MT_OK) return st;
  *bytes = p.bytes;
  return MT_OK;
}

mt_status mt_logmel(const float* wav, const mt_batch* wav_b, float* mel, void* ws, size_t ws_bytes,
                    void* stream) {
  MelPlan p;
  mt_status st = plan_mel(wav_b, p);
  if (st != MT_OK) return st;
  if (!wav || !mel || !ws) return fail(MT_ERR_INVALID_ARG, "mt_logmel: NULL device pointer");
  if ((uintptr_t)ws % ALIGN || (uintptr_t)mel % 16)
    return fail(MT_ERR_INVALID_ARG, "mt_logmel: ws must be 256-byte and mel 16-byte aligned");
  if (ws_bytes < p.bytes)
    return fail(MT_ERR_WORKSPACE, "mt_logmel: workspace %zu bytes < required %zu", ws_bytes, p.bytes);
  return run_logmel(wav, wav_b, p, mel, (char*)ws, (hipStream_t)stream);
}

mt_status mt_logmel_noalloc(const float* wav, const mt_batch* wav_b, float* mel, void* stream) {
  MelPlan p;
  mt_status st = plan_mel(wav_b, p);
  if (st != MT_OK) return st;
  if (!wav || !mel) return fail(MT_ERR_INVALID_ARG, "mt_logmel_noalloc: NULL device pointer");
  if ((uintptr_t)mel % 16) return fail(MT_ERR_INVALID_ARG, "mt_logmel_noalloc: mel must be 16-byte aligned");
  // 4096 sequences take 131 584 bytes of tables and maxima (one slot each)
  if (p.B > MT_LOGMEL_NOALLOC_MAX_SEQS || p.bytes > NOALLOC_SCRATCH_BYTES)
    return fail(MT_ERR_WORKSPACE,
                "mt_logmel_noalloc: %d sequences need %zu bytes of scratch, more than the library's "
                "fixed %zu (at most %d sequences)", p.B, p.bytes, NOALLOC_SCRATCH_BYTES,
                MT_LOGMEL_NOALLOC_MAX_SEQS);
  char* w = nullptr;
  st = scratch_for_current_device(&w);
  if (st != MT_OK) return st;
  return run_logmel(wav, wav_b, p, mel, w, (hipStream_t)stream);
}

int32_t mt_encoder_n_weights(const mt_encoder_config* cfg) {
  if (check_config(cfg) != MT_OK) return -1;
  return n_weights_of(*cfg);
}

mt_status mt_encoder_packed_bytes(const mt_encoder_config* cfg, size_t* bytes) {
  mt_status st = check_config(cfg);
  if (st != MT_OK) return st;
  if (!bytes) return fail(MT_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = packed_layout(*cfg).bytes;
  return MT_OK;
}

mt_status mt_encoder_create(const mt_encoder_config* cfg, const float* const* wts, int32_t n_weights,
                            void* packed, size_t packed_bytes, void* stream, mt_encoder** out) {
  mt_status st = check_config(cfg);
  if (st != MT_OK) return st;
  if (!out) return fail(MT_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  const mt_encoder_config c = *cfg;
  if (!wts) return fail(MT_ERR_INVALID_ARG, "weights is NULL");
  if (n_weights != n_weights_of(c))
    return fail(MT_ERR_INVALID_ARG, "expected %d weight tensors, got %d", n_weights_of(c), n_weights);
  for (int i = 0; i < n_weights; ++i)
    if (!wts[i]) return fail(MT_ERR_INVALID_ARG, "weights[%d] is NULL", i);
  const PackedLayout L = packed_layout(c);
  if (!packed) return fail(MT_ERR_INVALID_ARG, "packed is NULL");
  if ((uintptr_t)packed % ALIGN) return fail(MT_ERR_INVALID_ARG, "packed must be 256-byte aligned");
  if (packed_bytes < L.bytes)
    return fail(MT_ERR_WORKSPACE, "packed buffer %zu bytes < required %zu", packed_bytes, L.bytes);

  hipStream_t s = (hipStream_t)stream;
  const int bf = c.dtype == MT_BF16 ? DT_BF16 : c.dtype == MT_F16 ? DT_F16 : DT_F32;  // element type
  const bool half = bf != DT_F32;
  char* P = (char*)packed;
  const int64_t C = c.conv_ch, D = c.d_model, F = c.d_ffn, O = c.d_out, A = c.adapter_hidden;
  const size_t es = half ? 2 : 4;
  int wi = 0;
  auto next = [&]() { return wts[wi++]; };
  const bool two_x = c.frontend == MT_FRONTEND_CONV1D_2X;
  if (two_x) {
    HIP_TRY(launch_pack_conv1d(next(), P + L.conv1_w, (int)D, c.n_mels, bf, s), "pack conv1");
    HIP_TRY(launch_copy_f32(next(), (float*)(P + L.conv1_b), D, s), "pack conv1 bias");
    HIP_TRY(launch_pack_conv1d(next(), P + L.conv2_w, (int)D, (int)D, bf, s), "pack conv2");
    HIP_TRY(launch_copy_f32(next(), (float*)(P + L.conv2_b), D, s), "pack conv2 bias");
  } else {
    HIP_TRY(launch_copy_f32(next(), (float*)(P + L.conv1_w), C * 9, s), "pack conv1");
    HIP_TRY(launch_copy_f32(next(), (float*)(P + L.conv1_b), C, s), "pack conv1 bias");
    HIP_TRY(launch_pack_conv(next(), P + L.conv2_w, (int)C, bf, s), "pack conv2");
    HIP_TRY(launch_copy_f32(next(), (float*)(P + L.conv2_b), C, s), "pack conv2 bias");
    HIP_TRY(launch_pack_conv(next(), P + L.conv3_w, (int)C, bf, s), "pack conv3");
    HIP_TRY(launch_copy_f32(next(), (float*)(P + L.conv3_b), C, s), "pack conv3 bias");
    HIP_TRY(launch_pack_conv_out(next(), P + L.conv_out_w, (int)D, (int)C, 16, bf, s), "pack conv_out");
  }
  for (int l = 0; l < c.n_layers; ++l) {
    const auto& Ll = L.layers[l];
    HIP_TRY(launch_copy_f32(next(), (float*)(P + Ll.ln1_g), D, s), "pack ln1");
    HIP_TRY(launch_copy_f32(next(), (float*)(P + Ll.ln1_b), D, s), "pack ln1");
    for (int j = 0; j < 3; ++j) {  // q, k, v stacked into [3D][D]
      HIP_TRY(launch_convert(next(), P + Ll.wqkv + (size_t)j * D * D * es, D, D, D, 0, bf, s),
              "pack qkv");
      HIP_TRY(launch_copy_f32(next(), (float*)(P + Ll.bqkv) + j * D, D, s), "pack qkv bias");
    }
    HIP_TRY(launch_convert(next(), P + Ll.wo, D, D, D, 0, bf, s), "pack o");
    HIP_TRY(launch_copy_f32(next(), (float*)(P + Ll.bo), D, s), "pack o bias");
    HIP_TRY(launch_copy_f32(next(), (float*)(P + Ll.ln2_g), D, s), "pack ln2");
    HIP_TRY(launch_copy_f32(next(), (float*)(P + Ll.ln2_b), D, s), "pack ln2");
    HIP_TRY(launch_convert(next(), P + Ll.w1, F, D, D, 0, bf, s), "pack fc1");
    HIP_TRY(launch_copy_f32(next(), (float*)(P + Ll.b1), F, s), "pack fc1 bias");
    HIP_TRY(launch_convert(next(), P + Ll.w2, D, F, F, 0, bf, s), "pack fc2");
    HIP_TRY(launch_copy_f32(next(), (float*)(P + Ll.b2), D, s), "pack fc2 bias");
  }
  HIP_TRY(launch_copy_f32(next(), (float*)(P + L.lnp_g), D, s), "pack ln_post");
  HIP_TRY(launch_copy_f32(next(), (float*)(P + L.lnp_b), D, s), "pack ln_post");
  const int64_t KD = half ? 2 * D : D;
  if (!two_x) {
  {
    const float* w = next();
    HIP_TRY(launch_convert(w, P + L.wp1, D, D, KD, 0, bf, s), "pack proj1");
    if (half) HIP_TRY(launch_convert(w, P + L.wp1, D, D, KD, D, bf, s), "pack proj1");
  }
  HIP_TRY(launch_copy_f32(next(), (float*)(P + L.bp1), D, s), "pack proj1 bias");
  {
    const float* w = next();
    HIP_TRY(launch_convert(w, P + L.wp2, O, D, KD, 0, bf, s), "pack proj2");
    if (half) HIP_TRY(launch_convert(w, P + L.wp2, O, D, KD, D, bf, s), "pack proj2");
  }
  HIP_TRY(launch_copy_f32(next(), (float*)(P + L.bp2), O, s), "pack proj2 bias");
  }
  if (A) {
    const float* g = next();
    const float* u = next();
    HIP_TRY(launch_pack_swiglu(g, u, P + L.wgu, (int)A, (int)O, bf, s), "pack adapter gate/up");
    HIP_TRY(launch_convert(next(), P + L.wd, O, A, A, 0, bf, s), "pack adapter down");
  }

  HIP_TRY(launch_fill_i32((int*)(P + L.zeros), 0, 64, s), "zero block");

  mt_encoder* e = new mt_encoder();
  e->cfg = c;
  e->dt = bf;  // DT_* code
  e->es = es;
  e->conv1_w = (const float*)(P + L.conv1_w);  // 2x: 16-bit [D][3 n_mels]
  e->conv1_b = (const float*)(P + L.conv1_b);
  e->conv2_w = P + L.conv2_w;
  e->conv2_b = (const float*)(P + L.conv2_b);
  e->conv3_w = two_x ? nullptr : P + L.conv3_w;
  e->conv3_b = two_x ? nullptr : (const float*)(P + L.conv3_b);
  e->conv_out_w = two_x ? nullptr : P + L.conv_out_w;
  e->layers.resize(c.n_layers);
  for (int l = 0; l < c.n_layers; ++l) {
    const auto& Ll = L.layers[l];
    Layer& y = e->layers[l];
    y.ln1_g = (const float*)(P + Ll.ln1_g);
    y.ln1_b = (const float*)(P + Ll.ln1_b);
    y.wqkv = P + Ll.wqkv;
    y.bqkv = (const float*)(P + Ll.bqkv);
    y.wo = P + Ll.wo;
    y.bo = (const float*)(P + Ll.bo);
    y.ln2_g = (const float*)(P + Ll.ln2_g);
    y.ln2_b = (const float*)(P + Ll.ln2_b);
    y.w1 = P + Ll.w1;
    y.b1 = (const float*)(P + Ll.b1);
    y.w2 = P + Ll.w2;
    y.b2 = (const float*)(P + Ll.b2);
  }
  e->lnp_g = (const float*)(P + L.lnp_g);
  e->lnp_b = (const float*)(P + L.lnp_b);
  e->wp1 = two_x ? nullptr : P + L.wp1;
  e->bp1 = two_x ? nullptr : (const float*)(P + L.bp1);
  e->wp2 = two_x ? nullptr : P + L.wp2;
  e->bp2 = two_x ? nullptr : (const float*)(P + L.bp2);
  e->wgu = A ? P + L.wgu : nullptr;
  e->wd = A ? P + L.wd : nullptr;
  e->zeros = P + L.zeros;
  *out = e;
  return MT_OK;
}

void mt_encoder_destroy(mt_encoder* enc) { delete enc; }

mt_status mt_trace_arm(const char* stage, int32_t max_launches) {
  g_trace.stage.clear();
  g_trace.used = 0;
  if (!stage || !*stage) return MT_OK;
  if (max_launches < 1 || max_launches > 1 << 16)
    return fail(MT_ERR_INVALID_ARG, "max_launches must be in [1, 65536]");
  while ((int)g_trace.ev.size() < 2 * max_launches) {
    hipEvent_t e;
    HIP_TRY(hipEventCreate(&e), "hipEventCreate");
    g_trace.ev.push_back(e);
  }
  g_trace.stage = stage;
  return MT_OK;
}

mt_status mt_trace_collect(double* total_ms, int32_t* launches) {
  if (!total_ms || !launches) return fail(MT_ERR_INVALID_ARG, "NULL output pointer");
  double tot = 0.0;
  for (int i = 0; i < g_trace.used; ++i) {
    HIP_TRY(hipEventSynchronize(g_trace.ev[2 * i + 1]), "hipEventSynchronize");
    float ms = 0.f;
    HIP_TRY(hipEventElapsedTime(&ms, g_trace.ev[2 * i], g_trace.ev[2 * i + 1]), "hipEventElapsedTime");
    tot += ms;
  }
  *total_ms = tot;
  *launches = g_trace.used;
  g_trace.used = 0;
  return MT_OK;
}

mt_status mt_encode_workspace_size(const mt_encoder* enc, const mt_batch* mel_b, int32_t window,
                                   size_t* bytes) {
  if (!enc) return fail(MT_ERR_INVALID_ARG, "encoder is NULL");
  if (!bytes) return fail(MT_ERR_INVALID_ARG, "bytes is NULL");
  EncPlan p;
  mt_status st = plan_encode(enc, mel_b, window, p);
  if (st != MT_OK) return st;
  *bytes = p.bytes;
  return MT_OK;
}

mt_status mt_encode(const mt_encoder* enc, const float* mel, const mt_batch* mel_b, int32_t window,
                    float* out, void* ws, size_t ws_bytes, void* stream) {
  if (!enc) return fail(MT_ERR_INVALID_ARG, "encoder is NULL");
  EncPlan p;
  mt_status st = plan_encode(enc, mel_b, window, p);
  if (st != MT_OK) return st;
  if (!mel || !out || !ws) return fail(MT_ERR_INVALID_ARG, "mt_encode: NULL device pointer");
  if ((uintptr_t)ws % ALIGN || (uintptr_t)out % 16 || (uintptr_t)mel % 16)
    return fail(MT_ERR_INVALID_ARG, "mt_encode: ws must be 256-byte, mel and out 16-byte aligned");
  if (ws_bytes < p.bytes)
    return fail(MT_ERR_WORKSPACE, "mt_encode: workspace %zu bytes < required %zu", ws_bytes, p.bytes);

  return run_encode(enc, p, mel, window, out, (char*)ws, (hipStream_t)stream, nullptr, nullptr);
}


mt_status mt_encode_stream_workspace_size(const mt_encoder* enc, int64_t n_samples, int32_t window,
                                          int32_t chunk_windows, size_t* bytes) {
  if (!bytes) return fail(MT_ERR_INVALID_ARG, "bytes is NULL");
  StreamPlan sp;
  mt_status st = plan_stream(enc, n_samples, window, chunk_windows, sp);
  if (st != MT_OK) return st;
  *bytes = sp.bytes;
  return MT_OK;
}

mt_status mt_encode_stream(const mt_encoder* enc, const float* wav, int64_t n_samples, int32_t window,
                           int32_t chunk_windows, float* out, void* ws, size_t ws_bytes, void* stream) {
  StreamPlan sp;
  mt_status st = plan_stream(enc, n_samples, window, chunk_windows, sp);
  if (st != MT_OK) return st;
  if (!wav || !out || !ws) return fail(MT_ERR_INVALID_ARG, "mt_encode_stream: NULL device pointer");
  if ((uintptr_t)ws % ALIGN || (uintptr_t)out % 16)
    return fail(MT_ERR_INVALID_ARG, "mt_encode_stream: ws must be 256-byte and out 16-byte aligned");
  if (ws_bytes < sp.bytes)
    return fail(MT_ERR_WORKSPACE, "mt_encode_stream: workspace %zu bytes < required %zu", ws_bytes,
                sp.bytes);
  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  float* mel = (float*)(w + sp.off_mel);
  const int d_out = enc->cfg.with_head ? enc->cfg.d_out : enc->cfg.d_model;

  // pass 1: the stream's log-mel maximum (values discarded)
  const float ninf = -INFINITY;
  int key;
  memcpy(&key, &ninf, 4);
  key = key >= 0 ? key : key ^ 0x7fffffff;
  HIP_TRY(launch_fill_i32((int*)(w + sp.off_gmax), key, 1, s), "fill");
  HIP_TRY(launch_fill_i32((int*)(w + sp.off_sat), 0, 1, s), "fill");
  for (int64_t m0 = 0; m0 < sp.T; m0 += sp.Tc) {
    st = stream_mel(wav, sp.n, m0, std::min(sp.Tc, sp.T - m0), mel, w, sp, false, s);
    if (st != MT_OK) return st;
  }
  // pass 2: chunk by chunk, mel (normalised by the stream's maximum) -> encoder
  for (int64_t e0 = 0; e0 < sp.N; e0 += sp.Fc) {
    const int64_t e1 = std::min(sp.N, e0 + sp.Fc);
    const int drop = e0 > 0 ? 1 : 0;
    const int64_t m0 = std::max<int64_t>(0, 8 * e0 - 8), m1 = std::min(sp.T, 8 * e1);
    int64_t lens[1] = {m1 - m0};
    if (half_up(half_up(half_up(lens[0]))) != e1 - e0 + drop)
      return fail(MT_ERR_INVALID_ARG, "mt_encode_stream: internal chunk geometry error");
    st = stream_mel(wav, sp.n, m0, m1 - m0, mel, w, sp, true, s);
    if (st != MT_OK) return st;
    mt_batch b;
    b.layout = MT_PACKED;
    b.n_seqs = 1;
    b.len = lens;
    b.max_len = 0;
    EncPlan ep;
    st = plan_encode(enc, &b, window, ep);
    if (st != MT_OK) return st;
    StreamChunk ch;
    ch.pos = (int)(e0 - drop);
    ch.drop = drop;
    ch.keep = (int)(e1 - e0);
    st = run_encode(enc, ep, mel, window, out + e0 * d_out, w + sp.off_enc, s, &ch, (int*)(w + sp.off_sat));
    if (st != MT_OK) return st;
  }
  return MT_OK;
}


mt_status mt_stream_state_bytes(const mt_encoder* enc, int32_t window, int64_t max_push, size_t* bytes) {
  if (!bytes) return fail(MT_ERR_INVALID_ARG, "bytes is NULL");
  LivePlan lp;
  mt_status st = plan_live(enc, window, max_push, lp);
  if (st != MT_OK) return st;
  *bytes = lp.bytes;
  return MT_OK;
}

mt_status mt_stream_open(const mt_encoder* enc, int32_t window, int64_t max_push, void* state, size_t state_bytes,
                         void* stream, mt_stream** out) {
  if (!out) return fail(MT_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  LivePlan lp;
  mt_status st = plan_live(enc, window, max_push, lp);
  if (st != MT_OK) return st;
  if (!state) return fail(MT_ERR_INVALID_ARG, "mt_stream_open: state is NULL");
  if ((uintptr_t)state % ALIGN) return fail(MT_ERR_INVALID_ARG, "mt_stream_open: state must be 256-byte aligned");
  if (state_bytes < lp.bytes)
    return fail(MT_ERR_WORKSPACE, "mt_stream_open: state %zu bytes < required %zu", state_bytes, lp.bytes);
  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)state;
  const float ninf = -INFINITY;
  int key;
  memcpy(&key, &ninf, 4);
  key = key >= 0 ? key : key ^ 0x7fffffff;
  HIP_TRY(launch_fill_i32((int*)(w + lp.off_gmax), key, 1, s), "fill");
  HIP_TRY(launch_fill_i32((int*)(w + lp.off_sat), 0, 1, s), "fill");
  mt_stream* h = new mt_stream();
  h->enc = enc;
  h->window = window;
  h->max_push = max_push;
  h->state = w;
  *out = h;
  return MT_OK;
}

int64_t mt_stream_pending_frames(const mt_stream* st, int64_t n_more, int32_t finish) {
  if (!st || st->finished || n_more < 0 || (finish != 0 && finish != 1)) return -1;
  const int64_t have = st->have + n_more;
  if (!finish) return (live_complete(st->window, have) - st->next) * st->window;
  if (have < 201) return -1;
  return half_up(half_up(half_up(have / HOP))) - st->next * st->window;
}

mt_status mt_stream_push(mt_stream* st, const float* samples, int64_t n, float* out, int64_t out_frames,
                         int64_t* n_frames, void* stream) {
  if (!st) return fail(MT_ERR_INVALID_ARG, "stream is NULL");
  if (!n_frames) return fail(MT_ERR_INVALID_ARG, "n_frames is NULL");
  *n_frames = 0;
  if (st->finished) return fail(MT_ERR_INVALID_ARG, "mt_stream_push: the stream has finished");
  if (n < 0 || n > st->max_push)
    return fail(MT_ERR_INVALID_ARG, "mt_stream_push: %lld samples outside [0, max_push = %lld]", (long long)n,
                (long long)st->max_push);
  if (n > 0 && !samples) return fail(MT_ERR_INVALID_ARG, "mt_stream_push: samples is NULL");
  if (st->have + n > LIVE_MAX_SAMPLES)
    return fail(MT_ERR_UNSUPPORTED, "mt_stream_push: a stream of more than %lld samples", (long long)LIVE_MAX_SAMPLES);
  LivePlan lp;
  mt_status r = plan_live(st->enc, st->window, st->max_push, lp);
  if (r != MT_OK) return r;
  const int W = st->window;
  const int d = st->enc->cfg.with_head ? st->enc->cfg.d_out : st->enc->cfg.d_model;
  const int64_t k_end = live_complete(W, st->have + n);
  const int64_t frames = (k_end - st->next) * W;
  if (frames > 0 && (!out || (uintptr_t)out % 16))
    return fail(MT_ERR_INVALID_ARG, "mt_stream_push: out is NULL or not 16-byte aligned");
  if (frames > out_frames)
    return fail(MT_ERR_WORKSPACE, "mt_stream_push: %lld frames complete, out holds %lld", (long long)frames,
                (long long)out_frames);
  hipStream_t s = (hipStream_t)stream;
  char* w = st->state;
  if (n > 0) {
    if (st->have + n - st->base > lp.cap) {
      // keep what the next window can still read, in the other buffer
      const int64_t q0 = live_keep_from(W, st->next);
      if (q0 < st->base || st->have - q0 + n > lp.cap)
        return fail(MT_ERR_INVALID_ARG, "mt_stream_push: internal buffer plan error");
      if (st->have > q0)
        HIP_TRY(launch_copy_f32((const float*)(w + lp.off_buf[st->cur]) + (q0 - st->base),
                                (float*)(w + lp.off_buf[st->cur ^ 1]), st->have - q0, s), "keep samples");
      st->cur ^= 1;
      st->base = q0;
    }
    HIP_TRY(launch_copy_f32(samples, (float*)(w + lp.off_buf[st->cur]) + (st->have - st->base), n, s),
            "append samples");
    st->have += n;
  }
  for (int64_t k = st->next; k < k_end; ++k) {
    r = live_encode_window(st, lp, k, false, out + (k - st->next) * W * (int64_t)d, s);
    if (r != MT_OK) return r;
  }
  st->next = k_end;
  *n_frames = frames;
  return MT_OK;
}

mt_status mt_stream_finish(mt_stream* st, float* out, int64_t out_frames, int64_t* n_frames, void* stream) {
  if (!st) return fail(MT_ERR_INVALID_ARG, "stream is NULL");
  if (!n_frames) return fail(MT_ERR_INVALID_ARG, "n_frames is NULL");
  *n_frames = 0;
  if (st->finished) return fail(MT_ERR_INVALID_ARG, "mt_stream_finish: the stream has finished");
  if (st->have < 201)
    return fail(MT_ERR_INVALID_ARG, "mt_stream_finish: %lld samples; reflection padding by 200 needs more than 200",
                (long long)st->have);
  LivePlan lp;
  mt_status r = plan_live(st->enc, st->window, st->max_push, lp);
  if (r != MT_OK) return r;
  const int W = st->window;
  const int d = st->enc->cfg.with_head ? st->enc->cfg.d_out : st->enc->cfg.d_model;
  const int64_t N = half_up(half_up(half_up(st->have / HOP)));
  const int64_t n_win = (N + W - 1) / W;
  const int64_t frames = N - st->next * W;
  if (frames > 0 && (!out || (uintptr_t)out % 16))
    return fail(MT_ERR_INVALID_ARG, "mt_stream_finish: out is NULL or not 16-byte aligned");
  if (frames > out_frames)
    return fail(MT_ERR_WORKSPACE, "mt_stream_finish: %lld frames remain, out holds %lld", (long long)frames,
                (long long)out_frames);
  hipStream_t s = (hipStream_t)stream;
  for (int64_t k = st->next; k < n_win; ++k) {
    r = live_encode_window(st, lp, k, true, out + (k - st->next) * W * (int64_t)d, s);
    if (r != MT_OK) return r;
  }
  st->next = n_win;
  st->finished = true;
  *n_frames = frames;
  return MT_OK;
}

void mt_stream_close(mt_stream* st) { delete st; }

mt_status mt_prompt_embed_workspace_size(int64_t n_tokens, size_t* bytes) {
  if (!bytes) return fail(MT_ERR_INVALID_ARG, "bytes is NULL");
  if (n_tokens < 1 || n_tokens > INT32_MAX)
    return fail(MT_ERR_INVALID_ARG, "mt_prompt_embed: n_tokens %lld out of range", (long long)n_tokens);
  *bytes = ((size_t)n_tokens * 8 + ALIGN - 1) / ALIGN * ALIGN;
  return MT_OK;
}

mt_status mt_prompt_embed(const int32_t* tokens, int64_t n_tokens, int32_t audio_token, const void* table,
                          int32_t table_dtype, int64_t vocab, int32_t d, const float* audio,
                          int64_t n_audio, float* out, void* ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  mt_status st = mt_prompt_embed_workspace_size(n_tokens, &need);
  if (st != MT_OK) return st;
  if (!tokens) return fail(MT_ERR_INVALID_ARG, "mt_prompt_embed: tokens is NULL");
  if (table_dtype != MT_F32 && table_dtype != MT_BF16 && table_dtype != MT_F16)
    return fail(MT_ERR_INVALID_ARG, "mt_prompt_embed: table_dtype %d unknown", table_dtype);
  if (d < 4 || d % 4) return fail(MT_ERR_INVALID_ARG, "mt_prompt_embed: d = %d must be a positive multiple of 4", d);
  if (vocab < 1) return fail(MT_ERR_INVALID_ARG, "mt_prompt_embed: vocab must be >= 1");
  if (n_audio < 0) return fail(MT_ERR_INVALID_ARG, "mt_prompt_embed: n_audio < 0");
  std::vector<int64_t> map((size_t)n_tokens);
  int64_t k = 0;
  for (int64_t i = 0; i < n_tokens; ++i) {
    const int32_t t = tokens[i];
    if (t == audio_token) {
      map[i] = -(++k);
    } else {
      if (t < 0 || t >= vocab)
        return fail(MT_ERR_INVALID_ARG, "mt_prompt_embed: tokens[%lld] = %d outside [0, %lld)",
                    (long long)i, t, (long long)vocab);
      map[i] = t;
    }
  }
  if (k != n_audio)
    return fail(MT_ERR_INVALID_ARG, "mt_prompt_embed: %lld audio placeholders for %lld audio frames",
                (long long)k, (long long)n_audio);
  if (!table || !out || !ws || (n_audio > 0 && !audio))
    return fail(MT_ERR_INVALID_ARG, "mt_prompt_embed: NULL device pointer");
  if ((uintptr_t)ws % ALIGN || (uintptr_t)out % 16 || (uintptr_t)audio % 16 ||
      (uintptr_t)table % (table_dtype == MT_F32 ? 16 : 8))
    return fail(MT_ERR_INVALID_ARG, "mt_prompt_embed: misaligned pointer");
  if (ws_bytes < need)
    return fail(MT_ERR_WORKSPACE, "mt_prompt_embed: workspace %zu bytes < required %zu", ws_bytes, need);
  hipStream_t s = (hipStream_t)stream;
  HIP_TRY(upload_words((uint32_t*)ws, (const uint32_t*)map.data(), 2 * n_tokens, s), "upload tables");
  const int dt = table_dtype == MT_F32 ? DT_F32 : table_dtype == MT_BF16 ? DT_BF16 : DT_F16;
  HIP_TRY(launch_splice((const int64_t*)ws, n_tokens, table, dt, audio, out, d, s), "splice");
  return MT_OK;
}

}  // extern "C"
