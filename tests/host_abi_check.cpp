// Host-side check of the C ABI (include/mt.h) without a GPU: built with g++
// under AddressSanitizer and UndefinedBehaviorSanitizer together with api.cpp
// and the stub launchers of csrc/host_stubs.cpp, in which every "device"
// pointer is host memory and every launcher touches the first and last byte
// of each range its kernel would access.
//
// It calls every entry point with each kind of invalid argument the library
// rejects and checks the status (nothing may be launched, nothing may be
// touched), then runs valid calls of every entry point on buffers of exactly
// the size the size queries report, so that a wrongly carved workspace or a
// wrongly sized output is an out-of-bounds access the sanitizer reports.
// Exit status 0 and a last line "host_abi_check: N checks passed" when every
// check passed.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "mt.h"

static int g_checks = 0, g_failed = 0;

#define EXPECT(call, want)                                                                        \
  do {                                                                                            \
    ++g_checks;                                                                                   \
    const mt_status got_ = (call);                                                                \
    if (got_ != (want)) {                                                                         \
      ++g_failed;                                                                                 \
      fprintf(stderr, "FAIL %s:%d: %s -> %s (want %s): %s\n", __FILE__, __LINE__, #call,          \
              mt_status_string(got_), mt_status_string(want), mt_last_error());                  \
    }                                                                                             \
  } while (0)

#define EXPECT_TRUE(cond)                                                  \
  do {                                                                     \
    ++g_checks;                                                            \
    if (!(cond)) {                                                         \
      ++g_failed;                                                          \
      fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);      \
    }                                                                      \
  } while (0)

// Host buffers standing in for device memory: exactly `bytes` long (the
// sanitizer's redzone starts right after), 256-byte aligned.
struct Buf {
  void* p = nullptr;
  size_t n = 0;
  explicit Buf(size_t bytes) : n(bytes) {
    if (posix_memalign(&p, 256, bytes ? bytes : 1)) abort();
    memset(p, 0, bytes);
  }
  ~Buf() { free(p); }
  Buf(const Buf&) = delete;
  Buf& operator=(const Buf&) = delete;
  float* f() const { return (float*)p; }
};

static mt_batch batch(int layout, const std::vector<int64_t>& len, int64_t max_len = 0) {
  mt_batch b;
  b.layout = layout;
  b.n_seqs = (int32_t)len.size();
  b.len = len.data();
  b.max_len = max_len;
  return b;
}

// ------------------------------------------------------------------ log-mel
static void check_logmel() {
  std::vector<int64_t> lens = {201, 16077, 3200};
  mt_batch b = batch(MT_PACKED, lens);
  size_t ws_bytes = 0;
  EXPECT(mt_logmel_workspace_size(&b, nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_logmel_workspace_size(nullptr, &ws_bytes), MT_ERR_INVALID_ARG);
  EXPECT(mt_logmel_workspace_size(&b, &ws_bytes), MT_OK);
  {
    mt_batch bad = b;
    bad.layout = 7;
    EXPECT(mt_logmel_workspace_size(&bad, &ws_bytes), MT_ERR_INVALID_ARG);
    bad = b;
    bad.n_seqs = 0;
    EXPECT(mt_logmel_workspace_size(&bad, &ws_bytes), MT_ERR_INVALID_ARG);
    bad = b;
    bad.len = nullptr;
    EXPECT(mt_logmel_workspace_size(&bad, &ws_bytes), MT_ERR_INVALID_ARG);
    std::vector<int64_t> neg = {201, -1};
    bad = batch(MT_PACKED, neg);
    EXPECT(mt_logmel_workspace_size(&bad, &ws_bytes), MT_ERR_INVALID_ARG);
    std::vector<int64_t> short_clip = {200};
    bad = batch(MT_PACKED, short_clip);
    EXPECT(mt_logmel_workspace_size(&bad, &ws_bytes), MT_ERR_INVALID_ARG);
    std::vector<int64_t> huge = {(int64_t)INT32_MAX + 1};
    bad = batch(MT_PACKED, huge);
    EXPECT(mt_logmel_workspace_size(&bad, &ws_bytes), MT_ERR_UNSUPPORTED);
    std::vector<int64_t> over = {16000, 16001};
    bad = batch(MT_PADDED, over, 16000);
    EXPECT(mt_logmel_workspace_size(&bad, &ws_bytes), MT_ERR_INVALID_ARG);
    std::vector<int64_t> many(100, (int64_t)INT32_MAX);  // frames beyond the 32-bit tables
    bad = batch(MT_PACKED, many);
    EXPECT(mt_logmel_workspace_size(&bad, &ws_bytes), MT_ERR_UNSUPPORTED);
  }
  EXPECT(mt_logmel_workspace_size(&b, &ws_bytes), MT_OK);
  int64_t n = 0, T = 0;
  for (int64_t x : lens) {
    n += x;
    T += mt_mel_frames(x);
  }
  Buf wav(4 * n), mel(4 * 128 * T), ws(ws_bytes);
  EXPECT(mt_logmel(nullptr, &b, mel.f(), ws.p, ws_bytes, nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_logmel(wav.f(), &b, nullptr, ws.p, ws_bytes, nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_logmel(wav.f(), &b, mel.f(), nullptr, ws_bytes, nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_logmel(wav.f(), &b, mel.f(), (char*)ws.p + 16, ws_bytes - 16, nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_logmel(wav.f(), &b, (float*)((char*)mel.p + 4), ws.p, ws_bytes, nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_logmel(wav.f(), &b, mel.f(), ws.p, ws_bytes - 1, nullptr), MT_ERR_WORKSPACE);
  EXPECT(mt_logmel(wav.f(), &b, mel.f(), ws.p, ws_bytes, nullptr), MT_OK);
  EXPECT(mt_logmel_noalloc(wav.f(), &b, mel.f(), nullptr), MT_OK);
  EXPECT(mt_logmel_noalloc(nullptr, &b, mel.f(), nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_logmel_noalloc(wav.f(), &b, (float*)((char*)mel.p + 4), nullptr), MT_ERR_INVALID_ARG);
  // padded layout: [B, max_len] samples, [B, max_len / 160, 128] frames
  {
    const int64_t max_len = 16077;
    mt_batch pb = batch(MT_PADDED, lens, max_len);
    size_t pws = 0;
    EXPECT(mt_logmel_workspace_size(&pb, &pws), MT_OK);
    Buf pwav(4 * 3 * max_len), pmel(4 * 128 * 3 * (max_len / 160)), pw(pws);
    EXPECT(mt_logmel(pwav.f(), &pb, pmel.f(), pw.p, pws, nullptr), MT_OK);
    EXPECT(mt_logmel_noalloc(pwav.f(), &pb, pmel.f(), nullptr), MT_OK);
  }
  // the largest batch the fixed scratch array takes, and one more sequence
  {
    std::vector<int64_t> many(MT_LOGMEL_NOALLOC_MAX_SEQS, 201);
    mt_batch mb = batch(MT_PACKED, many);
    Buf w2(4 * 201 * many.size()), m2(4 * 128 * many.size());
    EXPECT(mt_logmel_noalloc(w2.f(), &mb, m2.f(), nullptr), MT_OK);
    many.push_back(201);
    mb = batch(MT_PACKED, many);
    EXPECT(mt_logmel_noalloc(w2.f(), &mb, m2.f(), nullptr), MT_ERR_WORKSPACE);
  }
  EXPECT_TRUE(mt_mel_frames(-1) == -1 && mt_mel_frames(16077) == 100);
  EXPECT_TRUE(mt_encoder_frames(-1) == -1 && mt_encoder_frames(3000) == 375 && mt_encoder_frames(1) == 1);
  EXPECT_TRUE(mt_encoder_frames_for(MT_FRONTEND_CONV1D_2X, 3000) == 1500);
  EXPECT_TRUE(mt_encoder_frames_for(5, 3000) == -1);
}

// ------------------------------------------------------------------ encoder
static mt_encoder_config small_cfg(int dtype, int adapter, int frontend = MT_FRONTEND_CONV2D_8X) {
  mt_encoder_config c;
  c.n_mels = 128;
  c.conv_ch = 32;
  c.d_model = 256;
  c.n_layers = 2;
  c.n_heads = 4;
  c.head_dim = 64;
  c.d_ffn = 512;
  c.d_out = frontend == MT_FRONTEND_CONV1D_2X ? 256 : 192;
  c.adapter_hidden = adapter;
  c.dtype = dtype;
  c.with_head = 1;
  c.ln_eps = 1e-5f;
  c.frontend = frontend;
  return c;
}

// Element counts of the weight tensors in the canonical order of mt.h.
static std::vector<size_t> weight_sizes(const mt_encoder_config& c) {
  const size_t C = c.conv_ch, D = c.d_model, F = c.d_ffn, O = c.d_out, A = c.adapter_hidden;
  std::vector<size_t> s;
  if (c.frontend == MT_FRONTEND_CONV1D_2X) {
    s = {D * c.n_mels * 3, D, D * D * 3, D};
  } else {
    s = {C * 9, C, C * C * 9, C, C * C * 9, C, D * C * 16};
  }
  for (int l = 0; l < c.n_layers; ++l) {
    const size_t per[16] = {D, D, D * D, D, D * D, D, D * D, D, D * D, D, D, D, F * D, F, D * F, D};
    s.insert(s.end(), per, per + 16);
  }
  s.push_back(D);
  s.push_back(D);
  if (c.frontend == MT_FRONTEND_CONV1D_2X) return s;
  const size_t head[4] = {D * D, D, O * D, O};
  s.insert(s.end(), head, head + 4);
  if (A) {
    s.push_back(A * O);
    s.push_back(A * O);
    s.push_back(O * A);
  }
  return s;
}

struct Weights {
  std::vector<Buf*> bufs;
  std::vector<const float*> ptrs;
  explicit Weights(const mt_encoder_config& c) {
    for (size_t n : weight_sizes(c)) {
      bufs.push_back(new Buf(4 * n));
      ptrs.push_back(bufs.back()->f());
    }
  }
  ~Weights() {
    for (Buf* b : bufs) delete b;
  }
};

static void check_config_rejections() {
  size_t bytes = 0;
  EXPECT(mt_encoder_packed_bytes(nullptr, &bytes), MT_ERR_INVALID_ARG);
  mt_encoder_config c = small_cfg(MT_F16, 0);
  EXPECT(mt_encoder_packed_bytes(&c, nullptr), MT_ERR_INVALID_ARG);
  struct Case {
    void (*edit)(mt_encoder_config&);
    mt_status want;
  };
  const Case cases[] = {
      {[](mt_encoder_config& c) { c.dtype = 9; }, MT_ERR_INVALID_ARG},
      {[](mt_encoder_config& c) { c.n_layers = -1; }, MT_ERR_INVALID_ARG},
      {[](mt_encoder_config& c) { c.d_ffn = 0; }, MT_ERR_INVALID_ARG},
      {[](mt_encoder_config& c) { c.adapter_hidden = -64; }, MT_ERR_INVALID_ARG},
      {[](mt_encoder_config& c) { c.ln_eps = 0.f; }, MT_ERR_INVALID_ARG},
      {[](mt_encoder_config& c) { c.with_head = 2; }, MT_ERR_INVALID_ARG},
      {[](mt_encoder_config& c) { c.frontend = 3; }, MT_ERR_INVALID_ARG},
      {[](mt_encoder_config& c) { c.n_mels = 80; }, MT_ERR_UNSUPPORTED},
      {[](mt_encoder_config& c) { c.head_dim = 32; c.n_heads = 8; }, MT_ERR_UNSUPPORTED},
      {[](mt_encoder_config& c) { c.n_heads = 3; }, MT_ERR_UNSUPPORTED},
      {[](mt_encoder_config& c) { c.d_model = 320; c.n_heads = 5; }, MT_ERR_UNSUPPORTED},
      {[](mt_encoder_config& c) { c.d_model = 2304; c.n_heads = 36; }, MT_ERR_UNSUPPORTED},
      {[](mt_encoder_config& c) { c.d_ffn = 500; }, MT_ERR_UNSUPPORTED},
      {[](mt_encoder_config& c) { c.conv_ch = 40; }, MT_ERR_UNSUPPORTED},
      {[](mt_encoder_config& c) { c.conv_ch = 2080; }, MT_ERR_UNSUPPORTED},
      {[](mt_encoder_config& c) { c.adapter_hidden = 256; c.with_head = 0; }, MT_ERR_INVALID_ARG},
      {[](mt_encoder_config& c) { c.frontend = MT_FRONTEND_CONV1D_2X; c.d_out = 256; c.dtype = MT_F32; },
       MT_ERR_UNSUPPORTED},
      {[](mt_encoder_config& c) { c.frontend = MT_FRONTEND_CONV1D_2X; c.d_out = 256; c.adapter_hidden = 64; },
       MT_ERR_INVALID_ARG},
      {[](mt_encoder_config& c) { c.frontend = MT_FRONTEND_CONV1D_2X; c.d_out = 192; }, MT_ERR_INVALID_ARG},
  };
  for (const Case& k : cases) {
    mt_encoder_config b = small_cfg(MT_F16, 0);
    k.edit(b);
    EXPECT(mt_encoder_packed_bytes(&b, &bytes), k.want);
    EXPECT_TRUE(mt_encoder_n_weights(&b) == -1);
  }
  EXPECT_TRUE(mt_encoder_n_weights(&c) == 7 + 16 * 2 + 6);
}

static mt_encoder* create(const mt_encoder_config& c, Weights& w, Buf*& packed) {
  size_t bytes = 0;
  EXPECT(mt_encoder_packed_bytes(&c, &bytes), MT_OK);
  packed = new Buf(bytes);
  mt_encoder* e = nullptr;
  const int nw = mt_encoder_n_weights(&c);
  EXPECT(mt_encoder_create(&c, w.ptrs.data(), nw, packed->p, bytes, nullptr, &e), MT_OK);
  return e;
}

static void check_create_rejections() {
  mt_encoder_config c = small_cfg(MT_F16, 0);
  Weights w(c);
  const int nw = mt_encoder_n_weights(&c);
  size_t bytes = 0;
  EXPECT(mt_encoder_packed_bytes(&c, &bytes), MT_OK);
  Buf packed(bytes);
  mt_encoder* e = nullptr;
  EXPECT(mt_encoder_create(&c, w.ptrs.data(), nw, packed.p, bytes, nullptr, nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_encoder_create(&c, nullptr, nw, packed.p, bytes, nullptr, &e), MT_ERR_INVALID_ARG);
  EXPECT(mt_encoder_create(&c, w.ptrs.data(), nw - 1, packed.p, bytes, nullptr, &e), MT_ERR_INVALID_ARG);
  std::vector<const float*> holes = w.ptrs;
  holes[5] = nullptr;
  EXPECT(mt_encoder_create(&c, holes.data(), nw, packed.p, bytes, nullptr, &e), MT_ERR_INVALID_ARG);
  EXPECT(mt_encoder_create(&c, w.ptrs.data(), nw, nullptr, bytes, nullptr, &e), MT_ERR_INVALID_ARG);
  EXPECT(mt_encoder_create(&c, w.ptrs.data(), nw, (char*)packed.p + 64, bytes - 64, nullptr, &e),
         MT_ERR_INVALID_ARG);
  EXPECT(mt_encoder_create(&c, w.ptrs.data(), nw, packed.p, bytes - 1, nullptr, &e), MT_ERR_WORKSPACE);
  EXPECT_TRUE(e == nullptr);
}

// One valid mt_encode on exactly sized buffers, packed or padded.
static void encode_once(mt_encoder* e, const mt_encoder_config& c, const std::vector<int64_t>& T, int layout,
                        int window) {
  int64_t max_len = 0, rows = 0, out_rows = 0;
  for (int64_t t : T) {
    max_len = t > max_len ? t : max_len;
    rows += t;
    out_rows += mt_encoder_frames_for(c.frontend, t);
  }
  mt_batch b = batch(layout, T, layout == MT_PADDED ? max_len : 0);
  size_t ws_bytes = 0;
  EXPECT(mt_encode_workspace_size(e, &b, window, &ws_bytes), MT_OK);
  const int d = c.with_head ? c.d_out : c.d_model;
  if (layout == MT_PADDED) {
    rows = (int64_t)T.size() * max_len;
    out_rows = (int64_t)T.size() * mt_encoder_frames_for(c.frontend, max_len);
  }
  Buf mel(4 * 128 * rows), out(4 * (size_t)d * out_rows), ws(ws_bytes);
  EXPECT(mt_encode(e, mel.f(), &b, window, out.f(), ws.p, ws_bytes, nullptr), MT_OK);
}

static void check_encode() {
  for (int dtype : {MT_F16, MT_BF16, MT_F32}) {
    for (int adapter : {0, 128}) {
      mt_encoder_config c = small_cfg(dtype, adapter);
      Weights w(c);
      Buf* packed = nullptr;
      mt_encoder* e = create(c, w, packed);
      const std::vector<int64_t> T = {1, 9, 200, 3000};
      encode_once(e, c, T, MT_PACKED, 104);
      encode_once(e, c, T, MT_PADDED, 104);
      encode_once(e, c, T, MT_PACKED, 1);
      if (dtype != MT_F32) {
        encode_once(e, c, {2400, 17}, MT_PACKED, 300);  // streamed keys (window > 256)
        encode_once(e, c, {2400, 17}, MT_PADDED, 1 << 30);
      } else {
        size_t bytes = 0;
        std::vector<int64_t> lt = {2400};
        mt_batch lb = batch(MT_PACKED, lt);
        EXPECT(mt_encode_workspace_size(e, &lb, 300, &bytes), MT_ERR_UNSUPPORTED);
        encode_once(e, c, {200}, MT_PACKED, 300);  // window >= every sequence: allowed
      }
      mt_encoder_destroy(e);
      delete packed;
    }
  }
  // the tower alone (with_head = 0) and the 2x front-end
  {
    mt_encoder_config c = small_cfg(MT_BF16, 0);
    c.with_head = 0;
    Weights w(c);
    Buf* packed = nullptr;
    mt_encoder* e = create(c, w, packed);
    encode_once(e, c, {3000, 5}, MT_PADDED, 104);
    mt_encoder_destroy(e);
    delete packed;
  }
  {
    mt_encoder_config c = small_cfg(MT_F16, 0, MT_FRONTEND_CONV1D_2X);
    Weights w(c);
    Buf* packed = nullptr;
    mt_encoder* e = create(c, w, packed);
    encode_once(e, c, {3000, 1, 77}, MT_PACKED, 1 << 30);
    encode_once(e, c, {3000, 1, 77}, MT_PADDED, 64);
    mt_encoder_destroy(e);
    delete packed;
  }
  // rejections of mt_encode
  mt_encoder_config c = small_cfg(MT_F16, 0);
  Weights w(c);
  Buf* packed = nullptr;
  mt_encoder* e = create(c, w, packed);
  std::vector<int64_t> T = {3000, 640};
  mt_batch b = batch(MT_PACKED, T);
  size_t ws_bytes = 0;
  EXPECT(mt_encode_workspace_size(nullptr, &b, 104, &ws_bytes), MT_ERR_INVALID_ARG);
  EXPECT(mt_encode_workspace_size(e, &b, 104, nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_encode_workspace_size(e, &b, 0, &ws_bytes), MT_ERR_INVALID_ARG);
  std::vector<int64_t> zero = {3000, 0};
  mt_batch zb = batch(MT_PACKED, zero);
  EXPECT(mt_encode_workspace_size(e, &zb, 104, &ws_bytes), MT_ERR_INVALID_ARG);
  std::vector<int64_t> toolong = {(int64_t)70000000};  // conv1 rows x 64 past 32 bits
  mt_batch tb = batch(MT_PACKED, toolong);
  EXPECT(mt_encode_workspace_size(e, &tb, 104, &ws_bytes), MT_ERR_UNSUPPORTED);
  // a window so long that the streamed-key attention's 32-bit byte offsets
  // into the qkv buffer would wrap (3 x 256 values of 2 bytes per row)
  std::vector<int64_t> longseq = {(int64_t)8 * 1500000};
  mt_batch lb = batch(MT_PACKED, longseq);
  EXPECT(mt_encode_workspace_size(e, &lb, 1500000, &ws_bytes), MT_ERR_UNSUPPORTED);
  EXPECT(mt_encode_workspace_size(e, &lb, 100000, &ws_bytes), MT_OK);
  EXPECT(mt_encode_workspace_size(e, &b, 104, &ws_bytes), MT_OK);
  Buf mel(4 * 128 * 3640), out(4 * 192 * (375 + 80)), ws(ws_bytes);
  EXPECT(mt_encode(nullptr, mel.f(), &b, 104, out.f(), ws.p, ws_bytes, nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_encode(e, nullptr, &b, 104, out.f(), ws.p, ws_bytes, nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_encode(e, mel.f(), &b, 104, nullptr, ws.p, ws_bytes, nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_encode(e, mel.f(), &b, 104, out.f(), nullptr, ws_bytes, nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_encode(e, mel.f(), &b, 104, (float*)((char*)out.p + 8), ws.p, ws_bytes, nullptr),
         MT_ERR_INVALID_ARG);
  EXPECT(mt_encode(e, mel.f(), &b, 104, out.f(), (char*)ws.p + 128, ws_bytes - 128, nullptr),
         MT_ERR_INVALID_ARG);
  EXPECT(mt_encode(e, mel.f(), &b, 104, out.f(), ws.p, ws_bytes - 1, nullptr), MT_ERR_WORKSPACE);
  EXPECT(mt_encode(e, mel.f(), &b, 104, out.f(), ws.p, ws_bytes, nullptr), MT_OK);

  // mt_encode_stream
  const int64_t n = 16000 * 7 + 77;
  for (int cw : {1, 3, 1000}) {
    size_t sb = 0;
    EXPECT(mt_encode_stream_workspace_size(e, n, 13, cw, &sb), MT_OK);
    Buf wav(4 * n), sout(4 * 192 * (size_t)mt_encoder_frames(mt_mel_frames(n))), sws(sb);
    EXPECT(mt_encode_stream(e, wav.f(), n, 13, cw, sout.f(), sws.p, sb, nullptr), MT_OK);
    if (cw == 3) {
      EXPECT(mt_encode_stream(e, wav.f(), n, 13, cw, sout.f(), sws.p, sb - 1, nullptr), MT_ERR_WORKSPACE);
      EXPECT(mt_encode_stream(e, nullptr, n, 13, cw, sout.f(), sws.p, sb, nullptr), MT_ERR_INVALID_ARG);
      EXPECT(mt_encode_stream(e, wav.f(), n, 13, cw, (float*)((char*)sout.p + 4), sws.p, sb, nullptr),
             MT_ERR_INVALID_ARG);
    }
  }
  size_t sb = 0;
  EXPECT(mt_encode_stream_workspace_size(e, n, 13, 1, nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_encode_stream_workspace_size(nullptr, n, 13, 1, &sb), MT_ERR_INVALID_ARG);
  EXPECT(mt_encode_stream_workspace_size(e, 200, 13, 1, &sb), MT_ERR_INVALID_ARG);
  EXPECT(mt_encode_stream_workspace_size(e, (int64_t)INT32_MAX + 1, 13, 1, &sb), MT_ERR_INVALID_ARG);
  EXPECT(mt_encode_stream_workspace_size(e, n, 0, 1, &sb), MT_ERR_INVALID_ARG);
  EXPECT(mt_encode_stream_workspace_size(e, n, 13, 0, &sb), MT_ERR_INVALID_ARG);
  {
    mt_encoder_config c2 = small_cfg(MT_F16, 0, MT_FRONTEND_CONV1D_2X);
    Weights w2(c2);
    Buf* p2 = nullptr;
    mt_encoder* e2 = create(c2, w2, p2);
    EXPECT(mt_encode_stream_workspace_size(e2, n, 13, 1, &sb), MT_ERR_UNSUPPORTED);
    mt_encoder_destroy(e2);
    delete p2;
  }
  mt_encoder_destroy(e);
  delete packed;
}

// ------------------------------------------------------------------ live stream
static void check_live() {
  mt_encoder_config c = small_cfg(MT_F16, 0);
  Weights w(c);
  Buf* packed = nullptr;
  mt_encoder* e = create(c, w, packed);
  const int W = 5;                 // 6400 samples per window
  const int64_t max_push = 20000;  // several windows per push, and buffer compaction
  size_t sb = 0;
  EXPECT(mt_stream_state_bytes(e, W, max_push, nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_stream_state_bytes(nullptr, W, max_push, &sb), MT_ERR_INVALID_ARG);
  EXPECT(mt_stream_state_bytes(e, 0, max_push, &sb), MT_ERR_INVALID_ARG);
  EXPECT(mt_stream_state_bytes(e, W, 0, &sb), MT_ERR_INVALID_ARG);
  EXPECT(mt_stream_state_bytes(e, W, (int64_t)INT32_MAX + 1, &sb), MT_ERR_INVALID_ARG);
  EXPECT(mt_stream_state_bytes(e, W, max_push, &sb), MT_OK);
  Buf state(sb);
  mt_stream* st = nullptr;
  EXPECT(mt_stream_open(e, W, max_push, state.p, sb, nullptr, nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_stream_open(e, W, max_push, nullptr, sb, nullptr, &st), MT_ERR_INVALID_ARG);
  EXPECT(mt_stream_open(e, W, max_push, (char*)state.p + 16, sb - 16, nullptr, &st), MT_ERR_INVALID_ARG);
  EXPECT(mt_stream_open(e, W, max_push, state.p, sb - 1, nullptr, &st), MT_ERR_WORKSPACE);
  EXPECT(mt_stream_open(e, W, max_push, state.p, sb, nullptr, &st), MT_OK);
  const int d = c.d_out;
  Buf chunk(4 * max_push);
  int64_t total = 0, frames = 0, got = 0;
  // pushes of many sizes: single samples, exactly a window, the largest push
  const int64_t sizes[] = {1, 39, 6400, 0, 20000, 3, 12345, 20000, 20000, 777, 6401, 19999, 20000};
  for (int64_t n : sizes) {
    const int64_t want = mt_stream_pending_frames(st, n, 0);
    EXPECT_TRUE(want >= 0 && want % W == 0);
    Buf out(4 * (size_t)d * (size_t)(want > 0 ? want : 1));
    if (want > 0)
      EXPECT(mt_stream_push(st, chunk.f(), n, out.f(), want - 1, &got, nullptr), MT_ERR_WORKSPACE);
    EXPECT(mt_stream_push(st, chunk.f(), n, out.f(), want, &got, nullptr), MT_OK);
    EXPECT_TRUE(got == want);
    total += n;
    frames += got;
  }
  EXPECT(mt_stream_push(st, chunk.f(), max_push + 1, nullptr, 0, &got, nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_stream_push(st, nullptr, 5, nullptr, 0, &got, nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_stream_push(st, chunk.f(), 5, nullptr, 0, nullptr, nullptr), MT_ERR_INVALID_ARG);
  const int64_t rest = mt_stream_pending_frames(st, 0, 1);
  const int64_t N = mt_encoder_frames(mt_mel_frames(total));
  EXPECT_TRUE(rest == N - frames && rest > 0);
  {
    Buf out(4 * (size_t)d * (size_t)rest);
    EXPECT(mt_stream_finish(st, out.f(), rest - 1, &got, nullptr), MT_ERR_WORKSPACE);
    EXPECT(mt_stream_finish(st, out.f(), rest, &got, nullptr), MT_OK);
    EXPECT_TRUE(got == rest);
  }
  EXPECT(mt_stream_push(st, chunk.f(), 5, nullptr, 0, &got, nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_stream_finish(st, nullptr, 0, &got, nullptr), MT_ERR_INVALID_ARG);
  EXPECT_TRUE(mt_stream_pending_frames(st, 0, 1) == -1);
  mt_stream_close(st);
  // a stream that ends before its first window, and one too short to frame
  EXPECT(mt_stream_open(e, W, max_push, state.p, sb, nullptr, &st), MT_OK);
  EXPECT(mt_stream_push(st, chunk.f(), 150, nullptr, 0, &got, nullptr), MT_OK);
  EXPECT(mt_stream_finish(st, nullptr, 0, &got, nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_stream_push(st, chunk.f(), 51, nullptr, 0, &got, nullptr), MT_OK);
  {
    Buf out(4 * (size_t)d);
    EXPECT(mt_stream_finish(st, out.f(), 1, &got, nullptr), MT_OK);
    EXPECT_TRUE(got == 1);
  }
  mt_stream_close(st);
  mt_encoder_destroy(e);
  delete packed;
}

// ------------------------------------------------------------------ prompt splice
static void check_prompt() {
  const int64_t vocab = 100;
  const int d = 64, audio_tok = 99;
  std::vector<int32_t> toks = {1, 2, audio_tok, audio_tok, 3, audio_tok, 7};
  size_t bytes = 0;
  EXPECT(mt_prompt_embed_workspace_size(0, &bytes), MT_ERR_INVALID_ARG);
  EXPECT(mt_prompt_embed_workspace_size(7, nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_prompt_embed_workspace_size(7, &bytes), MT_OK);
  for (int dt : {MT_F32, MT_BF16, MT_F16}) {
    Buf table((dt == MT_F32 ? 4 : 2) * vocab * d), audio(4 * 3 * d), out(4 * 7 * d), ws(bytes);
    EXPECT(mt_prompt_embed(toks.data(), 7, audio_tok, table.p, dt, vocab, d, audio.f(), 3, out.f(), ws.p, bytes,
                           nullptr), MT_OK);
  }
  Buf table(2 * vocab * d), audio(4 * 3 * d), out(4 * 7 * d), ws(bytes);
  EXPECT(mt_prompt_embed(nullptr, 7, audio_tok, table.p, MT_F16, vocab, d, audio.f(), 3, out.f(), ws.p, bytes,
                         nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_prompt_embed(toks.data(), 7, audio_tok, table.p, 5, vocab, d, audio.f(), 3, out.f(), ws.p, bytes,
                         nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_prompt_embed(toks.data(), 7, audio_tok, table.p, MT_F16, vocab, 6, audio.f(), 3, out.f(), ws.p, bytes,
                         nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_prompt_embed(toks.data(), 7, audio_tok, table.p, MT_F16, 0, d, audio.f(), 3, out.f(), ws.p, bytes,
                         nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_prompt_embed(toks.data(), 7, audio_tok, table.p, MT_F16, vocab, d, audio.f(), -1, out.f(), ws.p,
                         bytes, nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_prompt_embed(toks.data(), 7, audio_tok, table.p, MT_F16, vocab, d, audio.f(), 2, out.f(), ws.p, bytes,
                         nullptr), MT_ERR_INVALID_ARG);
  std::vector<int32_t> bad = toks;
  bad[0] = 100;
  EXPECT(mt_prompt_embed(bad.data(), 7, audio_tok, table.p, MT_F16, vocab, d, audio.f(), 3, out.f(), ws.p, bytes,
                         nullptr), MT_ERR_INVALID_ARG);
  bad[0] = -2;
  EXPECT(mt_prompt_embed(bad.data(), 7, audio_tok, table.p, MT_F16, vocab, d, audio.f(), 3, out.f(), ws.p, bytes,
                         nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_prompt_embed(toks.data(), 7, audio_tok, table.p, MT_F16, vocab, d, nullptr, 3, out.f(), ws.p, bytes,
                         nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_prompt_embed(toks.data(), 7, audio_tok, table.p, MT_F16, vocab, d, audio.f(), 3,
                         (float*)((char*)out.p + 4), ws.p, bytes, nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_prompt_embed(toks.data(), 7, audio_tok, table.p, MT_F16, vocab, d, audio.f(), 3, out.f(), ws.p,
                         bytes - 1, nullptr), MT_ERR_WORKSPACE);
}

// ------------------------------------------------------------------ decoder
static mt_decoder_config dec_cfg() {
  mt_decoder_config c;
  c.vocab = 512;
  c.d_model = 256;
  c.n_layers = 2;
  c.n_heads = 4;
  c.n_kv_heads = 2;
  c.head_dim = 128;
  c.d_ffn = 512;
  c.dtype = MT_BF16;
  c.rms_eps = 1e-6f;
  c.rope_base = 1e6f;
  return c;
}

static void check_decoder() {
  size_t bytes = 0;
  EXPECT(mt_decoder_packed_bytes(nullptr, &bytes), MT_ERR_INVALID_ARG);
  struct Case {
    void (*edit)(mt_decoder_config&);
    mt_status want;
  };
  const Case cases[] = {
      {[](mt_decoder_config& c) { c.dtype = MT_F32; }, MT_ERR_UNSUPPORTED},
      {[](mt_decoder_config& c) { c.vocab = 0; }, MT_ERR_INVALID_ARG},
      {[](mt_decoder_config& c) { c.rms_eps = 0.f; }, MT_ERR_INVALID_ARG},
      {[](mt_decoder_config& c) { c.rope_base = 1.f; }, MT_ERR_INVALID_ARG},
      {[](mt_decoder_config& c) { c.head_dim = 64; }, MT_ERR_UNSUPPORTED},
      {[](mt_decoder_config& c) { c.n_heads = 6; }, MT_ERR_UNSUPPORTED},
      {[](mt_decoder_config& c) { c.d_ffn = 500; }, MT_ERR_UNSUPPORTED},
      {[](mt_decoder_config& c) { c.vocab = 513; }, MT_ERR_UNSUPPORTED},
  };
  for (const Case& k : cases) {
    mt_decoder_config c = dec_cfg();
    k.edit(c);
    EXPECT(mt_decoder_packed_bytes(&c, &bytes), k.want);
    EXPECT_TRUE(mt_decoder_n_weights(&c) == -1);
  }
  mt_decoder_config c = dec_cfg();
  EXPECT(mt_decoder_packed_bytes(&c, nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_decoder_packed_bytes(&c, &bytes), MT_OK);
  const int nw = mt_decoder_n_weights(&c);
  EXPECT_TRUE(nw == 1 + 11 * 2 + 1);
  const size_t V = c.vocab, D = c.d_model, F = c.d_ffn, NQ = 4 * 128, NKV = 2 * 128;
  std::vector<size_t> sizes = {V * D};
  for (int l = 0; l < c.n_layers; ++l) {
    const size_t per[11] = {D, NQ * D, NKV * D, NKV * D, 128, 128, D * NQ, D, F * D, F * D, D * F};
    sizes.insert(sizes.end(), per, per + 11);
  }
  sizes.push_back(D);
  std::vector<Buf*> bufs;
  std::vector<const float*> ptrs;
  for (size_t s : sizes) {
    bufs.push_back(new Buf(4 * s));
    ptrs.push_back(bufs.back()->f());
  }
  Buf packed(bytes);
  mt_decoder* dec = nullptr;
  EXPECT(mt_decoder_create(&c, ptrs.data(), nw, packed.p, bytes, nullptr, nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_decoder_create(&c, nullptr, nw, packed.p, bytes, nullptr, &dec), MT_ERR_INVALID_ARG);
  EXPECT(mt_decoder_create(&c, ptrs.data(), nw + 1, packed.p, bytes, nullptr, &dec), MT_ERR_INVALID_ARG);
  EXPECT(mt_decoder_create(&c, ptrs.data(), nw, (char*)packed.p + 8, bytes - 8, nullptr, &dec),
         MT_ERR_INVALID_ARG);
  EXPECT(mt_decoder_create(&c, ptrs.data(), nw, packed.p, bytes - 1, nullptr, &dec), MT_ERR_WORKSPACE);
  EXPECT(mt_decoder_create(&c, ptrs.data(), nw, packed.p, bytes, nullptr, &dec), MT_OK);
  EXPECT_TRUE(mt_decoder_embedding(dec) == packed.p);
  const int max_seqs = 3, max_pos = 200;
  size_t cache_bytes = 0;
  EXPECT(mt_decoder_cache_bytes(dec, 0, max_pos, &cache_bytes), MT_ERR_INVALID_ARG);
  EXPECT(mt_decoder_cache_bytes(dec, max_seqs, max_pos, nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_decoder_cache_bytes(dec, max_seqs, max_pos, &cache_bytes), MT_OK);
  Buf cache(cache_bytes);
  // a prompt of 5 rows, a decode step of 2 sequences, a 70-row prompt
  // (tiled products), each on exactly sized buffers
  auto decode = [&](std::vector<int32_t> seq, std::vector<int32_t> pos, bool with_next) {
    const int n = (int)seq.size();
    size_t wsb = 0;
    EXPECT(mt_decode_workspace_size(dec, n, seq.data(), pos.data(), max_seqs, max_pos, &wsb), MT_OK);
    Buf x(4 * n * D), logits(4 * n * V), next(4 * n), ws(wsb);
    EXPECT(mt_decode(dec, x.f(), n, seq.data(), pos.data(), cache.p, max_seqs, max_pos, logits.f(),
                     with_next ? (int32_t*)next.p : nullptr, ws.p, wsb, nullptr), MT_OK);
  };
  decode({0, 0, 0, 0, 0}, {0, 1, 2, 3, 4}, true);
  decode({0, 1}, {5, 0}, true);
  decode({2}, {0}, false);
  {
    std::vector<int32_t> s(70, 1), p(70);
    for (int i = 0; i < 70; ++i) p[i] = 1 + i;
    decode(s, p, true);
  }
  std::vector<int32_t> seq = {0, 1}, pos = {5, 5};
  size_t wsb = 0;
  EXPECT(mt_decode_workspace_size(dec, 2, seq.data(), pos.data(), max_seqs, max_pos, &wsb), MT_OK);
  Buf x(4 * 2 * D), logits(4 * 2 * V), ws(wsb);
  EXPECT(mt_decode_workspace_size(nullptr, 2, seq.data(), pos.data(), max_seqs, max_pos, &wsb), MT_ERR_INVALID_ARG);
  EXPECT(mt_decode_workspace_size(dec, 0, seq.data(), pos.data(), max_seqs, max_pos, &wsb), MT_ERR_INVALID_ARG);
  EXPECT(mt_decode_workspace_size(dec, 2, nullptr, pos.data(), max_seqs, max_pos, &wsb), MT_ERR_INVALID_ARG);
  EXPECT(mt_decode_workspace_size(dec, 2, seq.data(), pos.data(), 0, max_pos, &wsb), MT_ERR_INVALID_ARG);
  EXPECT(mt_decode_workspace_size(dec, 2, seq.data(), pos.data(), max_seqs, max_pos, nullptr), MT_ERR_INVALID_ARG);
  std::vector<int32_t> bad_seq = {0, 3}, bad_pos = {5, 200}, dup_seq = {1, 1};
  EXPECT(mt_decode_workspace_size(dec, 2, bad_seq.data(), pos.data(), max_seqs, max_pos, &wsb), MT_ERR_INVALID_ARG);
  EXPECT(mt_decode_workspace_size(dec, 2, seq.data(), bad_pos.data(), max_seqs, max_pos, &wsb), MT_ERR_INVALID_ARG);
  EXPECT(mt_decode_workspace_size(dec, 2, dup_seq.data(), pos.data(), max_seqs, max_pos, &wsb), MT_ERR_INVALID_ARG);
  EXPECT(mt_decode_workspace_size(dec, 2, seq.data(), pos.data(), max_seqs, max_pos, &wsb), MT_OK);
  EXPECT(mt_decode(dec, nullptr, 2, seq.data(), pos.data(), cache.p, max_seqs, max_pos, logits.f(), nullptr, ws.p,
                   wsb, nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_decode(dec, x.f(), 2, seq.data(), pos.data(), nullptr, max_seqs, max_pos, logits.f(), nullptr, ws.p,
                   wsb, nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_decode(dec, x.f(), 2, seq.data(), pos.data(), cache.p, max_seqs, max_pos, logits.f(), nullptr,
                   (char*)ws.p + 16, wsb - 16, nullptr), MT_ERR_INVALID_ARG);
  EXPECT(mt_decode(dec, x.f(), 2, seq.data(), pos.data(), cache.p, max_seqs, max_pos, logits.f(), nullptr, ws.p,
                   wsb - 1, nullptr), MT_ERR_WORKSPACE);
  mt_decoder_destroy(dec);
  for (Buf* b : bufs) delete b;
}

static void check_misc() {
  EXPECT(mt_trace_arm("fc1", 0), MT_ERR_INVALID_ARG);
  EXPECT(mt_trace_arm("fc1", (1 << 16) + 1), MT_ERR_INVALID_ARG);
  EXPECT(mt_trace_arm("mel", 4), MT_OK);
  double ms = 0;
  int32_t n = 0;
  EXPECT(mt_trace_collect(nullptr, &n), MT_ERR_INVALID_ARG);
  EXPECT(mt_trace_collect(&ms, &n), MT_OK);
  EXPECT(mt_trace_arm(nullptr, 0), MT_OK);
  EXPECT_TRUE(mt_max_window() == 256);
  EXPECT_TRUE(strcmp(mt_status_string(MT_ERR_WORKSPACE), "MT_ERR_WORKSPACE") == 0);
  EXPECT_TRUE(strcmp(mt_status_string((mt_status)42), "unknown mt_status") == 0);
}

int main() {
  check_logmel();
  check_config_rejections();
  check_create_rejections();
  check_encode();
  check_live();
  check_prompt();
  check_decoder();
  check_misc();
  if (g_failed) {
    fprintf(stderr, "host_abi_check: %d of %d checks failed\n", g_failed, g_checks);
    return 1;
  }
  printf("host_abi_check: %d checks passed\n", g_checks);
  return 0;
}
