/*
 * mt.h -- C ABI of the windowed-attention audio encoder for AMD MI355X (gfx950).
 *
 * The library computes the forward pass of the audio encoder described in the
 * model card "MOSS-Transcribe-preview-2B-GGUF":
 *   - Architecture table, row "Audio": 16 kHz mono input, 128 mel bins,
 *     n_fft 400, hop 160, matching Whisper's feature extractor;
 *   - gotcha list: Whisper drops the trailing STFT frame, so a clip of n
 *     samples gives exactly n / hop mel frames;
 *   - row "Conv front-end": three 3x3 stride-2 Conv2D (1 -> 480 -> 480 -> 480),
 *     conv_out 480*16 = 7680 -> 1280 without bias, sinusoidal positions;
 *   - row "Audio encoder": 32 pre-LN Transformer layers, d 1280, 20 heads of
 *     64, FFN 5120, windowed (block-diagonal) attention;
 *   - row "Encoder head": ln_post -> proj1 (1280 -> 1280) -> GELU -> proj2
 *     (1280 -> 2048);
 *   - row "Adapter": gated MLP (SwiGLU) 2048 -> 8192 -> 2048 (optional).
 *
 * Conventions for every entry point
 *   - Device pointers point to memory of the current HIP device; host pointers
 *     are read before the call returns and may be freed afterwards.
 *   - The caller owns every device buffer (inputs, outputs, packed weights,
 *     workspace).  The library never allocates device memory; it owns only
 *     the small host handle of an encoder.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call is
 *     asynchronous on that stream and does not synchronise the host.
 *   - Errors are returned as mt_status; nothing is launched when a call
 *     fails validation.  mt_last_error() gives a thread-local description.
 *   - Calls that share a workspace, or that write the same output, must be
 *     ordered by the caller (for example by issuing them on one stream).
 */
#ifndef MT_H
#define MT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MT_OK = 0,
  MT_ERR_INVALID_ARG = 1, /* null pointer, bad length, bad layout, ... */
  MT_ERR_UNSUPPORTED = 2, /* geometry or window the kernels are not built for */
  MT_ERR_WORKSPACE = 3,   /* workspace or packed buffer too small */
  MT_ERR_HIP = 4          /* a HIP runtime call failed */
} mt_status;

/* Compute type of the matrix operands (accumulation is fp32 in every case;
 * the residual stream, LayerNorm statistics, softmax and epilogues are fp32).
 *   MT_F32   fp32 operands everywhere;
 *   MT_BF16  bf16 weights and activations at the matrix cores.  Against the
 *            fp64 definition (per output row: cosine >= 0.999 and max |diff|
 *            <= 0.02 RMS) it holds on single clips, batches and long streams
 *            without the adapter (measured 0.016 - 0.019), but NOT through the
 *            SwiGLU adapter: the product of its two projections doubles the
 *            tower's relative error (measured up to 0.027 on 2..60 s clips);
 *   MT_F16   fp16 weights and activations at the matrix cores (weights given
 *            as bf16 values are held exactly in fp16 unless |w| < 2^-17,
 *            which moves by at most 2^-25; activations saturate at +-65504).
 *            Meets that bar on every workload (measured <= 0.004): the
 *            16-bit type to use when the bar matters.
 * With 16-bit operands the head's activations enter its two products as
 * hi/lo pairs of the operand type. */
typedef enum { MT_F32 = 0, MT_BF16 = 1, MT_F16 = 2 } mt_dtype;

typedef enum {
  MT_PACKED = 0, /* sequences stored back to back, no padding */
  MT_PADDED = 1  /* sequence i starts at row i * max_len */
} mt_layout;

/* A batch of variable-length sequences.  `len` is a HOST array of n_seqs
 * lengths (samples for a waveform batch, mel frames for a log-mel batch).
 * For MT_PADDED, max_len is the row stride per sequence and every len[i]
 * must be <= max_len; for MT_PACKED max_len is ignored. */
typedef struct {
  int32_t layout;
  int32_t n_seqs;
  const int64_t* len;
  int64_t max_len;
} mt_batch;

/* Front-end variants (mt_encoder_config.frontend).
 *   MT_FRONTEND_CONV2D_8X  model card "MOSS-Transcribe-preview-2B-GGUF",
 *       Architecture table, Conv front-end row: three 3x3 stride-2 Conv2D
 *       (1 -> C -> C -> C channels, GELU after each) over the mel image, then
 *       conv_out (C * 16 -> d_model) and sinusoids; windowed attention; head
 *       ln_post -> proj1 -> GELU -> proj2 (+ optional SwiGLU adapter).
 *   MT_FRONTEND_CONV1D_2X  the whisper geometries of page "CrisperWhisper ->
 *       ONNX (with cross-attentions)" (sections What this exports instead and
 *       Results: 1500 encoder frames per 30 s, full attention).  The page does
 *       not describe the front-end; the one implemented is two 1-D
 *       convolutions over time with kernel 3 and padding 1, the mel bins as
 *       input channels: conv1 n_mels -> d_model stride 1, conv2 d_model ->
 *       d_model stride 2, GELU after each, then the same sinusoids; the head
 *       is ln_post only (d_out = d_model), no adapter; 16-bit dtypes only. */
typedef enum {
  MT_FRONTEND_CONV2D_8X = 0,
  MT_FRONTEND_CONV1D_2X = 1
} mt_frontend;

/* Encoder geometry and compute type.  The production geometry is
 * {128, 480, 1280, 32, 20, 64, 5120, 2048, 0 or 8192}.  The kernels require
 * n_mels == 128, head_dim == 64, n_heads * head_dim == d_model, conv_ch a
 * multiple of 32 (at most 2048), d_ffn, d_out, adapter_hidden multiples of
 * 64, and d_model a multiple of 256 (at most 2048).  n_layers may be 0
 * (front-end only). */
typedef struct {
  int32_t n_mels;
  int32_t conv_ch;
  int32_t d_model;
  int32_t n_layers;
  int32_t n_heads;
  int32_t head_dim;
  int32_t d_ffn;
  int32_t d_out;
  int32_t adapter_hidden; /* 0: no adapter */
  int32_t dtype;          /* mt_dtype */
  int32_t with_head;      /* 1: full output (d_out wide); 0: stop after the
                             tower and return the fp32 residual stream
                             (d_model wide) */
  float ln_eps;           /* LayerNorm epsilon, 1e-5 */
  int32_t frontend;       /* mt_frontend (0: the 8x Conv2D front-end).  With
                             MT_FRONTEND_CONV1D_2X conv_ch is ignored. */
} mt_encoder_config;

typedef struct mt_encoder mt_encoder; /* opaque host handle */

/* ---- lengths ---------------------------------------------------------- */

/* Mel frames of a clip of n samples: floor(n / 160) (trailing frame dropped).
 * Returns -1 for n < 0. */
int64_t mt_mel_frames(int64_t n_samples);

/* Encoder frames for T mel frames: three stride-2 convs, ceil(ceil(ceil(T/2)/2)/2).
 * Returns -1 for T < 0. */
int64_t mt_encoder_frames(int64_t mel_frames);

/* Encoder frames for T mel frames with front-end `frontend` (mt_frontend):
 * the 8x one as mt_encoder_frames, the 2x one ceil(T / 2).  Returns -1 for
 * T < 0 or an unknown front-end. */
int64_t mt_encoder_frames_for(int32_t frontend, int64_t mel_frames);

/* ---- log-mel ---------------------------------------------------------- */

/* Workspace bytes for mt_logmel on this batch. */
mt_status mt_logmel_workspace_size(const mt_batch* wav, size_t* bytes);

/* Waveform -> normalised log-mel (Architecture table, row "Audio").
 *   wav   device fp32 samples: packed [sum n_i] or padded [n_seqs, max_len];
 *         each n_i >= 201 (reflect padding by 200 needs more than 200).
 *   mel   device fp32 output, frame-major: packed [sum T_i, 128] or padded
 *         [n_seqs, max_len / 160, 128] with rows t >= T_i set to 0;
 *         T_i = floor(n_i / 160).
 * Per clip: periodic Hann 400, reflect-padded centred frames, |rFFT|^2,
 * Slaney mel filterbank (0..8 kHz), log10(max(., 1e-10)), clamp at the clip's
 * own maximum minus 8, then (x + 4) / 4. */
mt_status mt_logmel(const float* wav, const mt_batch* wav_b, float* mel, void* ws,
                    size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation and output as mt_logmel, without a workspace argument.  The
 * per-call tables and per-clip maxima live in a fixed array of the library,
 * 256 KiB per device, reserved until the process ends; batches of more than
 * MT_LOGMEL_NOALLOC_MAX_SEQS sequences get MT_ERR_WORKSPACE before anything
 * runs.  Nothing is allocated on any call.  Every call on one device uses that
 * device's array: calls that can overlap on one device (several streams or
 * threads) race, and the caller must order them (for example on one
 * stream).  Each call resets what it reads before use. */
#define MT_LOGMEL_NOALLOC_MAX_SEQS 4096
mt_status mt_logmel_noalloc(const float* wav, const mt_batch* wav_b, float* mel, void* stream);

/* ---- encoder ---------------------------------------------------------- */

/* Number of weight tensors create() expects for this geometry:
 * 7 + 16 * n_layers + 6 (+ 3 with the adapter); with MT_FRONTEND_CONV1D_2X,
 * 4 + 16 * n_layers + 2.  Returns -1 for an invalid configuration. */
int32_t mt_encoder_n_weights(const mt_encoder_config* cfg);

/* Bytes of the packed-weight buffer create() needs. */
mt_status mt_encoder_packed_bytes(const mt_encoder_config* cfg, size_t* bytes);

/* Build an encoder.  `weights` is a HOST array of n_weights DEVICE pointers to
 * contiguous fp32 tensors in this canonical order (torch layouts: Linear
 * [out, in], Conv2d [out, in, k_freq, k_time]):
 *   conv1.weight [C,1,3,3], conv1.bias [C], conv2.weight [C,C,3,3], conv2.bias,
 *   conv3.weight, conv3.bias, conv_out.weight [D, C*16];
 *   per layer l: ln1.weight [D], ln1.bias, q.weight [D,D], q.bias, k.weight,
 *     k.bias, v.weight, v.bias, o.weight, o.bias, ln2.weight, ln2.bias,
 *     fc1.weight [F,D], fc1.bias [F], fc2.weight [D,F], fc2.bias [D];
 *   ln_post.weight, ln_post.bias, proj1.weight [D,D], proj1.bias,
 *   proj2.weight [O,D], proj2.bias [O];
 *   adapter only: gate.weight [A,O], up.weight [A,O], down.weight [O,A].
 * Feature j of conv_out's input is conv3 channel j / 16 at frequency j % 16.
 * MT_FRONTEND_CONV1D_2X instead: conv1.weight [D, n_mels, 3], conv1.bias [D],
 *   conv2.weight [D, D, 3], conv2.bias [D] (torch Conv1d [out, in, k]; tap k
 *   reads input frame stride * t + k - 1), the same 16 per layer, then
 *   ln_post.weight, ln_post.bias.
 * `packed` (device, >= mt_encoder_packed_bytes, 256-byte aligned) receives
 * the weights in kernel layouts (rounded to nearest-even for 16-bit types);
 * it must stay alive and unchanged until mt_encoder_destroy.  The source
 * tensors may be freed once the repacking work on `stream` has completed. */
mt_status mt_encoder_create(const mt_encoder_config* cfg, const float* const* weights,
                            int32_t n_weights, void* packed, size_t packed_bytes,
                            void* stream, mt_encoder** out);

void mt_encoder_destroy(mt_encoder* enc);

/* Largest window (encoder frames) whose keys the attention kernel keeps on
 * chip.  16-bit encoders accept any window: longer windows (up to window >=
 * every sequence, i.e. full attention) stream their keys through LDS.  fp32
 * encoders accept a larger `window` only when no sequence is longer than
 * this (the attention is then the same as with window = the longest
 * sequence); otherwise mt_encode returns MT_ERR_UNSUPPORTED. */
int32_t mt_max_window(void);

/* Workspace bytes for mt_encode on this batch and window. */
mt_status mt_encode_workspace_size(const mt_encoder* enc, const mt_batch* mel_b, int32_t window,
                                   size_t* bytes);

/* Log-mel -> encoder frames (N_i below is mt_encoder_frames_for(frontend, T_i)).
 *   mel     device fp32, [sum T_i, n_mels] packed or [n_seqs, max_len, n_mels]
 *           padded (rows t >= T_i are not read); each T_i >= 1.
 *   window  W >= 1, in encoder frames: frames [kW, (k+1)W) of each sequence
 *           attend only to each other, in every layer.
 *   out     device fp32, packed [sum N_i, d] or padded
 *           [n_seqs, N(max_len), d] with rows >= N_i set to 0; d = d_out (or
 *           d_model when with_head == 0).  MT_FRONTEND_CONV1D_2X with
 *           with_head == 1: ln_post of the residual stream, fp32.
 *   ws      device workspace of >= mt_encode_workspace_size bytes, 256-byte
 *           aligned; its contents on entry do not matter.
 * fp16 range: with MT_F16 operands every value converted to fp16 is clamped
 * to +-65504, and the clamps are reported: once the call's work has run (in
 * stream order), the first 32-bit word of ws holds a mask of MT_SAT_* bits,
 * one per stage that clamped at least one value (0: none).  Other operand
 * types leave it 0.  The attention kernel's fp16 values need no report: its
 * probabilities lie in [0, 256] and its outputs within the range of v. */
#define MT_SAT_FRONTEND 1 /* conv1, conv2, conv3 outputs (2x: conv1) */
#define MT_SAT_LN 2       /* LayerNorm outputs (ln1, ln2) */
#define MT_SAT_QKV 4      /* q, k, v */
#define MT_SAT_FFN 8      /* FFN hidden (GELU of fc1) */
#define MT_SAT_HEAD 16    /* ln_post and GELU(proj1) hi/lo pairs */
#define MT_SAT_ADAPTER 32 /* proj2 output into the adapter, SwiGLU hidden */
mt_status mt_encode(const mt_encoder* enc, const float* mel, const mt_batch* mel_b,
                    int32_t window, float* out, void* ws, size_t ws_bytes, void* stream);

/* Bounded-memory encode of one long stream (model card "MOSS-Transcribe-
 * preview-2B-GGUF", Architecture table; the windows make encoder frames
 * independent beyond the convolutions' receptive field of 15 mel frames).
 *   wav            device fp32 [n_samples], one stream, n_samples >= 201.
 *   window         W >= 1 as in mt_encode.
 *   chunk_windows  windows encoded per chunk (>= 1): the workspace holds one
 *                  chunk's activations and does not grow with the stream.
 *   out            device fp32 [N, d], N = mt_encoder_frames(mt_mel_frames(n)).
 * Two passes over the waveform: the stream's log-mel maximum first (the
 * normalisation needs it), then each chunk's mel frames with their receptive
 * field (8 frames before, none after) and the encoder.  The result equals
 * mt_logmel + mt_encode of the whole stream with the same window.  Only the
 * 8x front-end streams: an MT_FRONTEND_CONV1D_2X encoder gives
 * MT_ERR_UNSUPPORTED.  The first 32-bit word of ws holds the fp16 saturation
 * mask of the whole stream, as for mt_encode. */
mt_status mt_encode_stream_workspace_size(const mt_encoder* enc, int64_t n_samples, int32_t window,
                                          int32_t chunk_windows, size_t* bytes);
mt_status mt_encode_stream(const mt_encoder* enc, const float* wav, int64_t n_samples,
                           int32_t window, int32_t chunk_windows, float* out, void* ws,
                           size_t ws_bytes, void* stream);

/* Live encoding of one stream whose audio arrives piece by piece (model card
 * "MOSS-Transcribe-preview-2B-GGUF", Architecture table, rows "Audio" and
 * "Audio encoder": windowed attention makes each window depend only on its
 * own audio beyond the convolutions' receptive field).  The pages do not say
 * how the log clamp's clip maximum is found when the clip is not yet
 * complete; the reading taken is a causal running maximum: window k (encoder
 * frames [kW, (k+1)W)) is clamped at the maximum of the unclamped log-mel
 * over mel frames 0 .. 8 (k+1) W - 1, the frames its receptive field reaches,
 * minus 8.  Each window is therefore encoded exactly as the whole-clip path
 * would encode the stream prefix it needs; the result does not depend on how
 * the audio is split into pushes, the last window sees the maximum of the
 * whole stream, and once the stream's loudest frame has arrived the windows
 * equal mt_encode_stream / mt_logmel + mt_encode of the whole stream.
 *
 * A window is encoded as soon as its samples are in (samples up to
 * 1280 (k+1) W + 39, i.e. W * 80 ms plus 2.5 ms of look-ahead); the state keeps
 * about 1280 W + max_push recent samples, whatever the stream's length (up to
 * 2^31 - 1 samples).  8x front-end only.
 *
 *   mt_stream_state_bytes  device state bytes for this window and the largest
 *                          push (max_push samples).
 *   mt_stream_open         starts a stream in `state` (device, caller-owned,
 *                          256-byte aligned, >= mt_stream_state_bytes; it must
 *                          stay alive and be used by this stream only until
 *                          mt_stream_close).  The first 32-bit word of the
 *                          state holds the fp16 saturation mask (MT_SAT_*) of
 *                          everything the stream has encoded.
 *   mt_stream_push         appends n <= max_push samples (device fp32) and
 *                          encodes every window whose samples are now all in,
 *                          writing their frames to out (device fp32
 *                          [out_frames, d], d as for mt_encode) in order;
 *                          *n_frames (host) = frames written.  The count is
 *                          known on the host before the work runs:
 *                          mt_stream_pending_frames(st, n, 0) gives it.
 *   mt_stream_finish       marks the end of the stream (at least 201 samples in
 *                          all) and encodes the remaining frames, the last
 *                          window partial, with the reflection and zero padding
 *                          of the stream's real end;
 *                          mt_stream_pending_frames(st, 0, 1) gives the count.
 *   mt_stream_close        frees the host handle (not the state).
 * Every call is asynchronous on `stream`; pushes of one stream must be ordered
 * (one stream).  Errors: MT_ERR_INVALID_ARG (push after finish, n > max_push,
 * a finish before 201 samples, NULL pointers), MT_ERR_WORKSPACE (state or out
 * too small), MT_ERR_UNSUPPORTED (the 2x front-end, a stream longer than
 * 2^31 - 1 samples); nothing runs and the stream is unchanged when a call
 * fails its checks (after MT_ERR_HIP the stream must be closed). */
typedef struct mt_stream mt_stream;
mt_status mt_stream_state_bytes(const mt_encoder* enc, int32_t window, int64_t max_push, size_t* bytes);
mt_status mt_stream_open(const mt_encoder* enc, int32_t window, int64_t max_push, void* state,
                         size_t state_bytes, void* stream, mt_stream** out);
/* Frames that a push of n_more samples (finish = 0) or the finish (finish = 1,
 * n_more = 0) would write; -1 if that call would be refused. */
int64_t mt_stream_pending_frames(const mt_stream* st, int64_t n_more, int32_t finish);
mt_status mt_stream_push(mt_stream* st, const float* samples, int64_t n, float* out, int64_t out_frames,
                         int64_t* n_frames, void* stream);
mt_status mt_stream_finish(mt_stream* st, float* out, int64_t out_frames, int64_t* n_frames, void* stream);
void mt_stream_close(mt_stream* st);

/* Prompt embedding with the audio spliced in (model card "MOSS-Transcribe-
 * preview-2B-GGUF", Architecture table, rows Prompt and Audio injection): row
 * i of the output is the token-embedding row of tokens[i], except that each
 * position holding audio_token takes the next audio frame instead.
 *   tokens       host int32 [n_tokens]; every id other than audio_token in
 *                [0, vocab).
 *   table        device [vocab, d], MT_F32, MT_BF16 or MT_F16 (the tied
 *                embedding is kept at F16 by the model card); 16-byte (fp32) or
 *                8-byte aligned rows.
 *   audio        device fp32 [n_audio, d], n_audio = the number of
 *                placeholders in tokens (e.g. the adapter output of one clip).
 *   out          device fp32 [n_tokens, d].
 *   ws           device workspace of >= mt_prompt_embed_workspace_size bytes
 *                (the row map), 256-byte aligned.
 * A count mismatch or an id out of range is reported before any launch. */
mt_status mt_prompt_embed_workspace_size(int64_t n_tokens, size_t* bytes);
mt_status mt_prompt_embed(const int32_t* tokens, int64_t n_tokens, int32_t audio_token,
                          const void* table, int32_t table_dtype, int64_t vocab, int32_t d,
                          const float* audio, int64_t n_audio, float* out, void* ws,
                          size_t ws_bytes, void* stream);

/* ---- diagnostics -------------------------------------------------------- */

/* Stage timer.  Arms timing of one stage of mt_logmel / mt_encode, named
 * "mel", "mel_norm", "conv1", "conv2", "conv3", "conv_out", "ln1", "qkv",
 * "attn", "o", "ln2", "fc1", "fc2", "ln_post", "proj1", "proj2",
 * "adapter_gu", "adapter_down", "copy_rows" or "zero_pad": each later launch
 * of that stage is bracketed by two hipEvents recorded on the call's stream,
 * for up to max_launches launches.  NULL or "" disarms.  Timing only; results
 * are unchanged.  Process-wide state, not thread-safe. */
mt_status mt_trace_arm(const char* stage, int32_t max_launches);

/* Waits for the recorded events, returns the summed duration (ms) and the
 * number of timed launches, and clears the record (the stage stays armed). */
mt_status mt_trace_collect(double* total_ms, int32_t* launches);

/* ---- errors ----------------------------------------------------------- */

const char* mt_status_string(mt_status s);
const char* mt_last_error(void);

/* ---- language-model decoder (model card "MOSS-Transcribe-preview-2B-GGUF",
 *      Architecture table, row LLM: Qwen3-1.7B) ---------------------------- */

/* Decoder geometry.  The card's: {151936, 2048, 28, 16, 8, 128, 6144}.  The
 * kernels require head_dim == 128, n_heads == 2 * n_kv_heads, d_model and
 * d_ffn multiples of 256, vocab a multiple of 16, dtype MT_BF16 or MT_F16
 * (weights, matrix operands and the KV cache; fp32 accumulation and residual
 * stream). */
typedef struct {
  int32_t vocab;
  int32_t d_model;
  int32_t n_layers;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t d_ffn;
  int32_t dtype;
  float rms_eps;   /* RMSNorm epsilon: 1e-6 */
  float rope_base; /* rotary base: 1e6 */
} mt_decoder_config;

typedef struct mt_decoder mt_decoder; /* opaque host handle */

/* 1 + 11 * n_layers + 1, or -1 for an invalid configuration. */
int32_t mt_decoder_n_weights(const mt_decoder_config* cfg);
mt_status mt_decoder_packed_bytes(const mt_decoder_config* cfg, size_t* bytes);

/* Build a decoder.  `weights`: HOST array of DEVICE pointers to contiguous
 * fp32 tensors (Linear [out, in], no biases) in this order:
 *   embed.weight [vocab, D] (also the output head: tied);
 *   per layer: input_norm.weight [D], q.weight [Hq*128, D], k.weight
 *     [Hkv*128, D], v.weight [Hkv*128, D], q_norm.weight [128],
 *     k_norm.weight [128], o.weight [D, Hq*128], post_norm.weight [D],
 *     gate.weight [F, D], up.weight [F, D], down.weight [D, F];
 *   norm.weight [D].
 * `packed` (device, >= mt_decoder_packed_bytes, 256-byte aligned) receives
 * the kernel layouts and must outlive the handle. */
mt_status mt_decoder_create(const mt_decoder_config* cfg, const float* const* weights, int32_t n_weights,
                            void* packed, size_t packed_bytes, void* stream, mt_decoder** out);
void mt_decoder_destroy(mt_decoder* dec);

/* The packed embedding table (device, [vocab][d_model] of the decoder's
 * dtype): the table mt_prompt_embed reads token rows from. */
const void* mt_decoder_embedding(const mt_decoder* dec);

/* Bytes of a KV cache for max_seqs sequences of up to max_pos positions:
 * [n_layers][max_seqs][2 (K, V)][n_kv_heads][max_pos][128] of the dtype.
 * The caller allocates it; K entries are stored after K-norm and rotation. */
mt_status mt_decoder_cache_bytes(const mt_decoder* dec, int32_t max_seqs, int32_t max_pos, size_t* bytes);

/* Workspace bytes for mt_decode with these rows (HOST seq / pos arrays). */
mt_status mt_decode_workspace_size(const mt_decoder* dec, int32_t n_rows, const int32_t* seq, const int32_t* pos,
                                   int32_t max_seqs, int32_t max_pos, size_t* bytes);

/* One forward step of the decoder over n_rows new rows.
 *   x       device fp32 [n_rows, d_model]: the rows' input embeddings (token
 *           rows of the table, or adapter frames; see mt_prompt_embed).
 *   seq     HOST int32 [n_rows]: cache slot (0 .. max_seqs-1) of each row.
 *   pos     HOST int32 [n_rows]: each row's position (0 .. max_pos-1);
 *           (seq, pos) pairs distinct.  A row attends to positions 0 .. pos
 *           of its slot: positions below pos must hold K/V written by an
 *           earlier call or by another row of this one (rows of one call
 *           write their K/V before any row attends).  A prompt is one call
 *           with positions 0 .. S-1; a decode step one row per sequence.
 *   cache   device KV cache of mt_decoder_cache_bytes(max_seqs, max_pos)
 *           (may be NULL for a decoder of 0 layers).
 *   logits  device fp32 [n_rows, vocab] (tied head on the final RMSNorm).
 *   next    device int32 [n_rows] or NULL: the first index of each row's
 *           largest logit.
 * Up to 64 rows run the skinny matrix-vector kernels (the weights stream
 * once for all rows); more rows run the tiled products. */
mt_status mt_decode(const mt_decoder* dec, const float* x, int32_t n_rows, const int32_t* seq, const int32_t* pos,
                    void* cache, int32_t max_seqs, int32_t max_pos, float* logits, int32_t* next, void* ws,
                    size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MT_H */
