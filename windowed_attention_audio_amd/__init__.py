"""Python binding of libmt.so, the MI355X (gfx950) windowed-attention audio
encoder.  Argument marshalling only: every step of the forward pass runs in
the library's HIP kernels.  PyTorch provides device memory and streams.

The functions carry the names of the C entry points (include/mt.h):

    mt_mel_frames(n)                 floor(n / 160)
    mt_encoder_frames(T)             ceil(ceil(ceil(T / 2) / 2) / 2)
    mt_encoder_frames_for(f, T)      the same for front-end f (2x: ceil(T / 2))
    mt_logmel(wav, lens, ...)        waveform -> normalised log-mel
    mt_encoder_create(cfg, weights)  -> Encoder (packed weights on device)
    mt_encode(enc, mel, lens, W)     log-mel -> encoder frames

Importing the package does not need a GPU; calling the compute entry points
does, and raises if the compiled library is missing.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmt.so")

MT_OK, MT_ERR_INVALID_ARG, MT_ERR_UNSUPPORTED, MT_ERR_WORKSPACE, MT_ERR_HIP = range(5)
MT_F32, MT_BF16, MT_F16 = 0, 1, 2
MT_PACKED, MT_PADDED = 0, 1
MT_FRONTEND_CONV2D_8X, MT_FRONTEND_CONV1D_2X = 0, 1
FRONTENDS = {"conv2d_8x": MT_FRONTEND_CONV2D_8X, "conv1d_2x": MT_FRONTEND_CONV1D_2X}

EXPORTS = (
    "mt_mel_frames", "mt_encoder_frames", "mt_encoder_frames_for", "mt_logmel_workspace_size",
    "mt_logmel", "mt_logmel_noalloc",
    "mt_encoder_n_weights", "mt_encoder_packed_bytes", "mt_encoder_create",
    "mt_encoder_destroy", "mt_max_window", "mt_encode_workspace_size", "mt_encode",
    "mt_encode_stream_workspace_size", "mt_encode_stream",
    "mt_stream_state_bytes", "mt_stream_open", "mt_stream_pending_frames", "mt_stream_push",
    "mt_stream_finish", "mt_stream_close",
    "mt_prompt_embed_workspace_size", "mt_prompt_embed",
    "mt_decoder_n_weights", "mt_decoder_packed_bytes", "mt_decoder_create", "mt_decoder_destroy",
    "mt_decoder_embedding", "mt_decoder_cache_bytes", "mt_decode_workspace_size", "mt_decode",
    "mt_status_string", "mt_last_error", "mt_trace_arm", "mt_trace_collect",
)


class MtError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class Batch(ctypes.Structure):
    _fields_ = [("layout", ctypes.c_int32), ("n_seqs", ctypes.c_int32),
                ("len", ctypes.POINTER(ctypes.c_int64)), ("max_len", ctypes.c_int64)]


class EncoderConfig(ctypes.Structure):
    _fields_ = [("n_mels", ctypes.c_int32), ("conv_ch", ctypes.c_int32),
                ("d_model", ctypes.c_int32), ("n_layers", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("d_ffn", ctypes.c_int32), ("d_out", ctypes.c_int32),
                ("adapter_hidden", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("with_head", ctypes.c_int32), ("ln_eps", ctypes.c_float),
                ("frontend", ctypes.c_int32)]


class DecoderConfig(ctypes.Structure):
    _fields_ = [("vocab", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_layers", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("d_ffn", ctypes.c_int32), ("dtype", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("rope_base", ctypes.c_float)]


_lib = None


def lib():
    """The loaded libmt.so.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m windowed_attention_audio_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        c_sz = ctypes.c_size_t
        vp = ctypes.c_void_p
        L.mt_mel_frames.restype = ctypes.c_int64
        L.mt_mel_frames.argtypes = [ctypes.c_int64]
        L.mt_encoder_frames.restype = ctypes.c_int64
        L.mt_encoder_frames.argtypes = [ctypes.c_int64]
        L.mt_encoder_frames_for.restype = ctypes.c_int64
        L.mt_encoder_frames_for.argtypes = [ctypes.c_int32, ctypes.c_int64]
        L.mt_logmel_workspace_size.argtypes = [ctypes.POINTER(Batch), ctypes.POINTER(c_sz)]
        L.mt_logmel.argtypes = [vp, ctypes.POINTER(Batch), vp, vp, c_sz, vp]
        L.mt_logmel_noalloc.argtypes = [vp, ctypes.POINTER(Batch), vp, vp]
        L.mt_encoder_n_weights.argtypes = [ctypes.POINTER(EncoderConfig)]
        L.mt_encoder_packed_bytes.argtypes = [ctypes.POINTER(EncoderConfig), ctypes.POINTER(c_sz)]
        L.mt_encoder_create.argtypes = [ctypes.POINTER(EncoderConfig), ctypes.POINTER(vp),
                                        ctypes.c_int32, vp, c_sz, vp, ctypes.POINTER(vp)]
        L.mt_encoder_destroy.argtypes = [vp]
        L.mt_encoder_destroy.restype = None
        L.mt_max_window.restype = ctypes.c_int32
        L.mt_encode_workspace_size.argtypes = [vp, ctypes.POINTER(Batch), ctypes.c_int32,
                                               ctypes.POINTER(c_sz)]
        L.mt_encode.argtypes = [vp, vp, ctypes.POINTER(Batch), ctypes.c_int32, vp, vp, c_sz, vp]
        L.mt_encode_stream_workspace_size.argtypes = [vp, ctypes.c_int64, ctypes.c_int32,
                                                      ctypes.c_int32, ctypes.POINTER(c_sz)]
        L.mt_encode_stream.argtypes = [vp, vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, vp,
                                       vp, c_sz, vp]
        i64p = ctypes.POINTER(ctypes.c_int64)
        L.mt_stream_state_bytes.argtypes = [vp, ctypes.c_int32, ctypes.c_int64, ctypes.POINTER(c_sz)]
        L.mt_stream_open.argtypes = [vp, ctypes.c_int32, ctypes.c_int64, vp, c_sz, vp, ctypes.POINTER(vp)]
        L.mt_stream_pending_frames.argtypes = [vp, ctypes.c_int64, ctypes.c_int32]
        L.mt_stream_pending_frames.restype = ctypes.c_int64
        L.mt_stream_push.argtypes = [vp, vp, ctypes.c_int64, vp, ctypes.c_int64, i64p, vp]
        L.mt_stream_finish.argtypes = [vp, vp, ctypes.c_int64, i64p, vp]
        L.mt_stream_close.argtypes = [vp]
        L.mt_stream_close.restype = None
        L.mt_prompt_embed_workspace_size.argtypes = [ctypes.c_int64, ctypes.POINTER(c_sz)]
        L.mt_prompt_embed.argtypes = [ctypes.POINTER(ctypes.c_int32), ctypes.c_int64, ctypes.c_int32,
                                      vp, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, vp,
                                      ctypes.c_int64, vp, vp, c_sz, vp]
        i32p = ctypes.POINTER(ctypes.c_int32)
        dcp = ctypes.POINTER(DecoderConfig)
        L.mt_decoder_n_weights.argtypes = [dcp]
        L.mt_decoder_packed_bytes.argtypes = [dcp, ctypes.POINTER(c_sz)]
        L.mt_decoder_create.argtypes = [dcp, ctypes.POINTER(vp), ctypes.c_int32, vp, c_sz, vp,
                                        ctypes.POINTER(vp)]
        L.mt_decoder_destroy.argtypes = [vp]
        L.mt_decoder_destroy.restype = None
        L.mt_decoder_embedding.argtypes = [vp]
        L.mt_decoder_embedding.restype = vp
        L.mt_decoder_cache_bytes.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(c_sz)]
        L.mt_decode_workspace_size.argtypes = [vp, ctypes.c_int32, i32p, i32p, ctypes.c_int32,
                                               ctypes.c_int32, ctypes.POINTER(c_sz)]
        L.mt_decode.argtypes = [vp, vp, ctypes.c_int32, i32p, i32p, vp, ctypes.c_int32, ctypes.c_int32,
                                vp, vp, vp, c_sz, vp]
        L.mt_trace_arm.argtypes = [ctypes.c_char_p, ctypes.c_int32]
        L.mt_trace_arm.restype = ctypes.c_int
        L.mt_trace_collect.argtypes = [ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_int32)]
        L.mt_trace_collect.restype = ctypes.c_int
        L.mt_status_string.restype = ctypes.c_char_p
        L.mt_status_string.argtypes = [ctypes.c_int]
        L.mt_last_error.restype = ctypes.c_char_p
        for name in ("mt_logmel_workspace_size", "mt_logmel", "mt_logmel_noalloc",
                     "mt_encoder_packed_bytes",
                     "mt_encoder_create", "mt_encode_workspace_size", "mt_encode",
                     "mt_encode_stream_workspace_size", "mt_encode_stream",
                     "mt_stream_state_bytes", "mt_stream_open", "mt_stream_push", "mt_stream_finish",
                     "mt_prompt_embed_workspace_size", "mt_prompt_embed",
                     "mt_decoder_packed_bytes", "mt_decoder_create", "mt_decoder_cache_bytes",
                     "mt_decode_workspace_size", "mt_decode"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status):
    if status != MT_OK:
        L = lib()
        raise MtError(status, L.mt_status_string(status).decode() + ": " +
                      L.mt_last_error().decode())


def make_batch(lens, layout=MT_PACKED, max_len=0):
    arr = (ctypes.c_int64 * len(lens))(*[int(x) for x in lens])
    b = Batch(layout, len(lens), arr, int(max_len))
    b._keep = arr
    return b


def _check_input(t, lens, layout, width, what):
    """The library takes raw device pointers and cannot see buffer sizes: a
    tensor whose shape does not match the host lengths would be read past its
    end.  Raise here instead.  width: trailing row width (0 for waveforms)."""
    lens = [int(x) for x in lens]
    tail = (width,) if width else ()
    if layout == MT_PADDED:
        ok = t.dim() == 2 + len(tail) and t.shape[0] >= len(lens) and t.shape[1] >= max(lens, default=0) \
            and tuple(t.shape[2:]) == tail
        want = f"[>= {len(lens)}, >= {max(lens, default=0)}" + (f", {width}]" if width else "]")
    else:
        ok = t.dim() == 1 + len(tail) and t.shape[0] >= sum(lens) and tuple(t.shape[1:]) == tail
        want = f"[>= {sum(lens)}" + (f", {width}]" if width else "]")
    if not ok:
        raise ValueError(f"{what}: shape {tuple(t.shape)} does not match the lengths (expected {want})")


def _check_output(t, shape, what):
    import math
    if t.numel() < math.prod(shape):
        raise ValueError(f"{what}: {t.numel()} elements, the call writes {math.prod(shape)} ({shape})")


def _stream_ptr(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def mt_mel_frames(n: int) -> int:
    return lib().mt_mel_frames(int(n))


def mt_encoder_frames(T: int) -> int:
    return lib().mt_encoder_frames(int(T))


def mt_encoder_frames_for(frontend: int, T: int) -> int:
    return lib().mt_encoder_frames_for(int(frontend), int(T))


def mt_max_window() -> int:
    return lib().mt_max_window()


def mt_logmel_workspace_size(lens, layout=MT_PACKED, max_len=0) -> int:
    b = make_batch(lens, layout, max_len)
    n = ctypes.c_size_t()
    _check(lib().mt_logmel_workspace_size(ctypes.byref(b), ctypes.byref(n)))
    return n.value


def mt_logmel(wav, lens, layout=MT_PACKED, max_len=0, mel=None, ws=None, stream=None):
    """wav: fp32 CUDA tensor, packed [sum n] or padded [B, max_len].
    Returns the fp32 log-mel tensor [sum T, 128] or [B, max_len // 160, 128]."""
    import torch
    assert wav.is_cuda and wav.dtype == torch.float32 and wav.is_contiguous()
    _check_input(wav, lens, layout, 0, "mt_logmel wav")
    if layout == MT_PADDED:
        max_len = wav.shape[1]
        shape = (len(lens), max_len // 160, 128)
    else:
        shape = (sum(int(n) // 160 for n in lens), 128)
    b = make_batch(lens, layout, max_len)
    if mel is None:
        mel = torch.empty(shape, dtype=torch.float32, device=wav.device)
    _check_output(mel, shape, "mt_logmel mel")
    nbytes = mt_logmel_workspace_size(lens, layout, max_len)
    if ws is None:
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=wav.device)
    _check(lib().mt_logmel(ctypes.c_void_p(wav.data_ptr()), ctypes.byref(b),
                           ctypes.c_void_p(mel.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
                           ws.numel(), _stream_ptr(stream)))
    return mel


def mt_logmel_noalloc(wav, lens, layout=MT_PACKED, max_len=0, mel=None, stream=None):
    """mt_logmel without a workspace (the library's fixed per-device scratch
    array holds the tables and per-clip maxima; at most
    MT_LOGMEL_NOALLOC_MAX_SEQS sequences; calls on one device must not
    overlap)."""
    import torch
    assert wav.is_cuda and wav.dtype == torch.float32 and wav.is_contiguous()
    _check_input(wav, lens, layout, 0, "mt_logmel_noalloc wav")
    if layout == MT_PADDED:
        max_len = wav.shape[1]
        shape = (len(lens), max_len // 160, 128)
    else:
        shape = (sum(int(n) // 160 for n in lens), 128)
    b = make_batch(lens, layout, max_len)
    if mel is None:
        mel = torch.empty(shape, dtype=torch.float32, device=wav.device)
    _check_output(mel, shape, "mt_logmel_noalloc mel")
    _check(lib().mt_logmel_noalloc(ctypes.c_void_p(wav.data_ptr()), ctypes.byref(b),
                                   ctypes.c_void_p(mel.data_ptr()), _stream_ptr(stream)))
    return mel


MT_LOGMEL_NOALLOC_MAX_SEQS = 4096

# fp16 saturation mask (first 32-bit word of an encode workspace after the call)
MT_SAT_FRONTEND, MT_SAT_LN, MT_SAT_QKV, MT_SAT_FFN, MT_SAT_HEAD, MT_SAT_ADAPTER = 1, 2, 4, 8, 16, 32


def saturation_mask(ws) -> int:
    """The MT_SAT_* mask an mt_encode / mt_encode_stream call left in its
    workspace `ws` (a uint8 CUDA tensor); synchronises the stream."""
    import torch
    return int(ws[:4].view(torch.int32).item())


def encoder_config(geom: dict, dtype: int, with_head: bool = True, ln_eps: float = 1e-5):
    """geom["frontend"]: "conv2d_8x" (default) or "conv1d_2x"."""
    return EncoderConfig(geom["n_mels"], geom["conv_ch"], geom["d_model"], geom["n_layers"],
                         geom["n_heads"], geom["head_dim"], geom["d_ffn"], geom["d_out"],
                         geom.get("adapter_hidden", 0), dtype, 1 if with_head else 0, ln_eps,
                         FRONTENDS[geom.get("frontend", "conv2d_8x")])


class Encoder:
    """An encoder whose packed weights live in a torch-owned device buffer."""

    def __init__(self, handle, cfg, packed):
        self.handle = handle
        self.cfg = cfg
        self.packed = packed

    @property
    def d_out(self):
        return self.cfg.d_out if self.cfg.with_head else self.cfg.d_model

    def close(self):
        if self.handle:
            lib().mt_encoder_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def mt_encoder_n_weights(cfg: EncoderConfig) -> int:
    return lib().mt_encoder_n_weights(ctypes.byref(cfg))


def mt_encoder_packed_bytes(cfg: EncoderConfig) -> int:
    n = ctypes.c_size_t()
    _check(lib().mt_encoder_packed_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def mt_encoder_create(cfg: EncoderConfig, weights, device="cuda", stream=None) -> Encoder:
    """weights: fp32 CUDA tensors in the canonical order of include/mt.h."""
    import torch
    for w in weights:
        assert w.is_cuda and w.dtype == torch.float32 and w.is_contiguous()
    nbytes = mt_encoder_packed_bytes(cfg)
    packed = torch.empty(nbytes, dtype=torch.uint8, device=device)
    ptrs = (ctypes.c_void_p * len(weights))(*[w.data_ptr() for w in weights])
    h = ctypes.c_void_p()
    _check(lib().mt_encoder_create(ctypes.byref(cfg), ptrs, len(weights),
                                   ctypes.c_void_p(packed.data_ptr()), nbytes,
                                   _stream_ptr(stream), ctypes.byref(h)))
    return Encoder(h, cfg, packed)


def mt_encode_workspace_size(enc: Encoder, lens, window, layout=MT_PACKED, max_len=0) -> int:
    b = make_batch(lens, layout, max_len)
    n = ctypes.c_size_t()
    _check(lib().mt_encode_workspace_size(enc.handle, ctypes.byref(b), int(window),
                                          ctypes.byref(n)))
    return n.value


def mt_encode(enc: Encoder, mel, lens, window, layout=MT_PACKED, out=None, ws=None, stream=None):
    """mel: fp32 CUDA tensor [sum T, 128] (packed) or [B, max_len, 128] (padded).
    Returns fp32 [sum N, d] or [B, N(max_len), d]."""
    import torch
    assert mel.is_cuda and mel.dtype == torch.float32 and mel.is_contiguous()
    _check_input(mel, lens, layout, enc.cfg.n_mels, "mt_encode mel")
    max_len = mel.shape[1] if layout == MT_PADDED else 0
    d = enc.d_out
    fe = enc.cfg.frontend
    if layout == MT_PADDED:
        shape = (len(lens), mt_encoder_frames_for(fe, max_len), d)
    else:
        shape = (sum(mt_encoder_frames_for(fe, int(t)) for t in lens), d)
    b = make_batch(lens, layout, max_len)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=mel.device)
    _check_output(out, shape, "mt_encode out")
    if ws is None:
        nbytes = mt_encode_workspace_size(enc, lens, window, layout, max_len)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=mel.device)
    _check(lib().mt_encode(enc.handle, ctypes.c_void_p(mel.data_ptr()), ctypes.byref(b),
                           int(window), ctypes.c_void_p(out.data_ptr()),
                           ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream_ptr(stream)))
    return out


def mt_encode_stream_workspace_size(enc: Encoder, n_samples, window, chunk_windows) -> int:
    n = ctypes.c_size_t()
    _check(lib().mt_encode_stream_workspace_size(enc.handle if enc is not None else None,
                                                 int(n_samples), int(window), int(chunk_windows),
                                                 ctypes.byref(n)))
    return n.value


def mt_encode_stream(enc: Encoder, wav, window, chunk_windows, out=None, ws=None, stream=None):
    """wav: fp32 CUDA tensor [n] (one stream).  Encodes it chunk_windows
    windows at a time with a workspace that does not grow with the stream;
    returns fp32 [N, d], equal to mt_logmel + mt_encode over the whole stream."""
    import torch
    assert wav.is_cuda and wav.dtype == torch.float32 and wav.is_contiguous() and wav.dim() == 1
    n = wav.numel()
    N = mt_encoder_frames(mt_mel_frames(n))
    if out is None:
        out = torch.empty((N, enc.d_out), dtype=torch.float32, device=wav.device)
    if ws is None:
        nbytes = mt_encode_stream_workspace_size(enc, n, window, chunk_windows)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=wav.device)
    _check(lib().mt_encode_stream(enc.handle, ctypes.c_void_p(wav.data_ptr()), int(n), int(window),
                                  int(chunk_windows), ctypes.c_void_p(out.data_ptr()),
                                  ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream_ptr(stream)))
    return out


def mt_stream_state_bytes(enc: Encoder, window, max_push) -> int:
    n = ctypes.c_size_t()
    _check(lib().mt_stream_state_bytes(enc.handle if enc is not None else None, int(window), int(max_push),
                                       ctypes.byref(n)))
    return n.value


class LiveStream:
    """One live stream (mt_stream_open): push() appends audio and returns the
    frames of the windows it completed, finish() the rest.  The device state
    is a torch tensor owned by this object."""

    def __init__(self, enc: Encoder, window, max_push, stream=None):
        import torch
        self.enc = enc
        self.window = int(window)
        self.max_push = int(max_push)
        nbytes = mt_stream_state_bytes(enc, window, max_push)
        self.state = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        h = ctypes.c_void_p()
        _check(lib().mt_stream_open(enc.handle, self.window, self.max_push, ctypes.c_void_p(self.state.data_ptr()),
                                    nbytes, _stream_ptr(stream), ctypes.byref(h)))
        self.handle = h

    def pending_frames(self, n_more=0, finish=False) -> int:
        return lib().mt_stream_pending_frames(self.handle, int(n_more), 1 if finish else 0)

    def _out(self, n):
        import torch
        return torch.empty((max(n, 1), self.enc.d_out), dtype=torch.float32, device="cuda")

    def push(self, samples, out=None, stream=None):
        """samples: fp32 CUDA tensor [n]; returns fp32 [frames, d]."""
        import torch
        assert samples.is_cuda and samples.dtype == torch.float32 and samples.is_contiguous()
        n = samples.numel()
        want = self.pending_frames(n)
        if out is None:
            out = self._out(want)
        got = ctypes.c_int64()
        _check(lib().mt_stream_push(self.handle, ctypes.c_void_p(samples.data_ptr()), int(n),
                                    ctypes.c_void_p(out.data_ptr()), out.shape[0], ctypes.byref(got),
                                    _stream_ptr(stream)))
        return out[:got.value]

    def finish(self, out=None, stream=None):
        want = self.pending_frames(0, finish=True)
        if out is None:
            out = self._out(want)
        got = ctypes.c_int64()
        _check(lib().mt_stream_finish(self.handle, ctypes.c_void_p(out.data_ptr()), out.shape[0],
                                      ctypes.byref(got), _stream_ptr(stream)))
        return out[:got.value]

    def close(self):
        if self.handle:
            lib().mt_stream_close(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def mt_prompt_embed_workspace_size(n_tokens) -> int:
    n = ctypes.c_size_t()
    _check(lib().mt_prompt_embed_workspace_size(int(n_tokens), ctypes.byref(n)))
    return n.value


def mt_prompt_embed(tokens, table, audio, audio_token, out=None, ws=None, stream=None):
    """tokens: host int sequence [S]; table: CUDA tensor [vocab, d] (float32,
    bfloat16 or float16); audio: fp32 CUDA tensor [A, d] with A = the number of
    audio_token entries.  Returns fp32 [S, d]."""
    import torch
    dt = {torch.float32: MT_F32, torch.bfloat16: MT_BF16, torch.float16: MT_F16}[table.dtype]
    assert table.is_cuda and table.is_contiguous() and table.dim() == 2
    assert audio.is_cuda and audio.dtype == torch.float32 and audio.is_contiguous()
    toks = (ctypes.c_int32 * len(tokens))(*[int(t) for t in tokens])
    d = table.shape[1]
    if out is None:
        out = torch.empty((len(tokens), d), dtype=torch.float32, device=table.device)
    _check_output(out, (len(tokens), d), "mt_prompt_embed out")
    if audio.dim() != 2 or audio.shape[1] != d:
        raise ValueError(f"mt_prompt_embed: audio {tuple(audio.shape)} against a table of width {d}")
    if ws is None:
        ws = torch.empty(mt_prompt_embed_workspace_size(len(tokens)), dtype=torch.uint8,
                         device=table.device)
    _check(lib().mt_prompt_embed(toks, len(tokens), int(audio_token),
                                 ctypes.c_void_p(table.data_ptr()), dt, table.shape[0], d,
                                 ctypes.c_void_p(audio.data_ptr()), audio.shape[0],
                                 ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
                                 ws.numel(), _stream_ptr(stream)))
    return out


# ------------------------------------------------------------------ decoder


def decoder_config(geom: dict, dtype: int, rms_eps: float = 1e-6, rope_base: float = 1e6):
    return DecoderConfig(geom["vocab"], geom["d_model"], geom["n_layers"], geom["n_heads"],
                         geom["n_kv_heads"], geom["head_dim"], geom["d_ffn"], dtype, rms_eps, rope_base)


class Decoder:
    """A decoder whose packed weights live in a torch-owned device buffer."""

    def __init__(self, handle, cfg, packed):
        self.handle = handle
        self.cfg = cfg
        self.packed = packed

    def close(self):
        if self.handle:
            lib().mt_decoder_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def mt_decoder_n_weights(cfg: DecoderConfig) -> int:
    return lib().mt_decoder_n_weights(ctypes.byref(cfg))


def mt_decoder_packed_bytes(cfg: DecoderConfig) -> int:
    n = ctypes.c_size_t()
    _check(lib().mt_decoder_packed_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def mt_decoder_create(cfg: DecoderConfig, weights, device="cuda", stream=None) -> Decoder:
    """weights: fp32 CUDA tensors in the canonical order of include/mt.h."""
    import torch
    for w in weights:
        assert w.is_cuda and w.dtype == torch.float32 and w.is_contiguous()
    nbytes = mt_decoder_packed_bytes(cfg)
    packed = torch.empty(nbytes, dtype=torch.uint8, device=device)
    ptrs = (ctypes.c_void_p * len(weights))(*[w.data_ptr() for w in weights])
    h = ctypes.c_void_p()
    _check(lib().mt_decoder_create(ctypes.byref(cfg), ptrs, len(weights), ctypes.c_void_p(packed.data_ptr()),
                                   nbytes, _stream_ptr(stream), ctypes.byref(h)))
    return Decoder(h, cfg, packed)


def mt_decoder_embedding(dec: Decoder):
    """The packed [vocab, d_model] table as a torch view (bfloat16 / float16)."""
    import torch
    dt = torch.bfloat16 if dec.cfg.dtype == MT_BF16 else torch.float16
    ptr = lib().mt_decoder_embedding(dec.handle)
    off = ptr - dec.packed.data_ptr()
    n = dec.cfg.vocab * dec.cfg.d_model * 2
    return dec.packed[off:off + n].view(dt).view(dec.cfg.vocab, dec.cfg.d_model)


def mt_decoder_cache_bytes(dec: Decoder, max_seqs: int, max_pos: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().mt_decoder_cache_bytes(dec.handle, int(max_seqs), int(max_pos), ctypes.byref(n)))
    return n.value


def _i32(a):
    return (ctypes.c_int32 * len(a))(*[int(v) for v in a])


def mt_decode_workspace_size(dec: Decoder, seq, pos, max_seqs, max_pos) -> int:
    n = ctypes.c_size_t()
    _check(lib().mt_decode_workspace_size(dec.handle, len(seq), _i32(seq), _i32(pos), int(max_seqs),
                                          int(max_pos), ctypes.byref(n)))
    return n.value


def mt_decode(dec: Decoder, x, seq, pos, cache, max_seqs, max_pos, logits=None, next_ids=None, ws=None,
              stream=None):
    """x: fp32 CUDA tensor [n, d_model]; seq, pos: host int sequences [n];
    cache: CUDA byte tensor of mt_decoder_cache_bytes.  Returns (logits fp32
    [n, vocab], next int32 [n])."""
    import torch
    n = len(seq)
    assert x.is_cuda and x.dtype == torch.float32 and x.is_contiguous() and x.shape[0] == n
    if x.dim() != 2 or x.shape[1] != dec.cfg.d_model or len(pos) != n:
        raise ValueError(f"mt_decode: x {tuple(x.shape)} with {n} seq / {len(pos)} pos entries "
                         f"(expected [{n}, {dec.cfg.d_model}])")
    need = mt_decoder_cache_bytes(dec, max_seqs, max_pos)
    if cache.numel() * cache.element_size() < need:
        raise ValueError(f"mt_decode: cache of {cache.numel() * cache.element_size()} bytes, "
                         f"{max_seqs} x {max_pos} positions need {need}")
    if logits is None:
        logits = torch.empty((n, dec.cfg.vocab), dtype=torch.float32, device=x.device)
    if next_ids is None:
        next_ids = torch.empty(n, dtype=torch.int32, device=x.device)
    _check_output(logits, (n, dec.cfg.vocab), "mt_decode logits")
    _check_output(next_ids, (n,), "mt_decode next_ids")
    if ws is None:
        ws = torch.empty(max(mt_decode_workspace_size(dec, seq, pos, max_seqs, max_pos), 1), dtype=torch.uint8,
                         device=x.device)
    _check(lib().mt_decode(dec.handle, ctypes.c_void_p(x.data_ptr()), n, _i32(seq), _i32(pos),
                           ctypes.c_void_p(cache.data_ptr()), int(max_seqs), int(max_pos),
                           ctypes.c_void_p(logits.data_ptr()), ctypes.c_void_p(next_ids.data_ptr()),
                           ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream_ptr(stream)))
    return logits, next_ids


def mt_trace_arm(stage, max_launches=4096):
    """Time every launch of one named stage with HIP events (None disarms)."""
    _check(lib().mt_trace_arm(stage.encode() if stage else None, int(max_launches)))


def mt_trace_collect():
    """(total_ms, launches) of the armed stage since the last collect."""
    t = ctypes.c_double()
    n = ctypes.c_int32()
    _check(lib().mt_trace_collect(ctypes.byref(t), ctypes.byref(n)))
    return t.value, n.value
