"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every entry point include/mt.h declares, and
reject bad arguments on the host before any launch.  The length functions are
checked against the closed forms, and the build's log-mel tables against the
oracle's filterbank.
"""

import ctypes
import math
import os
import re

import numpy as np
import pytest

import synth
import windowed_attention_audio_amd as W
from oracle import encoder as OE
from oracle import logmel as OL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    # the in-tree library is what these checks are about: build it if this
    # checkout has not (hipcc cross-compiles gfx950 without a GPU)
    if not os.path.exists(W.LIB_PATH):
        from windowed_attention_audio_amd import build as B
        B.build()
    return W.lib()


def test_c_abi_under_sanitizers():
    # api.cpp built with g++ -fsanitize=address,undefined against stub
    # launchers that touch the ends of every range a kernel would access; the
    # driver calls every rejection path of every entry point and valid calls
    # on exactly sized buffers (tests/host_abi_check.cpp)
    import subprocess
    from windowed_attention_audio_amd import build as B
    exe = B.build_host_check()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-6000:]
    last = r.stdout.strip().splitlines()[-1]
    assert last.startswith("host_abi_check:") and last.endswith("checks passed"), last
    assert int(last.split()[1]) >= 250


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "mt.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mt_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_symbols()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), f"libmt.so does not export {n}"
    assert set(names) == set(W.EXPORTS)


@pytest.mark.parametrize("n", [0, 159, 160, 16000, 16077, 480000, 9600000])
def test_mel_frames(L, n):
    assert W.mt_mel_frames(n) == n // 160 == OL.frame_count(n)


@pytest.mark.parametrize("T", [0, 1, 2, 7, 8, 9, 100, 3000, 60000, 60001])
def test_encoder_frames(L, T):
    c = lambda x: -(-x // 2)
    assert W.mt_encoder_frames(T) == c(c(c(T))) == OE.encoder_frames(T) if T else True
    assert W.mt_encoder_frames(T) == math.ceil(math.ceil(math.ceil(T / 2) / 2) / 2)


def test_negative_lengths(L):
    assert W.mt_mel_frames(-1) == -1 and W.mt_encoder_frames(-5) == -1


def test_logmel_workspace_and_rejections(L):
    assert W.mt_logmel_workspace_size([16000]) > 0
    assert W.mt_logmel_workspace_size([16000] * 64) > W.mt_logmel_workspace_size([16000])
    for bad in ([200], [201, 100], [-5]):
        with pytest.raises(W.MtError) as e:
            W.mt_logmel_workspace_size(bad)
        assert e.value.status == W.MT_ERR_INVALID_ARG
    with pytest.raises(W.MtError) as e:  # padded: length above the row stride
        W.mt_logmel_workspace_size([3000, 5000], layout=W.MT_PADDED, max_len=4000)
    assert e.value.status == W.MT_ERR_INVALID_ARG
    b = W.make_batch([16000], layout=7)
    n = ctypes.c_size_t()
    assert L.mt_logmel_workspace_size(ctypes.byref(b), ctypes.byref(n)) == W.MT_ERR_INVALID_ARG
    b = W.Batch(0, 0, None, 0)
    assert L.mt_logmel_workspace_size(ctypes.byref(b), ctypes.byref(n)) == W.MT_ERR_INVALID_ARG
    b = W.Batch(0, 2, None, 0)
    assert L.mt_logmel_workspace_size(ctypes.byref(b), ctypes.byref(n)) == W.MT_ERR_INVALID_ARG
    assert b"len is NULL" in L.mt_last_error()
    # null device pointers are rejected before anything is launched
    b = W.make_batch([16000])
    assert L.mt_logmel(None, ctypes.byref(b), None, None, 0, None) == W.MT_ERR_INVALID_ARG


def test_config_validation(L):
    ok = W.encoder_config(synth.FULL_GEOM, W.MT_BF16)
    assert W.mt_encoder_n_weights(ok) == 7 + 16 * 32 + 6
    ad = W.encoder_config(dict(synth.FULL_GEOM, adapter_hidden=8192), W.MT_BF16)
    assert W.mt_encoder_n_weights(ad) == 7 + 16 * 32 + 6 + 3
    assert W.mt_encoder_n_weights(ad) == len(synth.weight_names(dict(synth.FULL_GEOM,
                                                                     adapter_hidden=8192)))
    for over, status in ((dict(n_mels=80), W.MT_ERR_UNSUPPORTED),
                         (dict(head_dim=128, n_heads=10), W.MT_ERR_UNSUPPORTED),
                         (dict(n_heads=19), W.MT_ERR_UNSUPPORTED),
                         (dict(conv_ch=100), W.MT_ERR_UNSUPPORTED),
                         (dict(d_ffn=0), W.MT_ERR_INVALID_ARG),
                         (dict(n_layers=-1), W.MT_ERR_INVALID_ARG)):
        cfg = W.encoder_config(dict(synth.FULL_GEOM, **over), W.MT_BF16)
        with pytest.raises(W.MtError) as e:
            W.mt_encoder_packed_bytes(cfg)
        assert e.value.status == status, over
    bad = W.encoder_config(synth.FULL_GEOM, 7)
    with pytest.raises(W.MtError):
        W.mt_encoder_packed_bytes(bad)


def test_packed_bytes(L):
    geom = synth.FULL_GEOM
    names = synth.weight_names(geom)
    n_params = sum(int(np.prod(s)) for _, s in names)
    # vectors and conv1's 9 taps stay fp32; matrices become bf16
    n_vec = sum(int(np.prod(s)) for n, s in names if len(s) == 1 or n == "conv1.weight")
    f32 = W.mt_encoder_packed_bytes(W.encoder_config(geom, W.MT_F32))
    b16 = W.mt_encoder_packed_bytes(W.encoder_config(geom, W.MT_BF16))
    assert abs(n_params - 647.9e6) < 0.1e6  # encoder parameters, about 648 M
    pad = 256 * len(names)
    assert 4 * n_params <= f32 <= 4 * n_params + pad
    # the head's two matrices are stored twice for the hi/lo-split activations
    head = 1280 * 1280 + 2048 * 1280
    expect = 2 * (n_params - n_vec + head) + 4 * n_vec
    assert expect <= b16 <= expect + pad


def test_create_rejects_before_launch(L):
    cfg = W.encoder_config(dict(synth.FULL_GEOM, n_layers=1), W.MT_BF16)
    n = W.mt_encoder_n_weights(cfg)
    ptrs = (ctypes.c_void_p * n)(*([1] * n))
    h = ctypes.c_void_p()
    assert L.mt_encoder_create(ctypes.byref(cfg), ptrs, n - 1, ctypes.c_void_p(256), 1 << 40,
                               None, ctypes.byref(h)) == W.MT_ERR_INVALID_ARG
    ptrs[3] = None
    assert L.mt_encoder_create(ctypes.byref(cfg), ptrs, n, ctypes.c_void_p(256), 1 << 40,
                               None, ctypes.byref(h)) == W.MT_ERR_INVALID_ARG
    ptrs[3] = 1
    assert L.mt_encoder_create(ctypes.byref(cfg), ptrs, n, ctypes.c_void_p(256), 16,
                               None, ctypes.byref(h)) == W.MT_ERR_WORKSPACE
    assert L.mt_encoder_create(ctypes.byref(cfg), ptrs, n, ctypes.c_void_p(100), 1 << 40,
                               None, ctypes.byref(h)) == W.MT_ERR_INVALID_ARG
    assert not h.value


def test_encode_rejects_null_encoder(L):
    b = W.make_batch([3000])
    n = ctypes.c_size_t()
    assert L.mt_encode_workspace_size(None, ctypes.byref(b), 104, ctypes.byref(n)) == \
        W.MT_ERR_INVALID_ARG
    assert L.mt_encode(None, None, ctypes.byref(b), 104, None, None, 0, None) == \
        W.MT_ERR_INVALID_ARG


def test_status_strings_and_trace(L):
    for s in range(5):
        assert L.mt_status_string(s).startswith(b"MT_")
    W.mt_trace_arm(None)
    assert W.mt_trace_collect() == (0.0, 0)
    assert W.mt_max_window() == 256


def test_library_tables_match_oracle_filterbank():
    from windowed_attention_audio_amd import gen_tables as G
    rows = G.filterbank()
    F = np.zeros((128, 201))
    for m, (first, w) in enumerate(rows):
        F[m, first:first + len(w)] = w
    assert np.max(np.abs(F - OL.mel_filterbank())) < 1e-12


def test_encode_stream_rejects_null_encoder(L):
    import ctypes as C
    n = C.c_size_t()
    assert L.mt_encode_stream_workspace_size(None, 16000, 104, 1, C.byref(n)) == W.MT_ERR_INVALID_ARG
    assert L.mt_encode_stream(None, None, 16000, 104, 1, None, None, 0, None) == W.MT_ERR_INVALID_ARG


def test_prompt_embed_rejects_before_launch(L):
    import ctypes as C
    n = C.c_size_t()
    assert L.mt_prompt_embed_workspace_size(0, C.byref(n)) == W.MT_ERR_INVALID_ARG
    assert L.mt_prompt_embed_workspace_size(10, C.byref(n)) == W.MT_OK and n.value >= 80

    def call(toks, dtype=W.MT_F16, d=8, n_audio=1, vocab=10):
        arr = (C.c_int32 * len(toks))(*toks)
        p = C.c_void_p(256)  # never dereferenced: validation fails first
        return L.mt_prompt_embed(arr, len(toks), 9, p, dtype, vocab, d, p, n_audio, p, p, 1 << 20, None)

    assert call([1, 9, 9]) == W.MT_ERR_INVALID_ARG          # 2 placeholders, 1 frame
    assert call([1, 11, 9]) == W.MT_ERR_INVALID_ARG         # id outside the vocabulary
    assert call([1, 9], dtype=7) == W.MT_ERR_INVALID_ARG    # unknown table type
    assert call([1, 9], d=6) == W.MT_ERR_INVALID_ARG        # d not a multiple of 4


@pytest.mark.parametrize("T", [0, 1, 2, 3, 3000, 3001])
def test_encoder_frames_for(L, T):
    from oracle import encoder2x as OE2
    assert W.mt_encoder_frames_for(W.MT_FRONTEND_CONV2D_8X, T) == W.mt_encoder_frames(T)
    want = OE2.frames_2x(T) if T else 0
    assert W.mt_encoder_frames_for(W.MT_FRONTEND_CONV1D_2X, T) == want == -(-T // 2)
    assert W.mt_encoder_frames_for(W.MT_FRONTEND_CONV1D_2X, -1) == -1
    assert W.mt_encoder_frames_for(5, T) == -1


def test_config_validation_2x(L):
    for geom in (synth.WHISPER_SMALL_GEOM, synth.WHISPER_LARGE_GEOM):
        cfg = W.encoder_config(geom, W.MT_F16)
        assert W.mt_encoder_n_weights(cfg) == 4 + 16 * geom["n_layers"] + 2 == \
            len(synth.weight_names(geom))
        # conv_ch is ignored by this front-end
        assert W.mt_encoder_packed_bytes(W.encoder_config(dict(geom, conv_ch=1), W.MT_F16)) == \
            W.mt_encoder_packed_bytes(cfg)
    for over, dt, status in ((dict(), W.MT_F32, W.MT_ERR_UNSUPPORTED),
                             (dict(adapter_hidden=1024), W.MT_BF16, W.MT_ERR_INVALID_ARG),
                             (dict(d_out=2048), W.MT_BF16, W.MT_ERR_INVALID_ARG)):
        cfg = W.encoder_config(dict(synth.WHISPER_SMALL_GEOM, **over), dt)
        with pytest.raises(W.MtError) as e:
            W.mt_encoder_packed_bytes(cfg)
        assert e.value.status == status, over
    cfg = W.encoder_config(synth.WHISPER_SMALL_GEOM, W.MT_BF16)
    cfg.frontend = 9
    with pytest.raises(W.MtError) as e:
        W.mt_encoder_packed_bytes(cfg)
    assert e.value.status == W.MT_ERR_INVALID_ARG


def test_packed_bytes_2x(L):
    geom = synth.WHISPER_SMALL_GEOM
    names = synth.weight_names(geom)
    n_mat = sum(int(np.prod(s)) for _, s in names if len(s) > 1)
    n_vec = sum(int(np.prod(s)) for _, s in names if len(s) == 1)
    b16 = W.mt_encoder_packed_bytes(W.encoder_config(geom, W.MT_BF16))
    expect = 2 * n_mat + 4 * n_vec
    assert expect <= b16 <= expect + 256 * (len(names) + 1)


def test_decoder_config_validation(L):
    cfg = W.decoder_config(synth.DEC_GEOM, W.MT_BF16)
    assert W.mt_decoder_n_weights(cfg) == 1 + 11 * 28 + 1 == len(synth.decoder_weight_names(synth.DEC_GEOM))
    names = synth.decoder_weight_names(synth.DEC_GEOM)
    n_mat = sum(int(np.prod(s)) for _, s in names if len(s) > 1)
    n_vec = sum(int(np.prod(s)) for _, s in names if len(s) == 1)
    b = W.mt_decoder_packed_bytes(cfg)
    assert 2 * n_mat + 4 * n_vec <= b <= 2 * n_mat + 4 * n_vec + 256 * (len(names) + 1)
    for over, dt, status in ((dict(), W.MT_F32, W.MT_ERR_UNSUPPORTED),
                             (dict(head_dim=64), W.MT_BF16, W.MT_ERR_UNSUPPORTED),
                             (dict(n_kv_heads=4), W.MT_BF16, W.MT_ERR_UNSUPPORTED),
                             (dict(d_model=1000), W.MT_BF16, W.MT_ERR_UNSUPPORTED),
                             (dict(d_ffn=0), W.MT_BF16, W.MT_ERR_INVALID_ARG)):
        c = W.decoder_config(dict(synth.DEC_GEOM, **over), dt)
        with pytest.raises(W.MtError) as e:
            W.mt_decoder_packed_bytes(c)
        assert e.value.status == status, over
    assert W.mt_decoder_n_weights(W.decoder_config(synth.DEC_GEOM, W.MT_F32)) == -1


def test_decode_rejects_null_decoder(L):
    n = ctypes.c_size_t()
    seq = (ctypes.c_int32 * 1)(0)
    pos = (ctypes.c_int32 * 1)(0)
    assert L.mt_decode_workspace_size(None, 1, seq, pos, 1, 8, ctypes.byref(n)) == W.MT_ERR_INVALID_ARG
    assert L.mt_decode(None, None, 1, seq, pos, None, 1, 8, None, None, None, 0, None) == W.MT_ERR_INVALID_ARG
    assert L.mt_decoder_embedding(None) is None


def test_with_adapter_equals_full_draw():
    # the bench's variable-length workload adds the adapter to the main
    # workload's weights; the result must be the full seeded draw
    g0 = dict(synth.FULL_GEOM, n_layers=1, conv_ch=32, d_model=64, n_heads=1, d_ffn=128, d_out=64,
              adapter_hidden=0)
    g1 = dict(g0, adapter_hidden=128)
    full = synth.make_weights(g1, bf16=True)
    built = synth.with_adapter(synth.make_weights(g0, bf16=True), g1, bf16=True)
    assert list(full) == list(built)
    assert any(k.startswith("adapter.") for k in full)
    for k in full:
        assert np.array_equal(full[k], built[k]), k


def test_binding_rejects_inputs_shorter_than_the_lengths():
    # The C ABI takes raw device pointers: a tensor smaller than its host
    # lengths say would be read past its end.  The binding compares shapes
    # with the lengths first and raises (no device needed: shape-only
    # stand-ins).
    class Shape:
        def __init__(self, *shape):
            self.shape = shape

        def dim(self):
            return len(self.shape)

        def numel(self):
            n = 1
            for x in self.shape:
                n *= x
            return n

    chk = W._check_input
    chk(Shape(48000, 128), [3000] * 16, W.MT_PACKED, 128, "mel")          # exact
    chk(Shape(48001, 128), [3000] * 16, W.MT_PACKED, 128, "mel")          # larger buffer: fine
    chk(Shape(16, 3000, 128), [3000] * 16, W.MT_PADDED, 128, "mel")
    chk(Shape(16 * 480000), [480000] * 16, W.MT_PACKED, 0, "wav")
    for t, lens, layout, width in [
            (Shape(48000, 128), [128] * 48000, W.MT_PACKED, 128),  # rows read as sequences
            (Shape(47999, 128), [3000] * 16, W.MT_PACKED, 128),
            (Shape(48000, 80), [3000] * 16, W.MT_PACKED, 128),
            (Shape(16, 2999, 128), [3000] * 16, W.MT_PADDED, 128),
            (Shape(15, 3000, 128), [3000] * 16, W.MT_PADDED, 128),
            (Shape(100), [200], W.MT_PACKED, 0)]:
        with pytest.raises(ValueError):
            chk(t, lens, layout, width, "x")
    W._check_output(Shape(6000, 2048), (6000, 2048), "out")
    with pytest.raises(ValueError):
        W._check_output(Shape(5999, 2048), (6000, 2048), "out")
