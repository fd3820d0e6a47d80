"""Pins for the live-stream oracle (CPU only).

oracle.live reads the clip maximum of a stream that arrives piece by piece as
a causal running maximum.  These tests tie it to the whole-clip definition
(oracle.logmel + oracle.encoder, pinned in their own tests), not to itself:

  * window k of the live stream equals the whole-clip encoding of the stream
    prefix that window k's receptive field needs (the first
    1280 (k+1) W + 40 samples: that prefix's own maximum is g_k, and none of
    its frames up to 8 (k+1) W - 1 reaches its end), rows [kW, (k+1)W);
  * the last window equals the whole-stream encoding;
  * when the stream's loudest frame lies in window 0's range, every window
    equals the whole-stream encoding;
  * g_k is non-decreasing and ends at the stream's maximum; a burst that comes
    later changes only the windows from its own on.
"""

import math

import numpy as np

import synth
from oracle import encoder as E
from oracle import live as LV
from oracle import logmel as LM

GEOM = dict(n_mels=128, conv_ch=4, d_model=16, n_layers=2, n_heads=2, head_dim=8, d_ffn=32, d_out=12,
            adapter_hidden=0)
W = 13  # encoder frames per window: 104 mel frames, 16640 samples


def weights():
    return E.as_f64(synth.make_weights(GEOM, bf16=False, seed=9, ln_random=True))


def stream(n, burst_at=None, seed=3):
    rng = np.random.default_rng(seed)
    t = np.arange(n) / 16000.0
    x = 0.2 * np.sin(2 * np.pi * 440 * t) + 0.05 * rng.standard_normal(n)
    x[int(0.3 * n):int(0.35 * n)] = 0.0  # a silent stretch
    if burst_at is not None:
        x[burst_at:burst_at + 3000] += 0.9 * np.sin(2 * np.pi * 1200 * t[burst_at:burst_at + 3000])
    return x.astype(np.float32)


def whole(wav, P):
    return E.encode_clip(LM.log_mel(wav), P, GEOM, W)


def test_live_window_equals_whole_clip_of_its_prefix():
    P = weights()
    wav = stream(16000 * 5 + 77, burst_at=16000 * 3)
    T = LM.frame_count(len(wav))
    N = E.encoder_frames(T)
    n_win = math.ceil(N / W)
    live = LV.encode_live(wav, P, GEOM, W)
    assert sorted(live) == list(range(n_win))
    for k in range(n_win - 1):  # full windows
        prefix = wav[:1280 * (k + 1) * W + 40]
        assert LM.frame_count(len(prefix)) == 8 * (k + 1) * W
        ref = whole(prefix, P)[k * W:(k + 1) * W]
        np.testing.assert_allclose(live[k], ref, rtol=1e-9, atol=1e-9 * np.abs(ref).max())
    ref = whole(wav, P)
    np.testing.assert_allclose(live[n_win - 1], ref[(n_win - 1) * W:], rtol=1e-9, atol=1e-9 * np.abs(ref).max())


def test_live_equals_whole_stream_when_loudest_frame_is_first():
    P = weights()
    wav = stream(16000 * 4 + 1234, burst_at=2000)
    L = LV.raw_log_mel(wav)
    assert L[:8 * W].max() == L.max()
    live = LV.encode_live(wav, P, GEOM, W)
    ref = whole(wav, P)
    got = np.concatenate([live[k] for k in sorted(live)])
    assert got.shape == ref.shape
    np.testing.assert_allclose(got, ref, rtol=1e-9, atol=1e-9 * np.abs(ref).max())


def test_running_max_monotone_and_late_burst_changes_only_later_windows():
    P = weights()
    burst = 16000 * 3
    wav = stream(16000 * 5, burst_at=burst)
    L = LV.raw_log_mel(wav)
    T = L.shape[0]
    N = E.encoder_frames(T)
    n_win = math.ceil(N / W)
    g = [LV.running_max(L, k, W) for k in range(n_win)]
    assert all(b >= a for a, b in zip(g, g[1:]))
    assert g[-1] == L.max()
    # brute force of the definition: the maximum over frames [0, min(T, 8 (k+1) W))
    for k in range(n_win):
        assert g[k] == max(L[t, m] for t in range(min(T, 8 * (k + 1) * W)) for m in range(128))
    kb = (burst // 160 + 2) // (8 * W)  # the burst's frames begin in window kb's range
    assert g[kb - 1] < g[kb] - 0.5
    live = LV.encode_live(wav, P, GEOM, W)
    ref = whole(wav, P)
    for k in range(n_win):
        r = ref[k * W:(k + 1) * W]
        same = np.allclose(live[k], r, rtol=1e-9, atol=1e-9 * np.abs(ref).max())
        # before the burst the floor g_k - 8 is lower than the stream's: some
        # entries differ; from the burst's window on, g_k is the stream maximum
        assert same == (g[k] == g[-1]), k
