"""Whisper-style log-mel front-end, float64.  TEST INFRASTRUCTURE ONLY.

Source: model card "MOSS-Transcribe-preview-2B-GGUF", Architecture table, row
"Audio" (16 kHz mono, 128 mel bins, n_fft 400, hop 160, matching Whisper's
feature extractor) and the gotcha on the trailing STFT frame (Whisper drops
the last frame, so a clip of n samples gives exactly n/hop frames).

Readings where the page is silent (each pinned by a test):
  * window: periodic Hann of length 400 (denominator 400);
  * framing: centred frames, the signal reflect-padded by n_fft/2 = 200 on
    both sides (mirror excludes the edge sample); frame t covers padded
    samples [160 t, 160 t + 400); T = floor(n / 160) frames are kept;
  * mel scale: Slaney (linear below 1 kHz, logarithmic above), 128 triangles
    spread evenly in mel between 0 Hz and 8 kHz, each scaled by 2/(bandwidth in
    Hz) (Slaney area normalisation), over the 201 linear bins at 40 Hz spacing;
  * log floor 1e-10; the clamp "max - 8" uses the maximum over this clip's
    own frames; then (x + 4) / 4.
"""

from __future__ import annotations

import numpy as np

SR = 16000
N_FFT = 400
HOP = 160
N_BINS = N_FFT // 2 + 1  # 201
PAD = N_FFT // 2  # 200


def frame_count(n_samples: int) -> int:
    """Mel frames for n samples: the trailing STFT frame is dropped, leaving
    exactly floor(n / hop)."""
    return int(n_samples) // HOP


def hann_periodic(n: int = N_FFT) -> np.ndarray:
    j = np.arange(n, dtype=np.float64)
    return 0.5 - 0.5 * np.cos(2.0 * np.pi * j / n)


def frames(wav: np.ndarray) -> np.ndarray:
    """Windowed frames [T, 400] of a clip (float64)."""
    x = np.asarray(wav, dtype=np.float64)
    n = x.shape[0]
    if n <= PAD:
        raise ValueError("reflect padding of 200 needs more than 200 samples")
    xp = np.pad(x, (PAD, PAD), mode="reflect")
    T = frame_count(n)
    idx = HOP * np.arange(T)[:, None] + np.arange(N_FFT)[None, :]
    return xp[idx] * hann_periodic()[None, :]


def power_spectrum(wav: np.ndarray) -> np.ndarray:
    """|DFT_400(frame)|^2 for bins 0..200, shape [T, 201]."""
    X = np.fft.rfft(frames(wav), n=N_FFT, axis=-1)
    return X.real ** 2 + X.imag ** 2


def hz_to_mel(f):
    """Slaney mel scale: 3 f / 200 below 1 kHz, logarithmic above."""
    f = np.asarray(f, dtype=np.float64)
    lin = 3.0 * f / 200.0
    log = 15.0 + 27.0 * np.log(np.maximum(f, 1e-300) / 1000.0) / np.log(6.4)
    return np.where(f < 1000.0, lin, log)


def mel_to_hz(m):
    m = np.asarray(m, dtype=np.float64)
    lin = 200.0 * m / 3.0
    log = 1000.0 * np.exp((m - 15.0) * np.log(6.4) / 27.0)
    return np.where(m < 15.0, lin, log)


def mel_filterbank(n_mels: int = 128, fmin: float = 0.0, fmax: float = 8000.0) -> np.ndarray:
    """Triangular Slaney filters, area-normalised, shape [n_mels, 201]."""
    fk = np.arange(N_BINS, dtype=np.float64) * SR / N_FFT
    h = mel_to_hz(np.linspace(hz_to_mel(fmin), hz_to_mel(fmax), n_mels + 2))
    F = np.zeros((n_mels, N_BINS), dtype=np.float64)
    for m in range(n_mels):
        lo, ce, hi = h[m], h[m + 1], h[m + 2]
        up = (fk - lo) / (ce - lo)
        down = (hi - fk) / (hi - ce)
        F[m] = np.maximum(0.0, np.minimum(up, down)) * (2.0 / (hi - lo))
    return F


def log_mel(wav: np.ndarray, n_mels: int = 128) -> np.ndarray:
    """Normalised log-mel of one clip, frame-major [T, n_mels], float64."""
    E = power_spectrum(wav) @ mel_filterbank(n_mels).T
    L = np.log10(np.maximum(E, 1e-10))
    g = L.max()
    L = np.maximum(L, g - 8.0)
    return (L + 4.0) / 4.0


def log_mel_batch(wavs: list, n_mels: int = 128) -> list:
    """Each clip is independent; the clamp uses each clip's own maximum."""
    return [log_mel(w, n_mels) for w in wavs]
