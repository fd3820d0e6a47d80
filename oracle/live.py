"""Live (incremental) encoding of one long stream, float64.  TEST INFRASTRUCTURE
ONLY.

Source: model card "MOSS-Transcribe-preview-2B-GGUF", Architecture table,
rows "Audio" (the log-mel front-end with the clamp at the clip's maximum minus
8) and "Audio encoder" (windowed, block-diagonal attention: encoder frames of
different windows never attend to each other, so beyond the convolutions'
receptive field a window depends only on its own audio).

Reading (the pages are silent on how the clip maximum of the log clamp is
found when the audio of one stream arrives piece by piece): a causal running
maximum.  Window k (encoder frames [kW, (k+1)W)) depends on mel frames
0 .. e_k - 1 with e_k = min(T, 8 (k+1) W) -- its last frame's receptive field
ends at mel frame 8 (k+1) W - 1 -- and its log-mel is clamped at

    g_k = max of the unclamped log-mel over mel frames [0, e_k)

minus 8, then (x + 4) / 4, as for a whole clip.  So g_k never decreases, the
last window uses the maximum of the whole stream, and every window from the
one whose range first contains the stream's loudest frame onwards equals the
whole-stream encoding.  The result does not depend on how the audio was split
into pushes.

Window k is then encoded from its receptive field, mel frames
[max(0, 8 (kW - 1)), e_k): a start on a multiple of 8 keeps the stride-2
convolutions aligned with the stream's, and the one encoder frame before kW
that this segment yields is dropped; positions count from the stream's start.
"""

from __future__ import annotations

import math

import numpy as np

from . import encoder as E
from . import logmel as LM


def raw_log_mel(wav: np.ndarray, n_mels: int = 128) -> np.ndarray:
    """log10(max(mel energy, 1e-10)) of every frame, before the clamp, [T, n_mels]."""
    En = LM.power_spectrum(wav) @ LM.mel_filterbank(n_mels).T
    return np.log10(np.maximum(En, 1e-10))


def window_end(k: int, window: int, T: int) -> int:
    """Exclusive end e_k of the mel frames window k depends on."""
    return min(T, 8 * (k + 1) * window)


def running_max(L: np.ndarray, k: int, window: int) -> float:
    """g_k: the largest unclamped log-mel value over mel frames [0, e_k)."""
    return float(L[:window_end(k, window, L.shape[0])].max())


def window_mel(L: np.ndarray, k: int, window: int):
    """(normalised mel of window k's receptive-field segment, its first mel frame)."""
    T = L.shape[0]
    e = window_end(k, window, T)
    s = max(0, 8 * (k * window - 1))
    g = running_max(L, k, window)
    return (np.maximum(L[s:e], g - 8.0) + 4.0) / 4.0, s


def encode_live(wav: np.ndarray, P: dict, geom: dict, window: int, windows=None, L=None) -> dict:
    """Encoder output of the windows of a live stream: {k: rows of window k}.
    windows: the window indices to compute (default: all)."""
    if L is None:
        L = raw_log_mel(wav, geom["n_mels"])
    T = L.shape[0]
    N = E.encoder_frames(T)
    n_win = math.ceil(N / window)
    out = {}
    for k in (range(n_win) if windows is None else windows):
        mel, s = window_mel(L, k, window)
        y = E.encode_clip(mel, P, geom, window, t0=s // 8)
        r0 = k * window - s // 8
        n = min(window, N - k * window)
        out[k] = y[r0:r0 + n]
    return out
