"""Full-attention encoder with a 2x time-downsampling front-end, float64.
TEST INFRASTRUCTURE ONLY.

Source: page "CrisperWhisper -> ONNX (with cross-attentions)":
  * section "What this exports instead": plain whisper-small geometry, 12
    encoder layers at d_model 768;
  * section "Results": the decoder's cross-attention spans 12 heads and 1500
    encoder frames for one 30 s window, i.e. 3000 log-mel frames reduced 2x
    in time, every encoder frame visible to every query (full attention);
  * opening paragraphs: large-v3's encoder has 32 layers and 2.5 GB of fp32
    weights (the 32 x 1280 geometry of the model card's tower).

Readings where the page is silent (each pinned by tests/test_oracle_encoder2x.py):
  * front-end: two 1-D convolutions over time with kernel 3 and padding 1
    (zero outside the clip); the log-mel bins are the first one's input
    channels; the first has stride 1 (n_mels -> d), the second stride 2
    (d -> d); biases present, GELU after each; a clip of T mel frames gives
    N = ceil(T / 2) encoder frames;
  * positions, pre-LN layers, LayerNorm, GELU, softmax scale: those of
    oracle.encoder (model card "MOSS-Transcribe-preview-2B-GGUF", Architecture
    table), the sinusoids added after the second convolution's GELU;
  * attention over the whole clip (a window of at least N frames; a smaller
    window is accepted and means block-diagonal attention as in oracle.encoder);
  * output: ln_post of the residual stream (with_head), else the stream itself;
  * n_mels = 128, the log-mel of oracle.logmel.
"""

from __future__ import annotations

import numpy as np

from .encoder import gelu, layer, layer_norm, sinusoids


def frames_2x(mel_frames: int) -> int:
    """Encoder frames of a clip of T >= 1 mel frames: ceil(T / 2)."""
    return (mel_frames - 1) // 2 + 1


def conv1d_k3(x, w, b, stride: int):
    """Cross-correlation over time with kernel 3, padding 1 (zeros).

    x [T, Cin], w [Cout, Cin, 3] (tap d multiplies input frame s*t + d - 1),
    b [Cout] -> [(T - 1) // s + 1, Cout].
    """
    T, Cin = x.shape
    n = (T - 1) // stride + 1
    xp = np.zeros((T + 2, Cin), dtype=np.float64)
    xp[1:T + 1] = x
    out = np.broadcast_to(np.asarray(b, dtype=np.float64), (n, w.shape[0])).copy()
    for d in range(3):
        rows = xp[d:d + stride * (n - 1) + 1:stride]  # input frames s*t + d - 1
        out += rows @ w[:, :, d].T
    return out


def front_end_2x(mel, P):
    """[T, n_mels] -> [ceil(T / 2), d]: conv (s1) -> GELU -> conv (s2) -> GELU,
    then the sinusoids."""
    h = gelu(conv1d_k3(mel, P["conv1.weight"], P["conv1.bias"], 1))
    x = gelu(conv1d_k3(h, P["conv2.weight"], P["conv2.bias"], 2))
    return x + sinusoids(x.shape[0], x.shape[1])


def encode_clip_2x(mel, P, geom: dict, window=None, n_layers=None, with_head: bool = True):
    """One clip's log-mel [T, n_mels] -> [ceil(T / 2), d_model].

    window     None: the whole clip (full attention)
    n_layers   run only the first n layers (default: all of geom["n_layers"])
    with_head  False stops after the tower, giving the residual stream
    """
    L = geom["n_layers"] if n_layers is None else n_layers
    x = front_end_2x(mel, P)
    W = x.shape[0] if window is None else window
    for l in range(L):
        x = layer(x, P, l, geom["n_heads"], W)
    if not with_head:
        return x
    return layer_norm(x, P["ln_post.weight"], P["ln_post.bias"])


def encode_2x(mels: list, P, geom: dict, window=None, **kw) -> list:
    """Clips are independent: a batch is the list of per-clip outputs."""
    return [encode_clip_2x(m, P, geom, window, **kw) for m in mels]
