"""Audio encoder forward pass, float64.  TEST INFRASTRUCTURE ONLY.

Source: model card "MOSS-Transcribe-preview-2B-GGUF", Architecture table:
  * "Conv front-end": three 3x3 stride-2 Conv2D (1 -> 480 -> 480 -> 480), then
    conv_out, a bias-free Linear 480*16 = 7680 -> 1280, then sinusoidal
    positions are added;
  * "Audio encoder": 32 pre-LN Transformer layers, d = 1280, 20 heads of 64,
    FFN 5120, windowed (block-diagonal) self-attention;
  * "Encoder head": ln_post -> proj1 (1280 -> 1280) -> GELU -> proj2
    (1280 -> 2048);
  * "Adapter": gated MLP (SwiGLU) 2048 -> 8192 -> 2048.

Readings where the page is silent (each pinned by a test under tests/):
  * conv: padding 1, GELU after each conv, conv biases present; the mel image
    has height = mel bin (128) and width = time, one input channel; zero
    outside the clip; heights 128 -> 64 -> 32 -> 16, widths T -> ceil(T/2)
    -> ceil(T/4) -> ceil(T/8);
  * flatten: feature index c*16 + f (channel-major) for conv_out's input;
  * positions: [sin | cos] halves, timescale_j = 10000^(-j/639) for
    j = 0..639, position t counted from the clip's first encoder frame;
  * layers: LayerNorm eps 1e-5 with biased variance, all q/k/v/o/fc Linears
    with bias, softmax scale 1/sqrt(64), exact erf GELU;
  * windows: encoder frames [kW, min((k+1)W, N)) of each clip form window k,
    identical in every layer; clips never share a window;
  * head Linears with bias; adapter Linears without bias:
    down(SiLU(gate(y)) * up(y)).
"""

from __future__ import annotations

import math

import numpy as np
from scipy.special import erf

LN_EPS = 1e-5


def gelu(x):
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def silu(x):
    return x / (1.0 + np.exp(-x))


def layer_norm(x, g, b, eps: float = LN_EPS):
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * g + b


def linear(x, w, b=None):
    y = x @ w.T
    if b is not None:
        y = y + b
    return y


def conv_len(n: int) -> int:
    """Output length of a 3-tap, stride-2, padding-1 convolution."""
    return (int(n) - 1) // 2 + 1


def encoder_frames(mel_frames: int) -> int:
    return conv_len(conv_len(conv_len(mel_frames)))


def conv3x3_s2(img, w, b):
    """y[o, i, j] = b[o] + sum_{c,di,dj} w[o,c,di,dj] * img[c, 2i+di-1, 2j+dj-1],
    zero outside the image.  img [C, H, W] -> [O, ceil(H/2), ceil(W/2)]."""
    C, H, W = img.shape
    O = w.shape[0]
    Ho, Wo = conv_len(H), conv_len(W)
    xp = np.zeros((C, H + 3, W + 3), dtype=np.float64)
    xp[:, 1:H + 1, 1:W + 1] = img
    y = np.empty((O, Ho * Wo), dtype=np.float64)
    y[:] = b[:, None]
    for di in range(3):
        for dj in range(3):
            tap = xp[:, di:di + 2 * Ho:2, dj:dj + 2 * Wo:2].reshape(C, Ho * Wo)
            y += np.ascontiguousarray(w[:, :, di, dj]) @ tap
    return y.reshape(O, Ho, Wo)


def front_end(mel, P):
    """Log-mel [T, n_mels] -> conv_out output [N, d_model] (positions not yet added)."""
    img = np.asarray(mel, dtype=np.float64).T[None]  # [1, n_mels, T]
    y = gelu(conv3x3_s2(img, P["conv1.weight"], P["conv1.bias"]))
    y = gelu(conv3x3_s2(y, P["conv2.weight"], P["conv2.bias"]))
    y = gelu(conv3x3_s2(y, P["conv3.weight"], P["conv3.bias"]))
    C, F8, N = y.shape
    z = y.transpose(2, 0, 1).reshape(N, C * F8)  # z[t, c*F8 + f] = y[c, f, t]
    return linear(z, P["conv_out.weight"])


def sinusoids(n: int, d: int, t0: int = 0):
    half = d // 2
    tau = np.exp(-np.arange(half, dtype=np.float64) * math.log(10000.0) / (half - 1))
    t = (t0 + np.arange(n, dtype=np.float64))[:, None]
    return np.concatenate([np.sin(t * tau[None]), np.cos(t * tau[None])], axis=1)


def window_bounds(n: int, window: int, t0: int = 0):
    """Windows [start, end) in segment rows; window k covers stream frames
    [kW, (k+1)W).  For a whole clip t0 = 0."""
    if window < 1:
        raise ValueError("window must be >= 1")
    out = []
    r = 0
    while r < n:
        k = (t0 + r) // window
        end = min(n, (k + 1) * window - t0)
        out.append((r, end))
        r = end
    return out


def softmax_rows(s):
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=-1, keepdims=True)


def windowed_attention(q, k, v, n_heads: int, window: int, t0: int = 0):
    """Block-diagonal attention: each row attends only to rows of its window."""
    n, d = q.shape
    hd = d // n_heads
    out = np.empty_like(q)
    for (a, e) in window_bounds(n, window, t0):
        qw = q[a:e].reshape(e - a, n_heads, hd).transpose(1, 0, 2)
        kw = k[a:e].reshape(e - a, n_heads, hd).transpose(1, 0, 2)
        vw = v[a:e].reshape(e - a, n_heads, hd).transpose(1, 0, 2)
        p = softmax_rows(qw @ kw.transpose(0, 2, 1) / math.sqrt(hd))
        out[a:e] = (p @ vw).transpose(1, 0, 2).reshape(e - a, d)
    return out


def layer(x, P, l: int, n_heads: int, window: int, t0: int = 0):
    p = f"layers.{l}."
    h = layer_norm(x, P[p + "ln1.weight"], P[p + "ln1.bias"])
    q = linear(h, P[p + "q.weight"], P[p + "q.bias"])
    k = linear(h, P[p + "k.weight"], P[p + "k.bias"])
    v = linear(h, P[p + "v.weight"], P[p + "v.bias"])
    a = windowed_attention(q, k, v, n_heads, window, t0)
    x = x + linear(a, P[p + "o.weight"], P[p + "o.bias"])
    h = layer_norm(x, P[p + "ln2.weight"], P[p + "ln2.bias"])
    x = x + linear(gelu(linear(h, P[p + "fc1.weight"], P[p + "fc1.bias"])),
                   P[p + "fc2.weight"], P[p + "fc2.bias"])
    return x


def head(x, P):
    h = layer_norm(x, P["ln_post.weight"], P["ln_post.bias"])
    return linear(gelu(linear(h, P["proj1.weight"], P["proj1.bias"])),
                  P["proj2.weight"], P["proj2.bias"])


def adapter(y, P):
    g = linear(y, P["adapter.gate.weight"])
    u = linear(y, P["adapter.up.weight"])
    return linear(silu(g) * u, P["adapter.down.weight"])


def encode_clip(mel, P, geom: dict, window: int, n_layers=None, with_head: bool = True,
                with_adapter=None, t0: int = 0):
    """One clip's log-mel [T, n_mels] -> encoder output.

    n_layers    run only the first n layers (default: all of geom["n_layers"])
    with_head   False stops after the tower, giving the residual stream
    t0          stream index of the segment's first encoder frame (0 for a
                whole clip); used for positions and window boundaries only
    """
    L = geom["n_layers"] if n_layers is None else n_layers
    if with_adapter is None:
        with_adapter = bool(geom.get("adapter_hidden", 0))
    x = front_end(mel, P)
    x = x + sinusoids(x.shape[0], x.shape[1], t0)
    for l in range(L):
        x = layer(x, P, l, geom["n_heads"], window, t0)
    if not with_head:
        return x
    y = head(x, P)
    if with_adapter:
        y = adapter(y, P)
    return y


def encode(mels: list, P, geom: dict, window: int, **kw) -> list:
    """Clips are independent: a batch is the list of per-clip outputs."""
    return [encode_clip(m, P, geom, window, **kw) for m in mels]


def as_f64(weights: dict) -> dict:
    return {k: np.asarray(v, dtype=np.float64) for k, v in weights.items()}
