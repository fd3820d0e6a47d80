"""Pins for the 2x-front-end, full-attention encoder oracle (CPU only).

Each test ties oracle.encoder2x to something other than itself: the frame
count the CrisperWhisper export page reports (section Results: 1500 encoder
frames for a 30 s window), torch CPU float64 library runs (conv1d,
TransformerEncoderLayer, layer_norm), closed-form special cases of the
convolution (identity and shift taps) and of the front-end (zero weights
leave only the sinusoids), and the equivalence of any window >= N with full
attention.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as TF

import synth
from oracle import encoder as E
from oracle import encoder2x as E2

from .test_oracle_encoder import torch_layer

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "counts.json")

TINY2X = dict(frontend="conv1d_2x", n_mels=16, conv_ch=16, d_model=16, n_layers=2, n_heads=2,
              head_dim=8, d_ffn=32, d_out=16, adapter_hidden=0)


def tiny2x_weights(geom=TINY2X, seed=6):
    return E.as_f64(synth.make_weights(geom, bf16=False, seed=seed, ln_random=True))


def test_frames_golden():
    g = json.load(open(GOLDEN))
    for c in g["two_x_cases"]:
        T = c["n_samples"] // 160
        assert T == c["mel_frames"]
        assert E2.frames_2x(T) == c["encoder_frames"]
    assert [E2.frames_2x(t) for t in (1, 2, 3, 4, 5)] == [1, 1, 2, 2, 3]


def test_front_end_shape_on_30s():
    geom = dict(TINY2X, n_mels=128, n_layers=0)
    P = tiny2x_weights(geom)
    mel = np.random.default_rng(1).standard_normal((3000, 128))
    assert E2.front_end_2x(mel, P).shape == (1500, geom["d_model"])


@pytest.mark.parametrize("T,Ci,Co,s", [(1, 3, 4, 1), (2, 3, 4, 2), (7, 5, 2, 1), (8, 2, 3, 2),
                                       (9, 4, 4, 2)])
def test_conv1d_matches_torch(T, Ci, Co, s):
    rng = np.random.default_rng(T * 10 + s)
    x = rng.standard_normal((T, Ci))
    w = rng.standard_normal((Co, Ci, 3))
    b = rng.standard_normal(Co)
    mine = E2.conv1d_k3(x, w, b, s)
    ref = TF.conv1d(torch.from_numpy(x.T[None].copy()), torch.from_numpy(w), torch.from_numpy(b),
                    stride=s, padding=1)[0].T.numpy()
    assert mine.shape == ref.shape
    assert np.max(np.abs(mine - ref)) < 1e-12


def test_conv1d_identity_and_shift_taps():
    x = np.arange(1.0, 13.0).reshape(6, 2)
    eye = np.eye(2)
    for d, shift in ((0, -1), (1, 0), (2, 1)):
        w = np.zeros((2, 2, 3))
        w[:, :, d] = eye
        out = E2.conv1d_k3(x, w, np.zeros(2), 1)
        for t in range(6):
            src = t + shift
            want = x[src] if 0 <= src < 6 else np.zeros(2)
            assert np.array_equal(out[t], want)
        # stride 2: output t reads input 2t + shift
        out2 = E2.conv1d_k3(x, w, np.zeros(2), 2)
        assert out2.shape == (3, 2)
        for t in range(3):
            src = 2 * t + shift
            want = x[src] if 0 <= src < 6 else np.zeros(2)
            assert np.array_equal(out2[t], want)


def test_zero_convs_leave_gelu_of_bias_plus_sinusoids():
    geom = dict(TINY2X, n_layers=0)
    P = tiny2x_weights(geom)
    for k in ("conv1.weight", "conv2.weight"):
        P[k] = np.zeros_like(P[k])
    P["conv1.bias"] = np.zeros_like(P["conv1.bias"])
    c = np.linspace(-2.0, 2.0, geom["d_model"])
    P["conv2.bias"] = c
    mel = np.random.default_rng(3).standard_normal((11, geom["n_mels"]))
    out = E2.front_end_2x(mel, P)
    D = geom["d_model"]
    pos = np.arange(6)[:, None]
    inv = np.exp(-math.log(10000.0) / (D // 2 - 1) * np.arange(D // 2))
    pe = np.concatenate([np.sin(pos * inv), np.cos(pos * inv)], axis=1)
    phi = 0.5 * (1.0 + np.array([math.erf(v / math.sqrt(2.0)) for v in c]))
    assert np.max(np.abs(out - (c * phi + pe))) < 1e-14


def torch_encoder_2x(mel, P, geom, with_head=True):
    """Independent composition from torch CPU float64 library modules, full
    attention (no mask)."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    x = t(mel).T[None]  # [1, n_mels, T]
    x = TF.gelu(TF.conv1d(x, t(P["conv1.weight"]), t(P["conv1.bias"]), stride=1, padding=1))
    x = TF.gelu(TF.conv1d(x, t(P["conv2.weight"]), t(P["conv2.bias"]), stride=2, padding=1))
    h = x[0].T
    N, D = h.shape
    pos = torch.arange(N, dtype=torch.float64)[:, None]
    inv = torch.exp(-math.log(10000.0) / (D // 2 - 1) * torch.arange(D // 2, dtype=torch.float64))
    h = h + torch.cat([torch.sin(pos * inv), torch.cos(pos * inv)], dim=1)
    with torch.no_grad():
        for l in range(geom["n_layers"]):
            h = torch_layer(P, l, geom)(h[None])[0]
    if with_head:
        h = TF.layer_norm(h, (D,), t(P["ln_post.weight"]), t(P["ln_post.bias"]), eps=1e-5)
    return h.numpy()


@pytest.mark.parametrize("T,with_head", [(1, True), (2, True), (37, True), (64, False)])
def test_encode_matches_torch_composition(T, with_head):
    P = tiny2x_weights()
    mel = np.random.default_rng(T).standard_normal((T, TINY2X["n_mels"]))
    mine = E2.encode_clip_2x(mel, P, TINY2X, with_head=with_head)
    ref = torch_encoder_2x(mel, P, TINY2X, with_head)
    assert mine.shape == (E2.frames_2x(T), TINY2X["d_model"])
    assert np.max(np.abs(mine - ref)) < 1e-10


def test_any_window_at_least_n_is_full_attention():
    P = tiny2x_weights()
    mel = np.random.default_rng(4).standard_normal((30, TINY2X["n_mels"]))
    full = E2.encode_clip_2x(mel, P, TINY2X)
    N = full.shape[0]
    for W in (N, N + 1, 10 * N):
        assert np.array_equal(E2.encode_clip_2x(mel, P, TINY2X, window=W), full)
    # a smaller window is block-diagonal attention and differs
    assert np.max(np.abs(E2.encode_clip_2x(mel, P, TINY2X, window=N // 2) - full)) > 1e-6


def test_weight_names_2x():
    names = [n for n, _ in synth.weight_names(synth.WHISPER_SMALL_GEOM)]
    assert names[:4] == ["conv1.weight", "conv1.bias", "conv2.weight", "conv2.bias"]
    assert names[-2:] == ["ln_post.weight", "ln_post.bias"]
    assert len(names) == 4 + 16 * 12 + 2
