"""Pins for the encoder oracle (CPU only).

Each test ties oracle.encoder to something other than itself: frame-count
closed forms from the model card (Architecture table, Conv front-end row:
three stride-2 convs, 480*16 = 7680 features), library runs of torch CPU
float64 (conv2d, layer_norm, gelu, silu, scaled_dot_product_attention,
TransformerEncoderLayer), closed forms of the sinusoids, brute force on tiny
inputs, and the window-locality invariant of block-diagonal attention
(Architecture table, Audio encoder row).
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

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "counts.json")

TINY = dict(n_mels=16, conv_ch=4, d_model=16, n_layers=2, n_heads=2, head_dim=8,
            d_ffn=32, d_out=12, adapter_hidden=0)


def tiny_weights(geom=TINY, ln_random=True, seed=5):
    return E.as_f64(synth.make_weights(geom, bf16=False, seed=seed, ln_random=ln_random))


def test_counts_golden():
    g = json.load(open(GOLDEN))
    for c in g["cases"]:
        assert E.encoder_frames(c["mel_frames"]) == c["encoder_frames"]
        n = c["encoder_frames"]
        wins = E.window_bounds(n, c["window"])
        if "windows" in c:
            assert [e - a for a, e in wins] == c["windows"]
        else:
            assert len(wins) == c["n_windows"]
            assert wins[-1][1] - wins[-1][0] == c["last_window"]
    assert 16 * E.encoder_frames(3000) == g["batch16x30s"]["total_encoder_frames"]
    assert 16 * len(E.window_bounds(375, 104)) == g["batch16x30s"]["n_windows"]
    assert g["conv_channels"] * (128 // 8) == g["conv_out_in_features"]


def test_front_end_shapes_full_geometry():
    geom = dict(synth.FULL_GEOM, n_layers=0)
    P = E.as_f64(synth.make_weights(geom, bf16=False))
    mel = np.random.default_rng(0).standard_normal((100, 128))
    z = E.front_end(mel, P)
    assert z.shape == (13, 1280)
    assert P["conv_out.weight"].shape == (1280, 7680)


@pytest.mark.parametrize("H,W,C,O", [(16, 11, 1, 5), (9, 7, 3, 4), (8, 1, 2, 2), (5, 2, 3, 3)])
def test_conv_matches_torch(H, W, C, O):
    rng = np.random.default_rng(H * 100 + W)
    img = rng.standard_normal((C, H, W))
    w = rng.standard_normal((O, C, 3, 3))
    b = rng.standard_normal(O)
    ref = TF.conv2d(torch.from_numpy(img)[None], torch.from_numpy(w), torch.from_numpy(b),
                    stride=2, padding=1)[0].numpy()
    mine = E.conv3x3_s2(img, w, b)
    assert mine.shape == ref.shape
    assert np.max(np.abs(mine - ref)) < 1e-12


def test_conv_centre_tap_is_subsampling():
    rng = np.random.default_rng(3)
    img = rng.standard_normal((3, 13, 10))
    w = np.zeros((3, 3, 3, 3))
    for c in range(3):
        w[c, c, 1, 1] = 1.0
    y = E.conv3x3_s2(img, w, np.zeros(3))
    assert np.array_equal(y, img[:, ::2, ::2])


def test_flatten_order_channel_major():
    # conv_out column c*F8 + f must read conv3 output channel c at frequency f
    P = tiny_weights()
    rng = np.random.default_rng(1)
    mel = rng.standard_normal((40, TINY["n_mels"]))
    img = mel.T[None]
    y = E.gelu(E.conv3x3_s2(img, P["conv1.weight"], P["conv1.bias"]))
    y = E.gelu(E.conv3x3_s2(y, P["conv2.weight"], P["conv2.bias"]))
    y = E.gelu(E.conv3x3_s2(y, P["conv3.weight"], P["conv3.bias"]))
    C, F8, N = y.shape
    Q = dict(P)
    sel = np.zeros((C * F8, C * F8))
    sel[np.arange(C * F8), np.arange(C * F8)] = 1.0
    Q["conv_out.weight"] = sel
    z = E.front_end(mel, Q)
    for c in range(C):
        for f in range(F8):
            assert np.array_equal(z[:, c * F8 + f], y[c, f, :])


def test_sinusoid_closed_forms():
    pe = E.sinusoids(50, 1280)
    assert np.array_equal(pe[0, :640], np.zeros(640))
    assert np.array_equal(pe[0, 640:], np.ones(640))
    t = np.arange(50.0)
    assert np.allclose(pe[:, 0], np.sin(t), atol=1e-15)
    assert np.allclose(pe[:, 640], np.cos(t), atol=1e-15)
    assert np.allclose(pe[:, 639], np.sin(t * 1e-4), atol=1e-15)
    assert np.allclose(pe[:, 1279], np.cos(t * 1e-4), atol=1e-15)
    # middle column: timescale 10000^(-320/639)
    assert np.allclose(pe[:, 320], np.sin(t * 10000.0 ** (-320.0 / 639.0)), atol=1e-14)
    seg = E.sinusoids(20, 1280, t0=30)
    assert np.allclose(seg, pe[30:50], atol=1e-12)


def test_layer_norm_gelu_silu_match_torch():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((7, 24)) * 3 + 1
    g = rng.standard_normal(24)
    b = rng.standard_normal(24)
    tx = torch.from_numpy(x)
    ref = TF.layer_norm(tx, (24,), torch.from_numpy(g), torch.from_numpy(b), eps=1e-5).numpy()
    assert np.max(np.abs(E.layer_norm(x, g, b) - ref)) < 1e-12
    assert np.max(np.abs(E.gelu(x) - TF.gelu(tx).numpy())) < 1e-13
    assert np.max(np.abs(E.gelu(x) - TF.gelu(tx, approximate="tanh").numpy())) > 1e-5
    assert np.max(np.abs(E.silu(x) - TF.silu(tx).numpy())) < 1e-13


def block_mask(n, window, t0=0):
    wid = (t0 + np.arange(n)) // window
    return wid[:, None] == wid[None, :]


@pytest.mark.parametrize("n,W,t0", [(11, 3, 0), (11, 4, 0), (9, 5, 3), (7, 7, 0), (13, 1, 0)])
def test_windowed_attention_vs_masked_sdpa(n, W, t0):
    rng = np.random.default_rng(n * 10 + W)
    H, hd = 2, 8
    q, k, v = (rng.standard_normal((n, H * hd)) for _ in range(3))
    mine = E.windowed_attention(q, k, v, H, W, t0)
    tq, tk, tv = (torch.from_numpy(a).reshape(n, H, hd).transpose(0, 1) for a in (q, k, v))
    mask = torch.from_numpy(block_mask(n, W, t0))
    ref = TF.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
    ref = ref.transpose(0, 1).reshape(n, H * hd).numpy()
    assert np.max(np.abs(mine - ref)) < 1e-12


def test_windowed_attention_brute_force():
    rng = np.random.default_rng(11)
    n, W, H, hd = 11, 3, 2, 8
    q, k, v = (rng.standard_normal((n, H * hd)) for _ in range(3))
    mine = E.windowed_attention(q, k, v, H, W)
    out = np.zeros((n, H * hd))
    for h in range(H):
        for i in range(n):
            js = [j for j in range(n) if j // W == i // W]
            s = [sum(q[i, h * hd + d] * k[j, h * hd + d] for d in range(hd)) / math.sqrt(hd)
                 for j in js]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = sum(e)
            for d in range(hd):
                out[i, h * hd + d] = sum(e[a] / z * v[j, h * hd + d] for a, j in enumerate(js))
    assert np.max(np.abs(mine - out)) < 1e-12


def test_window_one_returns_v_and_large_window_is_full_attention():
    rng = np.random.default_rng(4)
    n, H, hd = 10, 2, 8
    q, k, v = (rng.standard_normal((n, H * hd)) for _ in range(3))
    assert np.array_equal(E.windowed_attention(q, k, v, H, 1), v)
    tq, tk, tv = (torch.from_numpy(a).reshape(n, H, hd).transpose(0, 1) for a in (q, k, v))
    full = TF.scaled_dot_product_attention(tq, tk, tv).transpose(0, 1).reshape(n, H * hd).numpy()
    for W in (10, 11, 500):
        assert np.max(np.abs(E.windowed_attention(q, k, v, H, W) - full)) < 1e-12


def torch_layer(P, l, geom):
    D, H = geom["d_model"], geom["n_heads"]
    m = torch.nn.TransformerEncoderLayer(D, H, dim_feedforward=geom["d_ffn"], dropout=0.0,
                                         activation="gelu", layer_norm_eps=1e-5,
                                         batch_first=True, norm_first=True).double()
    p = f"layers.{l}."
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    with torch.no_grad():
        m.self_attn.in_proj_weight.copy_(t(np.concatenate([P[p + "q.weight"], P[p + "k.weight"],
                                                           P[p + "v.weight"]])))
        m.self_attn.in_proj_bias.copy_(t(np.concatenate([P[p + "q.bias"], P[p + "k.bias"],
                                                         P[p + "v.bias"]])))
        m.self_attn.out_proj.weight.copy_(t(P[p + "o.weight"]))
        m.self_attn.out_proj.bias.copy_(t(P[p + "o.bias"]))
        m.linear1.weight.copy_(t(P[p + "fc1.weight"]))
        m.linear1.bias.copy_(t(P[p + "fc1.bias"]))
        m.linear2.weight.copy_(t(P[p + "fc2.weight"]))
        m.linear2.bias.copy_(t(P[p + "fc2.bias"]))
        m.norm1.weight.copy_(t(P[p + "ln1.weight"]))
        m.norm1.bias.copy_(t(P[p + "ln1.bias"]))
        m.norm2.weight.copy_(t(P[p + "ln2.weight"]))
        m.norm2.bias.copy_(t(P[p + "ln2.bias"]))
    return m.eval()


@pytest.mark.parametrize("n,W", [(11, 4), (9, 9), (6, 1)])
def test_layer_matches_torch_encoder_layer(n, W):
    P = tiny_weights()
    rng = np.random.default_rng(n + W)
    x = rng.standard_normal((n, TINY["d_model"]))
    mine = E.layer(x, P, 1, TINY["n_heads"], W)
    m = torch_layer(P, 1, TINY)
    # torch bool mask: True = may NOT attend
    mask = torch.from_numpy(~block_mask(n, W))
    with torch.no_grad():
        ref = m(torch.from_numpy(x)[None], src_mask=mask)[0].numpy()
    assert np.max(np.abs(mine - ref)) < 1e-11


def torch_encoder(mel, P, geom, W):
    """Independent composition from torch CPU float64 library modules."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    x = t(mel).T[None, None]  # [1, 1, n_mels, T]
    for i in (1, 2, 3):
        x = TF.gelu(TF.conv2d(x, t(P[f"conv{i}.weight"]), t(P[f"conv{i}.bias"]), stride=2,
                              padding=1))
    _, C, F8, N = x.shape
    z = x[0].permute(2, 0, 1).reshape(N, C * F8)
    h = z @ t(P["conv_out.weight"]).T
    D = h.shape[1]
    pos = torch.arange(N, dtype=torch.float64)[:, None]
    inv = torch.exp(-math.log(10000.0) / (D // 2 - 1) * torch.arange(D // 2, dtype=torch.float64))
    h = h + torch.cat([torch.sin(pos * inv), torch.cos(pos * inv)], dim=1)
    mask = torch.from_numpy(~block_mask(N, W))
    with torch.no_grad():
        for l in range(geom["n_layers"]):
            h = torch_layer(P, l, geom)(h[None], src_mask=mask)[0]
    h = TF.layer_norm(h, (D,), t(P["ln_post.weight"]), t(P["ln_post.bias"]), eps=1e-5)
    h = TF.gelu(TF.linear(h, t(P["proj1.weight"]), t(P["proj1.bias"])))
    y = TF.linear(h, t(P["proj2.weight"]), t(P["proj2.bias"]))
    if geom.get("adapter_hidden", 0):
        y = TF.linear(TF.silu(TF.linear(y, t(P["adapter.gate.weight"]))) *
                      TF.linear(y, t(P["adapter.up.weight"])), t(P["adapter.down.weight"]))
    return y.numpy()


@pytest.mark.parametrize("T,W,adapter", [(77, 3, 0), (40, 100, 0), (64, 2, 24)])
def test_encode_matches_torch_composition(T, W, adapter):
    geom = dict(TINY, adapter_hidden=adapter)
    P = tiny_weights(geom)
    mel = np.random.default_rng(T).standard_normal((T, geom["n_mels"]))
    mine = E.encode_clip(mel, P, geom, W)
    ref = torch_encoder(mel, P, geom, W)
    assert mine.shape == (E.encoder_frames(T), geom["d_out"])
    assert np.max(np.abs(mine - ref)) < 1e-10


def test_window_locality():
    geom = TINY
    P = tiny_weights()
    T, W = 200, 4  # 25 encoder frames -> windows of 4
    rng = np.random.default_rng(9)
    mel = rng.standard_normal((T, geom["n_mels"]))
    base = E.encode_clip(mel, P, geom, W)
    N = base.shape[0]
    for k in (0, 2, 6):
        m2 = mel.copy()
        lo, hi = 8 * k * W, min(T - 1, 8 * (k + 1) * W - 8)
        m2[lo:hi + 1] += rng.standard_normal((hi + 1 - lo, geom["n_mels"]))
        out = E.encode_clip(m2, P, geom, W)
        inside = np.zeros(N, bool)
        inside[k * W:min(N, (k + 1) * W)] = True
        assert np.array_equal(out[~inside], base[~inside])
        assert np.max(np.abs(out[inside] - base[inside])) > 1e-7


def test_segment_with_offset_matches_whole_clip():
    # A mel segment with an 8-frame halo, encoded with t0 = its first encoder
    # frame, reproduces the whole clip's rows for the window it contains.
    geom = TINY
    P = tiny_weights()
    T, W = 240, 5
    mel = np.random.default_rng(12).standard_normal((T, geom["n_mels"]))
    whole = E.encode_clip(mel, P, geom, W)
    for k in (1, 3):
        s = 8 * (k * W - 1)
        e = min(T, 8 * (k + 1) * W + 8)
        seg = E.encode_clip(mel[s:e], P, geom, W, t0=s // 8)
        r0 = k * W - s // 8
        assert np.max(np.abs(seg[r0:r0 + W] - whole[k * W:(k + 1) * W])) < 1e-10
