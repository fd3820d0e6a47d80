"""Pins for the decoder oracle (CPU only).

Each test ties oracle.decoder to something other than itself: the model
card's total parameter count (Architecture table, row Parameters: about 2.4 B
for encoder, adapter and LLM together), torch CPU float64 library runs
(rms_norm, scaled_dot_product_attention with grouped-query heads, linear,
silu), a complex-number statement of the rotary positions and its
relative-position invariance, the equality of a multi-row step with
row-by-row steps through the KV cache, and the tied head recognising its own
token.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as TF

import synth
from oracle import decoder as D

TINY = dict(vocab=300, d_model=256, n_layers=2, n_heads=4, n_kv_heads=2, head_dim=128, d_ffn=384)


def tiny_weights(geom=TINY, seed=7):
    return {k: v.astype(np.float64) for k, v in synth.make_decoder_weights(geom, bf16=False, seed=seed).items()}


def test_total_parameters_match_card():
    enc = sum(int(np.prod(s)) for _, s in synth.weight_names(dict(synth.FULL_GEOM, adapter_hidden=8192)))
    dec = sum(int(np.prod(s)) for _, s in synth.decoder_weight_names(synth.DEC_GEOM))
    total = enc + dec
    assert abs(total - 2.4e9) / 2.4e9 < 0.02, total
    assert dec == 1720574976  # Qwen3-1.7B with the embedding counted once (tied)


def test_rms_norm_matches_torch():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 64)) * 3.0
    w = rng.standard_normal(64)
    ref = TF.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(w), eps=1e-6).numpy()
    assert np.max(np.abs(D.rms_norm(x, w) - ref)) < 1e-12


def test_rope_as_complex_rotation_and_relative_positions():
    rng = np.random.default_rng(2)
    hd = 128
    x = rng.standard_normal((3, 5, hd))
    pos = np.array([0, 1, 7, 1000, 123456])
    r = D.rope_neox(x, pos)
    # value j and j + 64 form z = a + i b, turned by pos * base^(-j/64)
    z = x[..., :64] + 1j * x[..., 64:]
    th = pos[:, None] * (1e6 ** (-np.arange(64) / 64.0))
    zr = z * np.exp(1j * th)
    assert np.max(np.abs(r[..., :64] - zr.real)) < 1e-9
    assert np.max(np.abs(r[..., 64:] - zr.imag)) < 1e-9
    assert np.allclose(r[:, 0], x[:, 0])  # position 0: identity
    # scores depend only on the distance between positions
    q, k = rng.standard_normal((1, hd)), rng.standard_normal((1, hd))
    for m, n, s in ((5, 2, 40), (100, 100, 7), (3, 90, 1000)):
        a = D.rope_neox(q[None], [m])[0, 0] @ D.rope_neox(k[None], [n])[0, 0]
        b = D.rope_neox(q[None], [m + s])[0, 0] @ D.rope_neox(k[None], [n + s])[0, 0]
        assert abs(a - b) < 1e-9


def test_attend_matches_torch_gqa_sdpa():
    rng = np.random.default_rng(3)
    P0, n, Hq, Hkv, hd = 9, 4, 4, 2, 16
    q = rng.standard_normal((n, Hq, hd))
    K = rng.standard_normal((P0 + n, Hkv, hd))
    V = rng.standard_normal((P0 + n, Hkv, hd))
    pos = np.arange(P0, P0 + n)
    mine = D.attend(q, K, V, pos)
    mask = torch.from_numpy(np.arange(P0 + n)[None, :] <= pos[:, None])  # True = may attend
    ref = TF.scaled_dot_product_attention(
        torch.from_numpy(q.transpose(1, 0, 2))[None], torch.from_numpy(K.transpose(1, 0, 2))[None],
        torch.from_numpy(V.transpose(1, 0, 2))[None], attn_mask=mask, enable_gqa=True)[0]
    assert np.max(np.abs(mine - ref.numpy().transpose(1, 0, 2))) < 1e-12


def torch_forward(x, P, geom, n_layers):
    """Independent composition from torch CPU float64 library calls: the
    whole sequence at once with a causal mask."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    Hq, Hkv, hd = geom["n_heads"], geom["n_kv_heads"], geom["head_dim"]
    n = x.shape[0]
    x = t(x)
    pos = torch.arange(n, dtype=torch.float64)
    inv = 1e6 ** (-torch.arange(hd // 2, dtype=torch.float64) / (hd // 2))
    ang = pos[:, None] * inv[None]
    cos, sin = torch.cos(ang), torch.sin(ang)

    def rope(z):  # [H, n, hd]
        a, b = z[..., :hd // 2], z[..., hd // 2:]
        return torch.cat([a * cos - b * sin, b * cos + a * sin], dim=-1)

    for l in range(n_layers):
        p = f"layers.{l}."
        h = TF.rms_norm(x, (x.shape[1],), t(P[p + "input_norm.weight"]), eps=1e-6)
        q = TF.linear(h, t(P[p + "q.weight"])).view(n, Hq, hd).transpose(0, 1)
        k = TF.linear(h, t(P[p + "k.weight"])).view(n, Hkv, hd).transpose(0, 1)
        v = TF.linear(h, t(P[p + "v.weight"])).view(n, Hkv, hd).transpose(0, 1)
        q = rope(TF.rms_norm(q, (hd,), t(P[p + "q_norm.weight"]), eps=1e-6))
        k = rope(TF.rms_norm(k, (hd,), t(P[p + "k_norm.weight"]), eps=1e-6))
        a = TF.scaled_dot_product_attention(q[None], k[None], v[None], is_causal=True, enable_gqa=True)[0]
        x = x + TF.linear(a.transpose(0, 1).reshape(n, Hq * hd), t(P[p + "o.weight"]))
        h = TF.rms_norm(x, (x.shape[1],), t(P[p + "post_norm.weight"]), eps=1e-6)
        x = x + TF.linear(TF.silu(TF.linear(h, t(P[p + "gate.weight"]))) * TF.linear(h, t(P[p + "up.weight"])),
                          t(P[p + "down.weight"]))
    h = TF.rms_norm(x, (x.shape[1],), t(P["norm.weight"]), eps=1e-6)
    return TF.linear(h, t(P["embed.weight"])).numpy()


@pytest.mark.parametrize("n", [1, 6])
def test_forward_matches_torch_composition(n):
    P = tiny_weights()
    tokens = np.random.default_rng(n).integers(0, TINY["vocab"], n)
    x = D.embed(tokens, P)
    mine = D.forward(x, P, TINY, D.empty_cache(TINY))
    ref = torch_forward(x, P, TINY, TINY["n_layers"])
    assert mine.shape == (n, TINY["vocab"])
    assert np.max(np.abs(mine - ref)) < 1e-9


def test_cache_steps_equal_one_pass():
    P = tiny_weights()
    tokens = np.random.default_rng(11).integers(0, TINY["vocab"], 7)
    x = D.embed(tokens, P)
    whole_cache = D.empty_cache(TINY)
    whole = D.forward(x, P, TINY, whole_cache)
    c = D.empty_cache(TINY)
    parts = [D.forward(x[:3], P, TINY, c)]            # a 3-row prefill
    for i in range(3, 7):                             # then one row per step
        parts.append(D.forward(x[i:i + 1], P, TINY, c))
    assert np.max(np.abs(np.concatenate(parts) - whole)) < 1e-10
    for l in range(TINY["n_layers"]):
        assert np.max(np.abs(c[l]["K"] - whole_cache[l]["K"])) < 1e-12
        assert c[l]["K"].shape == (7, TINY["n_kv_heads"], TINY["head_dim"])


def test_tied_head_recognises_its_token():
    # with the layers' output projections zeroed the stream is the embedding
    # itself, and the tied head scores the input token highest
    geom = dict(TINY, n_layers=1)
    P = tiny_weights(geom)
    P["layers.0.o.weight"][:] = 0.0
    P["layers.0.down.weight"][:] = 0.0
    P["norm.weight"][:] = 1.0
    tokens = np.array([0, 5, 299, 17])
    logits = D.forward(D.embed(tokens, P), P, geom, D.empty_cache(geom))
    assert np.array_equal(np.argmax(logits, axis=1), tokens)
