"""Language-model decoder forward with a KV cache, float64.  TEST INFRASTRUCTURE ONLY.

Source: model card "MOSS-Transcribe-preview-2B-GGUF", Architecture table, row
LLM: Qwen3-1.7B, 28 layers, hidden 2048, 16 query and 8 key/value heads
(grouped-query attention) of head_dim 128, FFN 6144 with SwiGLU, RMSNorm,
per-head Q-norm and K-norm, NEOX-style rotary positions with base 1e6, and
the token embedding tied to the output head; row Vocab: 151 936 tokens.

Readings where the card is silent (each pinned by tests/test_oracle_decoder.py):
  * pre-norm layers: x += o(attn(rms(x))); x += down(silu(gate(h)) * up(h)),
    h = rms(x) with the post-attention norm; a final RMSNorm before the head;
  * RMSNorm: x / sqrt(mean(x^2) + eps) * w, eps = 1e-6; no biases anywhere;
  * Q-norm / K-norm: RMSNorm over each head's 128 values with one weight
    vector per layer (shared by the heads), applied before the rotation;
  * rotary (NEOX): within a head, value j pairs with value j + 64; at position
    p the pair turns by the angle p * base^(-j / 64), j = 0..63;
  * attention: causal, scale 1 / sqrt(128); query head h reads key/value head
    h // 2 (consecutive query heads share a key/value head);
  * logits = rms_final(x) . E^T with E the [vocab, hidden] embedding table.

The cache holds, per layer, K and V of every earlier position of each
sequence (after K-norm and rotation for K).  A forward step takes new rows
(token embeddings) at consecutive positions starting at the cache length.
"""

from __future__ import annotations

import math

import numpy as np

RMS_EPS = 1e-6
ROPE_BASE = 1.0e6


def rms_norm(x, w, eps: float = RMS_EPS):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * w


def silu(x):
    return x / (1.0 + np.exp(-x))


def rope_neox(x, pos, base: float = ROPE_BASE):
    """x [..., n, head_dim] at integer positions pos [n] -> rotated copy."""
    hd = x.shape[-1]
    half = hd // 2
    inv = base ** (-np.arange(half, dtype=np.float64) / half)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]  # [n, half]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def attend(q, K, V, q_pos):
    """q [n, Hq, hd] at positions q_pos; K, V [P, Hkv, hd] for positions
    0..P-1; causal (query at p sees keys 0..p) -> [n, Hq, hd]."""
    n, Hq, hd = q.shape
    Hkv = K.shape[1]
    grp = Hq // Hkv
    out = np.empty_like(q)
    for i in range(n):
        L = q_pos[i] + 1
        for h in range(Hq):
            kh = h // grp
            s = K[:L, kh, :] @ q[i, h] / math.sqrt(hd)
            p = np.exp(s - s.max())
            p /= p.sum()
            out[i, h] = p @ V[:L, kh, :]
    return out


def layer_step(x, P, l: int, geom: dict, cache: dict, pos0: int):
    """New rows x [n, D] at positions pos0..pos0+n-1 of one sequence; cache
    {"K": [P, Hkv, hd], "V": ...} of layer l holds positions < pos0 and is
    extended in place with the new rows."""
    p = f"layers.{l}."
    Hq, Hkv, hd = geom["n_heads"], geom["n_kv_heads"], geom["head_dim"]
    n = x.shape[0]
    pos = np.arange(pos0, pos0 + n)
    h = rms_norm(x, P[p + "input_norm.weight"])
    q = (h @ P[p + "q.weight"].T).reshape(n, Hq, hd)
    k = (h @ P[p + "k.weight"].T).reshape(n, Hkv, hd)
    v = (h @ P[p + "v.weight"].T).reshape(n, Hkv, hd)
    q = rope_neox(rms_norm(q, P[p + "q_norm.weight"]).transpose(1, 0, 2), pos).transpose(1, 0, 2)
    k = rope_neox(rms_norm(k, P[p + "k_norm.weight"]).transpose(1, 0, 2), pos).transpose(1, 0, 2)
    cache["K"] = np.concatenate([cache["K"], k], axis=0)
    cache["V"] = np.concatenate([cache["V"], v], axis=0)
    a = attend(q, cache["K"], cache["V"], pos).reshape(n, Hq * hd)
    x = x + a @ P[p + "o.weight"].T
    h = rms_norm(x, P[p + "post_norm.weight"])
    g = h @ P[p + "gate.weight"].T
    u = h @ P[p + "up.weight"].T
    return x + (silu(g) * u) @ P[p + "down.weight"].T


def empty_cache(geom: dict) -> list:
    Hkv, hd = geom["n_kv_heads"], geom["head_dim"]
    return [{"K": np.zeros((0, Hkv, hd)), "V": np.zeros((0, Hkv, hd))} for _ in range(geom["n_layers"])]


def forward(x, P, geom: dict, cache: list, n_layers=None):
    """New rows x [n, D] (token embeddings) continuing one sequence whose cache
    holds its earlier positions -> logits [n, vocab]; the cache is extended."""
    L = geom["n_layers"] if n_layers is None else n_layers
    pos0 = cache[0]["K"].shape[0] if cache else 0  # a decoder of 0 layers keeps no cache
    x = np.asarray(x, dtype=np.float64)
    for l in range(L):
        x = layer_step(x, P, l, geom, cache[l], pos0)
    h = rms_norm(x, P["norm.weight"])
    return h @ P["embed.weight"].T


def embed(tokens, P):
    return P["embed.weight"][np.asarray(tokens, dtype=np.int64)]
