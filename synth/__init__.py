"""Seeded synthetic inputs: waveforms, clip durations and model weights.

This module only draws random numbers and lays them out.  It holds none of the
encoder's arithmetic, so the oracle and the HIP path can both take their inputs
from it without sharing any part of the computation.

Workloads (the model card "MOSS-Transcribe-preview-2B-GGUF", Architecture
table: 16 kHz mono audio, 128 mel bins, the encoder geometry):

  c0  1 s clip, batch 1, computed in fp32
  c1  30 s clip, batch 1, bf16 weights and activations
  c2  16 clips of 30 s, bf16 (throughput workload)
  c3  one 10-minute stream, bf16
  c4  32 clips of uniform 2..60 s, packed, window 52, SwiGLU adapter, bf16

Signal recipe: the sum of three sinusoids of amplitude 0.2 with frequencies
drawn uniformly in [100, 4000] Hz and zero phase, plus Gaussian noise of
standard deviation 0.01, clipped to [-1, 1].  With gaps, the clip is cut into
0.5 s blocks (8000 samples, the last one possibly shorter) and round(0.2 x
#blocks) of them, drawn without replacement, are set to exactly zero.  Draw
order per clip: frequencies, noise, gap blocks.  These inputs stand in for the
pages' own audio (a speech sample and a long meeting-recording benchmark),
which is not available here.

Weight recipe, in canonical order (the order the C-ABI's weight array uses):
linear weights and every bias ~ N(0, 0.02^2); convolution weights ~
N(0, 1/fan_in) (variance 1/fan_in); LayerNorm gamma = 1, beta = 0 unless
``ln_random`` is set (then gamma = 1 + N(0, 0.1^2), beta = N(0, 0.1^2), used
only to make sure gamma and beta are really applied).  For bf16 workloads
the fp32 draws are rounded to the nearest bf16 (ties to even) once, here, so
both sides start from the same bf16 weight values.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

SR = 16000
HOP = 160

FULL_GEOM = dict(
    n_mels=128,
    conv_ch=480,
    d_model=1280,
    n_layers=32,
    n_heads=20,
    head_dim=64,
    d_ffn=5120,
    d_out=2048,
    adapter_hidden=0,
)

# The full-attention variant with the 2x conv front-end, at the two whisper
# geometries the CrisperWhisper export page names (small: 12 layers, d 768,
# 12 heads; large-v3: 32 layers at the tower's 32 x 1280 geometry).  FFN 4d
# and 128 mel bins are readings (the page gives neither).
WHISPER_SMALL_GEOM = dict(
    frontend="conv1d_2x", n_mels=128, conv_ch=768, d_model=768, n_layers=12, n_heads=12,
    head_dim=64, d_ffn=3072, d_out=768, adapter_hidden=0,
)
WHISPER_LARGE_GEOM = dict(
    frontend="conv1d_2x", n_mels=128, conv_ch=1280, d_model=1280, n_layers=32, n_heads=20,
    head_dim=64, d_ffn=5120, d_out=1280, adapter_hidden=0,
)

# The language-model decoder of the model card (Architecture table, row LLM):
# Qwen3-1.7B geometry, vocabulary 151 936.
DEC_GEOM = dict(
    vocab=151936, d_model=2048, n_layers=28, n_heads=16, n_kv_heads=8, head_dim=128, d_ffn=6144,
)

WEIGHT_SEED = 1234
ADAPTER_SEED = 1235


@dataclass
class Workload:
    cid: int
    name: str
    n_samples: list
    gaps: bool
    dtype: str  # "f32" | "bf16"
    window: int
    adapter_hidden: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def audio_seconds(self) -> float:
        return float(sum(self.n_samples)) / SR


def c4_durations() -> np.ndarray:
    """32 clip durations in seconds, uniform in [2, 60], seeded."""
    rng = np.random.Generator(np.random.PCG64([4, 999]))
    return rng.uniform(2.0, 60.0, size=32)


def workload(cid: int) -> Workload:
    if cid == 0:
        return Workload(0, "1s_clip_fp32", [16000], False, "f32", 104)
    if cid == 1:
        return Workload(1, "30s_clip_bf16", [480000], True, "bf16", 104)
    if cid == 2:
        return Workload(2, "16x30s_bf16", [480000] * 16, True, "bf16", 104)
    if cid == 3:
        return Workload(3, "600s_stream_bf16", [9600000], True, "bf16", 104)
    if cid == 4:
        n = [int(math.floor(SR * d)) for d in c4_durations()]
        return Workload(4, "32_varlen_packed_adapter_bf16", n, True, "bf16", 52,
                        adapter_hidden=8192)
    raise ValueError(f"unknown workload {cid}")


def make_clip(cid: int, clip_idx: int, n_samples: int, gaps: bool) -> np.ndarray:
    """One synthetic 16 kHz clip as float32, seeded by (workload, clip index)."""
    rng = np.random.Generator(np.random.PCG64([cid, clip_idx]))
    freqs = rng.uniform(100.0, 4000.0, size=3)
    t = np.arange(n_samples, dtype=np.float64)
    sig = np.zeros(n_samples, dtype=np.float64)
    for f in freqs:
        sig += 0.2 * np.sin(2.0 * np.pi * f * t / SR)
    sig += rng.normal(0.0, 0.01, size=n_samples)
    np.clip(sig, -1.0, 1.0, out=sig)
    if gaps:
        nblk = -(-n_samples // 8000)
        nz = int(round(0.2 * nblk))
        if nz > 0:
            for b in rng.choice(nblk, size=nz, replace=False):
                sig[b * 8000:(b + 1) * 8000] = 0.0
    return sig.astype(np.float32)


def make_clips(w: Workload) -> list:
    return [make_clip(w.cid, i, n, w.gaps) for i, n in enumerate(w.n_samples)]


def tone(freq_hz: float, n_samples: int, amp: float = 0.2) -> np.ndarray:
    """A pure cosine, float64 (used by front-end tests)."""
    t = np.arange(n_samples, dtype=np.float64)
    return amp * np.cos(2.0 * np.pi * freq_hz * t / SR)


# --------------------------------------------------------------------------
# weights


def weight_names(geom: dict) -> list:
    """Canonical tensor order, with shapes (torch/nn conventions: Linear
    weights are [out, in]; Conv2d weights are [out, in, kh(freq), kw(time)])."""
    C = geom["conv_ch"]
    F8 = geom["n_mels"] // 8
    D = geom["d_model"]
    H = geom["d_ffn"]
    O = geom["d_out"]
    two_x = geom.get("frontend", "conv2d_8x") == "conv1d_2x"
    if two_x:  # Conv1d weights are [out, in, k(time)]
        out = [
            ("conv1.weight", (D, geom["n_mels"], 3)), ("conv1.bias", (D,)),
            ("conv2.weight", (D, D, 3)), ("conv2.bias", (D,)),
        ]
    else:
        out = [
            ("conv1.weight", (C, 1, 3, 3)), ("conv1.bias", (C,)),
            ("conv2.weight", (C, C, 3, 3)), ("conv2.bias", (C,)),
            ("conv3.weight", (C, C, 3, 3)), ("conv3.bias", (C,)),
            ("conv_out.weight", (D, C * F8)),
        ]
    for l in range(geom["n_layers"]):
        p = f"layers.{l}."
        out += [
            (p + "ln1.weight", (D,)), (p + "ln1.bias", (D,)),
            (p + "q.weight", (D, D)), (p + "q.bias", (D,)),
            (p + "k.weight", (D, D)), (p + "k.bias", (D,)),
            (p + "v.weight", (D, D)), (p + "v.bias", (D,)),
            (p + "o.weight", (D, D)), (p + "o.bias", (D,)),
            (p + "ln2.weight", (D,)), (p + "ln2.bias", (D,)),
            (p + "fc1.weight", (H, D)), (p + "fc1.bias", (H,)),
            (p + "fc2.weight", (D, H)), (p + "fc2.bias", (D,)),
        ]
    out += [("ln_post.weight", (D,)), ("ln_post.bias", (D,))]
    if two_x:
        return out
    out += [
        ("proj1.weight", (D, D)), ("proj1.bias", (D,)),
        ("proj2.weight", (O, D)), ("proj2.bias", (O,)),
    ]
    A = geom.get("adapter_hidden", 0)
    if A:
        out += [
            ("adapter.gate.weight", (A, O)),
            ("adapter.up.weight", (A, O)),
            ("adapter.down.weight", (O, A)),
        ]
    return out


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 value (ties to even), returned as fp32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def make_weights(geom: dict, bf16: bool, seed: int = WEIGHT_SEED,
                 adapter_seed: int = ADAPTER_SEED, ln_random: bool = False) -> dict:
    """Seeded weights as an ordered dict name -> float32 array."""
    rng = np.random.Generator(np.random.PCG64(seed))
    arng = np.random.Generator(np.random.PCG64(adapter_seed))
    lrng = np.random.Generator(np.random.PCG64([seed, 7]))
    out = {}
    for name, shape in weight_names(geom):
        if name.startswith("adapter."):
            a = arng.standard_normal(shape, dtype=np.float32) * np.float32(0.02)
        elif name.split(".")[-2].startswith("ln") or name.startswith("ln_post"):
            if ln_random:
                if name.endswith("weight"):
                    a = (1.0 + 0.1 * lrng.standard_normal(shape)).astype(np.float32)
                else:
                    a = (0.1 * lrng.standard_normal(shape)).astype(np.float32)
            else:
                a = (np.ones if name.endswith("weight") else np.zeros)(shape, np.float32)
        elif name.startswith("conv") and name.endswith(".weight") and len(shape) >= 3:
            fan_in = int(np.prod(shape[1:]))
            a = rng.standard_normal(shape, dtype=np.float32) * np.float32(1.0 / math.sqrt(fan_in))
        else:
            a = rng.standard_normal(shape, dtype=np.float32) * np.float32(0.02)
        if bf16:
            a = round_to_bf16(a)
        out[name] = np.ascontiguousarray(a, dtype=np.float32)
    return out


def with_adapter(weights: dict, geom: dict, bf16: bool, adapter_seed: int = ADAPTER_SEED) -> dict:
    """The weights of geom given those of the same geometry without the
    adapter: the encoder tensors reused, the adapter tensors drawn as
    make_weights draws them (their own generator), so the result equals
    make_weights(geom, bf16) without drawing the encoder again."""
    arng = np.random.Generator(np.random.PCG64(adapter_seed))
    out = {}
    for name, shape in weight_names(geom):
        if name.startswith("adapter."):
            a = arng.standard_normal(shape, dtype=np.float32) * np.float32(0.02)
            if bf16:
                a = round_to_bf16(a)
            out[name] = np.ascontiguousarray(a, dtype=np.float32)
        else:
            out[name] = weights[name]
    return out


def geom_for(w: Workload, **over) -> dict:
    g = dict(FULL_GEOM)
    g["adapter_hidden"] = w.adapter_hidden
    g.update(over)
    return g


def prompt_tokens(n_audio: int, vocab: int, audio_token: int, seed: int = 77) -> list:
    """A synthetic prompt in the model card's ChatML shape (Architecture
    table, row Prompt): some text tokens, a run of n_audio audio placeholders,
    more text tokens.  Text ids are seeded draws from [0, vocab) other than
    audio_token (no tokenizer is available; the ids only need to be valid)."""
    rng = np.random.Generator(np.random.PCG64(seed))

    def text(k):
        t = rng.integers(0, vocab - 1, k)
        return [int(x) + (1 if x >= audio_token else 0) for x in t]

    return text(7) + [audio_token] * n_audio + text(9)


# --------------------------------------------------------------------------
# decoder weights


def decoder_weight_names(geom: dict) -> list:
    """Canonical tensor order of the decoder, with shapes (Linear weights
    [out, in], no biases)."""
    V, D, F = geom["vocab"], geom["d_model"], geom["d_ffn"]
    Hq, Hkv, hd = geom["n_heads"], geom["n_kv_heads"], geom["head_dim"]
    out = [("embed.weight", (V, D))]
    for l in range(geom["n_layers"]):
        p = f"layers.{l}."
        out += [
            (p + "input_norm.weight", (D,)),
            (p + "q.weight", (Hq * hd, D)), (p + "k.weight", (Hkv * hd, D)), (p + "v.weight", (Hkv * hd, D)),
            (p + "q_norm.weight", (hd,)), (p + "k_norm.weight", (hd,)),
            (p + "o.weight", (D, Hq * hd)),
            (p + "post_norm.weight", (D,)),
            (p + "gate.weight", (F, D)), (p + "up.weight", (F, D)), (p + "down.weight", (D, F)),
        ]
    out.append(("norm.weight", (D,)))
    return out


def make_decoder_weights(geom: dict, bf16: bool = True, seed: int = 4321) -> dict:
    """Seeded decoder weights, name -> float32 array: matrices N(0, 0.02^2)
    (the embedding N(0, 1): its rows are the inputs), norm weights
    1 + N(0, 0.1^2); bf16-valued when bf16."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {}
    for name, shape in decoder_weight_names(geom):
        if len(shape) == 1:
            a = (1.0 + 0.1 * rng.standard_normal(shape)).astype(np.float32)
        elif name == "embed.weight":
            a = rng.standard_normal(shape, dtype=np.float32)
        else:
            a = rng.standard_normal(shape, dtype=np.float32) * np.float32(0.02)
        if bf16:
            a = round_to_bf16(a)
        out[name] = np.ascontiguousarray(a, dtype=np.float32)
    return out
