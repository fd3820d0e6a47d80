"""GPU parity of the 2x-front-end, full-attention encoder against the oracle
(oracle.encoder2x), through the C ABI.

  * a d = 256 geometry on a ragged packed batch (1, 2, 77, 300 and 513 mel
    frames: 1 to 257 encoder frames), full attention and a 64-frame window,
    fp16 and bf16 operands, with and without ln_post;
  * whisper-small geometry (12 layers, d 768, 12 heads) on one 30 s clip:
    1500 frames under full attention, the whole output against the oracle;
  * the 32 x 1280 geometry on the 16 x 30 s batch: a two-layer encoder
    against the oracle on sampled clips, and the full 32-layer encoder's
    batch rows equal (bitwise) to the same clip encoded alone;
  * packed == padded bitwise, and the stream entry point's rejection.
"""

import sys

import numpy as np
import pytest

import synth
from oracle import encoder as OE
from oracle import encoder2x as OE2
from tests.helpers import GpuModel, assert_bf16_rows, gpu_logmel, split_rows

pytestmark = pytest.mark.gpu

MID = dict(frontend="conv1d_2x", n_mels=128, conv_ch=256, d_model=256, n_layers=2, n_heads=4,
           head_dim=64, d_ffn=1024, d_out=256, adapter_hidden=0)
FULL_ATTN = 1 << 30


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def rand_mels(lens, seed):
    rng = np.random.default_rng(seed)
    return [(0.5 * rng.standard_normal((t, 128))).astype(np.float32) for t in lens]


@pytest.fixture(scope="module")
def mid_weights():
    return synth.make_weights(MID, bf16=True, seed=21, ln_random=True)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("window", [FULL_ATTN, 64])
def test_mid_geometry_ragged(mid_weights, dt, window):
    lens = [77, 1, 513, 2, 300]
    mels = rand_mels(lens, 3)
    say(f"2x d256: dt={dt} window={window} lens={lens}")
    model = GpuModel(MID, dt, mid_weights)
    out = model.encode(mels, window)
    ns = [OE2.frames_2x(t) for t in lens]
    assert out.shape == (sum(ns), 256)
    P = OE.as_f64(mid_weights)
    for i, (m, g) in enumerate(zip(mels, split_rows(out, ns))):
        ref = OE2.encode_clip_2x(m.astype(np.float64), P, MID,
                                 window=None if window == FULL_ATTN else window)
        r = assert_bf16_rows(g, ref, what=f"clip {i} (T={lens[i]})")
        say(f"  clip {i} T={lens[i]} N={ns[i]}: min cos {r['cos'].min():.6f} "
            f"worst {r['maxabs_rms'].max():.4f}")


def test_mid_geometry_stream_out_and_padded(mid_weights):
    import windowed_attention_audio_amd as W
    lens = [130, 41, 257]
    mels = rand_mels(lens, 4)
    say("2x d256: with_head=0, packed vs padded")
    model = GpuModel(MID, "f16", mid_weights, with_head=False)
    packed = model.encode(mels, FULL_ATTN)
    padded = model.encode(mels, FULL_ATTN, layout=W.MT_PADDED)
    ns = [OE2.frames_2x(t) for t in lens]
    P = OE.as_f64(mid_weights)
    for i, (m, g) in enumerate(zip(mels, split_rows(packed, ns))):
        ref = OE2.encode_clip_2x(m.astype(np.float64), P, MID, with_head=False)
        assert_bf16_rows(g, ref, what=f"residual stream clip {i}")
        assert np.array_equal(padded[i, :ns[i]], g)
        assert not padded[i, ns[i]:].any()


def test_whisper_small_30s():
    geom = synth.WHISPER_SMALL_GEOM
    w = synth.workload(2)
    clip = synth.make_clips(w)[0]
    say("whisper-small 30 s: GPU log-mel + encode")
    mel = gpu_logmel([clip])
    assert mel.shape == (3000, 128)
    weights = synth.make_weights(geom, bf16=True)
    model = GpuModel(geom, "f16", weights)
    out = model.encode([mel], FULL_ATTN)
    assert out.shape == (1500, 768)
    say("whisper-small 30 s: oracle")
    ref = OE2.encode_clip_2x(mel.astype(np.float64), OE.as_f64(weights), geom)
    r = assert_bf16_rows(out, ref, what="whisper-small 30 s")
    say(f"  min cos {r['cos'].min():.6f} worst {r['maxabs_rms'].max():.4f}")


@pytest.fixture(scope="module")
def batch16_mels():
    w = synth.workload(2)
    clips = synth.make_clips(w)
    mel = gpu_logmel(clips)
    return split_rows(mel, [len(c) // 160 for c in clips])


def test_large_geometry_16x30s_two_layers(batch16_mels):
    geom = dict(synth.WHISPER_LARGE_GEOM, n_layers=2)
    weights = synth.make_weights(geom, bf16=True)
    say("32x1280 geometry, 2 layers, 16 x 30 s")
    model = GpuModel(geom, "f16", weights)
    out = model.encode(batch16_mels, FULL_ATTN)
    ns = [OE2.frames_2x(m.shape[0]) for m in batch16_mels]
    assert out.shape == (16 * 1500, 1280)
    P = OE.as_f64(weights)
    rows = split_rows(out, ns)
    for i in (0, 9, 15):
        ref = OE2.encode_clip_2x(batch16_mels[i].astype(np.float64), P, geom)
        r = assert_bf16_rows(rows[i], ref, what=f"clip {i}")
        say(f"  clip {i}: min cos {r['cos'].min():.6f} worst {r['maxabs_rms'].max():.4f}")


def test_large_geometry_batch_equals_single(batch16_mels):
    geom = synth.WHISPER_LARGE_GEOM
    weights = synth.make_weights(geom, bf16=True)
    say("32x1280 geometry, 32 layers, 16 x 30 s vs clip 5 alone")
    model = GpuModel(geom, "f16", weights)
    out = model.encode(batch16_mels, FULL_ATTN)
    assert np.isfinite(out).all()
    alone = model.encode([batch16_mels[5]], FULL_ATTN)
    assert np.array_equal(out[5 * 1500:6 * 1500], alone)


def test_stream_rejects_2x(mid_weights):
    import torch
    import windowed_attention_audio_amd as W
    model = GpuModel(MID, "f16", mid_weights)
    wav = torch.zeros(16000, dtype=torch.float32, device="cuda")
    with pytest.raises(W.MtError) as e:
        W.mt_encode_stream(model.enc, wav, 64, 1)
    assert e.value.status == W.MT_ERR_UNSUPPORTED
