"""GPU parity, full-size workloads: every clip of the 16 x 30 s batch, bf16
matrix operands, and the bounded-memory stream against the oracle.

  * each of the 16 clips of the 16 x 30 s batch, encoded alone through all 32
    layers, equals its rows of the batch bitwise (fp16 and bf16 operands), so
    the oracle-sampled clips stand for every clip of the batch; the same for
    the 32 variable-length clips with the adapter;
  * bf16 activations at the matrix cores (MT_BF16): the 16 x 30 s batch and
    the 10-minute stream within the parity bar; the 32-clip adapter workload
    outside it (documented, bounded);
  * mt_encode_stream (the 10-minute stream chunk by chunk) against the
    oracle: the oracle's log-mel of the whole stream, each sampled window
    encoded from its receptive field with the window's stream position.
"""

import sys

import numpy as np
import pytest

import synth
from oracle import encoder as OE
from oracle import logmel as OL
from tests.helpers import GpuModel, assert_bf16_rows, gpu_logmel, row_metrics, split_rows

pytestmark = pytest.mark.gpu

FULL = synth.FULL_GEOM

# bf16 activations on the adapter workload: max |diff| / RMS measured 0.027
# (clip 9); the bound keeps a regression from going unnoticed, it is not the
# parity bar (0.02), which this operand type does not meet there.
BF16_ADAPTER_BOUND = 0.035


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(scope="module")
def weights_bf16():
    return synth.make_weights(FULL, bf16=True)


@pytest.fixture(scope="module")
def P64(weights_bf16):
    return OE.as_f64(weights_bf16)


@pytest.fixture(scope="module")
def models(weights_bf16):
    return {"f16": GpuModel(FULL, "f16", weights_bf16), "bf16": GpuModel(FULL, "bf16", weights_bf16)}


@pytest.fixture(scope="module")
def batch16():
    w = synth.workload(2)
    clips = synth.make_clips(w)
    mel = gpu_logmel(clips)
    return w, clips, split_rows(mel, [len(c) // 160 for c in clips])


@pytest.fixture(scope="module")
def stream10():
    w = synth.workload(3)
    wav = synth.make_clips(w)[0]
    return w, wav, OL.log_mel(wav)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_batch16x30s_every_clip_alone_bitwise(models, batch16, dt):
    w, _, mels = batch16
    m = models[dt]
    say(f"16x30s ({dt}): batch vs each clip alone")
    rows = split_rows(m.encode(mels, w.window), [375] * 16)
    for i, mel in enumerate(mels):
        alone = m.encode([mel], w.window)
        assert np.array_equal(alone, rows[i]), f"clip {i}: alone != its rows in the batch"


def test_bf16_batch16x30s_sampled(models, batch16, P64):
    w, clips, mels = batch16
    got = split_rows(models["bf16"].encode(mels, w.window), [375] * 16)
    for i in (0, 7, 15):
        ref = OE.encode_clip(OL.log_mel(clips[i]), P64, FULL, w.window)
        m = assert_bf16_rows(got[i], ref, what=f"bf16 16x30s clip {i}")
        say(f"  bf16 clip {i}: min cos {m['cos'].min():.6f} max|d|/rms {m['maxabs_rms'].max():.4f}")


def _stream_windows(got, ref_mel, P64, W, windows, N):
    T = ref_mel.shape[0]
    for k in windows:
        s = max(0, 8 * (k * W - 1))
        e = min(T, 8 * (k + 1) * W + 8)
        seg = OE.encode_clip(ref_mel[s:e], P64, FULL, W, t0=s // 8)
        r0 = k * W - s // 8
        n = min(W, N - k * W)
        yield k, got[k * W:k * W + n], seg[r0:r0 + n]


def test_bf16_stream_10min_sampled_windows(models, stream10, P64):
    w, wav, ref_mel = stream10
    say("bf16 10 min stream")
    got = models["bf16"].encode([gpu_logmel([wav])], w.window)
    assert got.shape == (7500, 2048)
    for k, g, r in _stream_windows(got, ref_mel, P64, w.window, (0, 1, 40, 72), 7500):
        m = assert_bf16_rows(g, r, what=f"bf16 stream window {k}")
        say(f"  window {k}: min cos {m['cos'].min():.6f} max|d|/rms {m['maxabs_rms'].max():.4f}")


@pytest.mark.parametrize("cw", [5, 1])
def test_encode_stream_vs_oracle(models, stream10, P64, cw):
    # the bounded-memory path itself (not the whole-stream path) against the
    # oracle's definition of the stream's windows
    import torch
    import windowed_attention_audio_amd as W
    w, wav, ref_mel = stream10
    say(f"mt_encode_stream, {cw} window(s) per chunk, vs oracle")
    got = W.mt_encode_stream(models["f16"].enc, torch.from_numpy(wav).cuda(), w.window, cw)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    assert got.shape == (7500, 2048)
    for k, g, r in _stream_windows(got, ref_mel, P64, w.window, (0, 1, 40, 72), 7500):
        m = assert_bf16_rows(g, r, what=f"stream chunk_windows={cw} window {k}")
        say(f"  window {k}: min cos {m['cos'].min():.6f} max|d|/rms {m['maxabs_rms'].max():.4f}")


def test_varlen_adapter_every_clip_alone_bitwise(weights_bf16):
    # the 32 variable-length clips of 2-60 s with the adapter, window 52:
    # each clip encoded alone (its products on the small-row kernels) equals
    # its rows of the packed batch (13 613 rows: the 256-row kernels)
    # bitwise, so the clips the oracle samples stand for all 32
    w = synth.workload(4)
    geom = synth.geom_for(w)
    wts = synth.with_adapter(weights_bf16, geom, bf16=True)
    ad = GpuModel(geom, "f16", wts)
    clips = synth.make_clips(w)
    mel = gpu_logmel(clips)
    T = [len(c) // 160 for c in clips]
    N = [OE.encoder_frames(t) for t in T]
    mels = split_rows(mel, T)
    say(f"32 varlen clips + adapter: batch ({sum(N)} rows) vs each clip alone")
    rows = split_rows(ad.encode(mels, w.window), N)
    for i, m in enumerate(mels):
        alone = ad.encode([m], w.window)
        assert np.array_equal(alone, rows[i]), f"clip {i} (N={N[i]}): alone != its rows in the batch"


def test_bf16_varlen_adapter_outside_bar(weights_bf16):
    # bf16 activations through the SwiGLU adapter: the product of the gate
    # and up projections doubles the tower's relative error, which puts the
    # worst row past the 0.02 bar.  Cosine still meets its bar; max|d|/RMS is
    # held to a documented bound.
    w = synth.workload(4)
    geom = synth.geom_for(w)
    wts = synth.with_adapter(weights_bf16, geom, bf16=True)
    ad = GpuModel(geom, "bf16", wts)
    clips = synth.make_clips(w)
    mel = gpu_logmel(clips)
    T = [len(c) // 160 for c in clips]
    N = [OE.encoder_frames(t) for t in T]
    got = split_rows(ad.encode(split_rows(mel, T), w.window), N)
    P = OE.as_f64(wts)
    worst = 0.0
    for i in (9, 6, 20):
        ref = OE.encode_clip(OL.log_mel(clips[i]), P, geom, w.window)
        m = row_metrics(got[i], ref)
        say(f"  bf16 adapter clip {i}: min cos {m['cos'].min():.6f} max|d|/rms {m['maxabs_rms'].max():.4f}")
        assert m["cos"].min() >= 0.999
        worst = max(worst, float(m["maxabs_rms"].max()))
    assert worst <= BF16_ADAPTER_BOUND


def test_fp16_saturation_is_reported(weights_bf16):
    # fp16 operands clamp at +-65504; the clamp must be reported in the
    # workspace's saturation mask, not pass silently.  One layer whose fc1
    # weights are scaled by 2^17 (exact in bf16 and fp16) drives the FFN hidden
    # activations far past the fp16 range.
    import torch
    import windowed_attention_audio_amd as W
    geom = dict(FULL, n_layers=1)
    names = [n for n, _ in synth.weight_names(geom)]
    base = {n: weights_bf16[n] for n in names}
    big = dict(base)
    big["layers.0.fc1.weight"] = (base["layers.0.fc1.weight"] * np.float32(2.0 ** 17)).astype(np.float32)
    mel = torch.from_numpy(OL.log_mel(synth.make_clips(synth.workload(1))[0]).astype(np.float32)).cuda()
    T = [mel.shape[0]]

    def mask(weights, dt):
        m = GpuModel(geom, dt, weights)
        ws = torch.full((W.mt_encode_workspace_size(m.enc, T, 104),), 255, dtype=torch.uint8, device="cuda")
        out = W.mt_encode(m.enc, mel, T, 104, ws=ws)
        return W.saturation_mask(ws), out

    assert mask(base, "f16")[0] == 0
    got, out = mask(big, "f16")
    say(f"  fp16 mask with fc1 x 2^17: {got}")
    assert got & W.MT_SAT_FFN
    assert bool(torch.isfinite(out).all())  # clamped, not inf
    assert mask(big, "bf16")[0] == 0  # bf16 keeps fp32's range: nothing clamps
    # the stream path reports into the first word of its own workspace
    m = GpuModel(geom, "f16", big)
    wav = torch.from_numpy(synth.make_clips(synth.workload(1))[0]).cuda()
    ws = torch.full((W.mt_encode_stream_workspace_size(m.enc, wav.numel(), 104, 1),), 255, dtype=torch.uint8,
                    device="cuda")
    W.mt_encode_stream(m.enc, wav, 104, 1, ws=ws)
    assert W.saturation_mask(ws) & W.MT_SAT_FFN


# One weight tensor per stage scaled by a power of two (an exponent shift:
# exact in bf16 and fp16; 2^15 for the tensors with entries near 1, so that
# every scaled entry stays below 65504) drives that stage's fp16 outputs past
# the fp16 range.  Each case must set its stage's
# bit; the front-end lies upstream of every other stage, so only the
# front-end cases may set the front-end bit.  The batch of 16 clips runs the
# 256-row tile kernels (their staged epilogues), the single clip the small
# tiles.
SAT_CASES = [
    ("conv1.weight", 15, "MT_SAT_FRONTEND"),
    ("conv2.weight", 17, "MT_SAT_FRONTEND"),
    ("conv3.weight", 17, "MT_SAT_FRONTEND"),
    ("layers.0.ln1.weight", 15, "MT_SAT_LN"),
    ("layers.0.q.weight", 17, "MT_SAT_QKV"),
    ("layers.0.fc1.weight", 17, "MT_SAT_FFN"),
    ("ln_post.weight", 15, "MT_SAT_HEAD"),
    ("proj1.weight", 17, "MT_SAT_HEAD"),
    ("proj2.weight", 17, "MT_SAT_ADAPTER"),
    ("adapter.gate.weight", 17, "MT_SAT_ADAPTER"),
]


@pytest.fixture(scope="module")
def sat_setup():
    import torch
    geom = synth.geom_for(synth.workload(4), n_layers=1)  # with the adapter
    base = synth.with_adapter(synth.make_weights(geom, bf16=True), geom, bf16=True)
    clips = synth.make_clips(synth.workload(2))
    # packed log-mel rows [sum T, 128] with their per-clip frame counts
    mels = {"16x30s": (gpu_logmel(clips), [len(c) // 160 for c in clips]),
            "1x30s": (gpu_logmel(clips[:1]), [len(clips[0]) // 160])}
    torch.cuda.synchronize()
    return geom, base, mels


@pytest.mark.parametrize("batch", ["16x30s", "1x30s"])
@pytest.mark.parametrize("name,e,bit", SAT_CASES)
def test_fp16_saturation_bit_per_stage(sat_setup, batch, name, e, bit):
    import torch
    import windowed_attention_audio_amd as W
    geom, base, mels = sat_setup
    mel, T = mels[batch]
    assert mel.shape == (sum(T), 128)
    scaled = dict(base)
    v = base[name] * np.float32(2.0 ** e)
    assert float(np.abs(v).max()) < 65504.0
    scaled[name] = v.astype(np.float32)

    def run(weights):
        m = GpuModel(geom, "f16", weights)
        ws = torch.full((W.mt_encode_workspace_size(m.enc, T, 104),), 255, dtype=torch.uint8, device="cuda")
        out = W.mt_encode(m.enc, torch.from_numpy(mel).cuda(), T, 104, ws=ws)
        torch.cuda.synchronize()
        return W.saturation_mask(ws), out

    if name == SAT_CASES[0][0]:
        assert run(base)[0] == 0
    got, out = run(scaled)
    say(f"  {batch} {name} x 2^{e}: mask {got}")
    assert got & getattr(W, bit), f"{name}: {bit} not reported (mask {got})"
    if bit != "MT_SAT_FRONTEND":
        assert not got & W.MT_SAT_FRONTEND
    assert bool(torch.isfinite(out).all())  # clamped, not inf
