"""GPU parity at the workloads' full sizes, plus invariants of the HIP path.

  * 16 x 30 s batch: the whole batch on the GPU, sampled clips on the oracle;
  * 10-minute stream: the whole stream on the GPU, sampled windows on the
    oracle (each from its receptive field, an 8-frame halo of mel frames,
    encoded with the window's stream position);
  * 32 clips of 2..60 s, packed, window 52, with the SwiGLU adapter: the
    whole batch on the GPU, sampled clips on the oracle;
  * packed == padded, run-to-run determinism, window locality (bitwise), a
    workspace poisoned with NaN bytes, degenerate windows and lengths, and
    the host-side rejections.
"""

import sys

import numpy as np
import pytest

import synth
from oracle import encoder as OE
from oracle import logmel as OL
from tests.helpers import GpuModel, assert_bf16_rows, gpu_logmel, split_rows

pytestmark = pytest.mark.gpu

FULL = synth.FULL_GEOM


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
def model(weights_bf16):
    # bf16-valued weights, fp16 matrix operands, fp32 accumulation
    return GpuModel(FULL, "f16", weights_bf16)


def test_batch16x30s_sampled(model, P64):
    w = synth.workload(2)
    clips = synth.make_clips(w)
    say("16x30s: GPU log-mel + encode")
    mel = gpu_logmel(clips)
    T = [len(c) // 160 for c in clips]
    mels = split_rows(mel, T)
    got = model.encode(mels, w.window)
    assert got.shape == (6000, 2048)
    rows = split_rows(got, [375] * 16)
    for i in (0, 7, 15):
        ref = OE.encode_clip(OL.log_mel(clips[i]), P64, FULL, w.window)
        m = assert_bf16_rows(rows[i], ref, what=f"16x30s clip {i}")
        say(f"  clip {i}: min cos {m['cos'].min():.6f} max|d|/rms {m['maxabs_rms'].max():.4f}")


def test_stream_10min_sampled_windows(model, P64):
    w = synth.workload(3)
    wav = synth.make_clips(w)[0]
    say("10 min stream: GPU log-mel + encode")
    mel = gpu_logmel([wav])
    got = model.encode([mel], w.window)
    assert got.shape == (7500, 2048)
    ref_mel = OL.log_mel(wav)
    T, W = ref_mel.shape[0], w.window
    for k in (0, 1, 40, 72):
        s = max(0, 8 * (k * W - 1))
        e = min(T, 8 * (k + 1) * W + 8)
        seg = OE.encode_clip(ref_mel[s:e], P64, FULL, W, t0=s // 8)
        r0 = k * W - s // 8
        n = min(W, 7500 - k * W)
        m = assert_bf16_rows(got[k * W:k * W + n], seg[r0:r0 + n], what=f"stream window {k}")
        say(f"  window {k} ({n} rows): min cos {m['cos'].min():.6f} "
            f"max|d|/rms {m['maxabs_rms'].max():.4f}")


def test_varlen_packed_adapter_sampled(weights_bf16):
    w = synth.workload(4)
    geom = synth.geom_for(w)
    wts = synth.make_weights(geom, bf16=True)
    for k in weights_bf16:  # the tower is shared with the other workloads
        assert np.array_equal(wts[k], weights_bf16[k])
    ad = GpuModel(geom, "f16", wts)
    clips = synth.make_clips(w)
    say("32 varlen clips + adapter, W=52")
    mel = gpu_logmel(clips)
    T = [len(c) // 160 for c in clips]
    got = ad.encode(split_rows(mel, T), w.window)
    N = [OE.encoder_frames(t) for t in T]
    assert got.shape == (sum(N), 2048)
    rows = split_rows(got, N)
    P = OE.as_f64(wts)
    order = np.argsort(N)
    # shortest, median, longest, clip 9 (the worst of the bf16 operands) and two more
    for i in (int(order[0]), int(order[len(order) // 2]), int(order[-1]), 9, 5, 20):
        ref = OE.encode_clip(OL.log_mel(clips[i]), P, geom, w.window)
        m = assert_bf16_rows(rows[i], ref, what=f"varlen clip {i} (N={N[i]})")
        say(f"  clip {i} N={N[i]}: min cos {m['cos'].min():.6f} "
            f"max|d|/rms {m['maxabs_rms'].max():.4f}")


def _mels(seed, Ts):
    rng = np.random.default_rng(seed)
    return [rng.uniform(-1.0, 1.5, (t, 128)).astype(np.float32) for t in Ts]


def test_packed_equals_padded(model):
    mels = _mels(3, [3000, 1, 17, 800, 2999])
    a = model.encode(mels, 104, layout=0)
    b = model.encode(mels, 104, layout=1)
    N = [OE.encoder_frames(m.shape[0]) for m in mels]
    assert b.shape == (5, OE.encoder_frames(3000), 2048)
    for i, r in enumerate(split_rows(a, N)):
        assert np.array_equal(b[i, :N[i]], r)
        assert np.all(b[i, N[i]:] == 0)


def test_deterministic(model):
    mels = _mels(4, [3000, 1200])
    a = model.encode(mels, 104)
    b = model.encode(mels, 104)
    assert np.array_equal(a, b)


def test_window_locality_bitwise(model):
    W = 104
    mel = _mels(5, [3000])[0]
    base = model.encode([mel], W)
    for k in (0, 1, 3):
        m2 = mel.copy()
        lo, hi = 8 * k * W, min(2999, 8 * (k + 1) * W - 8)
        m2[lo:hi + 1] += 0.5
        out = model.encode([m2], W)
        inside = np.zeros(375, bool)
        inside[k * W:min(375, (k + 1) * W)] = True
        assert np.array_equal(out[~inside], base[~inside]), f"window {k} leaked"
        assert np.abs(out[inside] - base[inside]).max() > 1e-3


def test_poisoned_workspace(model):
    import torch
    import windowed_attention_audio_amd as W
    mels = _mels(6, [3000, 640])
    ref = model.encode(mels, 104)
    lens = [m.shape[0] for m in mels]
    mel = torch.from_numpy(np.concatenate(mels)).cuda()
    ws = torch.full((W.mt_encode_workspace_size(model.enc, lens, 104),), 255, dtype=torch.uint8,
                    device="cuda")
    out = torch.full((sum(OE.encoder_frames(t) for t in lens), 2048), float("nan"),
                     device="cuda")
    W.mt_encode(model.enc, mel, lens, 104, out=out, ws=ws)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), ref)


def test_degenerate_windows_and_lengths(model, P64):
    mels = _mels(7, [1, 9, 200])
    N = [OE.encoder_frames(m.shape[0]) for m in mels]
    assert N == [1, 2, 25]
    for W in (1, 2, 25, 1000):
        got = split_rows(model.encode(mels, W), N)
        for g, m in zip(got, mels):
            ref = OE.encode_clip(m.astype(np.float64), P64, FULL, W)
            assert_bf16_rows(g, ref, what=f"W={W} T={m.shape[0]}")


def test_rejections(model):
    import torch
    import windowed_attention_audio_amd as W
    mel = torch.zeros((3000, 128), device="cuda")
    # fp32 encoders keep every window's keys on chip: 375 frames > 256 is refused
    geom1 = dict(FULL, n_layers=1)
    names = [n for n, _ in synth.weight_names(geom1)]
    w32 = synth.make_weights(geom1, bf16=False)
    m32 = GpuModel(geom1, "f32", {n: w32[n] for n in names})
    with pytest.raises(W.MtError) as e:
        W.mt_encode(m32.enc, mel, [3000], 300)
    assert e.value.status == W.MT_ERR_UNSUPPORTED
    with pytest.raises(W.MtError) as e:
        W.mt_encode(model.enc, mel, [3000], 0)
    assert e.value.status == W.MT_ERR_INVALID_ARG
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(W.MtError) as e:
        W.mt_encode(model.enc, mel, [3000], 104, ws=ws)
    assert e.value.status == W.MT_ERR_WORKSPACE
    with pytest.raises(W.MtError) as e:
        W.mt_logmel(torch.zeros(200, device="cuda"), [200])
    assert e.value.status == W.MT_ERR_INVALID_ARG


def test_long_windows_30s(model, P64):
    # windows longer than the 256 frames kept on chip stream their keys:
    # W = 300 (windows of 300 and 75) and W >= N (full attention, 375 frames)
    w = synth.workload(1)
    mel = OL.log_mel(synth.make_clips(w)[0])
    for W in (300, 1000):
        say(f"30 s clip, W = {W}")
        got = model.encode([mel], W)
        ref = OE.encode_clip(mel, P64, FULL, W)
        m = assert_bf16_rows(got, ref, what=f"W={W}")
        say(f"  min cos {m['cos'].min():.6f} max|d|/rms {m['maxabs_rms'].max():.4f}")


def test_long_windows_varlen_one_layer():
    # one layer with random LayerNorm parameters, a packed batch whose clips are
    # shorter than, equal to and longer than the window; W = 600 and 2000
    geom = dict(FULL, n_layers=1)
    wts = synth.make_weights(geom, bf16=True, ln_random=True)
    model1 = GpuModel(geom, "f16", wts)
    P = OE.as_f64(wts)
    mels = _mels(11, [6000, 77, 4801, 2100])
    N = [OE.encoder_frames(m.shape[0]) for m in mels]
    for W in (600, 2000):
        got = split_rows(model1.encode(mels, W), N)
        for g, m in zip(got, mels):
            ref = OE.encode_clip(m.astype(np.float64), P, geom, W)
            assert_bf16_rows(g, ref, what=f"1 layer W={W} T={m.shape[0]}")


def _full_stream(model, wav, W):
    mel = gpu_logmel([wav])
    return model.encode([mel], W)


def test_stream_chunked_equals_whole(model):
    # mt_encode_stream (bounded workspace, chunk by chunk) against mt_logmel +
    # mt_encode of the whole 10-minute stream: bitwise equal
    import torch
    import windowed_attention_audio_amd as W
    w = synth.workload(3)
    wav = synth.make_clips(w)[0]
    full = _full_stream(model, wav, w.window)
    dwav = torch.from_numpy(wav).cuda()
    for cw in (1, 5, 1000):
        say(f"10 min stream, {cw} window(s) per chunk")
        got = W.mt_encode_stream(model.enc, dwav, w.window, cw)
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy(), full), f"chunk_windows={cw}"
    # the workspace does not grow with the stream
    n = len(wav)
    assert (W.mt_encode_stream_workspace_size(model.enc, n, w.window, 5)
            == W.mt_encode_stream_workspace_size(model.enc, 6 * n, w.window, 5))


def test_stream_short_and_ragged(model):
    import torch
    import windowed_attention_audio_amd as W
    rng = np.random.default_rng(12)
    for n, Wn, cw in ((201, 104, 1), (16000, 104, 1), (16000 * 7 + 77, 3, 2), (16000 * 20 + 159, 52, 3)):
        wav = (rng.standard_normal(n) * 0.2).astype(np.float32)
        full = _full_stream(model, wav, Wn)
        got = W.mt_encode_stream(model.enc, torch.from_numpy(wav).cuda(), Wn, cw).cpu().numpy()
        assert np.array_equal(got, full), f"n={n} W={Wn} chunk_windows={cw}"


def test_stream_rejections(model):
    import torch
    import windowed_attention_audio_amd as W
    wav = torch.zeros(16000, device="cuda")
    for args, status in (((200, 104, 1), W.MT_ERR_INVALID_ARG), ((16000, 0, 1), W.MT_ERR_INVALID_ARG),
                         ((16000, 104, 0), W.MT_ERR_INVALID_ARG)):
        with pytest.raises(W.MtError) as e:
            W.mt_encode_stream_workspace_size(model.enc, *args)
        assert e.value.status == status
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(W.MtError) as e:
        W.mt_encode_stream(model.enc, wav, 104, 1, ws=ws)
    assert e.value.status == W.MT_ERR_WORKSPACE
