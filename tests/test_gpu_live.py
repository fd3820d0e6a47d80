"""GPU: live encoding of a stream whose audio arrives piece by piece
(mt_stream_open / push / finish) against the oracle's reading of the clip
maximum as a causal running maximum (oracle.live), plus the properties that
reading implies:

  * the 10-minute stream pushed in seeded pieces of 0.2 .. 20 s: sampled
    windows against the oracle;
  * the split into pushes does not matter (bitwise);
  * with the loudest frame at the start, every window equals mt_encode_stream
    over the whole stream (bitwise: the same chunk arithmetic and maximum);
  * a loud burst late in the stream: windows before it (lower maximum) and
    after it against the oracle;
  * streams that end before a full window, and the shortest legal stream.
"""

import math
import sys

import numpy as np
import pytest

import synth
from oracle import encoder as OE
from oracle import live as LV
from tests.helpers import GpuModel, assert_bf16_rows

pytestmark = pytest.mark.gpu

FULL = synth.FULL_GEOM
MAX_PUSH = 16000 * 20


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
    return GpuModel(FULL, "f16", weights_bf16)


def run_live(model, wav, window, sizes):
    """Pushes wav in pieces of the given sizes (cycled), then finishes;
    returns the concatenated frames (numpy)."""
    import torch
    import windowed_attention_audio_amd as W
    st = W.LiveStream(model.enc, window, MAX_PUSH)
    dwav = torch.from_numpy(wav).cuda()
    outs, i, j = [], 0, 0
    while i < len(wav):
        n = min(sizes[j % len(sizes)], len(wav) - i)
        outs.append(st.push(dwav[i:i + n]).clone())
        i += n
        j += 1
    outs.append(st.finish().clone())
    torch.cuda.synchronize()
    st.close()
    return torch.cat(outs).cpu().numpy()


def seeded_sizes(seed, lo=0.2, hi=20.0, count=200):
    rng = np.random.default_rng(seed)
    return [int(16000 * s) for s in rng.uniform(lo, hi, size=count)]


def windows_vs_oracle(got, wav, P64, window, ks, what):
    L = LV.raw_log_mel(wav)
    ref = LV.encode_live(wav, P64, FULL, window, windows=ks, L=L)
    for k in ks:
        g = got[k * window:k * window + ref[k].shape[0]]
        m = assert_bf16_rows(g, ref[k], what=f"{what} window {k}")
        say(f"  {what} window {k}: min cos {m['cos'].min():.6f} max|d|/rms {m['maxabs_rms'].max():.4f}")


@pytest.fixture(scope="module")
def stream10():
    return synth.make_clips(synth.workload(3))[0]


def test_live_10min_stream_vs_oracle_and_push_sizes(model, P64, stream10):
    wav = stream10
    say("live 10 min stream, seeded pushes of 0.2 .. 20 s")
    a = run_live(model, wav, 104, seeded_sizes(1))
    assert a.shape == (7500, 2048)
    windows_vs_oracle(a, wav, P64, 104, (0, 1, 40, 72), "live")
    say("live 10 min stream, 1 s pushes")
    b = run_live(model, wav, 104, [16000])
    assert np.array_equal(a, b), "the result depends on how the audio was pushed"


def test_live_equals_encode_stream_when_loudest_first(model):
    import torch
    import windowed_attention_audio_amd as W
    wav = synth.make_clips(synth.workload(3))[0][:16000 * 90].copy()
    t = np.arange(4000) / 16000.0
    wav[1000:5000] += (0.9 * np.sin(2 * np.pi * 1000.0 * t)).astype(np.float32)  # the loudest frames, first window
    say("live vs mt_encode_stream, loudest frame first")
    got = run_live(model, wav, 104, seeded_sizes(2, 0.05, 7.0))
    ref = W.mt_encode_stream(model.enc, torch.from_numpy(wav).cuda(), 104, 1)
    torch.cuda.synchronize()
    assert np.array_equal(got, ref.cpu().numpy())


def test_live_late_burst_vs_oracle(model, P64):
    wav = synth.make_clips(synth.workload(3))[0][:16000 * 60].copy()
    b0 = 16000 * 30  # the burst lands in window 3's range (windows of 104 x 80 ms = 8.32 s)
    t = np.arange(8000) / 16000.0
    wav[b0:b0 + 8000] += (0.9 * np.sin(2 * np.pi * 700.0 * t)).astype(np.float32)
    L = LV.raw_log_mel(wav)
    g = [LV.running_max(L, k, 104) for k in range(4)]
    assert g[2] < g[3] - 0.5 and g[3] == L.max()
    say("live stream with a late burst")
    got = run_live(model, wav, 104, seeded_sizes(3, 1.0, 15.0))
    windows_vs_oracle(got, wav, P64, 104, (0, 1, 2, 3), "late burst")


@pytest.mark.parametrize("n,window,pushes", [(201, 104, [201]), (16000 * 3 + 77, 13, [997]),
                                             (16000 * 9 + 5, 104, [4000, 1, 16000])])
def test_live_short_streams_vs_oracle(model, P64, n, window, pushes):
    rng = np.random.default_rng(n)
    wav = (0.2 * rng.standard_normal(n)).astype(np.float32)
    got = run_live(model, wav, window, pushes)
    N = OE.encoder_frames(n // 160)
    assert got.shape == (N, 2048)
    windows_vs_oracle(got, wav, P64, window, tuple(range(math.ceil(N / window))), f"n={n} W={window}")
