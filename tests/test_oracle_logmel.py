"""Pins for the log-mel oracle (CPU only).

Each test ties oracle.logmel to something other than itself: closed forms of
the DFT of a Hann-windowed cosine, Parseval's identity, the frame-count rule
of the model card's gotcha list, and a library run of the feature extractor
the model card names as the front-end's match (Architecture table, row Audio;
"Implementation notes", Mel row).
"""

import json
import os

import numpy as np
import pytest

import synth
from oracle import logmel as LM

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "counts.json")


def test_frame_count_golden():
    g = json.load(open(GOLDEN))
    for c in g["cases"]:
        assert LM.frame_count(c["n_samples"]) == c["mel_frames"]


@pytest.mark.parametrize("n", [201, 359, 16000, 16077, 16159, 16160, 48013])
def test_frame_count_matches_frames(n):
    x = synth.make_clip(9, n, n, False)
    assert LM.frames(x).shape == (n // 160, 400)
    assert LM.log_mel(x).shape == (n // 160, 128)


def test_too_short_rejected():
    with pytest.raises(ValueError):
        LM.frames(np.zeros(200))


@pytest.mark.parametrize("f", [100.0, 437.0, 1234.5, 2999.0, 3999.0])
def test_pure_sinusoid_peak_bin(f):
    n = 16000
    x = 0.2 * np.sin(2 * np.pi * f * np.arange(n) / 16000.0)
    P = LM.power_spectrum(x)
    interior = P[3:-3]
    assert np.all(np.argmax(interior, axis=1) == int(round(f / 40.0)))


@pytest.mark.parametrize("k0", [2, 7, 50, 128, 198])
def test_bin_centred_cosine_closed_form(k0):
    # A*cos(2 pi k0 j / 400) through a periodic Hann of length N=400 gives
    # |X[k0]| = A N / 4 and |X[k0 +- 1]| = A N / 8, zero elsewhere.
    A, N = 0.2, 400
    x = synth.tone(40.0 * k0, 16000, amp=A)
    P = LM.power_spectrum(x)
    # frames that do not touch the reflected edge: 160 t - 200 >= 0 and
    # 160 t + 199 < n
    inner = P[2:-2]
    expect = np.zeros(201)
    expect[k0] = (A * N / 4) ** 2
    expect[k0 - 1] = expect[k0 + 1] = (A * N / 8) ** 2
    assert np.max(np.abs(inner - expect[None])) < 1e-9
    assert abs(expect[k0] - 400.0) < 1e-12 and abs(expect[k0 + 1] - 100.0) < 1e-12


def test_symmetric_hann_would_fail_closed_form():
    # Guard that the closed-form test above really separates the windows.
    j = np.arange(400)
    sym = 0.5 - 0.5 * np.cos(2 * np.pi * j / 399)
    x = 0.2 * np.cos(2 * np.pi * 50 * j / 400)
    Xs = np.abs(np.fft.rfft(x * sym)) ** 2
    assert abs(Xs[50] - 400.0) > 1e-3 or abs(Xs[49] - 100.0) > 1e-3


def test_parseval():
    x = synth.make_clip(1, 0, 48000, True)
    F = LM.frames(x)
    P = LM.power_spectrum(x)
    lhs = (F ** 2).sum(axis=1)
    rhs = (P[:, 0] + 2 * P[:, 1:200].sum(axis=1) + P[:, 200]) / 400.0
    assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-15)


def test_reflect_padding_edges():
    # Frame 0 is centred on sample 0: its first 200 samples mirror x[200..1].
    x = np.arange(1000, dtype=np.float64)
    w = LM.hann_periodic()
    F = LM.frames(x)
    xp0 = np.concatenate([x[200:0:-1], x[:200]])
    assert np.array_equal(F[0], xp0 * w)
    T = LM.frame_count(1000)
    start = 160 * (T - 1) - 200
    assert np.array_equal(F[T - 1], x[start:start + 400] * w)


def test_all_zero_clip():
    L = LM.log_mel(np.zeros(16000))
    assert np.all(L == -1.5)


def test_filterbank_rows_are_triangles():
    F = LM.mel_filterbank()
    assert F.shape == (128, 201)
    assert np.all(F >= 0)
    # every filter is non-zero on a contiguous run of bins
    for m in range(128):
        nz = np.nonzero(F[m])[0]
        assert len(nz) >= 1 and nz[-1] - nz[0] + 1 == len(nz)


@pytest.fixture(scope="module")
def whisper_fe():
    tr = pytest.importorskip("transformers")
    return tr.WhisperFeatureExtractor(feature_size=128)


def test_filterbank_matches_named_extractor(whisper_fe):
    ref = np.asarray(whisper_fe.mel_filters, dtype=np.float64).T  # [128, 201]
    assert np.max(np.abs(LM.mel_filterbank() - ref)) < 1e-12


@pytest.mark.parametrize("n,cid", [(16000, 0), (16077, 4), (480000, 1), (37123, 4)])
def test_log_mel_matches_named_extractor(whisper_fe, n, cid):
    x = synth.make_clip(cid, 3, n, cid != 0)
    mine = LM.log_mel(x)
    kw = {} if n == 480000 else {"padding": "longest"}
    ref = whisper_fe(x, sampling_rate=16000, return_tensors="np", **kw)["input_features"][0].T
    assert ref.shape == mine.shape
    assert np.max(np.abs(mine - ref)) < 1e-4


def test_per_clip_clamp():
    a = synth.make_clip(2, 0, 32000, True)
    b = 0.01 * synth.make_clip(2, 1, 24000, True)
    La, Lb = LM.log_mel_batch([a, b])
    assert np.array_equal(La, LM.log_mel(a)) and np.array_equal(Lb, LM.log_mel(b))
    # silence sits at the clamp floor: 2 below the clip's own maximum, or
    # at the log floor (1e-10 -> -1.5) when that is higher
    for L in (La, Lb):
        assert abs(L.min() - max(L.max() - 2.0, -1.5)) < 1e-12
