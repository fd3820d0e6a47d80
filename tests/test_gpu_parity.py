"""GPU parity: the HIP path through the C ABI against the oracle.

Inputs are seeded and synthetic (module synth); the oracle gets the same
input values (weights already bf16-representable for bf16 runs).
"""

import sys

import numpy as np
import pytest

import synth
from oracle import encoder as OE
from oracle import logmel as OL
from tests.helpers import (MEL_TOL, GpuModel, assert_bf16_rows, assert_f32_rows, gpu_logmel,
                           split_rows)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# ------------------------------------------------------------------ log-mel

@pytest.mark.parametrize("cid", [0, 1])
def test_logmel_single_clip(cid):
    w = synth.workload(cid)
    wav = synth.make_clips(w)
    say("logmel", w.name)
    mel = gpu_logmel(wav)
    ref = OL.log_mel(wav[0])
    assert mel.shape == ref.shape == (len(wav[0]) // 160, 128)
    err = np.abs(mel - ref).max()
    say("  max abs", err)
    assert err <= MEL_TOL


def test_logmel_varlen_packed_and_padded():
    w = synth.workload(4)
    wavs = synth.make_clips(w)[:8]
    lens = [len(x) for x in wavs]
    say("logmel varlen", lens)
    packed = gpu_logmel(wavs, layout=0)
    padded = gpu_logmel(wavs, layout=1)
    T = [n // 160 for n in lens]
    assert packed.shape == (sum(T), 128)
    for i, (x, m) in enumerate(zip(wavs, split_rows(packed, T))):
        ref = OL.log_mel(x)
        assert np.abs(m - ref).max() <= MEL_TOL
        assert np.array_equal(padded[i, :T[i]], m)
        assert np.all(padded[i, T[i]:] == 0)


def test_logmel_edge_lengths():
    # shortest legal clip (201 samples -> 1 frame), a non-multiple of 16
    # frames, and an all-silent clip
    rng = np.random.default_rng(0)
    wavs = [rng.standard_normal(201).astype(np.float32) * 0.1,
            rng.standard_normal(16000 * 3 + 77).astype(np.float32) * 0.3,
            np.zeros(3200, np.float32)]
    mel = gpu_logmel(wavs)
    T = [len(x) // 160 for x in wavs]
    for x, m in zip(wavs, split_rows(mel, T)):
        ref = OL.log_mel(x)
        assert np.abs(m - ref).max() <= MEL_TOL
    assert np.all(split_rows(mel, T)[2] == -1.5)


@pytest.mark.parametrize("nseq", [128, 131])
def test_logmel_many_sequences(nseq):
    # the most sequences whose tables the kernel stages in LDS (128), and more
    # (the frame lookup then searches the tables in memory); short ragged
    # clips, packed and padded
    rng = np.random.default_rng(7)
    lens = [int(n) for n in rng.integers(201, 2400, size=nseq)]
    wavs = [rng.standard_normal(n).astype(np.float32) * 0.2 for n in lens]
    say("logmel many sequences", len(wavs))
    packed = gpu_logmel(wavs, layout=0)
    padded = gpu_logmel(wavs, layout=1)
    T = [n // 160 for n in lens]
    assert packed.shape == (sum(T), 128)
    err = 0.0
    for i, (x, m) in enumerate(zip(wavs, split_rows(packed, T))):
        err = max(err, float(np.abs(m - OL.log_mel(x)).max()))
        assert np.array_equal(padded[i, :T[i]], m)
    say("  max abs", err)
    assert err <= MEL_TOL


def test_logmel_long_stream_c3():
    w = synth.workload(3)
    wav = synth.make_clips(w)
    say("logmel c3", len(wav[0]))
    mel = gpu_logmel(wav)
    ref = OL.log_mel(wav[0])
    assert mel.shape == (60000, 128)
    assert np.abs(mel - ref).max() <= MEL_TOL


# ------------------------------------------------------------------ encoder

FULL = synth.FULL_GEOM


@pytest.fixture(scope="module")
def full_weights_f32():
    return synth.make_weights(FULL, bf16=False)


@pytest.fixture(scope="module")
def full_weights_bf16():
    return synth.make_weights(FULL, bf16=True)


def small_geom(n_layers, adapter=0):
    return dict(FULL, n_layers=n_layers, adapter_hidden=adapter)


def sub_weights(full: dict, geom):
    names = [n for n, _ in synth.weight_names(geom)]
    return {n: full[n] for n in names}


def oracle_rows(mels, weights, geom, W, **kw):
    P = OE.as_f64(weights)
    return [OE.encode_clip(m, P, geom, W, **kw) for m in mels]


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
def test_front_end_only(dt, full_weights_f32, full_weights_bf16):
    geom = small_geom(0)
    wts = sub_weights(full_weights_f32 if dt == "f32" else full_weights_bf16, geom)
    model = GpuModel(geom, dt, wts, with_head=False)
    rng = np.random.default_rng(1)
    mels = [rng.uniform(-1, 1.5, (T, 128)) for T in (100, 37, 8, 1)]
    say("front-end", dt)
    got = model.encode(mels, 104)
    ns = [OE.encoder_frames(m.shape[0]) for m in mels]
    refs = oracle_rows(mels, wts, geom, 104, with_head=False)
    for g, r in zip(split_rows(got, ns), refs):
        if dt == "f32":
            assert_f32_rows(g, r, what="front-end f32")
        else:
            assert_bf16_rows(g, r, what=f"front-end {dt}")


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
def test_one_layer_random_ln(dt):
    geom = small_geom(1)
    wts = synth.make_weights(geom, bf16=(dt != "f32"), ln_random=True)
    model = GpuModel(geom, dt, wts)
    rng = np.random.default_rng(2)
    mels = [rng.uniform(-1, 1.5, (T, 128)) for T in (300, 77, 1000)]
    say("one layer", dt)
    for W in (104, 5, 1, 500):
        got = model.encode(mels, W)
        ns = [OE.encoder_frames(m.shape[0]) for m in mels]
        refs = oracle_rows(mels, wts, geom, W)
        for g, r in zip(split_rows(got, ns), refs):
            if dt == "f32":
                assert_f32_rows(g, r, what=f"1 layer f32 W={W}")
            else:
                assert_bf16_rows(g, r, what=f"1 layer {dt} W={W}")


def test_c0_fp32_full(full_weights_f32):
    w = synth.workload(0)
    mel = OL.log_mel(synth.make_clips(w)[0])
    model = GpuModel(FULL, "f32", full_weights_f32)
    say("c0 fp32 full")
    got = model.encode([mel], w.window)
    ref = oracle_rows([mel], full_weights_f32, FULL, w.window)[0]
    assert got.shape == (13, 2048)
    m = assert_f32_rows(got, ref, what="c0")
    say("  worst rel", m["rel"].max())


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_c1_30s_full(full_weights_bf16, dt):
    # bf16-valued weights; matrix operands fp16 (the default 16-bit type) or bf16
    w = synth.workload(1)
    mel = OL.log_mel(synth.make_clips(w)[0])
    model = GpuModel(FULL, dt, full_weights_bf16)
    say("c1 30 s full,", dt, "operands")
    got = model.encode([mel], w.window)
    ref = oracle_rows([mel], full_weights_bf16, FULL, w.window)[0]
    assert got.shape == (375, 2048)
    m = assert_bf16_rows(got, ref, what=f"c1 {dt}")
    say("  min cos", m["cos"].min(), "max |d|/rms", m["maxabs_rms"].max())
