"""mt_logmel_noalloc (no workspace: the library's fixed per-device scratch
array) against mt_logmel (caller workspace): the same kernels, so the outputs
are equal bit for bit -- on two calls in a row, the second with a smaller
batch (what the first call left in the scratch array must not leak into the
second), packed and padded, and the host-side rejection of a batch larger
than the array."""

import sys

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _both(wavs, layout):
    import torch
    import windowed_attention_audio_amd as W
    lens = [len(x) for x in wavs]
    if layout == W.MT_PACKED:
        wav = torch.from_numpy(np.concatenate(wavs).astype(np.float32)).cuda()
    else:
        arr = np.zeros((len(wavs), max(lens)), np.float32)
        for i, x in enumerate(wavs):
            arr[i, :len(x)] = x
        wav = torch.from_numpy(arr).cuda()
    ref = W.mt_logmel(wav, lens, layout=layout)
    got = W.mt_logmel_noalloc(wav, lens, layout=layout)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), got.cpu().numpy()


@pytest.mark.parametrize("layout", [0, 1])
def test_noalloc_equals_workspace_path_twice(layout):
    w = synth.workload(4)
    big = synth.make_clips(w)[:12]          # 12 clips of 2..60 s
    rng = np.random.default_rng(21)
    small = [rng.standard_normal(n).astype(np.float32) * 0.1 for n in (201, 16000 * 3 + 77, 999)]
    for name, wavs in (("12 varlen clips", big), ("3 short clips", small)):
        say(f"noalloc vs workspace ({name}, layout {layout})")
        ref, got = _both(wavs, layout)
        assert got.shape == ref.shape
        assert np.array_equal(got, ref), name


def test_noalloc_rejects_too_many_sequences():
    import torch
    import windowed_attention_audio_amd as W
    n = W.MT_LOGMEL_NOALLOC_MAX_SEQS + 1
    wav = torch.zeros(201 * n, dtype=torch.float32, device="cuda")
    with pytest.raises(W.MtError) as e:
        W.mt_logmel_noalloc(wav, [201] * n)
    assert e.value.status == W.MT_ERR_WORKSPACE
    # the largest batch it takes runs and matches the workspace path
    rng = np.random.default_rng(5)
    m = W.MT_LOGMEL_NOALLOC_MAX_SEQS
    wavs = [rng.standard_normal(201 + (i % 7) * 160).astype(np.float32) * 0.1 for i in range(m)]
    ref, got = _both(wavs, W.MT_PACKED)
    assert np.array_equal(got, ref)
