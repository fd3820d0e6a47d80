"""GPU parity of mt_prompt_embed (audio frames spliced into the prompt's
token embeddings) against the oracle, for fp32, bf16 and fp16 tables."""

import numpy as np
import pytest

import synth
from oracle import prompt as OP

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("dt", ["float32", "bfloat16", "float16"])
@pytest.mark.parametrize("n_audio", [0, 1, 375])
def test_prompt_embed(dt, n_audio):
    import torch
    import windowed_attention_audio_amd as W
    vocab, d, audio_token = 1000, 2048, 777
    rng = np.random.default_rng(3)
    table = torch.from_numpy(rng.standard_normal((vocab, d)).astype(np.float32)).to(getattr(torch, dt))
    audio = rng.standard_normal((n_audio, d)).astype(np.float32)
    tokens = synth.prompt_tokens(n_audio, vocab, audio_token)
    got = W.mt_prompt_embed(tokens, table.cuda(), torch.from_numpy(audio).cuda(), audio_token)
    ref = OP.splice(tokens, table.float().numpy().astype(np.float64), audio, audio_token)
    assert got.shape == (len(tokens), d)
    assert np.array_equal(got.cpu().numpy().astype(np.float64), ref)


def test_prompt_embed_rejections():
    import torch
    import windowed_attention_audio_amd as W
    table = torch.zeros((10, 8), device="cuda")
    audio = torch.zeros((2, 8), device="cuda")
    for toks in ([1, 9, 9, 9], [1, 12, 9, 9], [-1, 9, 9]):  # 3 placeholders; id 12; id -1
        with pytest.raises(W.MtError) as e:
            W.mt_prompt_embed(toks, table, audio, 9)
        assert e.value.status == W.MT_ERR_INVALID_ARG
