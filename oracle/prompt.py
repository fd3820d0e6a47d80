"""Prompt embedding with the audio frames spliced in.  TEST INFRASTRUCTURE ONLY.

Model card "MOSS-Transcribe-preview-2B-GGUF", Architecture table, rows Prompt
and Audio injection: each audio placeholder position of the prompt takes the
next adapter output frame in place of its token embedding; every other
position takes its token's row of the (tied) token-embedding table.

Pinned by tests/test_oracle_prompt.py (a hand-written example under
tests/golden/, and the placeholder-count check).
"""

import numpy as np


def splice(tokens, table, audio, audio_token):
    """tokens [S] ints, table [V, d], audio [A, d] (A = number of placeholders)
    -> [S, d] float64."""
    tokens = np.asarray(tokens, dtype=np.int64)
    table = np.asarray(table, dtype=np.float64)
    audio = np.asarray(audio, dtype=np.float64)
    n_ph = int(np.sum(tokens == audio_token))
    if n_ph != audio.shape[0]:
        raise ValueError(f"{n_ph} audio placeholders for {audio.shape[0]} audio frames")
    out = np.empty((len(tokens), table.shape[1]), dtype=np.float64)
    k = 0
    for i, t in enumerate(tokens):
        if t == audio_token:
            out[i] = audio[k]
            k += 1
        else:
            out[i] = table[t]
    return out
