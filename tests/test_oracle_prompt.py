"""Pins of oracle.prompt.splice (the audio splice into the prompt embedding)."""

import json
import os

import numpy as np
import pytest

from oracle import prompt as OP

GOLD = os.path.join(os.path.dirname(__file__), "golden", "splice_small.json")


def test_splice_golden_example():
    ex = json.load(open(GOLD))
    got = OP.splice(ex["tokens"], ex["table"], ex["audio"], ex["audio_token"])
    assert np.array_equal(got, np.array(ex["expected"], dtype=np.float64))


def test_splice_count_mismatch():
    table = np.zeros((4, 2))
    with pytest.raises(ValueError):
        OP.splice([1, 3, 3], table, np.zeros((1, 2)), 3)
    with pytest.raises(ValueError):
        OP.splice([1, 2], table, np.zeros((1, 2)), 3)


def test_splice_no_audio_is_a_lookup():
    rng = np.random.default_rng(0)
    table = rng.standard_normal((50, 8))
    tok = rng.integers(0, 49, 30)
    assert np.array_equal(OP.splice(tok, table, np.zeros((0, 8)), 49), table[tok])
