"""Pins for greedy verification: exhaustive enumeration, planted prefixes and the
hand-worked fixtures in tests/golden/verify_cases.json."""
import itertools
import json
import os

import numpy as np
import pytest

import synth
from synth import gen
from oracle import verify

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "verify_cases.json")


def _definition(d, y):
    """Accept length straight from the definition: the largest k such that every
    j <= k has d_j == y_{j-1}; checked by trying every k from the top down."""
    G = len(y)
    for k in range(G - 1, -1, -1):
        if all(d[j - 1] == y[j - 1] for j in range(1, k + 1)):
            return k + 1
    raise AssertionError


@pytest.mark.parametrize("G", [2, 3, 4])
def test_verify_exhaustive_small_alphabet(G):
    for d in itertools.product(range(3), repeat=G - 1):
        for y in itertools.product(range(3), repeat=G):
            tau, com, nxt = verify(d, y)
            assert tau == _definition(d, y)
            assert list(com[:tau]) == list(y[:tau])
            assert all(c == -1 for c in com[tau:])
            assert nxt == y[tau - 1]


@pytest.mark.parametrize("G", [2, 8, 16])
def test_draft_equal_to_target_accepts_whole_block(G):
    rng = np.random.default_rng(G)
    y = rng.integers(0, 151936, size=G)
    tau, com, nxt = verify(y[:-1], y)
    assert tau == G and list(com) == list(y) and nxt == y[-1]


def test_planted_prefix_gives_planted_accept_length():
    cfg = synth.get_config("C3").with_(batch=64)
    d = gen.tokens(cfg, "plant_draft", (64, 15))
    k = gen.planted_accept(cfg, (64,), 16)
    y = gen.planted_targets(cfg, d, k)
    for b in range(64):
        tau, com, nxt = verify(d[b], y[b])
        assert tau == k[b] + 1
        assert nxt == y[b, k[b]]


def test_golden_cases():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    assert len(cases) >= 6
    for c in cases:
        tau, com, nxt = verify(c["draft"], c["target"])
        assert tau == c["accept_len"], c["name"]
        assert list(com) == c["committed"], c["name"]
        assert nxt == c["next_anchor"], c["name"]
