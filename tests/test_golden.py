"""The oracle still reproduces its committed tiny fixtures (written by tests/golden/make_golden.py)."""
import json
import os

import numpy as np

import sys
sys.path.insert(0, os.path.join(os.path.dirname(__file__), "golden"))
import make_golden  # noqa: E402


def test_oracle_matches_fixture():
    with open(os.path.join(os.path.dirname(__file__), "golden", "oracle_tiny.json")) as f:
        want = json.load(f)
    got = make_golden.build()
    for part, keys in (("attention", ("o1", "o2")), ("layer", ("out1", "out2"))):
        for k in keys:
            assert np.allclose(np.array(got[part][k]), np.array(want[part][k]), rtol=0, atol=1e-13), (part, k)
    for k in ("k1_bits", "v1_bits"):
        assert got["layer"][k] == want["layer"][k]
