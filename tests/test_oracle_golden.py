"""The oracle's output on the tiny configuration is frozen in
tests/golden/tiny_forward.json (written by tests/golden/make_golden.py, which
calls only the oracle); inputs and outputs must reproduce it."""
import json
import os

import numpy as np

from tests.golden.make_golden import build

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_forward.json")


def test_tiny_forward_matches_frozen_vector():
    with open(GOLDEN) as f:
        want = json.load(f)
    got = build()
    assert got["inputs_sha256"] == want["inputs_sha256"]
    assert got["acc_row0_first8_hex"] == want["acc_row0_first8_hex"]
    np.testing.assert_allclose(got["acc_row_l2"], want["acc_row_l2"], rtol=1e-12)
