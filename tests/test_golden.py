"""The oracle still reproduces the stored snapshot written by make_golden.py."""
import json
import os

import numpy as np

from tests.golden import make_golden

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_toy_snapshot_reproduces():
    with open(os.path.join(HERE, "toy_fp32_seed0.json")) as f:
        ref = json.load(f)
    now = make_golden.toy_case()
    assert now["k_in"] == ref["k_in"] == 256
    assert now["k"] == ref["k"] == 688
    assert now["sel"] == ref["sel"]
    assert now["codes_gate_row0"] == ref["codes_gate_row0"]
    assert now["scale_gate_row0"] == ref["scale_gate_row0"]
    np.testing.assert_allclose(now["y"], ref["y"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(now["score_head"], ref["score_head"], rtol=1e-12)
    assert abs(now["T"] - ref["T"]) <= 1e-12 * ref["T"]
