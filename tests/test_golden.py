"""Drift guard: the oracle on the seeded tiny fp32 workload reproduces the stored values
written by tests/golden/make_golden.py (which calls only the oracle and the generator)."""
import json
import os

import numpy as np

from tests.golden.make_golden import compute

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_oracle_matches_stored_tiny_values():
    with open(os.path.join(HERE, "tiny_f32_seed1.json")) as f:
        stored = json.load(f)
    now = compute()
    for name, vals in stored["samples"].items():
        if name.endswith("_sum_abs"):
            np.testing.assert_allclose(now["samples"][name], vals, rtol=1e-12)
        else:
            for (idx, val), (idx2, val2) in zip(vals, now["samples"][name]):
                assert idx == idx2
                np.testing.assert_allclose(val2, val, rtol=1e-12, atol=1e-14)
