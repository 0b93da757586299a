"""The oracle still reproduces the values it wrote once its pins passed
(tests/golden/make_golden.py); guards against silent drift of the oracle."""
import json
import os

from tests.golden.make_golden import compute

HERE = os.path.dirname(os.path.abspath(__file__))


def test_tiny_regression_fixture(oracle_lib):
    with open(os.path.join(HERE, "golden", "tiny_oracle.json")) as f:
        ref = json.load(f)["values"]
    now = compute()
    for k, rows in ref.items():
        for (idx, val), (idx2, val2) in zip(rows, now[k]):
            assert idx == idx2
            assert abs(val - val2) <= 1e-12 * max(1.0, abs(val)), (k, idx, val, val2)
