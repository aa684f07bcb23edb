"""Host-side logic of bench.py that needs no GPU."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_output_check_accepts_within_and_flags_past_the_bound():
    y = np.array([1.0, -2.0, 3.0], dtype=np.float32)
    mag = np.array([[10.0, 20.0, 30.0]])
    ok = bench.output_check(y, {"y64": np.array([[1.00005, -2.0001, 3.0]]), "mag": mag})
    assert ok["ok"] and ok["outputs"] == 3 and abs(ok["max_err_over_bound"] - 0.5) < 1e-3
    bad = bench.output_check(y, {"y64": np.array([[1.0, -2.0, 3.001]]), "mag": mag})
    assert not bad["ok"] and bad["max_err_over_bound"] > 3.0


def test_output_check_shapes_follow_the_outputs():
    y = np.zeros((2, 3), dtype=np.float32)
    ref = {"y64": np.zeros(6), "mag": np.ones(6)}
    assert bench.output_check(y, ref) == {"outputs": 6, "bound": bench.output_check(y, ref)["bound"],
                                          "max_err_over_bound": 0.0, "ok": True}
