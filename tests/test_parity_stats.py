"""The parity-statistics report (tests/parity_stats.py) on a small hand-made
record: grouping of parametrised cases, sums and maxima.  CPU only."""
import json

import parity_stats


def test_report_groups_and_sums():
    lines = [
        json.dumps({"kind": "bf16", "test": "tests/test_a.py::test_x[1]", "what": "a", "n": 10, "max_ulp": 3,
                    "n_gt2ulp": 1, "n_floor_only": 1, "n_exact": 8, "n_fail": 0}),
        json.dumps({"kind": "bf16", "test": "tests/test_a.py::test_x[2]", "what": "b", "n": 5, "max_ulp": 7,
                    "n_gt2ulp": 2, "n_floor_only": 2, "n_exact": 3, "n_fail": 0}),
        json.dumps({"kind": "f32", "test": "tests/test_b.py::test_y", "what": "c", "n": 4, "max_rel": 2e-5,
                    "n_rel_gt_1e-5": 1, "n_floor_only": 1, "n_fail": 0}),
        json.dumps({"kind": "drift", "test": "tests/test_c.py::test_z", "what": "chain", "n": 6,
                    "gpu_vs_exact_ulp": {"median": 1.0, "p99": 2.0, "max": 3},
                    "oracle_vs_exact_ulp": {"median": 1.0, "p99": 2.0, "max": 4},
                    "gpu_max_err_over_ulp(0.02)": 1.5, "oracle_max_err_over_ulp(0.02)": 2.5,
                    "gpu_vs_oracle_gt2ulp": 0}),
    ]
    bf, f32, drift = parity_stats.summarise(lines)
    a = bf["test_a.py::test_x"]
    assert (a["checks"], a["n"], a["max_ulp"], a["n_gt2ulp"], a["n_floor_only"], a["n_exact"]) == (2, 15, 7, 3, 3, 11)
    assert f32["test_b.py::test_y"]["n_rel_gt_1e-5"] == 1
    md = parity_stats.markdown(bf, f32, drift, "cmd")
    assert "| test_a.py::test_x | 2 | 15 | 11 | 7 | 3 | 3 | 0 |" in md
    assert "| chain | 6 | 1 / 2 / 3 | 1 / 2 / 4 | 1.5 | 2.5 | 0 |" in md
