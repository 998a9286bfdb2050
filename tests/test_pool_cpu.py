"""The oracle spread over host worker processes (oracle/pool.py), which the
full-size GPU parity tests and the CPU baseline use: its results equal one
oracle call, and its comparison finds a planted error and a planted NaN at
the right element."""
import numpy as np

from oracle import pool
from oracle import tri_attn_oracle as O
from oracle import tri_attn_train_oracle as TO
from workloads import Workload, make_inputs


def _inp():
    return make_inputs(Workload("pool", 2, 12, 64, 4, "f32", ("pad", 9), seed=17))


def test_forward_rows_equal_one_oracle_call():
    inp = _inp()
    rows = [(1, 3), (0, 0), (0, 11), (1, 10)]
    got = pool.forward_rows(inp, rows, workers=2)
    np.testing.assert_array_equal(got, O.forward_rows(inp, rows))
    got_e = pool.forward_rows(inp, [(0, 2), (1, 7)], workers=2, ending=True)
    np.testing.assert_array_equal(got_e, O.forward_ending_cols(inp, [(0, 2), (1, 7)]))


def test_compare_rows_finds_planted_error_and_nan():
    inp = _inp()
    y = O.forward(inp)
    rows = [(b, i) for b in range(2) for i in range(12)]
    r = pool.compare_rows(inp, y.astype(np.float32), rows, workers=3)["y"]
    assert r["same_nan_pattern"] and r["max_abs_err"] < 1e-6
    bad = y.copy()
    bad[1, 4, 2, 33] += 0.25
    r = pool.compare_rows(inp, bad, rows, workers=3)["y"]
    assert abs(r["max_abs_err"] - 0.25) < 1e-9 and r["where"] == (1, 4, 2, 33)
    bad[0, 7, 5, 1] = np.nan
    r = pool.compare_rows(inp, bad, rows, workers=3)["y"]
    assert not r["same_nan_pattern"]


def test_compare_rows_training_mode_and_lse():
    inp = _inp()
    y, lse = TO.forward_train(inp, 0.3, 5, 2)
    rows = [(0, 1), (1, 11)]
    r = pool.compare_rows(inp, y.astype(np.float32), rows, train={"rate": 0.3, "seed": 5, "offset": 2},
                          lse=lse.astype(np.float32), workers=2)
    assert r["y"]["max_abs_err"] < 1e-6 and r["lse"]["max_abs_err"] < 1e-5
    assert r["lse_dead_rel"]["max_abs_err"] < 1e-6
    # a different seed's output must not pass
    y2, _ = TO.forward_train(inp, 0.3, 6, 2)
    r = pool.compare_rows(inp, y2.astype(np.float32), rows, train={"rate": 0.3, "seed": 5, "offset": 2}, workers=2)
    assert r["y"]["max_abs_err"] > 1e-3


def test_time_rows_counts_rows_and_passes():
    r = pool.time_rows(_inp(), [(0, i) for i in range(12)], 0.2, workers=2)
    assert r["workers"] == 2 and r["passes"] >= 1 and r["rows"] == 12 * r["passes"] and r["seconds"] >= 0.2
