"""The oracle and the generator still reproduce the committed regression fixture."""
import json
import os

import numpy as np

from oracle.tri_attn_oracle import forward
from workloads import Workload, make_inputs

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_golden_tiny_forward():
    with open(os.path.join(HERE, "tiny_forward.json")) as f:
        cases = json.load(f)
    assert len(cases) == 2
    for name, c in cases.items():
        B, N, D, h, dtype, mask, seed = c["workload"]
        inp = make_inputs(Workload(name, B, N, D, h, dtype, tuple(mask), seed))
        for k, v in c["inputs"].items():
            np.testing.assert_array_equal(np.asarray(v, dtype=inp[k].dtype), inp[k], err_msg=k)
        np.testing.assert_allclose(forward(inp), np.asarray(c["y"]), rtol=0, atol=1e-13)
