"""Write tests/golden/tiny_forward.json from the oracle (the only code it calls).

The pages print no numeric worked example, so this fixture is a regression
record of the oracle itself: its inputs come from the seeded generator at a
tiny shape of the l2_p6 problem family (pair representation (B, N, N, D),
pair mask (B, N, N)); its expected output is the oracle's float64 forward.
Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle.tri_attn_oracle import forward  # noqa: E402
from workloads import Workload, make_inputs  # noqa: E402

CASES = {
    "tiny_bernoulli": Workload("tiny_bernoulli", 1, 3, 4, 2, "f32", ("bernoulli", 0.6), 4242),
    "tiny_padded_bf16": Workload("tiny_padded_bf16", 2, 4, 8, 2, "bf16", ("pad", 3), 4243),
}


def main():
    out = {}
    for name, w in CASES.items():
        inp = make_inputs(w)
        y = forward(inp)
        out[name] = {
            "workload": [w.B, w.N, w.D, w.h, w.dtype, list(w.mask), w.seed],
            "inputs": {k: v.tolist() for k, v in inp.items() if hasattr(v, "tolist")},
            "y": y.tolist(),
        }
    with open(os.path.join(HERE, "tiny_forward.json"), "w") as f:
        json.dump(out, f, indent=None, separators=(",", ":"))


if __name__ == "__main__":
    main()
