"""Write tests/golden/tiny_oracle.json from the oracle alone (inputs: the seeded generator).

The pages print no worked example, so this fixture is not a page value: it freezes
the oracle's answer on the tiny workload (B=1, H=16, Q=4, L=256, seed 0) so that a
later change to the oracle's arithmetic shows up as a diff of this file.
Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from speculative_decode_mla_amd import inputs as I  # noqa: E402

SAMPLE_ROWS = [(0, 0), (0, 15), (1, 7), (2, 3), (3, 0), (3, 15)]


def compute():
    x = I.make_inputs("tiny")
    out, lse = oracle.verify_attention(x.q, x.pool(), x.slot_idx, x.seq_lens, x.q_lens, x.scale)
    return {
        "workload": "tiny: B=1 H=16 Q=4 L=256, 4096-slot pool, seed 0, scale 1/sqrt(192)",
        "lse": [[float(v) for v in row] for row in lse],
        "out_row_sums": [[float(v) for v in out[t].sum(axis=1)] for t in range(out.shape[0])],
        "out_samples": {f"{t},{h}": [float(v) for v in out[t, h, :16]] for t, h in SAMPLE_ROWS},
    }


if __name__ == "__main__":
    with open(os.path.join(HERE, "tiny_oracle.json"), "w") as f:
        json.dump(compute(), f, indent=1)
