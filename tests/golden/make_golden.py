"""Write tests/golden/tiny_f32_seed1.json from the fp64 oracle alone.

The pages print no worked attention example (no input or output values), so
the stored numbers here are not the pages': they are the oracle's outputs on
the seeded tiny fp32 workload (B=1, H=2, S=64, D=32, scale 1/sqrt(32)),
kept to catch silent drift of the oracle or of the input generator.  The
oracle itself is pinned by tests/test_oracle.py.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import attention_bwd_ref  # noqa: E402
from workload import CONFIGS, make_inputs  # noqa: E402

SAMPLES = [(0, 0, 0, 0), (0, 0, 1, 5), (0, 1, 17, 31), (0, 1, 63, 0), (0, 0, 40, 12)]


def compute():
    x = make_inputs(CONFIGS["tiny_f32"], 1)
    r = attention_bwd_ref(*(x[n].astype(np.float64) for n in ("q", "k", "v", "do")), x["scale"])
    out = {"config": "tiny_f32", "seed": 1, "samples": {}}
    for name in ("o", "dq", "dk", "dv"):
        out["samples"][name] = [[list(idx), float(r[name][idx])] for idx in SAMPLES]
        out["samples"][name + "_sum_abs"] = float(np.abs(r[name]).sum())
    out["samples"]["lse"] = [[list(idx[:3]), float(r["lse"][idx[:3]])] for idx in SAMPLES]
    return out


if __name__ == "__main__":
    with open(os.path.join(HERE, "tiny_f32_seed1.json"), "w") as f:
        json.dump(compute(), f, indent=1)
        f.write("\n")
