"""Write tests/golden/oracle_small.json: a frozen snapshot of the fp64 oracle
on one small seeded case, so that any later change to the oracle's arithmetic
shows up as a test failure and has to be justified from the pages.

Calls only ``oracle/`` (and the seeded generator); run from the repo root:
    python tests/golden/make_golden.py
"""

import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from workloads import numpy_inputs  # noqa: E402

B, H, N, D, M, SEED = 1, 2, 9, 3, 4, 1234


def main():
    q, k, v, g = numpy_inputs(B, H, N, D, M, seed=SEED, scale=1.0)
    rec = {"shape": [B, H, N, D, M], "seed": SEED, "scale": 1.0,
           "recipe": "workloads.numpy_inputs (default_rng(seed); Q, K, V, dout)",
           "source": "oracle.forward_quadratic / oracle.backward, fp64"}
    for causal in (True, False):
        out, den = oracle.forward_quadratic(q, k, v, causal)
        dq, dk, dv, _, _ = oracle.backward(q, k, v, g, causal)
        key = "causal" if causal else "noncausal"
        rec[key] = {"out": out.tolist(), "den": den.tolist(),
                    "dq": dq.tolist(), "dk": dk.tolist(), "dv": dv.tolist()}
    with open(os.path.join(HERE, "oracle_small.json"), "w") as f:
        json.dump(rec, f, indent=1)


if __name__ == "__main__":
    main()
