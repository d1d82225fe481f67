"""Write tests/golden/oracle_samples.json: oracle outputs on seeded workloads.

Calls only the oracle and the input generator.  The file is a drift check on
the oracle (a later change to its arithmetic must change this file in the same
commit, with the reason); it is not a pin -- the pins are in tests/pins.py.
Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_samples.json")


def sample(name, rows, n_cols=16, seed=0):
    wl = synth.get_workload(name)
    inp = synth.make_inputs(wl, seed=seed, rows=rows)
    eps = oracle.eps_as_passed(wl.eps)
    rng = np.random.default_rng(1234)
    cols = np.sort(rng.choice(wl.N, size=n_cols, replace=False))
    W1 = inp.W1[:, cols]
    if wl.gated:
        Y = oracle.rmsnorm_gated_mlp(inp.X, inp.g, W1, inp.W3[:, cols], eps)
    else:
        Y = oracle.rmsnorm_matmul(inp.X, inp.g, W1, eps)
    return {"workload": name, "seed": seed, "rows": [int(r) for r in rows],
            "cols": [int(c) for c in cols], "Y": [[float(v) for v in row] for row in Y]}


def main():
    cases = [
        sample("f32_m8_k1024_n1024", list(range(8))),
        sample("decode_m16_k4096_n6144", [0, 7, 15]),
        sample("gated_m64_k4096_n14336", [0, 33, 63]),
        sample("prefill_m4096_k4096_n4096", [0, 1000, 4095]),
    ]
    with open(OUT, "w") as f:
        json.dump({"note": "oracle outputs written by tests/golden/make_golden.py",
                   "cases": cases}, f, indent=1)


if __name__ == "__main__":
    main()
