"""Drift check: the oracle reproduces the outputs stored by make_golden.py."""
import json
import os

import numpy as np

import oracle
import synth

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_oracle_matches_stored_samples():
    with open(os.path.join(HERE, "oracle_samples.json")) as f:
        data = json.load(f)
    for case in data["cases"]:
        wl = synth.get_workload(case["workload"])
        inp = synth.make_inputs(wl, seed=case["seed"], rows=case["rows"])
        cols = case["cols"]
        eps = oracle.eps_as_passed(wl.eps)
        if wl.gated:
            Y = oracle.rmsnorm_gated_mlp(inp.X, inp.g, inp.W1[:, cols], inp.W3[:, cols], eps)
        else:
            Y = oracle.rmsnorm_matmul(inp.X, inp.g, inp.W1[:, cols], eps)
        np.testing.assert_allclose(Y, np.array(case["Y"]), rtol=1e-12, atol=1e-14)
