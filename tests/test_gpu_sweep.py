"""Seeded random-shape sweep of every variant against the CPU oracle (needs
an MI355X).

For each drawn shape (ragged M, K and N, including K and N that are not
multiples of 8, both storage types, plain and gated) every variant the
planner accepts for that shape is run -- the automatic choice and each forced
one -- and compared with the oracle within the storage type's tolerance.
Forced variants a shape cannot take must be refused with RMM_ERR_VARIANT.
Every output, plain or gated, is held to the elementwise bound
tol (|Y_ref| + 1) of its storage type.
"""
import numpy as np
import pytest
import torch

import synth
import tensor_program_amd as tpa
from tests.gpu_util import assert_within_tol, from_device, run_gpu, run_oracle, tol_for

pytestmark = pytest.mark.gpu

VARIANTS = ("auto", "generic", "decode", "prefill", "stream")


def _check(y, ref, dtype, what):
    assert_within_tol(y, ref, tol_for(dtype), what)


def _shapes(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(rng.choice([1, 2, 5, 8, 13, 16, 17, 31, 32, 40, 64, 65, 130, 257, 300]))
        K = int(rng.integers(1, 160)) * 8 + int(rng.choice([0, 0, 0, 4]))
        N = int(rng.integers(1, 120)) * 8 + int(rng.choice([0, 0, 0, 2]))
        dtype = str(rng.choice(["bf16", "bf16", "f32"]))
        gated = bool(rng.random() < 0.3)
        out.append((M, K, N, dtype, gated))
    return out


CASES = _shapes(20260, 24) + _shapes(777, 16)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_sweep(case, require_gpu):
    M, K, N, dtype, gated = case
    print(f"sweep {case}", flush=True)
    wl = synth.Workload("sweep", dtype, M, K, N, 1e-6, gated, None)
    inp = synth.make_inputs(wl, seed=M * 7 + K)
    ref = run_oracle(inp, wl.eps)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    ran = 0
    for variant in VARIANTS:
        st = tpa.plan(M, N, K, dtype=tdt, gated=gated, variant=variant)[0]
        if st != 0:
            with pytest.raises(tpa.RmmError):
                run_gpu(inp, wl.eps, variant=variant)
            continue
        y = from_device(run_gpu(inp, wl.eps, variant=variant))
        _check(y, ref, dtype, f"{case}/{variant}")
        ran += 1
    assert ran >= 2  # the automatic choice and the generic kernel at least
