"""The two calls of the C ABI that the path is defined by, rmsnorm_matmul and
rmsnorm_gated_mlp (include/rmm.h), called directly through ctypes -- not
through the _ex forms or the Python front end -- with and without a
caller-owned workspace, against the CPU oracle (needs an MI355X)."""
import ctypes

import numpy as np
import pytest
import torch

import synth
import tensor_program_amd as tpa
from tests.gpu_util import assert_within_tol, from_device, run_oracle, to_device, tol_for

pytestmark = pytest.mark.gpu

CASES = [
    # (M, K, N, gated): decode, stream, prefill and generic shapes
    (16, 4096, 6144, False),
    (64, 1024, 2048, False),
    (512, 1024, 1024, False),
    (7, 100, 36, False),
    (16, 1024, 2048, True),
    (64, 1024, 2048, True),
    (200, 264, 1032, True),
]


@pytest.mark.parametrize("with_ws", [False, True])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_plain_entry_points(case, with_ws, require_gpu):
    M, K, N, gated = case
    print(f"entry point {case} workspace {with_ws}", flush=True)
    lib = tpa.load_library()
    wl = synth.Workload("entry", "bf16", M, K, N, 1e-6, gated, None)
    inp = synth.make_inputs(wl, seed=21)
    x, g, w1 = to_device(inp, "X"), to_device(inp, "g"), to_device(inp, "W1")
    w3 = to_device(inp, "W3") if gated else None
    y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws, ws_bytes = None, 0
    if with_ws:
        ws_bytes = int(lib.rmm_workspace_bytes(tpa._binding.DTYPE_BF16, M, N, K, int(gated)))
        if ws_bytes:
            wst = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
            ws = wst.data_ptr()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for _ in range(2):  # a second call on the same workspace: counters were reset
        if gated:
            st = lib.rmsnorm_gated_mlp(x.data_ptr(), g.data_ptr(), w1.data_ptr(), w3.data_ptr(),
                                       y.data_ptr(), ctypes.c_float(wl.eps), M, N, K,
                                       tpa._binding.DTYPE_BF16, ws, ws_bytes, stream)
        else:
            st = lib.rmsnorm_matmul(x.data_ptr(), g.data_ptr(), w1.data_ptr(), y.data_ptr(),
                                    ctypes.c_float(wl.eps), M, N, K, tpa._binding.DTYPE_BF16, ws,
                                    ws_bytes, stream)
        assert st == 0, tpa._binding.status_string(st)
        torch.cuda.synchronize()
        worst = assert_within_tol(from_device(y), run_oracle(inp, wl.eps), tol_for("bf16"),
                                  f"{case}")
    print(f"  worst err/tol {worst:.3f}", flush=True)
