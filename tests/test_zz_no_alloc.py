"""rmsnorm_matmul_noalloc, the entry point for callers that cannot allocate
(its split-K scratch is a fixed device array inside the library), called
through the C ABI and checked against rmsnorm_matmul with a caller-owned
workspace: the same kernels and plan, so the same bits, and within the
elementwise bound of the CPU oracle.  Two calls in a row, the second smaller
(the array keeps the first call's contents), then shapes of the other
variants (needs an MI355X)."""
import ctypes

import numpy as np
import pytest
import torch

import synth
import tensor_program_amd as tpa
from tests.gpu_util import assert_within_tol, from_device, run_oracle, to_device, tol_for

pytestmark = pytest.mark.gpu

# (M, K, N, dtype): decode with 4 splits, then a smaller decode layout (8
# splits over 16 tiles), the stream split form, prefill and generic shapes
# (no scratch), the fp32 decode split form, and the first shape again
SEQUENCE = [(16, 4096, 6144, "bf16"), (8, 1024, 2048, "bf16"), (64, 1024, 2048, "bf16"),
            (300, 512, 1024, "bf16"), (7, 100, 36, "bf16"), (8, 1024, 1024, "f32"),
            (16, 4096, 6144, "bf16")]


def _call(lib, fn, x, g, w, y, eps, dtype, ws=None, ws_bytes=0):
    M, K = x.shape
    N = w.shape[1]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if fn == "noalloc":
        return lib.rmsnorm_matmul_noalloc(x.data_ptr(), g.data_ptr(), w.data_ptr(), y.data_ptr(),
                                          ctypes.c_float(eps), M, N, K, dtype, stream)
    return lib.rmsnorm_matmul(x.data_ptr(), g.data_ptr(), w.data_ptr(), y.data_ptr(),
                              ctypes.c_float(eps), M, N, K, dtype, ws, ws_bytes, stream)


def test_noalloc_matches_the_workspace_call(require_gpu):
    lib = tpa.load_library()
    for i, (M, K, N, dt) in enumerate(SEQUENCE):
        print(f"noalloc call {i}: {M}x{K}x{N} {dt}", flush=True)
        wl = synth.Workload("noalloc", dt, M, K, N, 1e-6, False, None)
        inp = synth.make_inputs(wl, seed=60 + i)
        x, g, w = to_device(inp, "X"), to_device(inp, "g"), to_device(inp, "W1")
        tdt = torch.bfloat16 if dt == "bf16" else torch.float32
        dcode = tpa._binding.DTYPE_BF16 if dt == "bf16" else tpa._binding.DTYPE_F32
        y0 = torch.full((M, N), float("nan"), dtype=tdt, device="cuda")
        y1 = torch.full((M, N), float("nan"), dtype=tdt, device="cuda")
        st = _call(lib, "noalloc", x, g, w, y0, wl.eps, dcode)
        assert st == 0, tpa._binding.status_string(st)
        need = int(lib.rmm_workspace_bytes(dcode, M, N, K, 0))
        wst = torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda")
        st = _call(lib, "ws", x, g, w, y1, wl.eps, dcode, wst.data_ptr() if need else None, need)
        assert st == 0, tpa._binding.status_string(st)
        torch.cuda.synchronize()
        assert torch.equal(y0.view(torch.int16 if dt == "bf16" else torch.int32),
                           y1.view(torch.int16 if dt == "bf16" else torch.int32)), f"call {i}"
        assert_within_tol(from_device(y0), run_oracle(inp, wl.eps), tol_for(dt), f"call {i}")


def test_noalloc_errors(require_gpu):
    lib = tpa.load_library()
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    g = torch.ones(64, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((64, 32), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((4, 32), dtype=torch.bfloat16, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    bf = tpa._binding.DTYPE_BF16
    assert lib.rmsnorm_matmul_noalloc(None, g.data_ptr(), w.data_ptr(), y.data_ptr(), 1e-6, 4, 32,
                                      64, bf, stream) == 1
    assert lib.rmsnorm_matmul_noalloc(x.data_ptr(), g.data_ptr(), w.data_ptr(), y.data_ptr(), -1.0,
                                      4, 32, 64, bf, stream) == 3
    assert lib.rmsnorm_matmul_noalloc(x.data_ptr(), g.data_ptr(), w.data_ptr(), x.data_ptr(), 1e-6,
                                      4, 32, 64, bf, stream) == 5
