"""The unfused two-kernel program (needs an MI355X).

The worked example of the Mirage paper review ("核心概念 / μGraph示例")
compares the fused kernel with what existing systems run: an RMSNorm kernel
that writes the normalised activations to memory and a MatMul kernel that
reads them back.  rmm_rmsnorm / rmm_matmul / rmm_gated_matmul are that
program; each piece is checked against the matching oracle step, and the
composition against the oracle's whole definition.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import tensor_program_amd as tpa
from tests.gpu_util import (assert_within_tol, bits_of, expected_exact, from_device, to_device,
                            tol_for)

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _check_rows(xn, ref, dtype, what):
    # One rounding of an fp32 value that is within a few fp32 ulps of the
    # exact one: 2^-8 relative for bf16 storage, 1e-6 for fp32.
    rel = 2.0 ** -8 if dtype == "bf16" else 1e-6
    err = np.abs(xn - ref)
    lim = rel * np.abs(ref) + 1e-30
    bad = err > lim
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} rows elements outside {rel:g} relative"


@pytest.mark.parametrize("name", ["f32_m8_k1024_n1024", "decode_m16_k4096_n6144",
                                  "prefill_m4096_k4096_n4096", "large_m8192_k8192_n28672"])
def test_rmsnorm_rows(name, require_gpu):
    wl = synth.get_workload(name)
    rows = np.arange(min(wl.M, 512))  # the large workload: its first 512 rows
    _log(f"rmsnorm {name} rows {len(rows)}")
    inp = synth.make_inputs(wl, rows=rows if wl.M > 512 else None, weights=False)
    xn = from_device(tpa.rmsnorm(to_device(inp, "X"), to_device(inp, "g"), wl.eps))
    torch.cuda.synchronize()
    ref = oracle.rmsnorm(inp.X, inp.g, oracle.eps_as_passed(wl.eps))
    _check_rows(xn, ref, wl.dtype, name)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(5, 37), (3, 64), (1, 8)])
def test_rmsnorm_odd_and_unaligned(shape, dtype, require_gpu):
    M, K = shape
    wl = synth.Workload("odd", dtype, M, K, 8, 1e-6, False, None)
    inp = synth.make_inputs(wl, weights=False)
    x = to_device(inp, "X")
    big = torch.empty(M * K + 1, dtype=x.dtype, device="cuda")
    xs = big[1:].view(M, K)  # one element off: not 16-byte aligned
    xs.copy_(x)
    xn = from_device(tpa.rmsnorm(xs, to_device(inp, "g"), 1e-6))
    _check_rows(xn, oracle.rmsnorm(inp.X, inp.g, oracle.eps_as_passed(1e-6)), dtype, "odd")


# (M, K, N, dtype, variant the plain product is expected to run)
PLAIN_CASES = [
    (16, 4096, 6144, "bf16", "decode"),
    (64, 4096, 14336, "bf16", "stream"),
    (512, 1024, 1024, "bf16", "prefill"),
    (8, 1024, 1024, "f32", "decode"),
    (24, 1024, 1024, "f32", "decode"),      # two 16-row launches
    (40, 1024, 1024, "f32", "generic"),
    (7, 100, 36, "bf16", "generic"),
]


@pytest.mark.parametrize("case", PLAIN_CASES, ids=lambda c: "x".join(map(str, c)))
def test_matmul_exact(case, require_gpu):
    M, K, N, dtype, variant = case
    assert tpa.plan(M, N, K, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)[1] == variant
    _log(f"matmul exact {case}")
    inp = synth.make_exact_inputs(M, K, N, dtype, seed=3)
    y = tpa.matmul(to_device(inp, "X"), to_device(inp, "W1"))
    torch.cuda.synchronize()
    want = expected_exact(oracle.matmul(inp.X, inp.W1), dtype)
    got = bits_of(y) if dtype == "bf16" else y.cpu().numpy()
    mism = np.argwhere(got != want)
    assert mism.size == 0, f"{len(mism)} mismatches, first at {tuple(mism[0])}"


@pytest.mark.parametrize("shape", [(13, 520, 392), (64, 1024, 14336), (200, 1032, 1032)])
def test_gated_matmul(shape, require_gpu):
    M, K, N = shape
    wl = synth.Workload("gated_plain", "bf16", M, K, N, 1e-6, True, None)
    inp = synth.make_inputs(wl)
    y = from_device(tpa.gated_matmul(to_device(inp, "X"), to_device(inp, "W1"),
                                     to_device(inp, "W3")))
    ref = oracle.gated_matmul(inp.X, inp.W1, inp.W3)
    assert_within_tol(y, ref, tol_for("bf16"), "gated_matmul")


@pytest.mark.parametrize("name", ["decode_m16_k4096_n6144", "gated_m64_k4096_n14336"])
def test_unfused_program_matches_definition(name, require_gpu):
    wl = synth.get_workload(name)
    _log(f"unfused program {name}")
    inp = synth.make_inputs(wl)
    x, g, w1 = to_device(inp, "X"), to_device(inp, "g"), to_device(inp, "W1")
    xn = tpa.rmsnorm(x, g, wl.eps)
    cols = None
    if wl.gated:
        y = tpa.gated_matmul(xn, w1, to_device(inp, "W3"))
        cols = np.sort(np.random.default_rng(9).choice(wl.N, size=1024, replace=False))
    else:
        y = tpa.matmul(xn, w1)
    y = from_device(y)
    e = oracle.eps_as_passed(wl.eps)
    if wl.gated:
        ref = oracle.rmsnorm_gated_mlp(inp.X, inp.g, inp.W1[:, cols], inp.W3[:, cols], e)
        y = y[:, cols]
    else:
        ref = oracle.rmsnorm_matmul(inp.X, inp.g, inp.W1, e)
    assert_within_tol(y, ref, tol_for(wl.dtype), f"unfused {name}")


@pytest.mark.parametrize("shape", [(1, 64), (33, 64), (31, 128), (1000, 128), (9, 256),
                                   (300, 512), (65536, 128)], ids=lambda s: "x".join(map(str, s)))
def test_rmsnorm_short_rows(shape, require_gpu):
    # Rows of 64 .. 512 (many rows per workgroup, a ragged last workgroup):
    # the per-key normalisation of the unfused QKNorm program.
    M, K = shape
    _log(f"rmsnorm short rows {shape}")
    wl = synth.Workload("rows", "bf16", M, K, 8, 1e-6, False, None)
    inp = synth.make_inputs(wl, weights=False)
    x = to_device(inp, "X")
    big = torch.full((M * K + 512,), 7.0, dtype=x.dtype, device="cuda")
    out = big[256:256 + M * K].view(M, K)
    xn = from_device(tpa.rmsnorm(x, to_device(inp, "g"), 1e-6, out=out))
    ref = oracle.rmsnorm(inp.X, inp.g, oracle.eps_as_passed(1e-6))
    _check_rows(xn, ref, "bf16", f"short rows {shape}")
    assert torch.all(big[:256] == 7.0) and torch.all(big[256 + M * K:] == 7.0)
