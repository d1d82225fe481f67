"""Parity of the low-rank adapter calls with the CPU oracle (needs an MI355X).

rmsnorm_lora computes Nrm W + (Nrm A^T) B and lora_matmul X W + (X A^T) B
(the LoRA row of the Mirage paper review's benchmark table, "五、实验结果").

* exact-arithmetic cases, bit for bit after the one rounding of Y: the
  decode kernel at every split count (the down-projection partials ride the
  split-K combine), ranks below, at and between its 16-wide blocks, ragged
  N and K, both 16-row blocks, and several 32-row launches (M up to 128);
  the prefill tile (T = (X g) A^T from its own kernel, then one more k-step
  of the two-part tile) for more rows and ranks above 32; the generic kernel
  for fp32;
* the adapter workload within tolerance, and B = 0 against the plain fused
  call on the same kernels.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import tensor_program_amd as tpa
from tests.gpu_util import assert_within_tol, bits_of, expected_exact, from_device, to_device, tol_for

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _lora_gpu(inp, eps, variant="auto", splits=0, norm=True):
    x, w = to_device(inp, "X"), to_device(inp, "W1")
    a, b = to_device(inp, "LA"), to_device(inp, "LB")
    if norm:
        y = tpa.rmsnorm_lora(x, to_device(inp, "g"), w, a, b, eps, variant=variant, splits=splits)
    else:
        y = tpa.lora_matmul(x, w, a, b)
    torch.cuda.synchronize()
    return y


LORA_EXACT = [
    # (M, K, N, R, dtype, variant, splits)
    (16, 4096, 6144, 16, "bf16", "decode", 0),
    (16, 4096, 6144, 16, "bf16", "decode", 1),
    (16, 4096, 6144, 32, "bf16", "decode", 4),
    (16, 4096, 6144, 8, "bf16", "decode", 3),
    (5, 136, 264, 24, "bf16", "decode", 2),     # ragged N, rank between blocks
    (32, 1024, 1032, 32, "bf16", "decode", 5),  # two row blocks
    (17, 1000, 520, 1, "bf16", "decode", 4),    # ragged K chunks
    (32, 4096, 1032, 16, "bf16", "decode", 1),  # A operand re-staged in segments
    (1, 8, 8, 16, "bf16", "decode", 0),
    (16, 1024, 1024, 64, "bf16", "generic", 0),
    (33, 200, 136, 48, "bf16", "generic", 0),
    (8, 1024, 1024, 16, "f32", "generic", 0),
    (5, 40, 24, 3, "f32", "generic", 0),
    (64, 1024, 2048, 16, "bf16", "auto", 0),    # M > 32: two 32-row decode launches
    (100, 520, 1032, 16, "bf16", "decode", 3),  # four launches, ragged last block
    (129, 200, 136, 8, "bf16", "generic", 0),   # the generic kernel above 128 rows
    # the prefill tile: ragged rows, columns and last k-step, every rank
    # block count, zero-padded ranks, K past the in-LDS gain
    (129, 200, 136, 8, "bf16", "auto", 0),
    (300, 1032, 520, 16, "bf16", "prefill", 0),
    (256, 4096, 1024, 64, "bf16", "prefill", 0),
    (130, 520, 264, 40, "bf16", "auto", 0),
    (16, 1024, 1032, 48, "bf16", "auto", 0),    # R > 32 at decode size: the prefill tile
    (200, 136, 16392, 1, "bf16", "prefill", 0),
    (129, 10248, 264, 16, "bf16", "prefill", 0),
    # the prefill tile with K split into ranges (T B added by the last one)
    (300, 1032, 520, 16, "bf16", "prefill", 4),
    (256, 4096, 1024, 64, "bf16", "prefill", 8),
    (129, 10248, 264, 16, "bf16", "prefill", 7),
    (200, 136, 16392, 1, "bf16", "prefill", 2),
    (130, 520, 264, 40, "bf16", "prefill", 3),
    (100, 1032, 1032, 16, "bf16", "auto", 0),   # above 64 rows with a workspace: the split tile
]


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("case", LORA_EXACT, ids=lambda c: "x".join(map(str, c)))
def test_lora_exact_bitwise(case, seed, require_gpu):
    M, K, N, R, dtype, variant, splits = case
    _log(f"lora exact {case} seed {seed}")
    inp = synth.make_exact_inputs(M, K, N, dtype, seed=seed, row_pow2=(seed == 1), lora=R)
    if variant != "auto":
        assert tpa.plan_lora(M, N, K, R, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32,
                             variant=variant, splits=splits)[0] == 0
    y = _lora_gpu(inp, 0.0, variant=variant, splits=splits)
    want = expected_exact(oracle.rmsnorm_lora(inp.X, inp.g, inp.W1, inp.LA, inp.LB, 0.0), dtype)
    got = bits_of(y) if dtype == "bf16" else y.cpu().numpy()
    mism = np.argwhere(got != want)
    assert mism.size == 0, f"{len(mism)} mismatches, first at {tuple(mism[0])}"


@pytest.mark.parametrize("case", [(16, 4096, 6144, 16, "bf16"), (7, 100, 36, 5, "bf16"),
                                  (8, 1024, 1024, 16, "f32"), (200, 1000, 520, 16, "bf16")],
                         ids=lambda c: "x".join(map(str, c)))
def test_lora_matmul_exact(case, require_gpu):
    M, K, N, R, dtype = case
    _log(f"lora_matmul exact {case}")
    inp = synth.make_exact_inputs(M, K, N, dtype, seed=5, lora=R)
    y = _lora_gpu(inp, 0.0, norm=False)
    want = expected_exact(oracle.lora_matmul(inp.X, inp.W1, inp.LA, inp.LB), dtype)
    got = bits_of(y) if dtype == "bf16" else y.cpu().numpy()
    mism = np.argwhere(got != want)
    assert mism.size == 0, f"{len(mism)} mismatches, first at {tuple(mism[0])}"


@pytest.mark.parametrize("variant,splits", [("auto", 0), ("decode", 1), ("generic", 0)])
def test_lora_workload(variant, splits, require_gpu):
    wl = synth.get_workload("lora_m16_k4096_n6144_r16")
    _log(f"lora workload variant {variant} splits {splits}")
    inp = synth.make_inputs(wl)
    y = from_device(_lora_gpu(inp, wl.eps, variant=variant, splits=splits))
    e = oracle.eps_as_passed(wl.eps)
    ref = oracle.rmsnorm_lora(inp.X, inp.g, inp.W1, inp.LA, inp.LB, e)
    # the elementwise bound tol (|Y_ref| + 1), also where the frozen product
    # and the adapter term cancel
    worst = assert_within_tol(y, ref, tol_for(wl.dtype), f"lora/{variant}")
    _log(f"  worst err/tol {worst:.3f}")


@pytest.mark.parametrize("M", [256, 512, 1000])
def test_lora_prefill_workload_recipe(M, require_gpu):
    """The adapter workload's shape and value recipe with more rows (the
    prefill tile), on every output at the elementwise bound."""
    base = synth.get_workload("lora_m16_k4096_n6144_r16")
    wl = synth.Workload("lora_prefill", base.dtype, M, base.K, base.N, base.eps, False, None,
                        base.lora)
    assert tpa.plan_lora(M, wl.N, wl.K, wl.lora)[1] == "prefill"
    _log(f"lora prefill workload recipe M={M}")
    inp = synth.make_inputs(wl)
    y = from_device(_lora_gpu(inp, wl.eps))
    ref = oracle.rmsnorm_lora(inp.X, inp.g, inp.W1, inp.LA, inp.LB, oracle.eps_as_passed(wl.eps))
    worst = assert_within_tol(y, ref, tol_for(wl.dtype), "lora/prefill")
    _log(f"  worst err/tol {worst:.3f}")


def test_lora_zero_b_is_the_exact_operand_product(require_gpu):
    """With B = 0 the adapter call is the frozen product alone, computed from
    the exact (two-part) operand X*g: within the output's own bf16 rounding
    (2^-8 relative) plus fp32 summation noise of the oracle's plain product,
    far inside the tolerance."""
    wl = synth.get_workload("lora_m16_k4096_n6144_r16")
    inp = synth.make_inputs(wl)
    x, g, w = to_device(inp, "X"), to_device(inp, "g"), to_device(inp, "W1")
    a = to_device(inp, "LA")
    b0 = torch.zeros((wl.lora, wl.N), dtype=x.dtype, device=x.device)
    y_lora = from_device(tpa.rmsnorm_lora(x, g, w, a, b0, wl.eps))
    torch.cuda.synchronize()
    ref = oracle.rmsnorm_matmul(inp.X, inp.g, inp.W1, oracle.eps_as_passed(wl.eps))
    err = np.abs(y_lora - ref)
    assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-5), float((err - 2.0 ** -8 * np.abs(ref)).max())


def test_lora_canaries_and_repeat(require_gpu):
    # Y inside a larger buffer: the guard elements stay untouched, and a
    # second call on the same workspace (counters reset by the first) gives
    # the same bits.
    M, K, N, R = 17, 1000, 520, 24
    inp = synth.make_exact_inputs(M, K, N, "bf16", seed=2, lora=R)
    x, g, w = to_device(inp, "X"), to_device(inp, "g"), to_device(inp, "W1")
    a, b = to_device(inp, "LA"), to_device(inp, "LB")
    big = torch.full((M * N + 256,), 7.0, dtype=torch.bfloat16, device="cuda")
    out = big[128:128 + M * N].view(M, N)
    ws = tpa.Workspace(tpa._binding.lora_workspace_bytes(tpa._binding.DTYPE_BF16, M, N, K, R,
                                                         "decode", 4), "cuda")
    tpa.rmsnorm_lora(x, g, w, a, b, 0.0, out=out, variant="decode", splits=4, workspace=ws)
    first = bits_of(out).copy()
    tpa.rmsnorm_lora(x, g, w, a, b, 0.0, out=out, variant="decode", splits=4, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(out), first)
    want = expected_exact(oracle.rmsnorm_lora(inp.X, inp.g, inp.W1, inp.LA, inp.LB, 0.0), "bf16")
    assert np.array_equal(first, want)
    guard = torch.cat([big[:128], big[128 + M * N:]]).float()
    assert torch.all(guard == 7.0)
    # the arrival counters (one per 128-column tile, at the start) are reset
    tiles = (N + 127) // 128
    assert torch.count_nonzero(ws.tensor[:4 * tiles]) == 0
