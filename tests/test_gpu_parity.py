"""Parity of the HIP path with the CPU oracle (needs an MI355X).

* exact-arithmetic cases: inputs on which every product and partial sum is
  exact in fp32 in any order, so the kernels must reproduce the oracle's
  result bit for bit (after its one rounding to the storage type), for every
  variant and forced split count -- the float analogue of the randomised
  equivalence test of the Mirage paper review ("等价性验证");
* the five workloads within tolerance, on all outputs where the oracle is
  quick and on sampled rows/columns at the full sizes;
* edge cases: empty, ragged, unaligned, zero rows, canaries around Y.
"""
import numpy as np
import pytest
import torch

import synth
import tensor_program_amd as tpa
from tests.gpu_util import (GATE_TINY, assert_within_tol, bits_of, expected_exact,
                            expected_gated_exact, from_device, run_gpu, run_oracle, to_device,
                            tol_for)

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


# ---------------------------------------------------------------- exact cases
EXACT_CASES = [
    # (M, K, N, dtype, variant, splits)
    (1, 8, 8, "f32", "generic", 0),
    (5, 40, 24, "f32", "generic", 0),
    (33, 200, 136, "bf16", "generic", 0),
    (8, 1024, 1024, "f32", "generic", 0),
    (8, 1024, 1024, "f32", "decode", 0),     # 32 tiles x 8 K ranges, split-K combine
    (8, 1024, 1024, "f32", "decode", 1),     # one range: 4 chunks of 256 in one workgroup
    (1, 8, 8, "f32", "decode", 0),
    (5, 40, 24, "f32", "decode", 0),
    (16, 1000, 520, "f32", "decode", 3),     # ragged K ranges, N % 32 != 0
    (13, 4096, 136, "f32", "decode", 0),     # 32 ranges of 128
    (11, 1000, 72, "f32", "decode", 1),      # multi-chunk loop with a partial last chunk
    (32, 1024, 1024, "f32", "decode", 0),    # two 16-row launches
    (21, 520, 136, "f32", "decode", 3),      # a ragged second block
    (16, 4096, 6144, "bf16", "generic", 0),
    (16, 4096, 6144, "bf16", "decode", 1),
    (16, 4096, 6144, "bf16", "decode", 3),
    (16, 4096, 6144, "bf16", "decode", 16),
    (16, 4096, 6144, "bf16", "decode", 32),
    (5, 136, 264, "bf16", "decode", 1),
    (5, 136, 264, "bf16", "decode", 2),
    (1, 8, 8, "bf16", "decode", 0),
    (32, 1024, 1032, "bf16", "decode", 5),
    (17, 1000, 520, "bf16", "decode", 4),
    (32, 4096, 1032, "bf16", "decode", 1),   # A operand re-staged in 8 segments
    (16, 8192, 264, "bf16", "decode", 2),    # 8 waves, 4 segments per split
    (256, 64, 256, "bf16", "prefill", 0),
    (300, 200, 264, "bf16", "prefill", 0),
    (513, 1032, 520, "bf16", "prefill", 0),
    (1, 8, 8, "bf16", "prefill", 0),
    (40, 4096, 2048, "bf16", "prefill", 0),
    (4096, 4096, 4096, "bf16", "prefill", 0),
    (1024, 8192, 28672, "bf16", "prefill", 0),
    # prefill with K split into ranges (few output tiles): forced counts,
    # ragged ranges, a last range ending inside a step, an odd last range
    (256, 4096, 4096, "bf16", "prefill", 1),
    (256, 4096, 4096, "bf16", "prefill", 16),
    (129, 1000, 520, "bf16", "prefill", 5),
    (300, 1032, 264, "bf16", "prefill", 3),
    (513, 200, 1032, "bf16", "prefill", 2),
    (200, 2048, 1032, "bf16", "prefill", 8),
    (384, 4096, 4096, "bf16", "prefill", 0),
    (64, 4096, 14336, "bf16", "stream", 0),
    (33, 1000, 520, "bf16", "stream", 0),
    (1, 8, 8, "bf16", "stream", 0),
    (64, 136, 4104, "bf16", "stream", 0),
    # stream at wide N: 256 strips (one per CU), 257 (a second round with an
    # 8-column last strip), 219 and 96 strips with 48- and 56-column last
    # strips
    (16, 136, 16384, "bf16", "stream", 0),
    (8, 200, 16392, "bf16", "stream", 0),
    (20, 264, 14000, "bf16", "stream", 0),
    (16, 520, 6136, "bf16", "stream", 0),
    # two 64-row launches: a full and a ragged second block, split and unsplit
    (100, 264, 1032, "bf16", "stream", 0),
    (128, 136, 16392, "bf16", "stream", 0),
    (200, 136, 1032, "bf16", "stream", 0),   # four launches, ragged last block
]

EXACT_SAMPLE_ROWS = 48  # above ~1e10 multiply-adds the oracle checks sampled rows


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("case", EXACT_CASES, ids=lambda c: "x".join(map(str, c)))
def test_exact_bitwise(case, seed, require_gpu):
    M, K, N, dtype, variant, splits = case
    _log(f"exact {case} seed {seed}")
    inp = synth.make_exact_inputs(M, K, N, dtype, seed=seed, row_pow2=(seed == 1))
    y = run_gpu(inp, 0.0, variant=variant, splits=splits)
    rows = None
    if M * K * N > 10**10:
        rng = np.random.default_rng(seed)
        rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, EXACT_SAMPLE_ROWS, replace=False)]))
    want = expected_exact(run_oracle(inp, 0.0, rows=rows), dtype)
    got = bits_of(y) if dtype == "bf16" else y.cpu().numpy()
    if rows is not None:
        got = got[rows]
    mism = np.argwhere(got != want)
    assert mism.size == 0, f"{len(mism)} mismatches, first at {tuple(mism[0])}"


# ------------------------------------------------------------ the workloads
def _check_workload(name, variant="auto", splits=0, rows=None, cols=None):
    wl = synth.get_workload(name)
    _log(f"workload {name} variant {variant} splits {splits}")
    inp = synth.make_inputs(wl)
    y = from_device(run_gpu(inp, wl.eps, variant=variant, splits=splits))
    if rows is not None:
        y = y[rows]
    if cols is not None:
        y = y[:, cols]
    ref = run_oracle(inp, wl.eps, rows=rows, cols=cols)
    worst = assert_within_tol(y, ref, tol_for(wl.dtype), f"{name}/{variant}")
    _log(f"  worst err/tol {worst:.3f}")


@pytest.mark.parametrize("variant,splits", [("auto", 0), ("generic", 0), ("decode", 1),
                                            ("decode", 16)])
def test_f32_m8_k1024_n1024(variant, splits, require_gpu):
    _check_workload("f32_m8_k1024_n1024", variant, splits)


@pytest.mark.parametrize("variant,splits", [("auto", 0), ("generic", 0), ("decode", 1),
                                            ("decode", 8)])
def test_decode_m16_k4096_n6144(variant, splits, require_gpu):
    _check_workload("decode_m16_k4096_n6144", variant, splits)


def _sample_rows(wl, n_random=48):
    rng = np.random.default_rng(7)
    rows = set(rng.choice(wl.M, size=n_random, replace=False).tolist()) | {0, wl.M - 1}
    scale = synth.row_scales(wl)
    if scale is not None:
        # every scaled-by-100 row, and the smallest and largest LogUniform scales
        if wl.row_scale == "pick_x100":
            rows |= set(np.nonzero(scale == 100.0)[0].tolist())
        else:
            order = np.argsort(scale)
            rows |= set(order[:8].tolist()) | set(order[-8:].tolist())
    return np.array(sorted(rows))


@pytest.mark.parametrize("variant", ["auto", "generic", "prefill"])
def test_prefill_m4096_k4096_n4096_sampled(variant, require_gpu):
    wl = synth.get_workload("prefill_m4096_k4096_n4096")
    _check_workload(wl.name, variant=variant, rows=_sample_rows(wl))


_GATED_REF = {}


@pytest.mark.parametrize("variant", ["auto", "stream", "decode", "generic"])
def test_gated_m64_k4096_n14336_full(variant, require_gpu):
    """The gated workload on every one of its 64 x 14336 outputs, at the
    elementwise bound (decode: 16-row launches are refused above 16 rows, so
    it runs on the first 16 rows)."""
    wl = synth.get_workload("gated_m64_k4096_n14336")
    inp = synth.make_inputs(wl)
    if "ref" not in _GATED_REF:
        _GATED_REF["ref"] = run_oracle(inp, wl.eps)
    ref = _GATED_REF["ref"]
    _log(f"workload {wl.name} variant {variant} (all outputs)")
    if variant == "decode":
        x16 = to_device(inp, "X")[:16].contiguous()
        y = from_device(run_gpu(inp, wl.eps, variant=variant, x=x16))
        ref = ref[:16]
    else:
        y = from_device(run_gpu(inp, wl.eps, variant=variant))
    worst = assert_within_tol(y, ref, tol_for(wl.dtype), f"{wl.name}/{variant}")
    _log(f"  worst err/tol {worst:.3f}")


def test_gated_m4096_k4096_n14336_sampled(require_gpu):
    """The gated product at prefill size (the 128-row gated tile, auto-selected
    above 128 rows): the gated workload's shape and value recipe with 4096
    rows, checked on sampled rows at the elementwise bound."""
    base = synth.get_workload("gated_m64_k4096_n14336")
    wl = synth.Workload("gated_m4096_k4096_n14336", base.dtype, 4096, base.K, base.N, base.eps,
                        True, None)
    assert tpa.plan(wl.M, wl.N, wl.K, gated=True)[1] == "prefill"
    rows = _sample_rows(wl, n_random=24)
    _log(f"gated prefill 4096 x 4096 x 14336, {len(rows)} sampled rows")
    inp = synth.make_inputs(wl)
    y = from_device(run_gpu(inp, wl.eps))[rows]
    worst = assert_within_tol(y, run_oracle(inp, wl.eps, rows=rows), tol_for(wl.dtype), wl.name)
    _log(f"  worst err/tol {worst:.3f}")


@pytest.mark.parametrize("M,K,N", [(129, 1000, 520), (200, 264, 1032), (300, 136, 264),
                                   (256, 4096, 384), (136, 10248, 136)])
def test_gated_prefill_shapes(M, K, N, require_gpu):
    """The gated prefill tile on ragged shapes: partial row and column tiles,
    a partial last k-step, and K past the in-LDS gain (10248), against the
    oracle at the elementwise bound."""
    wl = synth.Workload("gated_prefill", "bf16", M, K, N, 1e-6, True, None)
    _log(f"gated prefill M={M} K={K} N={N}")
    inp = synth.make_inputs(wl, seed=13)
    y = from_device(run_gpu(inp, wl.eps, variant="prefill"))
    worst = assert_within_tol(y, run_oracle(inp, wl.eps), 1e-2, "gated_prefill")
    _log(f"  worst err/tol {worst:.3f}")


@pytest.mark.parametrize("M,K,N,splits", [(384, 4096, 4096, 0), (256, 4096, 4096, 8),
                                          (129, 14336, 4096, 0), (1000, 1032, 2056, 0),
                                          (512, 4096, 4096, 7)])
def test_prefill_split_shapes(M, K, N, splits, require_gpu):
    """Plain prefill with K split into ranges (few output tiles), on the
    prefill workload's value recipe with rows scaled by 100, at the
    elementwise bound on every output."""
    wl = synth.Workload("prefill_split", "bf16", M, K, N, 1e-6, False, "pick_x100")
    st, variant, s = tpa.plan(M, N, K, variant="prefill", splits=splits)
    assert st == 0 and s > 1, (st, variant, s)
    _log(f"prefill split M={M} K={K} N={N} splits {splits} -> {s}")
    inp = synth.make_inputs(wl, seed=17)
    y = from_device(run_gpu(inp, wl.eps, variant="prefill", splits=splits))
    worst = assert_within_tol(y, run_oracle(inp, wl.eps), tol_for("bf16"), "prefill_split")
    _log(f"  worst err/tol {worst:.3f}")


@pytest.mark.parametrize("M,K,N,splits", [(256, 4096, 14336, 2), (512, 4096, 4096, 0),
                                          (129, 14336, 4096, 0), (300, 1032, 2056, 7)])
def test_gated_prefill_split_shapes(M, K, N, splits, require_gpu):
    """The gated tile with K split into ranges, on the gated workload's value
    recipe, at the elementwise bound on every output."""
    wl = synth.Workload("gated_split", "bf16", M, K, N, 1e-6, True, None)
    st, variant, s = tpa.plan(M, N, K, gated=True, variant="prefill", splits=splits)
    assert st == 0 and s > 1, (st, variant, s)
    _log(f"gated prefill split M={M} K={K} N={N} splits {splits} -> {s}")
    inp = synth.make_inputs(wl, seed=19)
    y = from_device(run_gpu(inp, wl.eps, variant="prefill", splits=splits))
    worst = assert_within_tol(y, run_oracle(inp, wl.eps), tol_for("bf16"), "gated_split")
    _log(f"  worst err/tol {worst:.3f}")


def test_large_m8192_k8192_n28672_sampled(require_gpu):
    wl = synth.get_workload("large_m8192_k8192_n28672")
    _check_workload(wl.name, rows=_sample_rows(wl, n_random=24))


# ----------------------------------------------------------------- gated small
@pytest.mark.parametrize("variant,splits", [("generic", 0), ("decode", 1), ("decode", 3),
                                            ("stream", 0)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gated_small(variant, splits, dtype, require_gpu):
    if dtype == "f32" and variant in ("decode", "stream"):
        pytest.skip("the gated product in fp32 runs the generic kernel only")
    wl = synth.Workload("gated_small", dtype, 13, 520, 392, 1e-6, True, None)
    _log(f"gated small {dtype} {variant} {splits}")
    inp = synth.make_inputs(wl, seed=5)
    y = from_device(run_gpu(inp, wl.eps, variant=variant, splits=splits))
    assert_within_tol(y, run_oracle(inp, wl.eps), tol_for(dtype), "gated_small")


# ------------------------------------------------------------------ edge cases
def _tensors(M, K, N, dtype=torch.bfloat16, seed=0):
    gen = torch.Generator().manual_seed(seed)
    x = torch.randn(M, K, generator=gen).to(dtype).cuda()
    g = (1 + 0.1 * torch.randn(K, generator=gen)).to(dtype).cuda()
    w = (torch.randn(K, N, generator=gen) / K ** 0.5).to(dtype).cuda()
    return x, g, w


def test_empty_is_noop(require_gpu):
    for (M, N) in ((0, 16), (4, 0)):
        x, g, w = _tensors(max(M, 1), 16, max(N, 1))
        x = x[:M].contiguous()
        w = w[:, :N].contiguous()
        y = tpa.rmsnorm_matmul(x, g, w, 1e-6)
        torch.cuda.synchronize()
        assert tuple(y.shape) == (M, N)


def test_zero_row_gives_zero(require_gpu):
    for variant in ("generic", "decode", "prefill", "stream"):
        x, g, w = _tensors(4, 256, 128)
        x[2] = 0
        y = tpa.rmsnorm_matmul(x, g, w, 1e-6, variant=variant)
        torch.cuda.synchronize()
        assert torch.all(y[2] == 0)
        assert torch.all(torch.isfinite(y.float()))


def test_canaries_around_output(require_gpu):
    """Y is written in full and nothing outside it is touched."""
    for variant, (M, K, N) in (("generic", (7, 72, 200)), ("decode", (7, 1024, 1032)),
                               ("decode", (16, 4096, 6144)), ("prefill", (300, 200, 264)),
                               ("prefill", (512, 256, 512)), ("stream", (40, 520, 328))):
        x, g, w = _tensors(M, K, N)
        guard = 4096
        buf = torch.full((guard + M * N + guard,), float("nan"), dtype=torch.bfloat16, device="cuda")
        buf[:guard] = 7.0
        buf[-guard:] = -7.0
        y = buf[guard:guard + M * N].view(M, N)
        tpa.rmsnorm_matmul(x, g, w, 1e-6, out=y, variant=variant)
        torch.cuda.synchronize()
        assert torch.all(torch.isfinite(y.float())), variant
        assert torch.all(buf[:guard] == 7.0) and torch.all(buf[-guard:] == -7.0), variant


def test_unaligned_pointers_take_generic_and_match(require_gpu):
    M, K, N = 6, 256, 264
    inp = synth.make_inputs(synth.Workload("unaligned", "bf16", M, K, N, 1e-6, False, None), seed=3)
    X = to_device(inp, "X")
    big = torch.empty(M * K + 1, dtype=torch.bfloat16, device="cuda")
    xs = big[1:].view(M, K)  # 2-byte offset: not 16-byte aligned
    xs.copy_(X)
    y = from_device(run_gpu(inp, 1e-6, x=xs))
    assert_within_tol(y, run_oracle(inp, 1e-6), 1e-2, "unaligned")


def test_workspace_reuse_and_streams(require_gpu):
    """Arrival counters reset themselves: repeated calls give identical bits,
    also on a second stream with its own workspace."""
    x, g, w = _tensors(16, 4096, 6144)
    y0 = tpa.rmsnorm_matmul(x, g, w, 1e-6, variant="decode", splits=16)
    ys = [tpa.rmsnorm_matmul(x, g, w, 1e-6, variant="decode", splits=16) for _ in range(5)]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ys.append(tpa.rmsnorm_matmul(x, g, w, 1e-6, variant="decode", splits=16))
    torch.cuda.synchronize()
    for y in ys:
        assert torch.equal(y.view(torch.int16), y0.view(torch.int16))


def test_errors_raise(require_gpu):
    x, g, w = _tensors(4, 64, 32)
    with pytest.raises(tpa.RmmError):
        tpa.rmsnorm_matmul(x, g, w, -1.0)
    with pytest.raises(tpa.RmmError):
        tpa.rmsnorm_matmul(x, g, w, 1e-6, variant="decode", splits=99)
    with pytest.raises(tpa.RmmError):  # output overlapping the input X
        tpa.rmsnorm_matmul(x, g, w, 1e-6, out=x.view(-1)[:128].view(4, 32))


@pytest.mark.parametrize("M", [1, 16, 40, 64, 65, 128, 256, 300])
def test_gated_stream_shapes(M, require_gpu):
    """Gated stream variant on ragged shapes (above 64 rows: several 64-row
    launches), against the oracle at the elementwise bound."""
    wl = synth.Workload("gated_stream", "bf16", M, 1032, 584, 1e-6, True, None)
    _log(f"gated stream M={M}")
    inp = synth.make_inputs(wl, seed=11)
    y = from_device(run_gpu(inp, wl.eps, variant="stream"))
    worst = assert_within_tol(y, run_oracle(inp, wl.eps), 1e-2, "gated_stream")
    _log(f"  worst err/tol {worst:.3f}")


@pytest.mark.parametrize("M,K,N", [(64, 264, 16392), (48, 264, 14336), (64, 136, 6136)])
def test_gated_stream_wide(M, K, N, require_gpu):
    """Gated stream variant at wide N (257 strips with an 8-column last one,
    224 strips, 96 strips with a 56-column last one), against the oracle at
    the elementwise bound."""
    wl = synth.Workload("gated_stream", "bf16", M, K, N, 1e-6, True, None)
    _log(f"gated stream wide M={M} K={K} N={N}")
    inp = synth.make_inputs(wl, seed=12)
    y = from_device(run_gpu(inp, wl.eps, variant="stream"))
    worst = assert_within_tol(y, run_oracle(inp, wl.eps), 1e-2, "gated_stream_wide")
    _log(f"  worst err/tol {worst:.3f}")


def test_one_workspace_for_every_layout(require_gpu):
    """One zero-filled workspace passed to a sequence of calls with different
    layouts (tile counts, variants, split counts, weight counts, dtypes):
    every call's exact result is right, so no call reads what another left
    in the workspace as its arrival counters.  (The second call has 72
    column tiles: in a layout whose counters were not in a fixed region, its
    counters would sit where the first call left its row-sum partials.)"""
    ws = tpa.Workspace(64 << 20, "cuda")
    seq = [(16, 4096, 1024, "bf16", False, "decode", 4), (16, 1024, 9216, "bf16", False, "decode", 2),
           (33, 1000, 520, "bf16", False, "stream", 0), (8, 1024, 1024, "f32", False, "decode", 0),
           (16, 4096, 6144, "bf16", False, "decode", 8), (13, 1000, 520, "bf16", True, "decode", 3),
           (200, 264, 1032, "bf16", True, "prefill", 3), (256, 1024, 1024, "bf16", False, "prefill", 4),
           (16, 4096, 1024, "bf16", False, "decode", 4)]
    for i, (M, K, N, dtype, gated, variant, splits) in enumerate(seq):
        _log(f"shared workspace call {i}: {M}x{K}x{N} {dtype} gated={gated} {variant} {splits}")
        inp = synth.make_exact_inputs(M, K, N, dtype, seed=40 + i, gated=gated)
        y = run_gpu(inp, 0.0, variant=variant, splits=splits, workspace=ws)
        ref = run_oracle(inp, 0.0)
        if gated:
            lo, hi = expected_gated_exact(ref)
            got = bits_of(y)
            for a in (got, lo, hi):
                a[a == 0x8000] = 0
            tiny = np.abs(ref) < GATE_TINY
            assert not np.any((got != lo) & (got != hi) & ~tiny), f"call {i}"
        else:
            got = bits_of(y) if dtype == "bf16" else y.cpu().numpy()
            assert np.array_equal(got, expected_exact(ref, dtype)), f"call {i}"
    # every call left the counters at zero
    assert torch.count_nonzero(ws.tensor[:64 * 1024]) == 0


# Gated exact-arithmetic cases: both products are exact, so every output must
# be the one bf16 rounding of silu(z1) z3 (up to fp32 noise in the gate).
GATED_EXACT = [
    (16, 4096, 6144, "decode", 4),
    (13, 1000, 520, "decode", 3),
    (5, 136, 264, "decode", 1),
    (64, 4096, 14336, "stream", 0),
    (33, 1000, 520, "stream", 0),     # split form (9 strips)
    (100, 264, 1032, "stream", 0),    # two 64-row launches
    (64, 264, 16392, "stream", 0),    # 257 strips
    (300, 200, 264, "stream", 0),
    (13, 1000, 520, "generic", 0),
    (200, 264, 1032, "prefill", 0),   # gated tile: 2 x 9 tiles, ragged
    (256, 4096, 512, "prefill", 0),
    # the gated tile with K split into ranges: a last range of one step, an
    # odd count rounded down, K past the in-LDS gain, the library's count
    (200, 264, 1032, "prefill", 3),
    (256, 4096, 512, "prefill", 8),
    (129, 1000, 520, "prefill", 5),
    (136, 10248, 136, "prefill", 6),
    (300, 1032, 264, "prefill", 0),
    (256, 4096, 4096, "prefill", 0),
    (100, 1032, 520, "auto", 0),      # above 64 rows with a workspace: the split tile
]


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("case", GATED_EXACT, ids=lambda c: "x".join(map(str, c)))
def test_gated_exact(case, seed, require_gpu):
    M, K, N, variant, splits = case
    _log(f"gated exact {case} seed {seed}")
    inp = synth.make_exact_inputs(M, K, N, "bf16", seed=seed, gated=True, row_pow2=(seed == 1))
    yt = run_gpu(inp, 0.0, variant=variant, splits=splits)
    y = bits_of(yt)
    ref = run_oracle(inp, 0.0)
    lo, hi = expected_gated_exact(ref)
    for a in (y, lo, hi):  # the sign of a zero output is not compared
        a[a == 0x8000] = 0
    tiny = np.abs(ref) < GATE_TINY
    assert np.all(np.abs(from_device(yt)[tiny]) < 2 * GATE_TINY)
    bad = np.argwhere((y != lo) & (y != hi) & ~tiny)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {tuple(bad[0])}"
    _log(f"  {int(tiny.sum())} outputs below 2^-100 of {tiny.size}")
