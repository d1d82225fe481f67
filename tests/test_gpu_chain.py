"""The layer chain in one persistent launch (needs an MI355X).

x_{l+1} = RMSNorm(x_l; g_l, eps) W_l for l = 0 .. L-1.  At these shapes the
chain uses the decode kernel's tiling, split count and summation order, so
every layer must equal -- bit for bit -- a single rmsnorm_matmul call (decode
variant) on the chain's own previous-layer output; the first and last layers
are also checked against the CPU oracle.  The wait flag must stay clear, and
the counters the kernel leaves behind must serve the next call.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import tensor_program_amd as tpa
from tests.gpu_util import assert_within_tol

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _chain_inputs(M, K, L, seed=0):
    layers = [synth.make_inputs(synth.Workload(f"chain_{l}", "bf16", M, K, K, 1e-6, False, None),
                                seed=seed + l) for l in range(L)]

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    x0 = dev(layers[0].bits["X"])
    G = dev(np.stack([lay.bits["g"] for lay in layers]))
    W = dev(np.stack([lay.bits["W1"] for lay in layers]))
    return x0, G, W, layers


def _as64(t):
    return t.float().cpu().numpy().astype(np.float64)


# (M, K, L, split count of the single-layer reference call: 0 = the
# automatic one, which equals the chain's at these shapes).  K = 4480 is the
# largest tiling the chain accepts: 35 tiles x 7 chunks of 640 rows (five
# tiles of the layer before per chunk, an odd number of 256-row steps), where
# the automatic decode split count (4) differs from the chain's, so the
# reference call is given 7.
@pytest.mark.parametrize("M,K,L,splits", [(16, 4096, 4, 0), (5, 1024, 3, 0), (1, 128, 2, 0),
                                          (16, 1024, 1, 0), (16, 4480, 3, 7)])
def test_chain_layers(M, K, L, splits, require_gpu):
    _log(f"chain M={M} K={K} L={L}")
    x0, G, W, layers = _chain_inputs(M, K, L)
    ws = tpa.Workspace(tpa._binding.chain_workspace_bytes(M, K, L), "cuda")
    xs = tpa.rmsnorm_matmul_chain(x0, G, W, 1e-6, workspace=ws)
    torch.cuda.synchronize()
    assert tpa.chain_wait_flag(ws, M, K, L) == 0
    prev = x0
    for layer in range(L):
        want = tpa.rmsnorm_matmul(prev, G[layer], W[layer], 1e-6, variant="decode", splits=splits)
        torch.cuda.synchronize()
        got = xs[layer]
        diff = (got.view(torch.int16) != want.view(torch.int16)).sum().item()
        assert diff == 0, f"layer {layer}: {diff} elements differ from the single call"
        prev = got.contiguous()
    for layer in sorted({0, L - 1}):
        xin = _as64(x0 if layer == 0 else xs[layer - 1])
        ref = oracle.rmsnorm_matmul(xin, layers[layer].g, layers[layer].W1, oracle.eps_as_passed(1e-6))
        assert_within_tol(_as64(xs[layer]), ref, 1e-2, f"layer {layer}")


def test_chain_repeated_calls_and_layouts(require_gpu):
    """Counters left by one call serve the next; other shapes use their own workspace."""
    x0, G, W, _ = _chain_inputs(16, 1024, 3, seed=4)
    first = tpa.rmsnorm_matmul_chain(x0, G, W, 1e-6).clone()
    y0, G2, W2, _ = _chain_inputs(3, 512, 2, seed=9)
    tpa.rmsnorm_matmul_chain(y0, G2, W2, 1e-6)
    for _ in range(3):
        again = tpa.rmsnorm_matmul_chain(x0, G, W, 1e-6)
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int16), first.view(torch.int16))


def test_chain_rejects(require_gpu):
    x0, G, W, _ = _chain_inputs(17, 256, 1)
    with pytest.raises(tpa.RmmError):
        tpa.rmsnorm_matmul_chain(x0, G, W, 1e-6)      # M > 16
