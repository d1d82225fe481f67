"""HIP-graph replay of every kernel variant (needs an MI355X).

The benchmark replays captured calls; the split-K combines rely on arrival
counters that each call resets itself (no memset is captured).  Each graph
below is replayed several times with eager calls and synchronisations in
between, and every replay must reproduce the eager result bit for bit.
"""
import numpy as np
import pytest
import torch

import synth
import tensor_program_amd as tpa
from tests.gpu_util import bits_of, to_device

pytestmark = pytest.mark.gpu


def _replays(fn, out, eager_between):
    want = None
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        fn()  # eager warm-up, also the reference
    torch.cuda.synchronize()
    want = bits_of(out).copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn()
    torch.cuda.synchronize()
    for i in range(4):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = bits_of(out)
        assert np.array_equal(got, want), f"replay {i}: {(got != want).sum()} elements differ"
        eager_between()
        torch.cuda.synchronize()


def test_graph_decode_split_k(require_gpu):
    wl = synth.get_workload("decode_m16_k4096_n6144")
    inp = synth.make_inputs(wl)
    x, g, w = to_device(inp, "X"), to_device(inp, "g"), to_device(inp, "W1")
    out = torch.empty((wl.M, wl.N), dtype=torch.bfloat16, device="cuda")
    ws = tpa.Workspace(tpa._binding.workspace_bytes(tpa._binding.DTYPE_BF16, wl.M, wl.N, wl.K,
                                                    False), "cuda")
    other = torch.empty_like(out)
    _replays(lambda: tpa.rmsnorm_matmul(x, g, w, wl.eps, out=out, workspace=ws), out,
             lambda: tpa.rmsnorm_matmul(x, g, w, wl.eps, out=other, workspace=ws))


def test_graph_decode_f32_split_k(require_gpu):
    wl = synth.get_workload("f32_m8_k1024_n1024")
    inp = synth.make_inputs(wl)
    x, g, w = to_device(inp, "X"), to_device(inp, "g"), to_device(inp, "W1")
    assert tpa.plan(wl.M, wl.N, wl.K, dtype=torch.float32)[1:] == ("decode", 16)
    out = torch.empty((wl.M, wl.N), dtype=torch.float32, device="cuda")
    ws = tpa.Workspace(tpa._binding.workspace_bytes(tpa._binding.DTYPE_F32, wl.M, wl.N, wl.K,
                                                    False), "cuda")
    other = torch.empty_like(out)
    _replays(lambda: tpa.rmsnorm_matmul(x, g, w, wl.eps, out=out, workspace=ws), out,
             lambda: tpa.rmsnorm_matmul(x, g, w, wl.eps, out=other, workspace=ws))


def test_graph_lora_and_attention(require_gpu):
    wl = synth.get_workload("lora_m16_k4096_n6144_r16")
    inp = synth.make_inputs(wl)
    x, g, w = to_device(inp, "X"), to_device(inp, "g"), to_device(inp, "W1")
    a, b = to_device(inp, "LA"), to_device(inp, "LB")
    out = torch.empty((wl.M, wl.N), dtype=torch.bfloat16, device="cuda")
    ws = tpa.Workspace(tpa._binding.lora_workspace_bytes(tpa._binding.DTYPE_BF16, wl.M, wl.N,
                                                         wl.K, wl.lora), "cuda")
    _replays(lambda: tpa.rmsnorm_lora(x, g, w, a, b, wl.eps, out=out, workspace=ws), out,
             lambda: tpa.rmsnorm_lora(x, g, w, a, b, wl.eps, workspace=ws))
    att = synth.make_attention_inputs(16, 1500, 128, seed=5)
    dv = {n: torch.from_numpy(np.ascontiguousarray(att.device_array(n)).view(np.int16)).cuda()
          .view(torch.bfloat16) for n in ("Q", "K", "V", "gq", "gk")}
    o = torch.empty((16, 128), dtype=torch.bfloat16, device="cuda")
    aws = tpa.Workspace(tpa._binding.attention_workspace_bytes(tpa._binding.DTYPE_BF16, 16, 1500,
                                                               128, 5), "cuda")
    call = lambda out: tpa.qknorm_attention(dv["Q"], dv["K"], dv["V"], dv["gq"], dv["gk"], 1e-6,
                                            out=out, splits=5, workspace=aws)
    _replays(lambda: call(o), o, lambda: call(None))


def test_graph_stream_prefill_and_chain(require_gpu):
    """The other variants under replay: the gated stream kernel, the prefill
    tile, and the persistent layer chain (its layer counters are cleared by
    the kernel itself, so a replay must find them as an eager call does)."""
    wl = synth.Workload("graph_gated", "bf16", 64, 1024, 2048, 1e-6, True, None)
    inp = synth.make_inputs(wl, seed=21)
    x, g = to_device(inp, "X"), to_device(inp, "g")
    w1, w3 = to_device(inp, "W1"), to_device(inp, "W3")
    out = torch.empty((wl.M, wl.N), dtype=torch.bfloat16, device="cuda")
    _replays(lambda: tpa.rmsnorm_gated_mlp(x, g, w1, w3, wl.eps, out=out, variant="stream"), out,
             lambda: tpa.rmsnorm_gated_mlp(x, g, w1, w3, wl.eps, variant="stream"))

    wl = synth.Workload("graph_prefill", "bf16", 520, 512, 1032, 1e-6, False, None)
    inp = synth.make_inputs(wl, seed=22)
    x, g, w = to_device(inp, "X"), to_device(inp, "g"), to_device(inp, "W1")
    out = torch.empty((wl.M, wl.N), dtype=torch.bfloat16, device="cuda")
    _replays(lambda: tpa.rmsnorm_matmul(x, g, w, wl.eps, out=out, variant="prefill"), out,
             lambda: tpa.rmsnorm_matmul(x, g, w, wl.eps, variant="prefill"))

    M, K, L = 16, 1024, 3
    layers = [synth.make_inputs(synth.Workload(f"graph_chain_{l}", "bf16", M, K, K, 1e-6, False,
                                               None), seed=30 + l) for l in range(L)]

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    x0 = dev(layers[0].bits["X"])
    G = dev(np.stack([lay.bits["g"] for lay in layers]))
    W = dev(np.stack([lay.bits["W1"] for lay in layers]))
    xs = torch.empty((L, M, K), dtype=torch.bfloat16, device="cuda")
    ws = tpa.Workspace(tpa._binding.chain_workspace_bytes(M, K, L), "cuda")
    _replays(lambda: tpa.rmsnorm_matmul_chain(x0, G, W, 1e-6, out=xs, workspace=ws,
                                                check_wait=False), xs,
             lambda: tpa.rmsnorm_matmul_chain(x0, G, W, 1e-6, workspace=ws))
    assert tpa.chain_wait_flag(ws, M, K, L) == 0
