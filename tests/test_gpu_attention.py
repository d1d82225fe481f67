"""Parity of QKNorm + attention with the CPU oracle (needs an MI355X).

o = softmax(norm(q) . norm(K)^T / sqrt(D)) V per batch-head (the QKNorm +
Attention row of the Mirage paper review's benchmark table, "五、实验结果").

* one-hot inputs (gains of 40, one key equal to q / 2): the softmax is
  exactly one-hot in fp32, so the output must be that key's value row bit for
  bit -- every key index, chunk boundary and merge is checked exactly, over
  head dims, key counts around the kernel's 64/128-key rounds and forced
  chunk counts;
* random inputs within tolerance, on all outputs for small shapes and on
  sampled batch-heads of the benchmark workload;
* canaries around O, repeat determinism, the workspace counters reset.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import tensor_program_amd as tpa
from tests.gpu_util import BF16_TOL

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _dev(inp, name):
    return torch.from_numpy(np.ascontiguousarray(inp.device_array(name)).view(np.int16)).to(
        "cuda").view(torch.bfloat16)


def _run(inp, eps, splits=0, out=None, workspace=None):
    o = tpa.qknorm_attention(_dev(inp, "Q"), _dev(inp, "K"), _dev(inp, "V"), _dev(inp, "gq"),
                             _dev(inp, "gk"), eps, out=out, splits=splits, workspace=workspace)
    torch.cuda.synchronize()
    return o


def _bits(t):
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


ONEHOT = [
    # (BH, S, D, splits)
    (8, 1, 128, 0), (8, 1, 64, 0),
    (5, 63, 128, 0), (5, 64, 128, 0), (5, 65, 128, 0),
    (3, 127, 64, 0), (3, 128, 64, 0), (3, 129, 64, 0),
    (16, 1000, 128, 1), (16, 1000, 128, 2), (16, 1000, 128, 3), (16, 1000, 128, 0),
    (7, 4096, 64, 5), (7, 4096, 64, 0),
    (4, 333, 128, 333),                     # one key per chunk
    (256, 2048, 128, 0),                    # the benchmark shape
]


@pytest.mark.parametrize("case", ONEHOT, ids=lambda c: "x".join(map(str, c)))
def test_attention_onehot_bitwise(case, require_gpu):
    BH, S, D, splits = case
    _log(f"attention one-hot {case}")
    inp, pick = synth.make_attention_onehot(BH, S, D, seed=BH + S)
    o = _run(inp, 0.0, splits=splits)
    want = synth.to_bf16_bits(inp.V[np.arange(BH), pick])
    got = _bits(o)
    mism = np.argwhere(got != want)
    assert mism.size == 0, f"{len(mism)} mismatches, first at {tuple(mism[0])}"


def _check(o, ref, what):
    y = o.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(y)), f"{what}: non-finite outputs"
    err = np.abs(y - ref)
    lim = BF16_TOL * (np.abs(ref) + 1.0)
    worst = float((err / lim).max())
    _log(f"  worst err/tol {worst:.3f}")
    assert worst <= 1.0, f"{what}: {(err > lim).sum()} outside tolerance, worst {worst:.3g}"


@pytest.mark.parametrize("case", [(16, 1, 128, 0), (16, 100, 64, 0), (16, 1000, 128, 0),
                                  (16, 1000, 128, 7), (8, 4096, 128, 0), (8, 4096, 64, 2)],
                         ids=lambda c: "x".join(map(str, c)))
@pytest.mark.parametrize("eps", [1e-6, 0.5])
def test_attention_random(case, eps, require_gpu):
    BH, S, D, splits = case
    _log(f"attention random {case} eps {eps}")
    inp = synth.make_attention_inputs(BH, S, D, seed=S)
    o = _run(inp, eps, splits=splits)
    ref = oracle.qknorm_attention(inp.Q, inp.K, inp.V, inp.gq, inp.gk, oracle.eps_as_passed(eps))
    _check(o, ref, f"random {case}")


def test_attention_workload_sampled(require_gpu):
    wl = synth.get_workload("attn_bh256_s2048_d128")
    inp = synth.make_attention_inputs(wl.BH, wl.S, wl.D)
    o = _run(inp, wl.eps)
    heads = np.unique(np.concatenate([[0, wl.BH - 1],
                                      np.random.default_rng(3).choice(wl.BH, 30, replace=False)]))
    ref = oracle.qknorm_attention(inp.Q[heads], inp.K[heads], inp.V[heads], inp.gq, inp.gk,
                                  oracle.eps_as_passed(wl.eps))
    _check(o[torch.from_numpy(heads).cuda()], ref, "workload")


def test_attention_canaries_repeat_and_counters(require_gpu):
    BH, S, D = 9, 777, 128
    inp, pick = synth.make_attention_onehot(BH, S, D, seed=4)
    big = torch.full((BH * D + 256,), 3.0, dtype=torch.bfloat16, device="cuda")
    out = big[128:128 + BH * D].view(BH, D)
    ws = tpa.Workspace(tpa._binding.attention_workspace_bytes(tpa._binding.DTYPE_BF16, BH, S, D,
                                                              4), "cuda")
    _run(inp, 0.0, splits=4, out=out, workspace=ws)
    first = _bits(out).copy()
    _run(inp, 0.0, splits=4, out=out, workspace=ws)
    assert np.array_equal(_bits(out), first)
    assert np.array_equal(first, synth.to_bf16_bits(inp.V[np.arange(BH), pick]))
    guard = torch.cat([big[:128], big[128 + BH * D:]]).float()
    assert torch.all(guard == 3.0)
    assert torch.count_nonzero(ws.tensor[:4 * BH]) == 0  # arrival counters reset


def test_binding_workspace_per_layout(require_gpu):
    # Regression: with one cached workspace per stream, a call with few
    # batch-heads (16 key chunks each) left partial sums at byte 256 onward,
    # which a later call with 256 batch-heads read as arrival counters.
    small = synth.make_attention_inputs(8, 4096, 128, seed=11)
    _run(small, 1e-6)
    wl = synth.get_workload("attn_bh256_s2048_d128")
    inp = synth.make_attention_inputs(wl.BH, wl.S, wl.D, seed=12)
    o = _run(inp, wl.eps, splits=4)  # 4 chunks: 256 arrival counters in bytes 0..1023
    heads = np.array([0, 63, 64, 200, 255])
    ref = oracle.qknorm_attention(inp.Q[heads], inp.K[heads], inp.V[heads], inp.gq, inp.gk,
                                  oracle.eps_as_passed(wl.eps))
    _check(o[torch.from_numpy(heads).cuda()], ref, "after a smaller call")


# The unfused program the benchmark table compares against: RMSNorm of q
# and of every key written to memory, then the attention step alone.

@pytest.mark.parametrize("case", [(16, 1, 128), (16, 100, 64), (16, 1000, 128), (8, 4096, 64),
                                  (3, 65, 128)], ids=lambda c: "x".join(map(str, c)))
def test_attention_step_random(case, require_gpu):
    BH, S, D = case
    _log(f"attention step {case}")
    inp = synth.make_attention_inputs(BH, S, D, seed=S + 1)
    o = tpa.attention(_dev(inp, "Q"), _dev(inp, "K"), _dev(inp, "V"))
    torch.cuda.synchronize()
    _check(o, oracle.attention(inp.Q, inp.K, inp.V), f"step {case}")


@pytest.mark.parametrize("case", [(16, 1000, 128), (8, 4096, 64)],
                         ids=lambda c: "x".join(map(str, c)))
def test_unfused_qknorm_program(case, require_gpu):
    BH, S, D = case
    eps = 1e-6
    _log(f"unfused qknorm program {case}")
    inp = synth.make_attention_inputs(BH, S, D, seed=S + 2)
    qn = tpa.rmsnorm(_dev(inp, "Q"), _dev(inp, "gq"), eps)
    kn = tpa.rmsnorm(_dev(inp, "K").view(BH * S, D), _dev(inp, "gk"), eps).view(BH, S, D)
    o = tpa.attention(qn, kn, _dev(inp, "V"))
    torch.cuda.synchronize()
    e = oracle.eps_as_passed(eps)
    _check(o, oracle.qknorm_attention(inp.Q, inp.K, inp.V, inp.gq, inp.gk, e), f"program {case}")


def test_unfused_qknorm_workload_sampled(require_gpu):
    wl = synth.get_workload("attn_bh256_s2048_d128")
    _log("unfused qknorm program, benchmark workload")
    inp = synth.make_attention_inputs(wl.BH, wl.S, wl.D)
    qn = tpa.rmsnorm(_dev(inp, "Q"), _dev(inp, "gq"), wl.eps)
    kn = tpa.rmsnorm(_dev(inp, "K").view(wl.BH * wl.S, wl.D), _dev(inp, "gk"), wl.eps)
    o = tpa.attention(qn, kn.view(wl.BH, wl.S, wl.D), _dev(inp, "V"))
    heads = np.unique(np.concatenate([[0, wl.BH - 1],
                                      np.random.default_rng(5).choice(wl.BH, 20, replace=False)]))
    ref = oracle.qknorm_attention(inp.Q[heads], inp.K[heads], inp.V[heads], inp.gq, inp.gk,
                                  oracle.eps_as_passed(wl.eps))
    _check(o[torch.from_numpy(heads).cuda()], ref, "unfused workload")


# Grouped queries: G query heads per key/value head, each key row read once
# for the group (G <= 2 on the vector ALUs, G >= 3 on the matrix cores).

def _run_gqa(inp, eps, splits=0):
    o = tpa.qknorm_attention_gqa(_dev(inp, "Q"), _dev(inp, "K"), _dev(inp, "V"), _dev(inp, "gq"),
                                 _dev(inp, "gk"), eps, splits=splits)
    torch.cuda.synchronize()
    return o


def _oracle_gqa(inp, G, eps, heads=None):
    # the definition per query row: its key/value head's keys and values
    K, V = np.repeat(inp.K, G, axis=0), np.repeat(inp.V, G, axis=0)
    Q = inp.Q
    if heads is not None:
        rows = (heads[:, None] * G + np.arange(G)[None, :]).reshape(-1)
        Q, K, V = Q[rows], K[rows], V[rows]
    return oracle.qknorm_attention(Q, K, V, inp.gq, inp.gk, oracle.eps_as_passed(eps))


GQA_ONEHOT = [
    # (BH, G, S, D, splits)
    (4, 2, 100, 128, 0), (3, 4, 64, 64, 0), (5, 7, 300, 128, 3), (2, 8, 129, 128, 0),
    (6, 8, 1000, 64, 4), (4, 3, 8, 128, 0), (2, 5, 4096, 128, 0),
    (2, 16, 300, 128, 0), (3, 12, 64, 64, 2), (5, 16, 33, 64, 0),
]


@pytest.mark.parametrize("case", GQA_ONEHOT, ids=lambda c: "x".join(map(str, c)))
def test_attention_gqa_onehot_bitwise(case, require_gpu):
    BH, G, S, D, splits = case
    _log(f"gqa one-hot {case}")
    inp, pick = synth.make_attention_onehot(BH, S, D, seed=BH + S + G, G=G)
    o = _run_gqa(inp, 0.0, splits=splits)
    heads = np.repeat(np.arange(BH), G)
    want = synth.to_bf16_bits(inp.V[heads, pick])
    got = _bits(o)
    mism = np.argwhere(got != want)
    assert mism.size == 0, f"{len(mism)} mismatches, first at {tuple(mism[0])}"


@pytest.mark.parametrize("case", [(8, 2, 1000, 128, 0), (4, 3, 777, 64, 0), (4, 4, 4096, 128, 0),
                                  (2, 8, 2048, 128, 5), (3, 6, 129, 64, 0), (16, 1, 1000, 128, 7),
                                  (4, 16, 1000, 128, 0), (2, 11, 3000, 64, 3)],
                         ids=lambda c: "x".join(map(str, c)))
@pytest.mark.parametrize("eps", [1e-6, 0.5])
def test_attention_gqa_random(case, eps, require_gpu):
    BH, G, S, D, splits = case
    _log(f"gqa random {case} eps {eps}")
    inp = synth.make_attention_inputs(BH, S, D, seed=S + G, G=G)
    o = _run_gqa(inp, eps, splits=splits)
    _check(o, _oracle_gqa(inp, G, eps), f"gqa {case}")


def test_attention_gqa_g1_is_qknorm_attention(require_gpu):
    inp = synth.make_attention_inputs(12, 1500, 128, seed=9)
    a = _bits(_run_gqa(inp, 1e-6))
    b = _bits(_run(inp, 1e-6))
    assert np.array_equal(a, b)


def test_attention_gqa_workload_sampled(require_gpu):
    wl = synth.get_workload("attn_gqa_bh32_g8_s2048_d128")
    _log("gqa workload, sampled heads")
    inp = synth.make_attention_inputs(wl.BH, wl.S, wl.D, G=wl.G)
    o = _run_gqa(inp, wl.eps)
    heads = np.unique(np.concatenate([[0, wl.BH - 1],
                                      np.random.default_rng(4).choice(wl.BH, 8, replace=False)]))
    rows = (heads[:, None] * wl.G + np.arange(wl.G)[None, :]).reshape(-1)
    _check(o[torch.from_numpy(rows).cuda()], _oracle_gqa(inp, wl.G, wl.eps, heads=heads),
           "gqa workload")


# Many queries per head (prefill): blocks of 64 positions per workgroup, the
# causal mask, grouped heads.

def _run_prefill(inp, eps, causal):
    o = tpa.qknorm_attention_prefill(_dev(inp, "Q"), _dev(inp, "K"), _dev(inp, "V"),
                                     _dev(inp, "gq"), _dev(inp, "gk"), eps, causal=causal)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("case", [(2, 2, 100, 128, True), (2, 2, 100, 128, False),
                                  (1, 3, 70, 64, True), (3, 1, 129, 128, True),
                                  # enough heads for two 16-row query blocks per wave
                                  (128, 2, 100, 128, False), (256, 4, 130, 64, True)],
                         ids=lambda c: "x".join(map(str, c)))
def test_attention_prefill_onehot_bitwise(case, require_gpu):
    # Query (g, i) of a head finds its own key at position g Sq + i (within its
    # horizon i + Skv - Sq when Skv = G Sq), equal to q / 2, gains of 40: the
    # softmax is exactly one-hot and the output is that key's value row.
    BH, G, Sq, D, causal = case
    Skv = G * Sq
    _log(f"prefill one-hot {case}")
    inp = synth.make_attention_prefill_inputs(BH, G, Sq, Skv, D, seed=Sq + G)
    Q, K = inp.Q.copy(), inp.K.copy()
    for qh in range(BH * G):
        K[qh // G, (qh % G) * Sq + np.arange(Sq)] = 0.5 * Q[qh]
    g40 = np.full(D, 40.0, np.float32)
    inp = synth.AttnInputs(Q, K, inp.V, g40, g40)
    o = _run_prefill(inp, 0.0, causal)
    want = np.stack([inp.V[qh // G, (qh % G) * Sq + np.arange(Sq)] for qh in range(BH * G)])
    got = _bits(o)
    mism = np.argwhere(got != synth.to_bf16_bits(want))
    assert mism.size == 0, f"{len(mism)} mismatches, first at {tuple(mism[0])}"


@pytest.mark.parametrize("case", [(2, 1, 200, 200, 128, True), (2, 4, 130, 300, 64, True),
                                  (1, 2, 64, 1000, 128, False), (3, 1, 1, 50, 128, True),
                                  (1, 8, 257, 257, 128, True), (2, 3, 65, 90, 64, False),
                                  # two 16-row query blocks per wave (128-position
                                  # workgroups), a ragged last block
                                  (64, 4, 130, 200, 128, False), (128, 4, 200, 300, 64, True),
                                  # one block per wave with 32-key tiles (more than 256
                                  # workgroups; the smaller grids above take 64-key tiles)
                                  (50, 2, 256, 300, 64, False), (32, 4, 200, 260, 64, True)],
                         ids=lambda c: "x".join(map(str, c)))
@pytest.mark.parametrize("eps", [1e-6, 0.5])
def test_attention_prefill_random(case, eps, require_gpu):
    BH, G, Sq, Skv, D, causal = case
    _log(f"prefill random {case} eps {eps}")
    inp = synth.make_attention_prefill_inputs(BH, G, Sq, Skv, D, seed=Sq + Skv)
    o = _run_prefill(inp, eps, causal)
    ref = oracle.qknorm_attention_prefill(inp.Q, inp.K, inp.V, inp.gq, inp.gk,
                                          oracle.eps_as_passed(eps), causal=causal)
    _check(o.reshape(-1, D), ref.reshape(-1, D), f"prefill {case}")


def test_attention_prefill_long_sampled(require_gpu):
    # 8 key/value heads x 4 queries each, 2048 positions, causal: two query
    # heads checked in full (every position against all its visible keys)
    BH, G, S, D = 8, 4, 2048, 128
    _log("prefill 8 x 4 heads x 2048, sampled heads")
    inp = synth.make_attention_prefill_inputs(BH, G, S, S, D)
    o = _run_prefill(inp, 1e-6, True)
    for qh in (0, BH * G - 1):
        ref = oracle.qknorm_attention_prefill(inp.Q[qh:qh + 1], inp.K[qh // G:qh // G + 1],
                                              inp.V[qh // G:qh // G + 1], inp.gq, inp.gk,
                                              oracle.eps_as_passed(1e-6), causal=True)
        _check(o[qh], ref[0], f"prefill head {qh}")


# The keys split into spans (whole 64-key tiles), combined per query row by a
# second kernel: forced counts, spans past a causal block's keys (stored
# empty), the library's own choice for few query blocks over many keys.
def _run_prefill_split(inp, eps, causal, splits):
    o = tpa.qknorm_attention_prefill(_dev(inp, "Q"), _dev(inp, "K"), _dev(inp, "V"),
                                     _dev(inp, "gq"), _dev(inp, "gk"), eps, causal=causal,
                                     splits=splits)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("case", [(2, 4, 130, 1000, 128, True, 3), (1, 2, 64, 1000, 64, False, 5),
                                  (2, 1, 200, 200, 128, True, 2), (1, 8, 70, 3000, 128, True, 0),
                                  (2, 2, 33, 700, 64, True, 11),
                                  # two query blocks per wave, the library's split
                                  (64, 4, 100, 2000, 64, False, 0)],
                         ids=lambda c: "x".join(map(str, c)))
@pytest.mark.parametrize("eps", [1e-6, 0.5])
def test_attention_prefill_split_random(case, eps, require_gpu):
    BH, G, Sq, Skv, D, causal, splits = case
    lib = tpa.load_library()
    need = lib.rmm_attention_prefill_workspace_bytes(BH, G, Sq, Skv, D, int(causal), splits)
    assert need > 0, "the case must run split"
    _log(f"prefill split {case} eps {eps}")
    inp = synth.make_attention_prefill_inputs(BH, G, Sq, Skv, D, seed=Sq + Skv + splits)
    o = _run_prefill_split(inp, eps, causal, splits)
    ref = oracle.qknorm_attention_prefill(inp.Q, inp.K, inp.V, inp.gq, inp.gk,
                                          oracle.eps_as_passed(eps), causal=causal)
    _check(o.reshape(-1, D), ref.reshape(-1, D), f"prefill split {case}")


@pytest.mark.parametrize("case", [(2, 2, 100, 128, True, 2), (1, 3, 70, 64, False, 3)],
                         ids=lambda c: "x".join(map(str, c)))
def test_attention_prefill_split_onehot_bitwise(case, require_gpu):
    # as test_attention_prefill_onehot_bitwise, with the keys in spans: the
    # span holding a query's own key gives o = v, every other span's weight
    # underflows to zero in the combine
    BH, G, Sq, D, causal, splits = case
    Skv = G * Sq
    _log(f"prefill split one-hot {case}")
    inp = synth.make_attention_prefill_inputs(BH, G, Sq, Skv, D, seed=Sq + G + 7)
    Q, K = inp.Q.copy(), inp.K.copy()
    for qh in range(BH * G):
        K[qh // G, (qh % G) * Sq + np.arange(Sq)] = 0.5 * Q[qh]
    g40 = np.full(D, 40.0, np.float32)
    inp = synth.AttnInputs(Q, K, inp.V, g40, g40)
    o = _run_prefill_split(inp, 0.0, causal, splits)
    want = np.stack([inp.V[qh // G, (qh % G) * Sq + np.arange(Sq)] for qh in range(BH * G)])
    got = _bits(o)
    mism = np.argwhere(got != synth.to_bf16_bits(want))
    assert mism.size == 0, f"{len(mism)} mismatches, first at {tuple(mism[0])}"


def test_attention_prefill_split_matches_unsplit_workload(require_gpu):
    # 8 key/value heads x 4 queries, 512 positions over 8192 keys (the library
    # splits the keys in three): two query heads against the oracle, every
    # head against the unsplit call at the elementwise bound
    BH, G, Sq, Skv, D = 8, 4, 512, 8192, 128
    assert tpa.load_library().rmm_attention_prefill_workspace_bytes(BH, G, Sq, Skv, D, 1, 0) > 0
    _log("prefill split 8 x 4 heads, 512 over 8192 keys")
    inp = synth.make_attention_prefill_inputs(BH, G, Sq, Skv, D, seed=3)
    o = _run_prefill_split(inp, 1e-6, True, 0)
    o1 = _run_prefill_split(inp, 1e-6, True, 1)
    _check(o.reshape(-1, D), o1.float().cpu().numpy().reshape(-1, D), "split against unsplit")
    for qh in (0, BH * G - 1):
        ref = oracle.qknorm_attention_prefill(inp.Q[qh:qh + 1], inp.K[qh // G:qh // G + 1],
                                              inp.V[qh // G:qh // G + 1], inp.gq, inp.gk,
                                              oracle.eps_as_passed(1e-6), causal=True)
        _check(o[qh], ref[0], f"prefill split head {qh}")
