"""Benchmark of the fused RMSNorm+MatMul hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

A step is one call of the library on one batch (one input set), i.e. one pass
of the whole hot path.  Inputs are seeded synthetic tensors already resident
in HBM.  R input sets are rotated so that each timed pass touches >= 1 GiB,
more than the 256 MB Infinity Cache, so W really streams from HBM.  The R
calls are captured once in a HIP graph (no allocation or memset inside) and
replayed; HIP events on the launch stream bracket the K timed steps.  Before
the W warm-up steps, untimed calls run for --settle-ms of wall time: after an
idle period the GPU takes some 10-20 ms under load to reach its steady clocks,
and a short timed region would otherwise measure that ramp.

Prints one JSON line.  `value` is the algorithmic HBM throughput (every input
byte once + Y once, per second) for bandwidth-bound workloads, or TFLOP/s for
matrix-core-bound ones.  `roofline` relates the dominant kernel to the MI355X
peak; `cpu_baseline` times the CPU oracle on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused RMSNorm+MatMul TFLOP/s and HBM GB/s (% of MI355X roofline)"
# the largest single-GPU workload (the headline line)
DEFAULT_WORKLOAD = "large_m8192_k8192_n28672"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6      # dense bf16 MFMA, 256 CU x 4096 flop/clk x 2.4 GHz
F32_VALU_PEAK_TFLOPS = 78.6    # fp32 FMA on the vector ALUs without packed math
RIDGE = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
ROTATE_BYTES = 1 << 30
# files each kernel is built from (their bytes, in order, make the source hash)
KERNEL_SOURCES = {"decode": ("rmm_decode.hip", "rmm_decode_core.h"),
                  "decode32": ("rmm_decode32.hip",), "generic": ("rmm_generic.hip",),
                  "prefill": ("rmm_prefill.hip",), "stream": ("rmm_stream.hip",),
                  "attention": ("rmm_attn.hip",), "chain": ("rmm_chain.hip", "rmm_decode_core.h")}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash(variant: str) -> str | None:
    files = KERNEL_SOURCES.get(variant)
    if not files:
        return None
    h = hashlib.sha256()
    for f in files:
        path = os.path.join(ROOT, "tensor_program_amd", "csrc", f)
        if not os.path.isfile(path):
            return None
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, variant: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.isfile(path):
        return None
    with open(path) as f:
        table = json.load(f)
    rec = table.get(f"{workload}/{variant}")
    if not rec or rec.get("kernel_source_sha256_16") != source_hash(variant):
        return None
    return rec.get("hbm_bytes_per_launch")


def host_cpu() -> dict:
    """The host's CPU model and logical CPU count (the oracle's machine)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "logical_cpus": os.cpu_count()}


def measure_peaks(stream, dev):
    """Achievable ceilings of this part, from the library's own probes
    (rmm_probe_hbm_read over a 2 GiB buffer, far past the 256 MB last-level
    cache; rmm_probe_mfma_bf16, a dense v_mfma_f32_32x32x16_bf16 loop),
    timed with HIP events on the launch stream."""
    import ctypes
    import torch
    import tensor_program_amd as tpa

    lib = tpa.load_library()
    nbytes = 2 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    h = ctypes.c_void_p(stream.cuda_stream)
    iters = 20000
    out = {}
    with torch.cuda.stream(stream):
        for name, launch, work in (
                ("hbm_read_gbs", lambda: lib.rmm_probe_hbm_read(buf.data_ptr(), nbytes,
                                                               sink.data_ptr(), h), nbytes / 1e9),
                ("mfma_bf16_tflops", lambda: lib.rmm_probe_mfma_bf16(iters, sink.data_ptr(), h),
                 lib.rmm_probe_mfma_flops(iters) / 1e12)):
            for _ in range(5):
                tpa._binding.check(launch())
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            n = 20
            e0.record(stream)
            for _ in range(n):
                launch()
            e1.record(stream)
            e1.synchronize()
            out[name] = work / (e0.elapsed_time(e1) / 1e3 / n)
    del buf
    torch.cuda.empty_cache()
    out["probes"] = ("rmm_probe_hbm_read (2 GiB linear read, 16-byte loads) and "
                     "rmm_probe_mfma_bf16 (4 chains of v_mfma_f32_32x32x16_bf16 per wave, 2 waves "
                     "per SIMD), 20 launches each after 5 untimed")
    return out


def synth_attn_type():
    import synth
    return synth.AttnWorkload


def cpu_baseline(wl, inp, budget_s: float):
    """The oracle, as it stands, on the host cores: whole workload if it fits
    the time budget, else a leading block of rows (rows are independent)."""
    import numpy as np
    import oracle

    eps = oracle.eps_as_passed(wl.eps)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    attn = isinstance(wl, synth_attn_type())
    # independent rows (key/value heads with their G queries for attention)
    total = wl.BH if attn else wl.M
    # Probe on a small block of rows, then size the sample to the budget.
    rows = min(total, max(1, threads))
    X = inp.Q[:rows] if attn else inp.X[:rows]

    def once(Xs):
        t0 = time.perf_counter()
        if attn:
            # the oracle takes one key/value head per query row: each head's
            # keys and values repeated for its G queries
            n = Xs.shape[0]
            G = wl.G
            oracle.qknorm_attention(inp.Q[:n * G], np.repeat(inp.K[:n], G, axis=0),
                                    np.repeat(inp.V[:n], G, axis=0), inp.gq, inp.gk, eps)
        elif wl.gated:
            oracle.rmsnorm_gated_mlp(Xs, inp.g, inp.W1, inp.W3, eps)
        elif wl.lora:
            oracle.rmsnorm_lora(Xs, inp.g, inp.W1, inp.LA, inp.LB, eps)
        else:
            oracle.rmsnorm_matmul(Xs, inp.g, inp.W1, eps)
        return time.perf_counter() - t0

    full = inp.Q if attn else inp.X
    unit_name = "key/value heads" if attn else "rows"
    t_probe = once(X)
    per_row = t_probe / rows
    rows_budget = int(budget_s / max(per_row, 1e-9))
    if rows_budget >= total:
        reps = max(1, int(budget_s / max(per_row * total, 1e-9)))
        reps = min(reps, 50)
        t = sum(once(full) for _ in range(reps)) / reps
        sample = f"full workload ({total} {unit_name}), mean of {reps} runs"
        frac = 1.0
    else:
        rows = max(rows, (rows_budget // threads) * threads)
        t = once(full[:rows])
        frac = rows / total
        sample = (f"first {rows} of {total} {unit_name} (they are independent), fp64 unfused; "
                  f"time extrapolated x{total / rows:.1f} to the whole workload")
    t_full = t / frac
    bound = "hbm" if wl.flops() / wl.algo_bytes() < RIDGE else "mfma"
    if bound == "hbm":
        value, unit = wl.algo_bytes() / t_full / 1e9, "GB/s"
    else:
        value, unit = wl.flops() / t_full / 1e12, "TFLOP/s"
    used = min(threads, rows)
    return {"value": value, "unit": unit, "cores": used, "kind": "oracle", "sample": sample,
            "seconds_full_workload": t_full, "omp_threads": threads} | host_cpu()


def bench_chain(args, name):
    """The persistent layer chain (rmsnorm_matmul_chain) on `chain_l{L}_m{M}_k{K}`:
    one call runs L layers x_{l+1} = RMSNorm(x_l; g_l) W_l with K x K weights.
    Timed beside the same L layers as separate calls of the single-layer
    kernel (decode variant), both as HIP-graph replays over rotating input
    sets; `value` is the chain's algorithmic GB/s (every weight, gain and
    activation byte once per layer)."""
    import re
    import numpy as np
    import torch

    import oracle
    import synth
    import tensor_program_amd as tpa

    m = re.fullmatch(r"chain_l(\d+)_m(\d+)_k(\d+)", name)
    if not m:
        raise SystemExit(f"unknown workload {name}")
    L, M, K = (int(v) for v in m.groups())
    eps = 1e-6
    dev = torch.device("cuda", 0)
    log(f"workload {name}: generating inputs")
    layers = [synth.make_inputs(synth.Workload(f"chain_{l}", "bf16", M, K, K, eps, False, None),
                                seed=l) for l in range(L)]

    def d(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    x0 = d(layers[0].bits["X"])
    G = d(np.stack([lay.bits["g"] for lay in layers]))
    W = d(np.stack([lay.bits["W1"] for lay in layers]))
    per_set = L * (K * K + K + 2 * M * K) * 2
    R = max(1, math.ceil(ROTATE_BYTES / (L * K * K * 2)))
    sets = [(x0, G, W if r == 0 else W.clone(), torch.empty((L, M, K), dtype=torch.bfloat16,
                                                            device=dev)) for r in range(R)]
    stream = torch.cuda.Stream(dev)
    results = {}
    for mode in ("chain", "separate"):
        def call(st):
            x, g, w, xs = st
            if mode == "chain":
                tpa.rmsnorm_matmul_chain(x, g, w, eps, out=xs, check_wait=False)
            else:
                prev = x
                for layer in range(L):
                    tpa.rmsnorm_matmul(prev, g[layer], w[layer], eps, out=xs[layer], variant="decode")
                    prev = xs[layer]
        with torch.cuda.stream(stream):
            for st in sets:
                call(st)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                for st in sets:
                    call(st)
            torch.cuda.synchronize()
            t0 = time.time()
            while time.time() - t0 < args.settle_ms / 1e3:
                graph.replay()
            def run(n):  # exactly n calls: whole rotations from the graph, the rest eager
                for _ in range(n // R):
                    graph.replay()
                for i in range(n % R):
                    call(sets[i])
            n_warm, n_steps = max(0, args.warmup), max(1, args.steps)
            run(n_warm)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            stream.synchronize()
            e0.record(stream)
            run(n_steps)
            e1.record(stream)
            e1.synchronize()
        results[mode] = (e0.elapsed_time(e1) / n_steps, n_steps, n_warm)
        log(f"{mode}: {results[mode][0] * 1e3:.1f} us per call ({results[mode][0] * 1e3 / L:.2f} "
            f"us per layer)")
    ms, steps, warm = results["chain"]
    # the graph-captured calls cannot synchronise; one checked call after them
    # raises if a layer wait ever gave up on this workspace
    tpa.rmsnorm_matmul_chain(*sets[0][:3], eps, out=sets[0][3])
    gbs = per_set / (ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        t0 = time.time()
        x = layers[0].X
        ref_layers = 0
        for layer in range(L):
            x = oracle.rmsnorm_matmul(x, layers[layer].g, layers[layer].W1, oracle.eps_as_passed(eps))
            ref_layers += 1
            if time.time() - t0 > args.cpu_budget:
                break
        sec = (time.time() - t0) / ref_layers
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        cpu = {"value": (per_set / L) / sec / 1e9, "unit": "GB/s", "cores": min(threads, M),
               "kind": "oracle", "sample": f"{ref_layers} of {L} layers (fp64, unfused), "
                                           f"{sec * 1e3:.1f} ms per layer"}
    out = {"metric": METRIC, "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": steps,
           "warmup": warm, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": name, "layers": L, "M": M, "K": K, "N": K, "eps": eps,
                      "rotating_input_sets": R, "hip_graph": True},
           "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": gbs / HBM_PEAK_GBS, "traffic": None, "kernel": "chain_kernel",
                        "algorithmic_bytes_per_launch": per_set},
           "cpu_baseline": cpu,
           "separate_calls": {"ms_per_step": results["separate"][0],
                              "chain_speedup": results["separate"][0] / ms,
                              "note": "the same layers as L graph-captured single-layer calls"}}
    print(json.dumps(out), flush=True)


def bench_attn_prefill(args, name):
    """QKNorm + attention for many queries per head on `attn_prefill_bh{BH}_g{G}_s{S}_d{D}`:
    BH key/value heads, G query heads each, S positions (Sq = Skv = S), causal.
    `value` is algorithmic TFLOP/s: 4 D flops (q.k and p.v) per visible
    (query, key) pair; rotating input sets replayed from a HIP graph."""
    import re
    import numpy as np
    import torch

    import oracle
    import synth
    import tensor_program_amd as tpa

    m = re.fullmatch(r"attn_prefill_bh(\d+)_g(\d+)_s(\d+)_d(\d+)", name)
    if not m:
        raise SystemExit(f"unknown workload {name}")
    BH, G, S, D = (int(v) for v in m.groups())
    eps = 1e-6
    dev = torch.device("cuda", 0)
    log(f"workload {name}: generating inputs")
    inp = synth.make_attention_prefill_inputs(BH, G, S, S, D)

    def d(nm):
        return torch.from_numpy(np.ascontiguousarray(inp.device_array(nm)).view(np.int16)).to(
            dev).view(torch.bfloat16)

    base = {nm: d(nm) for nm in ("Q", "K", "V", "gq", "gk")}
    per_set = (2 * BH * G * S * D + 2 * BH * S * D + 2 * D) * 2
    pairs = BH * G * S * (S + 1) // 2
    flops = 4 * D * pairs
    R = max(1, min(8, math.ceil(ROTATE_BYTES / per_set)))
    sets = []
    for r in range(R):
        st = {nm: (t if r == 0 else t.clone()) for nm, t in base.items()}
        st["O"] = torch.empty_like(st["Q"])
        sets.append(st)
    stream = torch.cuda.Stream(dev)

    def call(st):
        tpa.qknorm_attention_prefill(st["Q"], st["K"], st["V"], st["gq"], st["gk"], eps,
                                     causal=True, out=st["O"])
    with torch.cuda.stream(stream):
        for st in sets:
            call(st)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for st in sets:
                call(st)
        torch.cuda.synchronize()
        t0 = time.time()
        while time.time() - t0 < args.settle_ms / 1e3:
            graph.replay()

        def run(n):  # exactly n calls: whole rotations from the graph, the rest eager
            for _ in range(n // R):
                graph.replay()
            for i in range(n % R):
                call(sets[i])
        n_warm, n_steps = max(0, args.warmup), max(1, args.steps)
        run(n_warm)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        stream.synchronize()
        e0.record(stream)
        run(n_steps)
        e1.record(stream)
        e1.synchronize()
    ms = e0.elapsed_time(e1) / n_steps
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"{ms * 1e3:.1f} us per call, {tflops:.1f} TFLOP/s")
    cpu = None
    if not args.no_cpu_baseline:
        # the oracle on the first query heads, as many as fit the budget
        # (heads are independent), extrapolated to all of them
        t0 = time.time()
        n = 0
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        while n < BH * G and time.time() - t0 < args.cpu_budget:
            k = min(threads, BH * G - n)
            hs = np.arange(n, n + k)
            oracle.qknorm_attention_prefill(inp.Q[hs], np.stack([inp.K[h // G] for h in hs]),
                                            np.stack([inp.V[h // G] for h in hs]), inp.gq,
                                            inp.gk, oracle.eps_as_passed(eps), causal=True)
            n += k
        sec = (time.time() - t0) * (BH * G) / n
        cpu = {"value": flops / sec / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
               "sample": f"first {n} of {BH * G} query heads (fp64), extrapolated "
                         f"x{BH * G / n:.1f}"} | host_cpu()
    out = {"metric": METRIC, "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": n_steps,
           "warmup": n_warm, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": name, "BH": BH, "G": G, "Sq": S, "Skv": S, "D": D,
                      "causal": True, "eps": eps, "rotating_input_sets": R, "hip_graph": True},
           "roofline": {"bound": "mfma", "achieved": tflops, "peak": BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": tflops / BF16_PEAK_TFLOPS,
                        "traffic": stored_traffic(name, "attention"),
                        "kernel": "attn_prefill_kernel", "algorithmic_flops_per_launch": flops,
                        "note": "both products carry two bf16 parts: the matrix cores run "
                                "twice the algorithmic flops"},
           "cpu_baseline": cpu}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--variant", default="auto")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--no-graph", action="store_true", help="plain launches instead of a graph")
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed calls for this long before the warm-up steps (clock ramp)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds for the oracle leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-unfused", action="store_true",
                    help="skip timing the unfused two-kernel program beside the fused call")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the achievable-peak probes (HBM read, MFMA loop)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the fused RMSNorm+MatMul path is measured "
              "on one GPU's share (--gpus must be 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import tensor_program_amd as tpa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    tpa.load_library()  # fail loudly if the HIP library is not built
    if args.copy_calibration:
        n = 256 << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "launches": 10}))
        return
    if args.workload.startswith("chain_"):
        return bench_chain(args, args.workload)
    if args.workload.startswith("attn_prefill_"):
        return bench_attn_prefill(args, args.workload)
    wl = synth.get_workload(args.workload)
    attn = isinstance(wl, synth.AttnWorkload)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    log(f"workload {wl.name}: generating inputs")
    inp = synth.make_attention_inputs(wl.BH, wl.S, wl.D, G=wl.G) if attn else synth.make_inputs(wl)

    def dev_tensor(name):
        a = inp.device_array(name)
        if wl.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)

    if attn:
        names = ["Q", "K", "V", "gq", "gk"]
    else:
        names = (["X", "g", "W1"] + (["W3"] if wl.gated else []) + (["LA", "LB"] if wl.lora else []))
    base = {n: dev_tensor(n) for n in names}
    per_set = wl.algo_bytes()
    free = torch.cuda.mem_get_info(dev)[0]
    R = max(1, math.ceil(ROTATE_BYTES / per_set))
    R = max(1, min(R, int(0.6 * free // max(per_set, 1))))
    sets = []
    for r in range(R):
        s = {n: (t if r == 0 else t.clone()) for n, t in base.items()}
        s["Y"] = torch.empty((wl.BH * wl.G, wl.D) if attn else (wl.M, wl.N), dtype=torch.bfloat16
                             if wl.dtype == "bf16" else torch.float32, device=dev)
        sets.append(s)
    if attn:
        st, splits, _ = tpa.plan_attention(wl.BH, wl.S, wl.D, splits=args.splits, G=wl.G)
        variant = "attention"
    elif wl.lora:
        st, variant, splits = tpa.plan_lora(wl.M, wl.N, wl.K, wl.lora, dtype=sets[0]["Y"].dtype,
                                            variant=args.variant, splits=args.splits)
    else:
        st, variant, splits = tpa.plan(wl.M, wl.N, wl.K, dtype=sets[0]["Y"].dtype,
                                       gated=wl.gated, variant=args.variant, splits=args.splits)
    if st != 0:
        raise SystemExit(f"plan failed with status {st}")
    log(f"variant {variant}, splits {splits}, {R} rotating input sets "
        f"({R * per_set / 2**20:.0f} MiB)")
    stream = torch.cuda.Stream(dev)
    dcode = tpa._DTYPES[sets[0]["Y"].dtype]
    if attn:
        nbytes = tpa._binding.attention_gqa_workspace_bytes(dcode, wl.BH, wl.G, wl.S, wl.D,
                                                            args.splits)
    elif wl.lora:
        nbytes = tpa._binding.lora_workspace_bytes(dcode, wl.M, wl.N, wl.K, wl.lora, args.variant,
                                                   args.splits)
    else:
        nbytes = tpa._binding.workspace_bytes(dcode, wl.M, wl.N, wl.K, wl.gated, args.variant,
                                              args.splits)
    ws = tpa.Workspace(nbytes, dev) if nbytes > 0 else None
    torch.cuda.synchronize()

    def call(s):
        if attn and wl.G > 1:
            tpa.qknorm_attention_gqa(s["Q"], s["K"], s["V"], s["gq"], s["gk"], wl.eps,
                                     out=s["Y"], splits=args.splits, workspace=ws)
        elif attn:
            tpa.qknorm_attention(s["Q"], s["K"], s["V"], s["gq"], s["gk"], wl.eps, out=s["Y"],
                                 splits=args.splits, workspace=ws)
        elif wl.gated:
            tpa.rmsnorm_gated_mlp(s["X"], s["g"], s["W1"], s["W3"], wl.eps, out=s["Y"],
                                  variant=args.variant, splits=args.splits, workspace=ws)
        elif wl.lora:
            tpa.rmsnorm_lora(s["X"], s["g"], s["W1"], s["LA"], s["LB"], wl.eps, out=s["Y"],
                             variant=args.variant, splits=args.splits, workspace=ws)
        else:
            tpa.rmsnorm_matmul(s["X"], s["g"], s["W1"], wl.eps, out=s["Y"],
                               variant=args.variant, splits=args.splits, workspace=ws)

    def make_runner(fn, use_graph):
        """Returns run(n): n calls of fn(i) rotating over the R sets, replayed
        from a HIP graph of R calls when use_graph."""
        with torch.cuda.stream(stream):
            for i in range(R):  # eager warm-up of every set (also loads the code objects)
                fn(i)
        torch.cuda.synchronize()
        g = None
        if use_graph:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(R):
                    fn(i)
            torch.cuda.synchronize()

        def run(n):
            with torch.cuda.stream(stream):
                if g is not None:
                    reps = n // R
                    for _ in range(reps):
                        g.replay()
                    for i in range(n - reps * R):
                        fn(i)
                else:
                    for i in range(n):
                        fn(i % R)
        return run

    def time_steps(run, n):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            start.record(stream)
        run(n)
        with torch.cuda.stream(stream):
            end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end)

    run_steps = make_runner(lambda i: call(sets[i]), not args.no_graph)
    graph = None if args.no_graph else True

    # exactly the requested counts (run() replays whole rotations from the
    # graph and launches any remainder eagerly)
    steps = max(1, args.steps)
    warm = max(0, args.warmup)
    settle_calls = 0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < args.settle_ms:
        run_steps(R)
        settle_calls += R
        if settle_calls % (16 * R) == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    log(f"clock settle: {settle_calls} untimed calls in {(time.perf_counter() - t0) * 1e3:.0f} ms")
    log(f"warmup {warm} steps")
    run_steps(warm)
    torch.cuda.synchronize()
    log(f"timing {steps} steps")
    ms = time_steps(run_steps, steps)
    per_launch_s = ms / 1e3 / steps
    log(f"{ms:.3f} ms for {steps} steps: {per_launch_s * 1e6:.2f} us/step")

    # The unfused program the fused kernel replaces (the comparison of the
    # worked example): an RMSNorm kernel writes the normalised X, then a
    # product reads it back -- our plain-product kernels, and the vendor GEMM.
    unfused = None
    if not args.no_unfused and not attn:
        xn = [torch.empty_like(s["X"]) for s in sets]
        # the vendor leg multiplies by A^T as a K x R matrix (made once, untimed)
        at = [s["LA"].t().contiguous() for s in sets] if wl.lora else None

        def unfused_ours(i):
            s = sets[i]
            tpa.rmsnorm(s["X"], s["g"], wl.eps, out=xn[i])
            if wl.gated:
                tpa.gated_matmul(xn[i], s["W1"], s["W3"], out=s["Y"], workspace=ws)
            elif wl.lora:
                tpa.lora_matmul(xn[i], s["W1"], s["LA"], s["LB"], out=s["Y"], workspace=ws)
            else:
                tpa.matmul(xn[i], s["W1"], out=s["Y"], workspace=ws)

        def unfused_vendor(i):
            s = sets[i]
            tpa.rmsnorm(s["X"], s["g"], wl.eps, out=xn[i])
            if wl.gated:
                torch.mul(torch.nn.functional.silu(torch.matmul(xn[i], s["W1"])),
                          torch.matmul(xn[i], s["W3"]), out=s["Y"])
            elif wl.lora:
                torch.addmm(torch.matmul(xn[i], s["W1"]), torch.matmul(xn[i], at[i]), s["LB"],
                            out=s["Y"])
            else:
                torch.matmul(xn[i], s["W1"], out=s["Y"])

        run_u = make_runner(unfused_ours, not args.no_graph)
        run_u(warm)
        ms_u = time_steps(run_u, steps)
        run_v = make_runner(unfused_vendor, False)  # library GEMMs stay out of graphs
        run_v(warm)
        ms_v = time_steps(run_v, steps)
        unfused = {
            "ms_per_step": ms_u / steps, "fused_speedup": ms_u / ms,
            "vendor_gemm_ms_per_step": ms_v / steps, "fused_speedup_vs_vendor_gemm": ms_v / ms,
            "normalised_x_bytes": 2 * wl.M * wl.K * wl.elem_bytes,
            "note": "rmm_rmsnorm writes X*g/RMS to memory, then rmm_matmul (this library's "
                    "kernels; rmm_lora_matmul with the adapter) or torch.matmul (hipBLASLt; "
                    "with the adapter, three products) reads it back"}
        log(f"unfused: {ms_u / steps * 1e3:.2f} us/step (ours), {ms_v / steps * 1e3:.2f} us/step "
            f"(vendor GEMM); fused {ms / steps * 1e3:.2f}")
    elif not args.no_unfused and wl.G == 1:
        # QKNorm: RMSNorm of q and of every cached key written to memory, then
        # the attention step alone on the normalised copies.
        qn = [torch.empty_like(s["Q"]) for s in sets]
        kn = [torch.empty_like(s["K"]) for s in sets]
        na = tpa._binding.attention_workspace_bytes(dcode, wl.BH, wl.S, wl.D, 0)
        wsa = tpa.Workspace(na, dev) if na > 0 else None

        def unfused_attn(i):
            s = sets[i]
            tpa.rmsnorm(s["Q"], s["gq"], wl.eps, out=qn[i])
            tpa.rmsnorm(s["K"].view(wl.BH * wl.S, wl.D), s["gk"], wl.eps,
                        out=kn[i].view(wl.BH * wl.S, wl.D))
            tpa.attention(qn[i], kn[i], s["V"], out=s["Y"], workspace=wsa)

        run_u = make_runner(unfused_attn, not args.no_graph)
        run_u(warm)
        ms_u = time_steps(run_u, steps)
        unfused = {
            "ms_per_step": ms_u / steps, "fused_speedup": ms_u / ms,
            "normalised_k_bytes": 2 * wl.BH * wl.S * wl.D * 2,
            "note": "rmm_rmsnorm writes q*gq/RMS and every k*gk/RMS to memory, then "
                    "rmm_attention reads the normalised keys back"}
        log(f"unfused: {ms_u / steps * 1e3:.2f} us/step; fused {ms / steps * 1e3:.2f}")

    gbs = per_set / per_launch_s / 1e9
    tflops = wl.flops() / per_launch_s / 1e12
    bound = "hbm" if wl.flops() / per_set < RIDGE else "mfma"
    if bound == "hbm":
        value, unit = gbs, "GB/s"
        roof = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": gbs / HBM_PEAK_GBS}
    else:
        peak = BF16_PEAK_TFLOPS if wl.dtype == "bf16" else F32_VALU_PEAK_TFLOPS
        value, unit = tflops, "TFLOP/s"
        roof = {"bound": "mfma" if wl.dtype == "bf16" else "alu", "achieved": tflops,
                "peak": peak, "unit": "TFLOP/s", "frac": tflops / peak}
    # the fp32 decode variant is its own kernel (rmm_decode32.hip)
    kvar = "decode32" if (variant == "decode" and wl.dtype == "f32") else variant
    roof["traffic"] = stored_traffic(wl.name, kvar)
    peaks = None
    if not args.no_peaks:
        log("achievable-peak probes")
        peaks = measure_peaks(stream, dev)
        ach = peaks["hbm_read_gbs"] if roof["bound"] == "hbm" else (
            peaks["mfma_bf16_tflops"] if roof["bound"] == "mfma" else None)
        if ach:
            roof["achievable_peak"] = ach
            roof["frac_of_achievable"] = roof["achieved"] / ach
    roof["kernel"] = (("gqa_mfma_kernel" if wl.G >= 3 else "qknorm_attention_kernel") if attn
                      else f"{kvar}_kernel")
    roof["algorithmic_bytes_per_launch"] = per_set
    roof["algorithmic_flops_per_launch"] = wl.flops()

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        cpu = cpu_baseline(wl, inp, args.cpu_budget)

    line = {
        "metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": steps,
        "warmup": warm, "ms_per_step": ms / steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": ({"workload": wl.name, "BH": wl.BH, "G": wl.G, "S": wl.S, "D": wl.D} if attn else
                   {"workload": wl.name, "M": wl.M, "K": wl.K, "N": wl.N, "gated": wl.gated,
                    "lora_rank": wl.lora}) | {
                   "eps": wl.eps, "variant": variant, "splits": splits,
                   "rotating_input_sets": R, "hip_graph": graph is not None,
                   "clock_settle_calls": settle_calls},
        "tflops": tflops, "hbm_gbs_algorithmic": gbs,
        "roofline": roof, "cpu_baseline": cpu, "unfused_baseline": unfused,
        "achievable_peaks": peaks,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
