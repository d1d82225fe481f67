"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

Input generation only: nothing here computes any part of RMSNorm or the matmul.
The counter-based generator lives in ``synth.c`` (built to ``libsynth.so``);
this module wraps it with numpy and describes the five workloads.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .workloads import ATTN_WORKLOADS, WORKLOADS, AttnWorkload, Workload, get_workload  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_lib = None

# Tensor streams of the generator.
STREAM_X, STREAM_G, STREAM_W1, STREAM_W3, STREAM_ROWSCALE, STREAM_ROWPICK = 1, 2, 3, 4, 5, 6
STREAM_EXACT = 7
STREAM_LA, STREAM_LB = 20, 21  # adapter down- and up-projection (clear of the exact streams)
STREAM_Q, STREAM_K, STREAM_V, STREAM_GQ, STREAM_GK, STREAM_PICK = 22, 23, 24, 25, 26, 27


def build(force: bool = False) -> str:
    """Compile libsynth.so with gcc (host code only)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        u64, i64, i32, dbl, vp = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int,
                                  ctypes.c_double, ctypes.c_void_p)
        lib.synth_mix.argtypes = [u64]
        lib.synth_mix.restype = u64
        lib.synth_hash.argtypes = [u64, i32, i64, i64, i32, vp]
        lib.synth_uniform.argtypes = [u64, i32, i64, i64, i32, vp]
        lib.synth_normal_f32.argtypes = [u64, i32, i64, i64, dbl, dbl, vp, vp, vp]
        lib.synth_exact_f32.argtypes = [u64, i32, i64, i32, dbl, vp]
        lib.synth_f32_to_bf16.argtypes = [vp, vp, i64]
        lib.synth_bf16_to_f32.argtypes = [vp, vp, i64]
        for f in ("synth_hash", "synth_uniform", "synth_normal_f32", "synth_exact_f32",
                  "synth_f32_to_bf16", "synth_bf16_to_f32"):
            getattr(lib, f).restype = None
        _lib = lib
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def mix(x: int) -> int:
    return int(_load().synth_mix(x))


def hashes(seed: int, t: int, i0: int, n: int, j: int = 0) -> np.ndarray:
    out = np.empty(n, np.uint64)
    _load().synth_hash(seed, t, i0, n, j, _p(out))
    return out


def uniforms(seed: int, t: int, i0: int, n: int, j: int = 0) -> np.ndarray:
    out = np.empty(n, np.float64)
    _load().synth_uniform(seed, t, i0, n, j, _p(out))
    return out


def normals(seed: int, t: int, rows: int, cols: int, mul: float = 1.0, add: float = 0.0,
            row_scale: np.ndarray | None = None, row_idx: np.ndarray | None = None) -> np.ndarray:
    """float32 [rows, cols] of (float)(row_scale[r] * (add + mul * z(t, R*cols + c)))."""
    out = np.empty((rows, cols), np.float32)
    rs = None if row_scale is None else np.ascontiguousarray(row_scale, np.float64)
    ri = None if row_idx is None else np.ascontiguousarray(row_idx, np.int64)
    _load().synth_normal_f32(seed, t, rows, cols, mul, add, _p(rs), _p(ri), _p(out))
    return out


def exact_values(seed: int, t: int, shape, kind: int, density: float = 1.0) -> np.ndarray:
    """Small-integer values (see synth.c): kind 0 -> +-1, 1 -> {1,2}, 2 -> sparse {-2..2}."""
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    _load().synth_exact_f32(seed, t, n, kind, density, _p(out))
    return out.reshape(shape)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    a = np.ascontiguousarray(a, np.float32)
    out = np.empty(a.shape, np.uint16)
    _load().synth_f32_to_bf16(_p(a), _p(out), a.size)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, np.uint16)
    out = np.empty(b.shape, np.float32)
    _load().synth_bf16_to_f32(_p(b), _p(out), b.size)
    return out


def row_scales(wl: "Workload", seed: int = 0) -> np.ndarray | None:
    """Per-row scale of X for the workloads that have one (float64 [M]) else None."""
    M = wl.M
    if wl.row_scale == "pick_x100":
        # round(0.01*M) rows, the ones with the smallest h(6, m, 0), scaled by 100.
        count = int(round(0.01 * M))
        h = hashes(seed, STREAM_ROWPICK, 0, M, 0)
        picked = np.argsort(h, kind="stable")[:count]
        s = np.ones(M, np.float64)
        s[picked] = 100.0
        return s
    if wl.row_scale == "loguniform":
        # s_m = 10^(-2 + 4 u(5, m, 0)): LogUniform on [0.01, 100).
        u = uniforms(seed, STREAM_ROWSCALE, 0, M, 0)
        return np.power(10.0, -2.0 + 4.0 * u)
    return None


class Inputs:
    """Stored input values of one workload.

    ``X, g, W1, W3`` hold the stored values as float32 (bf16 workloads: the
    bf16 values decoded exactly); ``bits`` holds the uint16 patterns of the
    bf16 workloads, i.e. exactly what is handed to the library.
    """

    def __init__(self, wl, X, g, W1, W3, rows, LA=None, LB=None):
        self.wl, self.rows = wl, rows
        self.bits = {}
        self.LA, self.LB = LA, LB  # adapter: [R, K] and [R, N], or None
        if wl.dtype == "bf16":
            for name, a in (("X", X), ("g", g), ("W1", W1), ("W3", W3), ("LA", LA), ("LB", LB)):
                if a is not None:
                    b = to_bf16_bits(a)
                    self.bits[name] = b
                    a = bf16_bits_to_f32(b)
                setattr(self, name, a)
        else:
            self.X, self.g, self.W1, self.W3 = X, g, W1, W3

    def device_array(self, name):
        """The array handed to the library: uint16 bf16 bits or float32 values."""
        return self.bits[name] if self.wl.dtype == "bf16" else getattr(self, name)


def make_inputs(wl: "Workload", seed: int = 0, rows=None, weights: bool = True) -> Inputs:
    """Draw the inputs of ``wl``.  ``rows`` (optional index array) draws only those
    rows of X, bit-identical to the same rows of the full tensor."""
    M, K, N = wl.M, wl.K, wl.N
    scale = row_scales(wl, seed)
    if rows is None:
        X = normals(seed, STREAM_X, M, K, row_scale=scale)
    else:
        rows = np.asarray(rows, np.int64)
        X = normals(seed, STREAM_X, len(rows), K,
                    row_scale=None if scale is None else scale[rows], row_idx=rows)
    g = normals(seed, STREAM_G, 1, K, mul=0.1, add=1.0).reshape(K)
    W1 = W3 = LA = LB = None
    if weights:
        W1 = normals(seed, STREAM_W1, K, N, mul=1.0 / np.sqrt(K))
        if wl.gated:
            W3 = normals(seed, STREAM_W3, K, N, mul=1.0 / np.sqrt(K))
        if wl.lora:
            LA = normals(seed, STREAM_LA, wl.lora, K, mul=1.0 / np.sqrt(K))
            LB = normals(seed, STREAM_LB, wl.lora, N, mul=1.0 / np.sqrt(wl.lora))
    return Inputs(wl, X, g, W1, W3, rows, LA, LB)


def make_exact_inputs(M: int, K: int, N: int, dtype: str, seed: int = 0, gated: bool = False,
                      density: float = 0.25, row_pow2: bool = False, lora: int = 0) -> Inputs:
    """Inputs on which fp32 accumulation (and bf16 storage of X*g) is exact.

    X in {+-1} (optionally each row times 2^j, j in [-6, 6]), g in {1, 2},
    W (and the adapter's A and B) in {-2..2} with the given density; used with
    eps = 0, so the row RMS is 1 (or 2^j) exactly and every product and
    partial sum is a small integer times a power of two, whatever the order of
    summation (below 2^24 for K up to 2^12 and ranks up to 64).
    """
    wl = Workload("exact", dtype, M, K, N, 0.0, gated, None, lora)
    X = exact_values(seed, STREAM_EXACT, (M, K), 0)
    if row_pow2:
        j = (hashes(seed, STREAM_EXACT + 4, 0, M, 0) % np.uint64(13)).astype(np.int64) - 6
        X = (X * np.power(2.0, j)[:, None]).astype(np.float32)
    g = exact_values(seed, STREAM_EXACT + 1, (K,), 1)
    W1 = exact_values(seed, STREAM_EXACT + 2, (K, N), 2, density)
    W3 = exact_values(seed, STREAM_EXACT + 3, (K, N), 2, density) if gated else None
    LA = exact_values(seed, STREAM_EXACT + 5, (lora, K), 2, density) if lora else None
    LB = exact_values(seed, STREAM_EXACT + 6, (lora, N), 2, density) if lora else None
    return Inputs(wl, X, g, W1, W3, None, LA, LB)


class AttnInputs:
    """Stored values (float32, bf16-exact) and bf16 bit patterns of one
    attention call: Q [BH, D], K and V [BH, S, D], gq and gk [D]."""

    def __init__(self, Q, K, V, gq, gk):
        self.bits = {}
        for name, a in (("Q", Q), ("K", K), ("V", V), ("gq", gq), ("gk", gk)):
            b = to_bf16_bits(a)
            self.bits[name] = b
            setattr(self, name, bf16_bits_to_f32(b))

    def device_array(self, name):
        return self.bits[name]


def make_attention_inputs(BH: int, S: int, D: int, seed: int = 0, G: int = 1) -> AttnInputs:
    """BH key/value heads; Q has BH * G rows (G query heads per key/value head)."""
    Q = normals(seed, STREAM_Q, BH * G, D)
    K = normals(seed, STREAM_K, BH * S, D).reshape(BH, S, D)
    V = normals(seed, STREAM_V, BH * S, D).reshape(BH, S, D)
    gq = normals(seed, STREAM_GQ, 1, D, mul=0.1, add=1.0).reshape(D)
    gk = normals(seed, STREAM_GK, 1, D, mul=0.1, add=1.0).reshape(D)
    return AttnInputs(Q, K, V, gq, gk)


def make_attention_prefill_inputs(BH: int, G: int, Sq: int, Skv: int, D: int,
                                  seed: int = 0) -> AttnInputs:
    """Many queries per head: Q [BH * G, Sq, D], K and V [BH, Skv, D], gains [D]
    (the same distributions as make_attention_inputs)."""
    Q = normals(seed, STREAM_Q, BH * G * Sq, D).reshape(BH * G, Sq, D)
    K = normals(seed, STREAM_K, BH * Skv, D).reshape(BH, Skv, D)
    V = normals(seed, STREAM_V, BH * Skv, D).reshape(BH, Skv, D)
    gq = normals(seed, STREAM_GQ, 1, D, mul=0.1, add=1.0).reshape(D)
    gk = normals(seed, STREAM_GK, 1, D, mul=0.1, add=1.0).reshape(D)
    return AttnInputs(Q, K, V, gq, gk)


def make_attention_onehot(BH: int, S: int, D: int, seed: int = 0, G: int = 1):
    """Inputs whose softmax is exactly one-hot in fp32: gains of 40 and, per
    query, one key of its key/value head equal to q / 2 (exact in bf16),
    picked by the hash (the G queries of a head pick keys S // G apart, so
    they differ; needs S >= G); that key's score exceeds every other by
    thousands, so its weight is 1 and the others' are 0, and the output is
    that key's value row.  Returns (inputs, picked key index per query row,
    shape [BH * G])."""
    assert S >= G
    inp = make_attention_inputs(BH, S, D, seed, G=G)
    base = (hashes(seed, STREAM_PICK, 0, BH, 0) % np.uint64(S)).astype(np.int64)
    pick = (base[:, None] + np.arange(G)[None, :] * (S // G)) % S
    Q = inp.Q.copy()
    K = inp.K.copy()
    K[np.repeat(np.arange(BH), G), pick.reshape(-1)] = 0.5 * Q
    g = np.full(D, 40.0, np.float32)
    return AttnInputs(Q, K, inp.V, g, g), pick.reshape(-1)
