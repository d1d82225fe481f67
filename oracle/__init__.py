"""CPU oracle of the fused RMSNorm+MatMul path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (``tensor_program_amd``)
never does, and the two share no code.

``rmm_oracle.c`` is the plain unfused program in fp64 (see its header for the
passages it follows); this module marshals numpy arrays to it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rmm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-Wall"]
_lib = None


def build(force: bool = False, src: str = _SRC, out: str = _LIB, extra=()) -> str:
    """Compile the oracle with gcc."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, *extra, "-o", tmp, src, "-lm"])
        os.replace(tmp, out)
    return out


def load(path: str = _LIB):
    """Load an oracle build (the default one, or another build of the same source)."""
    lib = ctypes.CDLL(path)
    vp, dbl, i64 = ctypes.c_void_p, ctypes.c_double, ctypes.c_int64
    lib.rmm_oracle_rmsnorm_matmul_f64.argtypes = [vp, vp, vp, dbl, i64, i64, i64, vp]
    lib.rmm_oracle_rmsnorm_matmul_f64.restype = ctypes.c_int
    lib.rmm_oracle_rmsnorm_gated_mlp_f64.argtypes = [vp, vp, vp, vp, dbl, i64, i64, i64, vp]
    lib.rmm_oracle_rmsnorm_gated_mlp_f64.restype = ctypes.c_int
    lib.rmm_oracle_rmsnorm_f64.argtypes = [vp, vp, dbl, i64, i64, vp]
    lib.rmm_oracle_rmsnorm_f64.restype = ctypes.c_int
    lib.rmm_oracle_matmul_f64.argtypes = [vp, vp, i64, i64, i64, vp]
    lib.rmm_oracle_matmul_f64.restype = ctypes.c_int
    lib.rmm_oracle_gated_matmul_f64.argtypes = [vp, vp, vp, i64, i64, i64, vp]
    lib.rmm_oracle_gated_matmul_f64.restype = ctypes.c_int
    lib.rmm_oracle_rmsnorm_lora_f64.argtypes = [vp, vp, vp, vp, vp, dbl, i64, i64, i64, i64, vp]
    lib.rmm_oracle_rmsnorm_lora_f64.restype = ctypes.c_int
    lib.rmm_oracle_lora_matmul_f64.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, vp]
    lib.rmm_oracle_lora_matmul_f64.restype = ctypes.c_int
    lib.rmm_oracle_qknorm_attention_f64.argtypes = [vp, vp, vp, vp, vp, dbl, i64, i64, i64, vp]
    lib.rmm_oracle_qknorm_attention_f64.restype = ctypes.c_int
    lib.rmm_oracle_attention_f64.argtypes = [vp, vp, vp, i64, i64, i64, vp]
    lib.rmm_oracle_attention_f64.restype = ctypes.c_int
    lib.rmm_oracle_qknorm_attention_prefill_f64.argtypes = [vp, vp, vp, vp, vp, dbl, i64, i64,
                                                            i64, i64, i64, ctypes.c_int, vp]
    lib.rmm_oracle_qknorm_attention_prefill_f64.restype = ctypes.c_int
    return lib


def _default():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = load(_LIB)
    return _lib


def _d(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def rmsnorm_matmul(X, g, W, eps, lib=None) -> np.ndarray:
    """Y = RMSNorm(X; g, eps) @ W in fp64.  X: [M,K], g: [K], W: [K,N]."""
    lib = lib or _default()
    X, g, W = _d(X), _d(g), _d(W)
    M, K = X.shape
    K2, N = W.shape
    assert K2 == K and g.shape == (K,)
    Y = np.empty((M, N), np.float64)
    rc = lib.rmm_oracle_rmsnorm_matmul_f64(_p(X), _p(g), _p(W), float(eps), M, N, K, _p(Y))
    if rc != 0:
        raise ValueError(f"oracle error {rc}")
    return Y


def rmsnorm_gated_mlp(X, g, W1, W3, eps, lib=None) -> np.ndarray:
    """Y = silu(RMSNorm(X) @ W1) * (RMSNorm(X) @ W3) in fp64."""
    lib = lib or _default()
    X, g, W1, W3 = _d(X), _d(g), _d(W1), _d(W3)
    M, K = X.shape
    K2, N = W1.shape
    assert K2 == K and W3.shape == W1.shape and g.shape == (K,)
    Y = np.empty((M, N), np.float64)
    rc = lib.rmm_oracle_rmsnorm_gated_mlp_f64(_p(X), _p(g), _p(W1), _p(W3), float(eps), M, N,
                                              K, _p(Y))
    if rc != 0:
        raise ValueError(f"oracle error {rc}")
    return Y


def rmsnorm(X, g, eps, lib=None) -> np.ndarray:
    """The normalised, gained rows (X / r) * g in fp64 -- the tensor the fused
    kernels never write, produced by the first kernel of the unfused program."""
    lib = lib or _default()
    X, g = _d(X), _d(g)
    M, K = X.shape
    assert g.shape == (K,)
    out = np.empty((M, K), np.float64)
    rc = lib.rmm_oracle_rmsnorm_f64(_p(X), _p(g), float(eps), M, K, _p(out))
    if rc != 0:
        raise ValueError(f"oracle error {rc}")
    return out


def matmul(A, B, lib=None) -> np.ndarray:
    """Y = A @ B in fp64, the oracle's own i-k-j loops."""
    lib = lib or _default()
    A, B = _d(A), _d(B)
    M, K = A.shape
    K2, N = B.shape
    assert K2 == K
    Y = np.empty((M, N), np.float64)
    rc = lib.rmm_oracle_matmul_f64(_p(A), _p(B), M, N, K, _p(Y))
    if rc != 0:
        raise ValueError(f"oracle error {rc}")
    return Y


def gated_matmul(A, W1, W3, lib=None) -> np.ndarray:
    """Y = silu(A @ W1) * (A @ W3) in fp64."""
    lib = lib or _default()
    A, W1, W3 = _d(A), _d(W1), _d(W3)
    M, K = A.shape
    K2, N = W1.shape
    assert K2 == K and W3.shape == W1.shape
    Y = np.empty((M, N), np.float64)
    rc = lib.rmm_oracle_gated_matmul_f64(_p(A), _p(W1), _p(W3), M, N, K, _p(Y))
    if rc != 0:
        raise ValueError(f"oracle error {rc}")
    return Y


def rmsnorm_lora(X, g, W, A, B, eps, lib=None) -> np.ndarray:
    """Y = Nrm @ W + (Nrm @ A.T) @ B in fp64, Nrm = RMSNorm(X; g, eps).
    X: [M,K], g: [K], W: [K,N], A: [R,K] (down-projection rows), B: [R,N]."""
    lib = lib or _default()
    X, g, W, A, B = _d(X), _d(g), _d(W), _d(A), _d(B)
    M, K = X.shape
    K2, N = W.shape
    R = A.shape[0]
    assert K2 == K and g.shape == (K,) and A.shape == (R, K) and B.shape == (R, N)
    Y = np.empty((M, N), np.float64)
    rc = lib.rmm_oracle_rmsnorm_lora_f64(_p(X), _p(g), _p(W), _p(A), _p(B), float(eps), M, N, K,
                                         R, _p(Y))
    if rc != 0:
        raise ValueError(f"oracle error {rc}")
    return Y


def lora_matmul(X, W, A, B, lib=None) -> np.ndarray:
    """Y = X @ W + (X @ A.T) @ B in fp64 (the adapter without the norm)."""
    lib = lib or _default()
    X, W, A, B = _d(X), _d(W), _d(A), _d(B)
    M, K = X.shape
    K2, N = W.shape
    R = A.shape[0]
    assert K2 == K and A.shape == (R, K) and B.shape == (R, N)
    Y = np.empty((M, N), np.float64)
    rc = lib.rmm_oracle_lora_matmul_f64(_p(X), _p(W), _p(A), _p(B), M, N, K, R, _p(Y))
    if rc != 0:
        raise ValueError(f"oracle error {rc}")
    return Y


def qknorm_attention(Q, K, V, gq, gk, eps, lib=None) -> np.ndarray:
    """o = softmax(norm(q) . norm(K)^T / sqrt(D)) V per batch-head, in fp64.
    Q: [BH, D], K and V: [BH, S, D], gq and gk: [D] -> O: [BH, D]."""
    lib = lib or _default()
    Q, K, V, gq, gk = _d(Q), _d(K), _d(V), _d(gq), _d(gk)
    BH, D = Q.shape
    S = K.shape[1]
    assert K.shape == (BH, S, D) and V.shape == (BH, S, D) and gq.shape == (D,) and \
        gk.shape == (D,)
    O = np.empty((BH, D), np.float64)
    rc = lib.rmm_oracle_qknorm_attention_f64(_p(Q), _p(K), _p(V), _p(gq), _p(gk), float(eps), BH,
                                             S, D, _p(O))
    if rc != 0:
        raise ValueError(f"oracle error {rc}")
    return O


def qknorm_attention_prefill(Q, K, V, gq, gk, eps, causal=True, lib=None) -> np.ndarray:
    """QKNorm + attention for many queries per head, in fp64.  Q: [BH * G, Sq, D]
    (query head h * G + g reads key/value head h), K and V: [BH, Skv, D]; causal:
    query i sees keys 0 .. i + Skv - Sq.  -> O: [BH * G, Sq, D]."""
    lib = lib or _default()
    Q, K, V, gq, gk = _d(Q), _d(K), _d(V), _d(gq), _d(gk)
    BHq, Sq, D = Q.shape
    BH, Skv = K.shape[0], K.shape[1]
    assert BH > 0 and BHq % BH == 0 and K.shape == (BH, Skv, D) and V.shape == K.shape
    assert gq.shape == (D,) and gk.shape == (D,)
    O = np.empty((BHq, Sq, D), np.float64)
    rc = lib.rmm_oracle_qknorm_attention_prefill_f64(_p(Q), _p(K), _p(V), _p(gq), _p(gk),
                                                     float(eps), BH, BHq // BH, Sq, Skv, D,
                                                     int(bool(causal)), _p(O))
    if rc != 0:
        raise ValueError(f"oracle error {rc}")
    return O


def attention(Q, K, V, lib=None) -> np.ndarray:
    """o = softmax(q . K^T / sqrt(D)) V per batch-head, in fp64, on the vectors as
    given (the unfused program's second kernel).  Q: [BH, D], K and V: [BH, S, D]."""
    lib = lib or _default()
    Q, K, V = _d(Q), _d(K), _d(V)
    BH, D = Q.shape
    S = K.shape[1]
    assert K.shape == (BH, S, D) and V.shape == (BH, S, D)
    O = np.empty((BH, D), np.float64)
    rc = lib.rmm_oracle_attention_f64(_p(Q), _p(K), _p(V), BH, S, D, _p(O))
    if rc != 0:
        raise ValueError(f"oracle error {rc}")
    return O


def eps_as_passed(eps: float) -> float:
    """The eps the kernels see: the float32 value, widened exactly to double."""
    return float(np.float32(eps))
