"""ctypes binding of librmm.so: argument marshalling only.

Every step of the computation runs in the HIP kernels behind the C ABI
(include/rmm.h).  PyTorch provides device memory and the current stream.
If the library is missing this module raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librmm.so")

DTYPE_F32, DTYPE_BF16 = 0, 1
VARIANTS = {"auto": 0, "generic": 1, "decode": 2, "prefill": 3, "stream": 4}
VARIANT_NAMES = {v: k for k, v in VARIANTS.items()}
STATUS_OK = 0
# Not a status of the C ABI: raised by the Python front end when the layer
# chain's flag word reports a wait that gave up.
STATUS_CHAIN_WAIT = 100

# Exported symbols of include/rmm.h.
SYMBOLS = ("rmsnorm_matmul", "rmsnorm_gated_mlp", "rmsnorm_matmul_ex", "rmsnorm_gated_mlp_ex",
           "rmm_rmsnorm", "rmm_matmul", "rmm_gated_matmul", "rmm_workspace_bytes",
           "rmm_workspace_bytes_ex", "rmm_plan", "rmm_status_string", "rmm_last_hip_error",
           "rmm_abi_version", "rmsnorm_lora", "rmsnorm_lora_ex", "rmm_lora_matmul",
           "rmm_lora_workspace_bytes", "rmm_plan_lora", "qknorm_attention",
           "qknorm_attention_ex", "rmm_attention_workspace_bytes", "rmm_plan_attention",
           "rmm_attention", "qknorm_attention_gqa", "rmm_attention_gqa_workspace_bytes",
           "rmm_plan_attention_gqa", "qknorm_attention_prefill", "qknorm_attention_prefill_ex",
           "rmm_attention_prefill_workspace_bytes",
           "rmsnorm_matmul_chain", "rmm_chain_workspace_bytes", "rmm_chain_flag_offset",
           "rmm_probe_hbm_read", "rmm_probe_mfma_bf16", "rmm_probe_mfma_flops",
           "rmsnorm_matmul_noalloc")
LORA_MAX_RANK = 64

_lib = None


class RmmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def load_library(path: str = LIB_PATH):
    """Load librmm.so and declare its signatures.  Raises if it is not built."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m tensor_program_amd.build` "
                          "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(path)
    vp, f32, i64, i32, sz = (ctypes.c_void_p, ctypes.c_float, ctypes.c_int64, ctypes.c_int,
                             ctypes.c_size_t)
    lib.rmsnorm_matmul.argtypes = [vp, vp, vp, vp, f32, i64, i64, i64, i32, vp, sz, vp]
    lib.rmsnorm_gated_mlp.argtypes = [vp, vp, vp, vp, vp, f32, i64, i64, i64, i32, vp, sz, vp]
    lib.rmsnorm_matmul_noalloc.argtypes = [vp, vp, vp, vp, f32, i64, i64, i64, i32, vp]
    lib.rmsnorm_matmul_ex.argtypes = [vp, vp, vp, vp, f32, i64, i64, i64, i32, i32, i32, vp, sz,
                                      vp]
    lib.rmsnorm_gated_mlp_ex.argtypes = [vp, vp, vp, vp, vp, f32, i64, i64, i64, i32, i32, i32,
                                         vp, sz, vp]
    lib.rmm_rmsnorm.argtypes = [vp, vp, vp, f32, i64, i64, i32, vp]
    lib.rmm_matmul.argtypes = [vp, vp, vp, i64, i64, i64, i32, vp, sz, vp]
    lib.rmm_gated_matmul.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, vp, sz, vp]
    lib.rmsnorm_lora.argtypes = [vp, vp, vp, vp, vp, vp, f32, i64, i64, i64, i64, i32, vp, sz, vp]
    lib.rmsnorm_lora_ex.argtypes = [vp, vp, vp, vp, vp, vp, f32, i64, i64, i64, i64, i32, i32,
                                    i32, vp, sz, vp]
    lib.rmm_lora_matmul.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, vp, sz, vp]
    for f in ("rmsnorm_matmul", "rmsnorm_gated_mlp", "rmsnorm_matmul_ex", "rmsnorm_gated_mlp_ex",
              "rmsnorm_matmul_noalloc",
              "rmm_rmsnorm", "rmm_matmul", "rmm_gated_matmul", "rmsnorm_lora", "rmsnorm_lora_ex",
              "rmm_lora_matmul"):
        getattr(lib, f).restype = i32
    lib.rmm_lora_workspace_bytes.argtypes = [i32, i64, i64, i64, i64, i32, i32]
    lib.rmm_lora_workspace_bytes.restype = sz
    lib.rmm_plan_lora.argtypes = [vp, vp, vp, vp, vp, vp, f32, i64, i64, i64, i64, i32, i32, i32,
                                  vp, sz, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.rmm_plan_lora.restype = i32
    lib.qknorm_attention.argtypes = [vp, vp, vp, vp, vp, vp, f32, i64, i64, i64, i32, vp, sz, vp]
    lib.qknorm_attention.restype = i32
    lib.qknorm_attention_ex.argtypes = [vp, vp, vp, vp, vp, vp, f32, i64, i64, i64, i32, i32, vp,
                                        sz, vp]
    lib.qknorm_attention_ex.restype = i32
    lib.rmm_attention.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, vp, sz, vp]
    lib.rmm_attention.restype = i32
    lib.qknorm_attention_gqa.argtypes = [vp, vp, vp, vp, vp, vp, f32, i64, i64, i64, i64, i32, i32,
                                         vp, sz, vp]
    lib.qknorm_attention_gqa.restype = i32
    lib.rmm_attention_gqa_workspace_bytes.argtypes = [i32, i64, i64, i64, i64, i32]
    lib.rmm_attention_gqa_workspace_bytes.restype = sz
    lib.rmm_plan_attention_gqa.argtypes = [vp, vp, vp, vp, vp, vp, f32, i64, i64, i64, i64, i32, i32,
                                           vp, sz, ctypes.POINTER(i32), ctypes.POINTER(i64)]
    lib.rmm_plan_attention_gqa.restype = i32
    lib.qknorm_attention_prefill.argtypes = [vp, vp, vp, vp, vp, vp, f32, i64, i64, i64, i64, i64,
                                             i32, i32, vp]
    lib.qknorm_attention_prefill.restype = i32
    lib.qknorm_attention_prefill_ex.argtypes = [vp, vp, vp, vp, vp, vp, f32, i64, i64, i64, i64,
                                                i64, i32, i32, i32, vp, sz, vp]
    lib.qknorm_attention_prefill_ex.restype = i32
    lib.rmm_attention_prefill_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i32, i32]
    lib.rmm_attention_prefill_workspace_bytes.restype = sz
    lib.rmm_attention_workspace_bytes.argtypes = [i32, i64, i64, i64, i32]
    lib.rmm_attention_workspace_bytes.restype = sz
    lib.rmm_plan_attention.argtypes = [vp, vp, vp, vp, vp, vp, f32, i64, i64, i64, i32, i32, vp, sz,
                                       ctypes.POINTER(i32), ctypes.POINTER(i64)]
    lib.rmm_plan_attention.restype = i32
    lib.rmsnorm_matmul_chain.argtypes = [vp, vp, vp, vp, f32, i64, i64, i64, i32, vp, sz, vp]
    lib.rmsnorm_matmul_chain.restype = i32
    lib.rmm_chain_workspace_bytes.argtypes = [i64, i64, i64]
    lib.rmm_chain_workspace_bytes.restype = sz
    lib.rmm_chain_flag_offset.argtypes = [i64, i64, i64]
    lib.rmm_chain_flag_offset.restype = sz
    lib.rmm_probe_hbm_read.argtypes = [vp, sz, vp, vp]
    lib.rmm_probe_hbm_read.restype = i32
    lib.rmm_probe_mfma_bf16.argtypes = [i64, vp, vp]
    lib.rmm_probe_mfma_bf16.restype = i32
    lib.rmm_probe_mfma_flops.argtypes = [i64]
    lib.rmm_probe_mfma_flops.restype = i64
    lib.rmm_workspace_bytes.argtypes = [i32, i64, i64, i64, i32]
    lib.rmm_workspace_bytes.restype = sz
    lib.rmm_workspace_bytes_ex.argtypes = [i32, i64, i64, i64, i32, i32, i32]
    lib.rmm_workspace_bytes_ex.restype = sz
    lib.rmm_plan.argtypes = [vp, vp, vp, vp, vp, f32, i64, i64, i64, i32, i32, i32, i32, vp, sz,
                             ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.rmm_plan.restype = i32
    lib.rmm_status_string.argtypes = [i32]
    lib.rmm_status_string.restype = ctypes.c_char_p
    lib.rmm_last_hip_error.argtypes = []
    lib.rmm_last_hip_error.restype = i32
    lib.rmm_abi_version.argtypes = []
    lib.rmm_abi_version.restype = i32
    if path == LIB_PATH:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().rmm_status_string(status).decode()


def check(status: int):
    if status != STATUS_OK:
        msg = status_string(status)
        if status == 7:
            msg += f" (hipError_t {load_library().rmm_last_hip_error()})"
        raise RmmError(status, msg)


def workspace_bytes(dtype: int, M: int, N: int, K: int, gated: bool, variant: str = "auto",
                    splits: int = 0) -> int:
    return int(load_library().rmm_workspace_bytes_ex(dtype, M, N, K, int(gated),
                                                     VARIANTS[variant], splits))


def plan(X, g, W1, W3, Y, eps, M, N, K, dtype, gated, variant="auto", splits=0, ws=None,
         ws_bytes=0):
    """Host-only planning through rmm_plan: (status, variant name, splits)."""
    v = ctypes.c_int(-1)
    s = ctypes.c_int(-1)
    st = load_library().rmm_plan(X, g, W1, W3, Y, eps, M, N, K, dtype, int(gated),
                                 VARIANTS[variant], splits, ws, ws_bytes, ctypes.byref(v),
                                 ctypes.byref(s))
    return st, VARIANT_NAMES.get(v.value), s.value


def lora_workspace_bytes(dtype: int, M: int, N: int, K: int, R: int, variant: str = "auto",
                         splits: int = 0) -> int:
    return int(load_library().rmm_lora_workspace_bytes(dtype, M, N, K, R, VARIANTS[variant],
                                                       splits))


def plan_lora(X, g, W, A, B, Y, eps, M, N, K, R, dtype, variant="auto", splits=0, ws=None,
              ws_bytes=0):
    """Host-only planning through rmm_plan_lora: (status, variant name, splits)."""
    v = ctypes.c_int(-1)
    s = ctypes.c_int(-1)
    st = load_library().rmm_plan_lora(X, g, W, A, B, Y, eps, M, N, K, R, dtype, VARIANTS[variant],
                                      splits, ws, ws_bytes, ctypes.byref(v), ctypes.byref(s))
    return st, VARIANT_NAMES.get(v.value), s.value


def chain_workspace_bytes(M: int, K: int, L: int) -> int:
    return int(load_library().rmm_chain_workspace_bytes(M, K, L))


def chain_flag_offset(M: int, K: int, L: int) -> int:
    return int(load_library().rmm_chain_flag_offset(M, K, L))


def attention_workspace_bytes(dtype: int, BH: int, S: int, D: int, splits: int = 0) -> int:
    return int(load_library().rmm_attention_workspace_bytes(dtype, BH, S, D, splits))


def plan_attention(Q, K, V, gq, gk, O, eps, BH, S, D, dtype, splits=0, ws=None, ws_bytes=0,
                   G=1):
    """Host-only planning through rmm_plan_attention (rmm_plan_attention_gqa
    for G > 1): (status, chunks, keys per chunk)."""
    c = ctypes.c_int(-1)
    kc = ctypes.c_int64(-1)
    lib = load_library()
    if G == 1:
        st = lib.rmm_plan_attention(Q, K, V, gq, gk, O, eps, BH, S, D, dtype, splits, ws,
                                    ws_bytes, ctypes.byref(c), ctypes.byref(kc))
    else:
        st = lib.rmm_plan_attention_gqa(Q, K, V, gq, gk, O, eps, BH, G, S, D, dtype, splits, ws,
                                        ws_bytes, ctypes.byref(c), ctypes.byref(kc))
    return st, c.value, kc.value


def attention_gqa_workspace_bytes(dtype: int, BH: int, G: int, S: int, D: int,
                                  splits: int = 0) -> int:
    return int(load_library().rmm_attention_gqa_workspace_bytes(dtype, BH, G, S, D, splits))
