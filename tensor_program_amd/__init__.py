"""Fused RMSNorm+MatMul for MI355X (gfx950): Python front end of librmm.so.

    import tensor_program_amd as tpa
    y = tpa.rmsnorm_matmul(x, g, w, eps)             # Y = RMSNorm(x; g, eps) @ w
    y = tpa.rmsnorm_gated_mlp(x, g, w1, w3, eps)     # silu(norm(x) @ w1) * (norm(x) @ w3)

    # the unfused two-kernel program the fused calls replace (for comparison)
    xn = tpa.rmsnorm(x, g, eps)                       # normalised x, written to memory
    y = tpa.matmul(xn, w)                             # plain product
    y = tpa.gated_matmul(xn, w1, w3)                  # silu(xn @ w1) * (xn @ w3)

    # low-rank adapter (a: [R, K] down-projection rows, b: [R, N])
    y = tpa.rmsnorm_lora(x, g, w, a, b, eps)          # norm(x) @ w + (norm(x) @ a.T) @ b
    y = tpa.lora_matmul(x, w, a, b)                   # x @ w + (x @ a.T) @ b

    # QKNorm + attention, one query per batch-head (q: [BH, D], k, v: [BH, S, D])
    o = tpa.qknorm_attention(q, k, v, gq, gk, eps)

x: [M, K], g: [K], w/w1/w3: [K, N], all contiguous, on one GPU, all float32 or
all bfloat16.  The work is enqueued on torch's current stream; this module
only marshals arguments (see include/rmm.h for the contract).
"""
from __future__ import annotations

import torch

from . import _binding
from ._binding import RmmError, load_library  # noqa: F401

__all__ = ["rmsnorm_matmul", "rmsnorm_gated_mlp", "rmsnorm", "matmul", "gated_matmul",
           "rmsnorm_lora", "lora_matmul", "qknorm_attention", "qknorm_attention_gqa",
           "qknorm_attention_prefill", "attention",
           "rmsnorm_matmul_chain",
           "RmmError", "load_library", "Workspace"]

_DTYPES = {torch.float32: _binding.DTYPE_F32, torch.bfloat16: _binding.DTYPE_BF16}


class Workspace:
    """A zero-filled device workspace for the split-K and split-key combines.

    Every call keeps its arrival counters in the first 64 KiB, resets them,
    and overwrites its partial sums before reading them, so one workspace
    serves any sequence of calls on one stream without clearing (the
    functions below keep one per device and stream, grown when a call needs
    more).  Calls that may overlap (different streams) need different
    workspaces.
    """

    def __init__(self, nbytes: int, device):
        self.nbytes = int(nbytes)
        self.tensor = torch.zeros(max(self.nbytes, 1), dtype=torch.uint8, device=device)

    @property
    def ptr(self) -> int:
        return self.tensor.data_ptr()


_workspaces: dict = {}


def _workspace_for(device, stream_handle: int, nbytes: int) -> Workspace:
    """The binding's workspace for one device and stream, grown (a new
    zero-filled buffer) when a call needs more than it holds."""
    key = (str(device), stream_handle)
    ws = _workspaces.get(key)
    if ws is None or ws.nbytes < nbytes:
        ws = Workspace(nbytes, device)
        _workspaces[key] = ws
    return ws


def _check_operands(tensors, names):
    t0 = tensors[0]
    if t0.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t0.dtype}; use float32 or bfloat16")
    for t, n in zip(tensors, names):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{n} must be a torch.Tensor")
        if t.dtype != t0.dtype:
            raise TypeError(f"{n} has dtype {t.dtype}, expected {t0.dtype}")
        if t.device != t0.device or t.device.type != "cuda":
            raise ValueError(f"{n} must be on the same GPU as the others")
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")


def _call(x, g, w1, w3, eps, out, variant, splits, workspace):
    gated = w3 is not None
    tensors = [x, g, w1] + ([w3] if gated else [])
    names = ["x", "g", "w1", "w3"] if gated else ["x", "g", "w"]
    _check_operands(tensors, names)
    if x.dim() != 2 or g.dim() != 1 or w1.dim() != 2:
        raise ValueError("expected x: [M, K], g: [K], w: [K, N]")
    M, K = x.shape
    K2, N = w1.shape
    if K2 != K or g.shape[0] != K or (gated and tuple(w3.shape) != (K, N)):
        raise ValueError(f"shape mismatch: x {tuple(x.shape)}, g {tuple(g.shape)}, "
                         f"w {tuple(w1.shape)}")
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    else:
        _check_operands([x, out], ["x", "out"])
        if tuple(out.shape) != (M, N):
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {(M, N)}")
    lib = load_library()
    dtype = _DTYPES[x.dtype]
    stream = torch.cuda.current_stream(x.device).cuda_stream
    need = _binding.workspace_bytes(dtype, M, N, K, gated, variant, splits)
    if workspace is None and need > 0:
        workspace = _workspace_for(x.device, stream, need)
    ws_ptr = workspace.ptr if workspace is not None else None
    ws_bytes = workspace.nbytes if workspace is not None else 0
    v = _binding.VARIANTS[variant]
    if gated:
        st = lib.rmsnorm_gated_mlp_ex(x.data_ptr(), g.data_ptr(), w1.data_ptr(), w3.data_ptr(),
                                      out.data_ptr(), float(eps), M, N, K, dtype, v, splits,
                                      ws_ptr, ws_bytes, stream)
    else:
        st = lib.rmsnorm_matmul_ex(x.data_ptr(), g.data_ptr(), w1.data_ptr(), out.data_ptr(),
                                   float(eps), M, N, K, dtype, v, splits, ws_ptr, ws_bytes, stream)
    _binding.check(st)
    return out


def rmsnorm_matmul(x, g, w, eps: float, out=None, variant: str = "auto", splits: int = 0,
                   workspace: Workspace | None = None):
    """Y = RMSNorm(x; g, eps) @ w, fused (the normalised x is never stored)."""
    return _call(x, g, w, None, eps, out, variant, splits, workspace)


def rmsnorm_gated_mlp(x, g, w1, w3, eps: float, out=None, variant: str = "auto",
                      splits: int = 0, workspace: Workspace | None = None):
    """Y = silu(RMSNorm(x) @ w1) * (RMSNorm(x) @ w3), fused."""
    return _call(x, g, w1, w3, eps, out, variant, splits, workspace)


def rmsnorm(x, g, eps: float, out=None):
    """Xn = RMSNorm(x; g, eps), written to memory (first kernel of the unfused program)."""
    _check_operands([x, g], ["x", "g"])
    if x.dim() != 2 or g.dim() != 1 or g.shape[0] != x.shape[1]:
        raise ValueError("expected x: [M, K], g: [K]")
    M, K = x.shape
    if out is None:
        out = torch.empty_like(x)
    else:
        _check_operands([x, out], ["x", "out"])
        if tuple(out.shape) != (M, K):
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {(M, K)}")
    stream = torch.cuda.current_stream(x.device).cuda_stream
    _binding.check(load_library().rmm_rmsnorm(x.data_ptr(), g.data_ptr(), out.data_ptr(),
                                              float(eps), M, K, _DTYPES[x.dtype], stream))
    return out


def _plain(x, w1, w3, out, workspace):
    gated = w3 is not None
    tensors = [x, w1] + ([w3] if gated else [])
    _check_operands(tensors, ["x", "w1", "w3"] if gated else ["x", "w"])
    if x.dim() != 2 or w1.dim() != 2 or w1.shape[0] != x.shape[1] or \
            (gated and tuple(w3.shape) != tuple(w1.shape)):
        raise ValueError("expected x: [M, K], w: [K, N]")
    M, K = x.shape
    N = w1.shape[1]
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    else:
        _check_operands([x, out], ["x", "out"])
        if tuple(out.shape) != (M, N):
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {(M, N)}")
    lib = load_library()
    dtype = _DTYPES[x.dtype]
    stream = torch.cuda.current_stream(x.device).cuda_stream
    need = _binding.workspace_bytes(dtype, M, N, K, gated)
    if workspace is None and need > 0:
        workspace = _workspace_for(x.device, stream, need)
    ws_ptr = workspace.ptr if workspace is not None else None
    ws_bytes = workspace.nbytes if workspace is not None else 0
    if gated:
        st = lib.rmm_gated_matmul(x.data_ptr(), w1.data_ptr(), w3.data_ptr(), out.data_ptr(), M, N,
                                  K, dtype, ws_ptr, ws_bytes, stream)
    else:
        st = lib.rmm_matmul(x.data_ptr(), w1.data_ptr(), out.data_ptr(), M, N, K, dtype, ws_ptr,
                            ws_bytes, stream)
    _binding.check(st)
    return out


def matmul(x, w, out=None, workspace: Workspace | None = None):
    """Y = x @ w with the same kernels, no norm (second kernel of the unfused program)."""
    return _plain(x, w, None, out, workspace)


def gated_matmul(x, w1, w3, out=None, workspace: Workspace | None = None):
    """Y = silu(x @ w1) * (x @ w3) with the same kernels, no norm."""
    return _plain(x, w1, w3, out, workspace)


def _lora(x, g, w, a, b, eps, out, variant, splits, workspace, norm):
    tensors = [x, w, a, b] + ([g] if norm else [])
    _check_operands(tensors, ["x", "w", "a", "b", "g"][:len(tensors)])
    if x.dim() != 2 or w.dim() != 2 or a.dim() != 2 or b.dim() != 2 or (norm and g.dim() != 1):
        raise ValueError("expected x: [M, K], g: [K], w: [K, N], a: [R, K], b: [R, N]")
    M, K = x.shape
    N = w.shape[1]
    R = a.shape[0]
    if w.shape[0] != K or tuple(a.shape) != (R, K) or tuple(b.shape) != (R, N) or \
            (norm and g.shape[0] != K):
        raise ValueError(f"shape mismatch: x {tuple(x.shape)}, w {tuple(w.shape)}, "
                         f"a {tuple(a.shape)}, b {tuple(b.shape)}")
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    else:
        _check_operands([x, out], ["x", "out"])
        if tuple(out.shape) != (M, N):
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {(M, N)}")
    lib = load_library()
    dtype = _DTYPES[x.dtype]
    stream = torch.cuda.current_stream(x.device).cuda_stream
    need = _binding.lora_workspace_bytes(dtype, M, N, K, R, variant, splits)
    if workspace is None and need > 0:
        workspace = _workspace_for(x.device, stream, need)
    ws_ptr = workspace.ptr if workspace is not None else None
    ws_bytes = workspace.nbytes if workspace is not None else 0
    if norm:
        st = lib.rmsnorm_lora_ex(x.data_ptr(), g.data_ptr(), w.data_ptr(), a.data_ptr(),
                                 b.data_ptr(), out.data_ptr(), float(eps), M, N, K, R, dtype,
                                 _binding.VARIANTS[variant], splits, ws_ptr, ws_bytes, stream)
    else:
        if variant != "auto" or splits != 0:
            raise ValueError("lora_matmul takes no variant or split count")
        st = lib.rmm_lora_matmul(x.data_ptr(), w.data_ptr(), a.data_ptr(), b.data_ptr(),
                                 out.data_ptr(), M, N, K, R, dtype, ws_ptr, ws_bytes, stream)
    _binding.check(st)
    return out


def rmsnorm_lora(x, g, w, a, b, eps: float, out=None, variant: str = "auto", splits: int = 0,
                 workspace: Workspace | None = None):
    """Y = norm(x) @ w + (norm(x) @ a.T) @ b, fused; a: [R, K], b: [R, N], 1 <= R <= 64."""
    return _lora(x, g, w, a, b, eps, out, variant, splits, workspace, True)


def lora_matmul(x, w, a, b, out=None, workspace: Workspace | None = None):
    """Y = x @ w + (x @ a.T) @ b with the same kernels, no norm."""
    return _lora(x, None, w, a, b, 0.0, out, "auto", 0, workspace, False)


def plan_lora(M, N, K, R, dtype=torch.bfloat16, variant="auto", splits=0, with_workspace=True):
    """Which variant and split count an adapter call of this shape would run (host only)."""
    base = 1 << 40
    span = 1 << 36
    ptrs = [base + i * span for i in range(7)]
    d = _DTYPES[dtype]
    ws = ptrs[6] if with_workspace else None
    nb = _binding.lora_workspace_bytes(d, M, N, K, R, variant, splits) if with_workspace else 0
    return _binding.plan_lora(ptrs[0], ptrs[1], ptrs[2], ptrs[3], ptrs[4], ptrs[5], 1e-6, M, N, K,
                              R, d, variant, splits, ws, nb)


def qknorm_attention(q, k, v, gq, gk, eps: float, out=None, splits: int = 0,
                     workspace: Workspace | None = None):
    """o = softmax(norm(q) . norm(k)^T / sqrt(D)) v per batch-head, fused (bf16;
    q: [BH, D], k, v: [BH, S, D], gq, gk: [D], D = 64 or 128)."""
    _check_operands([q, k, v, gq, gk], ["q", "k", "v", "gq", "gk"])
    if q.dim() != 2 or k.dim() != 3 or gq.dim() != 1 or gk.dim() != 1:
        raise ValueError("expected q: [BH, D], k, v: [BH, S, D], gq, gk: [D]")
    BH, D = q.shape
    S = k.shape[1]
    if tuple(k.shape) != (BH, S, D) or tuple(v.shape) != (BH, S, D) or gq.shape[0] != D or \
            gk.shape[0] != D:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, "
                         f"v {tuple(v.shape)}")
    if out is None:
        out = torch.empty((BH, D), dtype=q.dtype, device=q.device)
    else:
        _check_operands([q, out], ["q", "out"])
        if tuple(out.shape) != (BH, D):
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {(BH, D)}")
    dtype = _DTYPES[q.dtype]
    stream = torch.cuda.current_stream(q.device).cuda_stream
    need = _binding.attention_workspace_bytes(dtype, BH, S, D, splits)
    if workspace is None and (need > 0 or splits > 1):  # a forced count needs one
        workspace = _workspace_for(q.device, stream, max(need, 256))
    ws_ptr = workspace.ptr if workspace is not None else None
    ws_bytes = workspace.nbytes if workspace is not None else 0
    _binding.check(load_library().qknorm_attention_ex(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), gq.data_ptr(), gk.data_ptr(), out.data_ptr(),
        float(eps), BH, S, D, dtype, splits, ws_ptr, ws_bytes, stream))
    return out


def qknorm_attention_gqa(q, k, v, gq, gk, eps: float, out=None, splits: int = 0,
                         workspace: Workspace | None = None):
    """Grouped-query QKNorm + attention (bf16): q: [BH * G, D] with query row
    h * G + g attending to key/value head h; k, v: [BH, S, D]; G = 1 .. 16."""
    _check_operands([q, k, v, gq, gk], ["q", "k", "v", "gq", "gk"])
    if q.dim() != 2 or k.dim() != 3 or gq.dim() != 1 or gk.dim() != 1:
        raise ValueError("expected q: [BH * G, D], k, v: [BH, S, D], gq, gk: [D]")
    BH, S, D = k.shape
    if BH == 0 or q.shape[0] % BH != 0:
        raise ValueError(f"q has {q.shape[0]} rows, not a multiple of {BH} key heads")
    G = q.shape[0] // BH
    if q.shape[1] != D or tuple(v.shape) != (BH, S, D) or gq.shape[0] != D or gk.shape[0] != D:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, "
                         f"v {tuple(v.shape)}")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_operands([q, out], ["q", "out"])
        if tuple(out.shape) != tuple(q.shape):
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {tuple(q.shape)}")
    dtype = _DTYPES[q.dtype]
    stream = torch.cuda.current_stream(q.device).cuda_stream
    lib = load_library()
    need = _binding.attention_gqa_workspace_bytes(dtype, BH, G, S, D, splits)
    if workspace is None and (need > 0 or splits > 1):  # a forced count needs one
        workspace = _workspace_for(q.device, stream, max(need, 256))
    ws_ptr = workspace.ptr if workspace is not None else None
    ws_bytes = workspace.nbytes if workspace is not None else 0
    _binding.check(lib.qknorm_attention_gqa(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), gq.data_ptr(), gk.data_ptr(), out.data_ptr(),
        float(eps), BH, G, S, D, dtype, splits, ws_ptr, ws_bytes, stream))
    return out


def qknorm_attention_prefill(q, k, v, gq, gk, eps: float, causal: bool = True, out=None,
                             splits: int = 0, workspace: Workspace | None = None):
    """QKNorm + attention for many queries per head (bf16): q: [BH * G, Sq, D]
    (query head h * G + g reads key/value head h), k, v: [BH, Skv, D]; causal:
    query position i sees keys 0 .. i + Skv - Sq.  splits: spans of the keys
    combined by a second kernel (0: the library's choice, 1: none)."""
    _check_operands([q, k, v, gq, gk], ["q", "k", "v", "gq", "gk"])
    if q.dim() != 3 or k.dim() != 3 or gq.dim() != 1 or gk.dim() != 1:
        raise ValueError("expected q: [BH * G, Sq, D], k, v: [BH, Skv, D], gq, gk: [D]")
    BH, Skv, D = k.shape
    BHq, Sq = q.shape[0], q.shape[1]
    if BH == 0 or BHq % BH != 0:
        raise ValueError(f"q has {BHq} heads, not a multiple of {BH} key heads")
    if q.shape[2] != D or tuple(v.shape) != (BH, Skv, D) or gq.shape[0] != D or \
            gk.shape[0] != D:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, "
                         f"v {tuple(v.shape)}")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_operands([q, out], ["q", "out"])
        if tuple(out.shape) != tuple(q.shape):
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {tuple(q.shape)}")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    lib = load_library()
    G = BHq // BH
    need = lib.rmm_attention_prefill_workspace_bytes(BH, G, Sq, Skv, D, int(bool(causal)), splits)
    if workspace is None and (need > 0 or splits > 1):  # a forced count needs one
        workspace = _workspace_for(q.device, stream, max(need, 256))
    ws_ptr = workspace.ptr if workspace is not None else None
    ws_bytes = workspace.nbytes if workspace is not None else 0
    _binding.check(lib.qknorm_attention_prefill_ex(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), gq.data_ptr(), gk.data_ptr(), out.data_ptr(),
        float(eps), BH, G, Sq, Skv, D, int(bool(causal)), _DTYPES[q.dtype], splits, ws_ptr,
        ws_bytes, stream))
    return out


def attention(q, k, v, out=None, workspace: Workspace | None = None):
    """o = softmax(q . k^T / sqrt(D)) v per batch-head, the attention step alone
    (q and k already normalised; bf16; q: [BH, D], k, v: [BH, S, D], D = 64 or 128)."""
    _check_operands([q, k, v], ["q", "k", "v"])
    if q.dim() != 2 or k.dim() != 3:
        raise ValueError("expected q: [BH, D], k, v: [BH, S, D]")
    BH, D = q.shape
    S = k.shape[1]
    if tuple(k.shape) != (BH, S, D) or tuple(v.shape) != (BH, S, D):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, "
                         f"v {tuple(v.shape)}")
    if out is None:
        out = torch.empty((BH, D), dtype=q.dtype, device=q.device)
    else:
        _check_operands([q, out], ["q", "out"])
        if tuple(out.shape) != (BH, D):
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {(BH, D)}")
    dtype = _DTYPES[q.dtype]
    stream = torch.cuda.current_stream(q.device).cuda_stream
    need = _binding.attention_workspace_bytes(dtype, BH, S, D, 0)
    if workspace is None and need > 0:
        workspace = _workspace_for(q.device, stream, need)
    ws_ptr = workspace.ptr if workspace is not None else None
    ws_bytes = workspace.nbytes if workspace is not None else 0
    _binding.check(load_library().rmm_attention(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), BH, S, D, dtype, ws_ptr,
        ws_bytes, stream))
    return out


def rmsnorm_matmul_chain(x0, g, w, eps: float, out=None, workspace: Workspace | None = None,
                         check_wait: bool = True):
    """L fused layers in one persistent launch, x_{l+1} = RMSNorm(x_l; g[l], eps) @ w[l]
    (bf16; x0: [M, K], g: [L, K], w: [L, K, K], M <= 16).  Returns every layer's
    output, [L, M, K] (out[l] = x_{l+1}).

    With check_wait (the default) the call synchronises the stream and reads
    the workspace's flag word: if a layer wait gave up (a workgroup of the
    grid was not resident, so the outputs are wrong) it clears the flag and
    raises RmmError.  Pass check_wait=False inside HIP graph capture or to
    keep the call asynchronous, and read chain_wait_flag() yourself."""
    _check_operands([x0, g, w], ["x0", "g", "w"])
    if x0.dim() != 2 or g.dim() != 2 or w.dim() != 3:
        raise ValueError("expected x0: [M, K], g: [L, K], w: [L, K, K]")
    M, K = x0.shape
    L = g.shape[0]
    if tuple(g.shape) != (L, K) or tuple(w.shape) != (L, K, K):
        raise ValueError(f"shape mismatch: x0 {tuple(x0.shape)}, g {tuple(g.shape)}, "
                         f"w {tuple(w.shape)}")
    if out is None:
        out = torch.empty((L, M, K), dtype=x0.dtype, device=x0.device)
    else:
        _check_operands([x0, out], ["x0", "out"])
        if tuple(out.shape) != (L, M, K):
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {(L, M, K)}")
    stream = torch.cuda.current_stream(x0.device).cuda_stream
    need = _binding.chain_workspace_bytes(M, K, L)
    if workspace is None and need > 0:
        workspace = _workspace_for(x0.device, stream, need)
    ws_ptr = workspace.ptr if workspace is not None else None
    ws_bytes = workspace.nbytes if workspace is not None else 0
    _binding.check(load_library().rmsnorm_matmul_chain(
        x0.data_ptr(), g.data_ptr(), w.data_ptr(), out.data_ptr(), float(eps), M, K, L,
        _DTYPES[x0.dtype], ws_ptr, ws_bytes, stream))
    if check_wait and workspace is not None:
        torch.cuda.current_stream(x0.device).synchronize()
        if chain_wait_flag(workspace, M, K, L):
            off = _binding.chain_flag_offset(M, K, L)
            workspace.tensor[off:off + 4].zero_()
            raise RmmError(_binding.STATUS_CHAIN_WAIT,
                           "rmsnorm_matmul_chain: a layer wait gave up (the grid was not "
                           "resident on the GPU); the outputs of this call are wrong")
    return out


def chain_wait_flag(workspace: Workspace, M: int, K: int, L: int) -> int:
    """The chain workspace's flag word (nonzero if a layer wait ever gave up)."""
    off = _binding.chain_flag_offset(M, K, L)
    return int(workspace.tensor[off:off + 4].view(torch.int32).item())


def plan_attention(BH, S, D, splits=0, with_workspace=True, G=1):
    """Chunks per key/value head and keys per chunk an attention call would run
    (host only); G query heads per key/value head."""
    base = 1 << 40
    span = 1 << 36
    ptrs = [base + i * span for i in range(7)]
    d = _binding.DTYPE_BF16
    ws = ptrs[6] if with_workspace else None
    nb = (_binding.attention_gqa_workspace_bytes(d, BH, G, S, D, splits)
          if with_workspace else 0)
    return _binding.plan_attention(ptrs[0], ptrs[1], ptrs[2], ptrs[3], ptrs[4], ptrs[5], 1e-6, BH,
                                   S, D, d, splits, ws, nb, G=G)


def plan(M, N, K, dtype=torch.bfloat16, gated=False, variant="auto", splits=0,
         with_workspace=True):
    """Which variant and split count a call of this shape would run (host only)."""
    # Distinct, 16-byte aligned stand-in addresses; rmm_plan never dereferences them.
    base = 1 << 40
    span = 1 << 36
    ptrs = [base + i * span for i in range(6)]
    d = _DTYPES[dtype]
    ws = ptrs[5] if with_workspace else None
    nb = _binding.workspace_bytes(d, M, N, K, gated, variant, splits) if with_workspace else 0
    return _binding.plan(ptrs[0], ptrs[1], ptrs[2], ptrs[3] if gated else None, ptrs[4], 1e-6,
                         M, N, K, d, gated, variant, splits, ws, nb)
