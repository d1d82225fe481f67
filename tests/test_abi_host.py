"""The C ABI on the host: the library loads, exports every symbol the header
declares, validates arguments in the documented order and plans variants --
all without touching a GPU (every call here fails validation or is empty,
so no HIP call is made)."""
import ctypes
import os
import re
import subprocess

import pytest

import tensor_program_amd as tpa
from tensor_program_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rmm.h")

OK, NULL, SHAPE, EPS, DTYPE, ALIAS, WORKSPACE, HIP, VARIANT = range(9)
BF16, F32 = _binding.DTYPE_BF16, _binding.DTYPE_F32
# Every workspace starts with a 64 KiB region holding the arrival counters.
CNT = 64 * 1024
# Fake, distinct, 16-byte aligned device addresses: never dereferenced here.
A = [(1 << 40) + i * (1 << 34) for i in range(8)]


@pytest.fixture(scope="module")
def lib():
    return tpa.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined"})


def test_header_symbols_exported(lib):
    names = declared_functions()
    assert set(names) == set(_binding.SYMBOLS), names
    out = subprocess.run(["nm", "-D", "--defined-only", _binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for n in names:
        assert n in exported, n
        getattr(lib, n)


def test_abi_version(lib):
    assert lib.rmm_abi_version() == 1


def call(lib, X=A[0], g=A[1], W=A[2], Y=A[3], eps=1e-6, M=16, N=64, K=64, dtype=BF16,
         variant=0, splits=0, ws=None, ws_bytes=0):
    return lib.rmsnorm_matmul_ex(X, g, W, Y, eps, M, N, K, dtype, variant, splits, ws, ws_bytes,
                                 None)


def call_gated(lib, W3=A[4], **kw):
    kw.setdefault("X", A[0])
    return lib.rmsnorm_gated_mlp_ex(kw.get("X"), A[1], A[2], W3, A[3], kw.get("eps", 1e-6),
                                    16, 64, 64, BF16, 0, 0, None, 0, None)


def test_validation_order(lib):
    assert call(lib, X=None) == NULL
    assert call(lib, Y=None) == NULL
    assert call_gated(lib, W3=None) == NULL
    assert call(lib, X=None, K=0) == NULL           # NULL is checked first
    assert call(lib, K=0) == SHAPE
    assert call(lib, M=-1) == SHAPE
    assert call(lib, N=-3) == SHAPE
    assert call(lib, M=1 << 62, K=1 << 4) == SHAPE  # element count overflow
    assert call(lib, K=0, eps=-1.0) == SHAPE        # shape before eps
    assert call(lib, eps=-1e-6) == EPS
    assert call(lib, eps=float("nan")) == EPS
    assert call(lib, eps=float("inf")) == EPS
    assert call(lib, eps=-1.0, dtype=7) == EPS      # eps before dtype
    assert call(lib, dtype=7) == DTYPE
    assert call(lib, Y=A[0] + 16) == ALIAS           # Y inside X
    assert call(lib, Y=A[2] - 8) == ALIAS            # Y overlapping the start of W
    assert call(lib, ws=A[3] + 64, ws_bytes=1 << 20) == ALIAS
    assert call(lib, variant=9) == VARIANT
    assert call(lib, variant=4, splits=2) == VARIANT  # splits only for decode
    assert call(lib, variant=4, dtype=F32) == VARIANT  # stream is bf16 only
    assert call(lib, variant=1, splits=2) == VARIANT  # splits only for decode
    assert call(lib, variant=2, dtype=F32, M=33) == VARIANT  # fp32 decode: M <= 32
    assert call(lib, variant=2, dtype=F32, X=A[0] + 4) == VARIANT  # fp32 decode: aligned
    assert call(lib, variant=2, M=33) == VARIANT
    assert call(lib, variant=2, N=60) == VARIANT      # N % 8 != 0
    assert call(lib, variant=2, X=A[0] + 2) == VARIANT  # unaligned
    assert call(lib, variant=2, splits=2) == VARIANT   # K=64: one 128-deep granule
    assert call(lib, variant=2, K=4096, N=6144, splits=8) == WORKSPACE  # needs a workspace
    need = lib.rmm_workspace_bytes_ex(BF16, 16, 6144, 4096, 0, 2, 8)
    assert need > 0
    assert call(lib, variant=2, K=4096, N=6144, splits=8, ws=A[6], ws_bytes=need - 1) == WORKSPACE
    # a workspace must be 16-byte aligned (its partial sums move 16 bytes at a time)
    assert call(lib, variant=2, K=4096, N=6144, splits=8, ws=A[6] + 8, ws_bytes=need) == WORKSPACE


def test_unfused_entry_points_validate(lib):
    # rmm_rmsnorm: NULL, SHAPE, EPS, DTYPE, ALIAS, in that order.
    def norm(X=A[0], g=A[1], Xn=A[3], eps=1e-6, M=16, K=64, dtype=BF16):
        return lib.rmm_rmsnorm(X, g, Xn, eps, M, K, dtype, None)
    assert norm(X=None) == NULL
    assert norm(Xn=None, K=0) == NULL
    assert norm(K=0) == SHAPE
    assert norm(M=-1) == SHAPE
    assert norm(M=1 << 62, K=1 << 4) == SHAPE
    assert norm(K=0, eps=-1.0) == SHAPE
    assert norm(eps=-1.0) == EPS
    assert norm(eps=float("nan"), dtype=7) == EPS
    assert norm(dtype=7) == DTYPE
    assert norm(Xn=A[0]) == ALIAS                     # in place is not allowed
    assert norm(Xn=A[1] - 8) == ALIAS                 # overlapping g
    assert norm(X=None, g=None, Xn=None, M=0) == OK   # empty: nothing launched
    # rmm_matmul / rmm_gated_matmul: the fused calls' rules, no eps.
    def mm(X=A[0], W=A[2], Y=A[3], M=16, N=64, K=64, dtype=BF16, ws=None, ws_bytes=0):
        return lib.rmm_matmul(X, W, Y, M, N, K, dtype, ws, ws_bytes, None)
    assert mm(X=None) == NULL
    assert mm(W=None) == NULL
    assert mm(K=0) == SHAPE
    assert mm(dtype=7) == DTYPE
    assert mm(Y=A[0] + 16) == ALIAS
    assert mm(Y=A[2] + 32) == ALIAS
    assert mm(X=None, W=None, Y=None, N=0) == OK
    assert lib.rmm_gated_matmul(A[0], A[2], None, A[3], 16, 64, 64, BF16, None, 0, None) == NULL
    assert lib.rmm_gated_matmul(A[0], A[2], A[4], A[4] + 8, 16, 64, 64, BF16, None, 0, None) == ALIAS


def test_lora_entry_points_validate(lib):
    # rmsnorm_lora: NULL (A, B too), SHAPE (rank 1..64), EPS, DTYPE, ALIAS
    # (Y against A and B as well), VARIANT, WORKSPACE, in that order.
    def lo(X=A[0], g=A[1], W=A[2], LA=A[5], LB=A[6], Y=A[3], eps=1e-6, M=16, N=64, K=64, R=16,
           dtype=BF16, variant=0, splits=0, ws=None, ws_bytes=0):
        return lib.rmsnorm_lora_ex(X, g, W, LA, LB, Y, eps, M, N, K, R, dtype, variant, splits,
                                   ws, ws_bytes, None)
    assert lo(LA=None) == NULL
    assert lo(LB=None, R=0) == NULL
    assert lo(R=0) == SHAPE
    assert lo(R=65) == SHAPE
    assert lo(R=-1, eps=-1.0) == SHAPE
    assert lo(eps=float("inf"), R=0) == SHAPE
    assert lo(eps=-1.0, dtype=7) == EPS
    assert lo(dtype=7, Y=A[5]) == DTYPE
    assert lo(Y=A[5] + 16) == ALIAS                 # Y overlapping A
    assert lo(Y=A[6] - 64) == ALIAS                 # Y overlapping B
    assert lo(variant=3) == WORKSPACE               # the adapter tile keeps T in the workspace
    # (a call that validates would launch: only the host-only plan takes these)
    assert _binding.plan_lora(A[0], A[1], A[2], A[5], A[6], A[3], 1e-6, 16, 64, 64, 16, BF16,
                              "prefill", 0, A[7], 1 << 30) == (OK, "prefill", 1)
    assert lo(variant=3, splits=2, ws=A[7], ws_bytes=1 << 30) == VARIANT   # no split with T
    assert lo(variant=3, ws=A[7], ws_bytes=1000) == WORKSPACE
    assert lo(variant=4) == VARIANT
    assert lo(M=129, variant=2) == VARIANT          # decode with the adapter: M <= 128 (32-row launches)
    assert lo(R=33, variant=2) == VARIANT           # decode: R <= 32
    assert lo(K=256, variant=2, splits=2) == WORKSPACE  # forced split count, no workspace
    assert lo(X=None, g=None, W=None, LA=None, LB=None, Y=None, M=0) == OK
    # rmm_lora_matmul: the same rules without eps and gain.
    assert lib.rmm_lora_matmul(A[0], A[2], None, A[6], A[3], 16, 64, 64, 16, BF16, None, 0,
                               None) == NULL
    assert lib.rmm_lora_matmul(A[0], A[2], A[5], A[6], A[3], 16, 64, 64, 0, BF16, None, 0,
                               None) == SHAPE
    assert lib.rmm_lora_matmul(A[0], A[2], A[5], A[6], A[6], 16, 64, 64, 16, BF16, None, 0,
                               None) == ALIAS


def test_lora_plans():
    import torch
    assert tpa.plan_lora(16, 6144, 4096, 16)[1:] == ("decode", 4)
    assert tpa.plan_lora(16, 6144, 4096, 32)[1:] == ("decode", 4)
    assert tpa.plan_lora(16, 6144, 4096, 1)[1] == "decode"
    assert tpa.plan_lora(32, 6144, 4096, 16)[1] == "decode"
    assert tpa.plan_lora(16, 6144, 4096, 33)[1] == "prefill"   # decode carries R <= 32
    assert tpa.plan_lora(16, 6144, 4096, 64)[1] == "prefill"
    assert tpa.plan_lora(16, 6144, 4096, 64, with_workspace=False)[1] == "generic"
    assert tpa.plan_lora(33, 6144, 4096, 16)[1] == "decode"    # 32-row launches
    assert tpa.plan_lora(64, 6144, 4096, 16)[1] == "decode"
    # above 64 rows with a workspace the prefill tile with K split into
    # ranges (128 x 6144 x 4096: 47 us against 85 us for four 32-row decode
    # launches); without one, decode up to 128 rows
    assert tpa.plan_lora(65, 6144, 4096, 16)[1] == "prefill"
    assert tpa.plan_lora(128, 6144, 4096, 16, with_workspace=False)[1:] == ("decode", 1)
    assert tpa.plan_lora(129, 6144, 4096, 16)[1:] == ("prefill", 5)
    assert tpa.plan_lora(1000, 6144, 4096, 16)[1:] == ("prefill", 1)   # 192 tiles: no split
    assert tpa.plan_lora(4096, 4096, 4096, 16)[1] == "prefill"
    assert tpa.plan_lora(4096, 4096, 4096, 16, with_workspace=False)[1] == "generic"
    assert tpa.plan_lora(4096, 4100, 4096, 16)[1] == "generic"    # N % 8 != 0
    assert tpa.plan_lora(8, 1024, 1024, 16, dtype=torch.float32)[1] == "generic"
    assert tpa.plan_lora(16, 6144, 4096, 16, with_workspace=False)[1:] == ("decode", 1)
    assert tpa.plan_lora(16, 6144, 4096, 16, variant="decode", splits=3)[1:] == ("decode", 3)
    assert tpa.plan_lora(16, 6144, 4096, 16, variant="prefill")[1] == "prefill"
    assert tpa.plan_lora(16, 6144, 4096, 16, variant="prefill", with_workspace=False)[0] == \
        WORKSPACE
    assert tpa.plan_lora(16, 6144, 4096, 16, variant="prefill", splits=2)[1:] == ("prefill", 2)
    assert tpa.plan_lora(16, 6144, 4096, 16, variant="prefill", splits=2,
                         with_workspace=False)[0] == WORKSPACE
    assert tpa.plan_lora(16, 6144, 4096, 16, variant="prefill", splits=65)[0] == VARIANT
    assert tpa.plan_lora(16, 6144, 4096, 65)[0] == SHAPE


def test_lora_workspace_sizes(lib):
    plain = lib.rmm_workspace_bytes(BF16, 16, 6144, 4096, 0)
    lora16 = lib.rmm_lora_workspace_bytes(BF16, 16, 6144, 4096, 16, 0, 0)
    lora32 = lib.rmm_lora_workspace_bytes(BF16, 16, 6144, 4096, 32, 0, 0)
    assert plain < lora16 < lora32   # the down-projection partials ride along
    # 4 splits x 48 tiles x (8 + 1) blocks of 16 x 16 fp32 beyond the plain partials' 8
    assert lora16 - plain == 4 * 48 * 1 * 256 * 4
    # R = 48: the prefill tile (decode carries R <= 32): T, 16 rows x 48 ranks
    # (3072 bytes, a multiple of 256), then the split's partial sums and row
    # sums of squares, S x (16 x 6144 + 16) fp32
    S = tpa.plan_lora(16, 6144, 4096, 48)[2]
    assert S > 1
    want = 65536 + 16 * 48 * 4 + S * (16 * 6144 + 16) * 4
    assert lib.rmm_lora_workspace_bytes(BF16, 16, 6144, 4096, 48, 0, 0) == want
    assert lib.rmm_lora_workspace_bytes(BF16, 16, 6144, 4096, 40, 0, 0) == want
    # unsplit: T alone
    assert lib.rmm_lora_workspace_bytes(BF16, 16, 6144, 4096, 48, 3, 1) == 65536 + 16 * 48 * 4
    # T not a multiple of 256 bytes: the partial sums start at the next one
    assert lib.rmm_lora_workspace_bytes(BF16, 3, 6144, 4096, 16, 3, 2) == \
        65536 + 256 + 2 * (3 * 6144 + 3) * 4
    assert lib.rmm_lora_workspace_bytes(F32, 16, 6144, 4096, 48, 0, 0) == 0   # generic: none
    assert lib.rmm_lora_workspace_bytes(BF16, 16, 6144, 4096, 0, 0, 0) == 0   # invalid rank
    assert lib.rmm_lora_workspace_bytes(BF16, 16, 6144, 4096, 16, 2, 1) == 0


def test_attention_entry_points_validate(lib):
    # qknorm_attention_ex: NULL, SHAPE, EPS, DTYPE, ALIAS, VARIANT, WORKSPACE.
    def at(Q=A[0], K=A[1], V=A[2], gq=A[3], gk=A[4], O=A[5], eps=1e-6, BH=16, S=512, D=128,
           dtype=BF16, splits=0, ws=None, ws_bytes=0):
        return lib.qknorm_attention_ex(Q, K, V, gq, gk, O, eps, BH, S, D, dtype, splits, ws,
                                       ws_bytes, None)
    assert at(V=None) == NULL
    assert at(gk=None, D=96) == NULL
    assert at(D=96) == SHAPE
    assert at(S=0) == SHAPE
    assert at(BH=-1) == SHAPE
    assert at(BH=1 << 40, S=1 << 20) == SHAPE          # element count overflows
    assert at(eps=float("nan")) == EPS
    assert at(eps=-1.0, dtype=F32) == EPS
    assert at(dtype=F32) == DTYPE                        # bf16 only
    assert at(O=A[1] + 256) == ALIAS                     # O inside K
    assert at(O=A[3] - 16) == ALIAS                      # O overlapping gq
    assert at(O=A[0] + 2) == ALIAS
    assert at(Q=A[0] + 8) == VARIANT                     # not 16-byte aligned
    assert at(S=1 << 23) == VARIANT                      # one head's keys need 32-bit offsets
    assert at(splits=513) == VARIANT                     # more chunks than keys
    assert at(splits=2) == WORKSPACE                     # forced chunks without a workspace
    assert at(splits=2, ws=A[6], ws_bytes=16) == WORKSPACE
    assert at(splits=2, ws=A[6] + 4, ws_bytes=1 << 24) == WORKSPACE   # not 16-byte aligned
    assert at(Q=None, K=None, V=None, gq=None, gk=None, O=None, BH=0) == OK


def test_attention_plans(lib):
    assert tpa.plan_attention(256, 2048, 128) == (0, 1, 2048)   # one workgroup per CU
    assert tpa.plan_attention(256, 2048, 128, with_workspace=False) == (0, 1, 2048)
    assert tpa.plan_attention(16, 4096, 128) == (0, 16, 256)    # 256 workgroups
    assert tpa.plan_attention(16, 4096, 128, splits=3) == (0, 3, 1408)
    assert tpa.plan_attention(4, 5, 64) == (0, 1, 128)          # chunks are whole 128-key rounds
    assert tpa.plan_attention(1, 1, 128) == (0, 1, 64)
    assert tpa.plan_attention(1, 100000, 64)[1] > 1
    assert lib.rmm_attention_workspace_bytes(BF16, 256, 2048, 128, 0) == 0
    nb = lib.rmm_attention_workspace_bytes(BF16, 256, 2048, 128, 4)
    assert nb == CNT + 256 * 4 * 130 * 4                  # counters, then (o, max, sum)
    assert lib.rmm_attention_workspace_bytes(BF16, 256, 2048, 128, 1) == 0
    assert lib.rmm_attention_workspace_bytes(F32, 256, 2048, 128, 0) == 0


def test_empty_shapes_are_noops(lib):
    # M == 0 or N == 0: RMM_OK, nothing launched (NULL pointers allowed).
    assert call(lib, X=None, g=None, W=None, Y=None, M=0) == OK
    assert call(lib, X=None, g=None, W=None, Y=None, N=0) == OK


def test_empty_shapes_plan_without_work(lib):
    # Regression: sizing an empty call used to divide by the (zero) tile count.
    for (M, N) in ((0, 6144), (16, 0), (0, 0)):
        assert lib.rmm_workspace_bytes(BF16, M, N, 4096, 0) == 0
        assert lib.rmm_workspace_bytes_ex(BF16, M, N, 4096, 1, 2, 0) == 0
        assert tpa.plan(M, N, 4096)[0] == OK


def test_status_strings(lib):
    for s in range(9):
        assert _binding.status_string(s).startswith("RMM_")
    assert "unknown" in _binding.status_string(99)


def test_variant_selection():
    import torch
    assert tpa.plan(16, 6144, 4096)[1:] == ("decode", 4)   # 48 tiles x 4 = 192 workgroups
    assert tpa.plan(16, 1024, 4096)[1:] == ("decode", 32)  # 8 tiles: 32 granules of 128
    assert tpa.plan(16, 32768, 4096)[1:] == ("decode", 1)  # 256 tiles already fill the CUs
    assert tpa.plan(16, 6144, 4096, with_workspace=False)[1:] == ("decode", 1)
    assert tpa.plan(64, 14336, 4096, gated=True)[1] == "stream"
    # gated, M <= 16: decode with a workspace (16 x 4096 x 14336: 45.9 vs 47.3 us), else stream
    assert tpa.plan(16, 14336, 4096, gated=True)[1] == "decode"
    assert tpa.plan(16, 14336, 4096, gated=True, with_workspace=False)[1] == "stream"
    assert tpa.plan(17, 14336, 4096, gated=True)[1] == "stream"
    # gated above 64 rows with a workspace: the 128-row tile with K split into
    # ranges (128 x 14336 x 4096: 75 us against 98 us for two 64-row stream
    # launches); without one, stream launches up to 128 rows
    assert tpa.plan(65, 14336, 4096, gated=True)[1:] == ("prefill", 2)
    assert tpa.plan(128, 14336, 4096, gated=True, with_workspace=False)[1] == "stream"
    assert tpa.plan(129, 14336, 4096, gated=True, with_workspace=False)[1:] == ("prefill", 1)
    assert tpa.plan(256, 4096, 4096, gated=True)[1:] == ("prefill", 4)
    assert tpa.plan(1024, 14336, 4096, gated=True)[1:] == ("prefill", 1)   # 896 tiles
    assert tpa.plan(129, 14336, 4100, gated=True)[1] == "generic"   # K % 8 != 0
    assert tpa.plan(48, 14336, 4096)[1] == "stream"
    # M <= 64 takes the stream kernel at any width (48 x 4096 x 4096: 21 us
    # against 107 us for the prefill tiles)
    assert tpa.plan(48, 2048, 4096)[1] == "stream"
    assert tpa.plan(129, 4104, 4096, variant="stream")[0] == VARIANT
    assert tpa.plan(257, 4096, 4096, variant="stream")[0] == VARIANT
    f32 = torch.float32
    assert tpa.plan(8, 1024, 1024, dtype=f32)[1:] == ("decode", 16)  # 8 tiles x 16 ranges of 64
    assert tpa.plan(8, 1024, 1024, dtype=f32, with_workspace=False)[1:] == ("decode", 1)
    assert tpa.plan(16, 64, 100, dtype=f32)[1:] == ("decode", 2)     # K ranges of >= 64 rows
    assert tpa.plan(32, 1024, 1024, dtype=f32)[1] == "decode"    # two 16-row launches
    assert tpa.plan(33, 1024, 1024, dtype=f32)[1] == "generic"
    assert tpa.plan(8, 1024, 1024, dtype=f32, gated=True)[1] == "generic"
    assert tpa.plan(8, 1024, 1024, dtype=f32, variant="decode", splits=5)[1:] == ("decode", 4)
    assert tpa.plan(4096, 4096, 4096)[1:] == ("prefill", 1)
    assert tpa.plan(8192, 28672, 8192)[1] == "prefill"
    assert tpa.plan(33, 520, 1000)[1] == "stream"
    # above 64 rows with a workspace: the prefill tile with K split into
    # ranges (256 x 4096 x 4096: 31 us against 89 us for four 64-row stream
    # launches); without one, 64-row stream launches up to 128 rows (256
    # when N <= 4096)
    assert tpa.plan(65, 520, 1000)[1] == "prefill"
    assert tpa.plan(65, 520, 1000, with_workspace=False)[1] == "stream"
    assert tpa.plan(129, 520, 1000, with_workspace=False)[1] == "stream"
    assert tpa.plan(257, 520, 1000, with_workspace=False)[1] == "prefill"
    assert tpa.plan(256, 4096, 4096)[1:] == ("prefill", 8)
    assert tpa.plan(129, 4096, 4096)[1:] == ("prefill", 11)
    assert tpa.plan(512, 14336, 4096)[1:] == ("prefill", 2)
    assert tpa.plan(1024, 14336, 4096)[1:] == ("prefill", 1)   # 224 tiles: no split
    assert tpa.plan(256, 4096, 4096, with_workspace=False)[1] == "stream"
    assert tpa.plan(512, 4096, 4096, with_workspace=False)[1:] == ("prefill", 1)
    # forced counts: whole, even ranges of 64-deep steps (K = 1000: 16 steps)
    assert tpa.plan(300, 264, 1000, variant="prefill", splits=5)[1:] == ("prefill", 4)
    assert tpa.plan(300, 264, 1000, variant="prefill", splits=3)[1:] == ("prefill", 3)
    assert tpa.plan(300, 264, 1000, variant="prefill", splits=16)[1:] == ("prefill", 8)
    assert tpa.plan(300, 264, 1000, variant="prefill", splits=17)[0] == VARIANT
    assert tpa.plan(300, 264, 1000, variant="prefill", splits=2,
                    with_workspace=False)[0] == WORKSPACE
    assert tpa.plan(300, 264, 1000, gated=True, variant="prefill", splits=5)[1:] == ("prefill", 4)
    assert tpa.plan(300, 264, 1000, gated=True, variant="prefill", splits=17)[0] == VARIANT
    assert tpa.plan(300, 264, 1000, variant="stream", splits=2)[0] == VARIANT
    assert tpa.plan(129, 4104, 1000)[1] == "prefill"
    assert tpa.plan(4096, 4096, 4095)[1] == "generic"   # K % 8 != 0
    assert tpa.plan(4096, 4096, 4096, variant="prefill", dtype=torch.float32)[0] == VARIANT
    assert tpa.plan(128, 256, 64, gated=True, variant="prefill")[1] == "prefill"
    assert tpa.plan(4096, 14336, 4096, gated=True)[1] == "prefill"
    assert tpa.plan(64, 14336, 4096, gated=True)[1] == "stream"
    assert tpa.plan(16, 6144, 4096, variant="decode", splits=3)[1:] == ("decode", 3)
    # split counts that do not divide K evenly are rounded to 128-deep chunks
    st, v, s = tpa.plan(17, 520, 1000, variant="decode", splits=4)
    assert (st, v, s) == (0, "decode", 4)
    st, v, s = tpa.plan(32, 1032, 1024, variant="decode", splits=5)
    assert (st, v, s) == (0, "decode", 4)


def test_workspace_sizes(lib):
    assert lib.rmm_workspace_bytes(BF16, 16, 6144, 4096, 0) == \
        lib.rmm_workspace_bytes_ex(BF16, 16, 6144, 4096, 0, 0, 0) > 0
    assert lib.rmm_workspace_bytes_ex(BF16, 16, 6144, 4096, 0, 2, 1) == 0
    # fp32 decode at 8 x 1024 x 1024: 32 tiles x 8 splits; the counter region,
    # 8-row sums of squares, 8 x 32 fp32 partials per tile and split
    # 16 K ranges x 8 tiles of 128 columns x 8 rows: sums of squares, then partials
    assert lib.rmm_workspace_bytes(F32, 8, 1024, 1024, 0) == \
        CNT + 16 * 8 * 8 * 4 + 16 * 8 * 8 * 128 * 4
    assert lib.rmm_workspace_bytes(F32, 8, 1024, 1024, 1) == 0   # gated fp32: generic kernel
    assert lib.rmm_workspace_bytes(BF16, 16, 6144, 0, 0) == 0  # invalid -> 0


def test_chain_validation_and_workspace(lib):
    def chain(X0=A[0], G=A[1], W=A[2], Xs=A[3], eps=1e-6, M=16, K=1024, L=4, dtype=BF16,
              ws=A[6], ws_bytes=1 << 30):
        return lib.rmsnorm_matmul_chain(X0, G, W, Xs, eps, M, K, L, dtype, ws, ws_bytes, None)
    assert chain(X0=None) == NULL
    assert chain(Xs=None, K=0) == NULL            # NULL before shape
    assert chain(K=0) == SHAPE
    assert chain(L=0) == SHAPE
    assert chain(M=-1) == SHAPE
    assert chain(K=1 << 40, L=1 << 30) == SHAPE   # element count overflow
    assert chain(eps=-1.0) == EPS
    assert chain(dtype=F32) == DTYPE              # bf16 only
    assert chain(Xs=A[0] + 64) == ALIAS           # output inside X0
    assert chain(Xs=A[6] - 64) == ALIAS           # output overlapping the workspace
    assert chain(M=17) == VARIANT
    assert chain(K=1000) == VARIANT               # K % 128 != 0
    assert chain(K=8192) == VARIANT               # 64 tiles x 4 chunks: not one workgroup per CU
    assert chain(X0=A[0] + 2) == VARIANT          # unaligned
    assert chain(ws=None) == WORKSPACE
    need = lib.rmm_chain_workspace_bytes(16, 1024, 4)
    assert need > 0 and chain(ws_bytes=need - 1) == WORKSPACE
    assert chain(ws=A[6] + 4) == WORKSPACE        # not 16-byte aligned
    assert chain(M=0, ws=None) == OK              # nothing to do, nothing launched
    # 8 tiles x 8 chunks of 128: the counter region (tile counters first, the
    # done + flag words in its last 256 bytes), 16-row sums, 8 x 64 floatx4 partials
    assert need == CNT + 8 * 8 * 16 * 4 + 8 * 8 * 8 * 64 * 16
    assert lib.rmm_chain_flag_offset(16, 1024, 4) == CNT - 256 + 4
    assert lib.rmm_chain_workspace_bytes(16, 8192, 4) == 0
    assert lib.rmm_chain_workspace_bytes(17, 1024, 4) == 0
    # The largest accepted tiling, K = 4480: 35 tiles x 7 chunks of 640.  The
    # 256-byte chain block (call-wide count, flag, one count per tile) holds
    # 2 + 35 words.
    need = lib.rmm_chain_workspace_bytes(16, 4480, 2)
    assert need == CNT + 15872 + 7 * 35 * 8 * 64 * 16  # row sums: 15,680 bytes, 256-aligned
    assert lib.rmm_chain_workspace_bytes(16, 4608, 2) == 0  # 36 tiles need 8 chunks: 288 workgroups


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(ImportError):
        _binding.load_library(str(tmp_path / "missing.so"))


def test_stream_split_workspace(lib):
    """The stream variant's split form: with at most 128 64-column strips
    (half the 256 workgroups) it needs a workspace (strip counters, then 2
    segments x 256 workgroups of fp32 sums per weight, then their row sums
    of squares); with more strips it needs none."""
    STREAM = 4
    # gated 64 x 4096 x 8192: 128 strips, two weights
    assert lib.rmm_workspace_bytes(BF16, 64, 8192, 4096, 1) == \
        CNT + 2 * 256 * 2 * 64 * 64 * 4 + 2 * 256 * 64 * 4
    # plain, forced stream, 96 strips: one weight
    assert lib.rmm_workspace_bytes_ex(BF16, 16, 6144, 4096, 0, STREAM, 0) == \
        CNT + 2 * 256 * 64 * 64 * 4 + 2 * 256 * 64 * 4
    assert lib.rmm_workspace_bytes(BF16, 64, 8200, 4096, 1) == 0       # 129 strips
    assert lib.rmm_workspace_bytes(BF16, 64, 14336, 4096, 1) == 0      # 224 strips
    # the split form is planned only with a workspace; without one the call is valid
    assert tpa.plan(64, 8192, 4096, gated=True)[:2] == (0, "stream")
    assert tpa.plan(64, 8192, 4096, gated=True, with_workspace=False)[:2] == (0, "stream")


def test_plain_entry_points_validate(lib):
    """rmsnorm_matmul and rmsnorm_gated_mlp themselves (not the _ex forms):
    every error in the documented order, and the empty no-op, with no HIP call."""
    def mm(X=A[0], g=A[1], W=A[2], Y=A[3], eps=1e-6, M=16, N=64, K=64, dtype=BF16, ws=None,
           ws_bytes=0):
        return lib.rmsnorm_matmul(X, g, W, Y, eps, M, N, K, dtype, ws, ws_bytes, None)

    def gm(X=A[0], g=A[1], W1=A[2], W3=A[4], Y=A[3], eps=1e-6, M=16, N=64, K=64, dtype=BF16,
           ws=None, ws_bytes=0):
        return lib.rmsnorm_gated_mlp(X, g, W1, W3, Y, eps, M, N, K, dtype, ws, ws_bytes, None)

    for f in (mm, gm):
        assert f(X=None) == NULL
        assert f(g=None) == NULL
        assert f(Y=None) == NULL
        assert f(X=None, K=0) == NULL          # NULL is checked before the shape
        assert f(K=0) == SHAPE
        assert f(M=-1) == SHAPE
        assert f(N=-1) == SHAPE
        assert f(M=1 << 62, K=1 << 10) == SHAPE
        assert f(K=0, eps=-1.0) == SHAPE        # shape before eps
        assert f(eps=-1e-6) == EPS
        assert f(eps=float("nan")) == EPS
        assert f(eps=float("inf")) == EPS
        assert f(eps=-1.0, dtype=7) == EPS     # eps before dtype
        assert f(dtype=7) == DTYPE
        assert f(Y=A[0]) == ALIAS              # Y on top of X
        assert f(Y=A[0], dtype=7) == DTYPE     # dtype before alias
        assert f(M=0) == OK and f(N=0) == OK   # empty: nothing launched
        assert f(M=0, X=None, Y=None) == OK
    assert gm(W3=None) == NULL
    assert gm(Y=A[4]) == ALIAS                 # Y on top of W3
    assert mm(W=None) == NULL
    # the documented workspace sizes are what the plain calls accept
    need = lib.rmm_workspace_bytes(BF16, 16, 6144, 4096, 0)
    assert need > 0
    assert mm(M=16, N=6144, K=4096, ws=A[5], ws_bytes=need - 1) == WORKSPACE
    needg = lib.rmm_workspace_bytes(BF16, 16, 6144, 4096, 1)
    assert needg > 0
    assert gm(M=16, N=6144, K=4096, ws=A[5], ws_bytes=needg - 1) == WORKSPACE


def test_forced_splits_beyond_the_counter_region(lib):
    """A split form needs one arrival counter per tile in the workspace's
    64 KiB counter region (16320 of them): forcing splits on more tiles is
    refused, the automatic choice runs without a combine there."""
    DECODE = 2
    N = 16321 * 128
    assert lib.rmm_workspace_bytes_ex(BF16, 16, N, 256, 0, DECODE, 2) == 0
    assert call(lib, M=16, N=N, K=256, variant=DECODE, splits=2, ws=A[5], ws_bytes=1 << 40) == VARIANT
    assert tpa.plan(16, N, 256, variant="decode")[1:] == ("decode", 1)
    N = 16320 * 128
    assert lib.rmm_workspace_bytes_ex(BF16, 16, N, 256, 0, DECODE, 2) > 0


def test_noalloc_validates_and_fits_its_scratch(lib):
    """rmsnorm_matmul_noalloc validates like rmsnorm_matmul (no HIP call on
    these failures), and every plain call's workspace fits its 16 MiB array:
    up to 64 rows the library's own choice needs no more; above, the prefill
    split is chosen to fit the workspace passed, which a plan with 16 MiB
    shows."""
    def na(X=A[0], g=A[1], W=A[2], Y=A[3], eps=1e-6, M=16, N=64, K=64, dtype=BF16):
        return lib.rmsnorm_matmul_noalloc(X, g, W, Y, eps, M, N, K, dtype, None)
    assert na(X=None) == NULL
    assert na(K=0) == SHAPE
    assert na(eps=-1.0) == EPS
    assert na(dtype=7) == DTYPE
    assert na(Y=A[0]) == ALIAS
    assert na(M=0) == OK and na(N=0, W=None) == OK and na(N=0) == OK  # empty: NULL allowed
    worst = 0
    split = 0
    for dtype in (BF16, F32):
        for M in (1, 8, 16, 17, 32, 33, 64, 100, 128, 200, 256, 1024):
            for K in (64, 1024, 4096, 8192):
                for N in (8, 128, 1024, 4096, 6144, 8192, 16384, 28672):
                    if M <= 64:
                        worst = max(worst, lib.rmm_workspace_bytes(dtype, M, N, K, 0))
                    st, v, sp = _binding.plan(A[0], A[1], A[2], None, A[3], 1e-6, M, N, K,
                                              dtype, False, ws=A[4], ws_bytes=16 << 20)
                    assert st == OK, (M, N, K, dtype, st)
                    split += v == "prefill" and sp > 1
    assert 0 < worst <= 16 << 20, worst
    assert split > 0


def test_attention_prefill_validation(lib):
    # qknorm_attention_prefill(_ex): NULL, SHAPE, EPS, DTYPE, ALIAS, VARIANT,
    # WORKSPACE, in that order; every call here fails before any launch.
    def at(Q=A[0], K=A[1], V=A[2], gq=A[3], gk=A[4], O=A[5], eps=1e-6, BH=2, G=2, Sq=100,
           Skv=1000, D=128, causal=1, dtype=BF16, splits=2, ws=None, ws_bytes=0):
        return lib.qknorm_attention_prefill_ex(Q, K, V, gq, gk, O, eps, BH, G, Sq, Skv, D, causal,
                                               dtype, splits, ws, ws_bytes, None)
    assert at(Q=None) == NULL
    assert at(G=0) == SHAPE
    assert at(D=96) == SHAPE
    assert at(Sq=1001) == SHAPE                           # causal needs Skv >= Sq
    assert at(eps=-1.0) == EPS
    assert at(dtype=F32) == DTYPE
    assert at(O=A[0]) == ALIAS                            # O on Q
    assert at(O=A[6] + 64, ws=A[6], ws_bytes=1 << 30) == ALIAS   # O inside the workspace
    assert at(Q=A[0] + 8) == VARIANT                      # not 16-byte aligned
    assert at(splits=17) == VARIANT                       # more spans than 64-key tiles
    assert at(splits=-1) == VARIANT
    assert at() == WORKSPACE                              # a forced split needs a workspace
    assert at(ws=A[6], ws_bytes=16) == WORKSPACE
    assert at(ws=A[6] + 4, ws_bytes=1 << 30) == WORKSPACE  # not 16-byte aligned
    assert at(Q=None, K=None, V=None, gq=None, gk=None, O=None, BH=0) == OK
    # the plain entry point: the same rules, no split
    assert lib.qknorm_attention_prefill(A[0], A[1], A[2], A[3], A[4], A[0], 1e-6, 2, 2, 100, 1000,
                                        128, 1, BF16, None) == ALIAS


def test_attention_prefill_workspace_sizes(lib):
    # 8 key/value heads x 4 queries, 512 positions over 8192 keys: 256
    # workgroups of 64 positions, so the library splits the keys in three
    # (spans of 2752 keys); the counter region, then 3 spans x 32 heads x 512
    # rows x (128 + 2) fp32
    assert lib.rmm_attention_prefill_workspace_bytes(8, 4, 512, 8192, 128, 1, 0) == \
        CNT + 3 * 32 * 512 * 130 * 4
    assert lib.rmm_attention_prefill_workspace_bytes(8, 4, 512, 8192, 128, 1, 3) == \
        CNT + 3 * 32 * 512 * 130 * 4
    assert lib.rmm_attention_prefill_workspace_bytes(8, 4, 512, 8192, 128, 1, 1) == 0
    # 2048 positions: 1024 workgroups already, no split
    assert lib.rmm_attention_prefill_workspace_bytes(8, 4, 2048, 2048, 128, 1, 0) == 0
    # 5 spans of 1000 keys round to 4 of 256 (whole 64-key tiles)
    assert lib.rmm_attention_prefill_workspace_bytes(1, 1, 64, 1000, 64, 0, 5) == \
        CNT + 4 * 64 * 66 * 4
    assert lib.rmm_attention_prefill_workspace_bytes(8, 4, 512, 8192, 128, 1, 200) == 0  # invalid
    # two query blocks per wave (256 workgroups of 128 positions), not causal: 3 spans
    assert lib.rmm_attention_prefill_workspace_bytes(16, 4, 512, 8192, 64, 0, 0) == \
        CNT + 3 * 64 * 512 * 66 * 4
