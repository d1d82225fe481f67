"""Build librmm.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m tensor_program_amd.build

Every source is compiled with hipcc for gfx950 only.  Packed fp32 VALU
instructions are switched off in device code (-packed-fp32-ops).  The
accumulating VOP2 form of the bf16 dot product is switched off too
(-dot13-insts): with it the compiler turns every zero-accumulator dot product
into a register clear plus the accumulating form, two instructions where the
VOP3P form takes the zero as a constant.  hipcc's host pass warns that it does
not know these features, which is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "librmm.so")
SOURCES = ["rmm_abi.cpp", "rmm_generic.hip", "rmm_decode.hip", "rmm_decode32.hip", "rmm_prefill.hip",
           "rmm_stream.hip", "rmm_norm.hip", "rmm_attn.hip",
           "rmm_chain.hip", "rmm_probe.hip", "rmm_noalloc.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
                 shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def cflags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Xclang", "-target-feature", "-Xclang", "-dot13-insts",
            "-Wall", "-Wno-unused-command-line-argument"]


def build(verbose: bool = False, save_temps: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *cflags(), "-c", os.path.join(CSRC, src), "-o", obj]
        if save_temps and src.endswith(".hip"):
            cmd += ["-save-temps=obj"]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [cc, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, save_temps="--save-temps" in sys.argv))
