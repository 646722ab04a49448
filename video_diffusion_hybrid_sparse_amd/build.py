"""Builds the HIP library libvdn_hybrid_attn.so in-tree for gfx950 with hipcc.

Usage: python -m video_diffusion_hybrid_sparse_amd.build  (or build() from Python).
Every call recompiles all sources.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libvdn_hybrid_attn.so")
SOURCES = ["api.hip", "gemm.hip", "proj_gemm.hip", "softmax_bf16.hip", "linear_bf16.hip", "scan.hip", "delta_bf16.hip", "backward.hip", "fp32_path.hip", "mxfp8.hip"]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", f"--offload-arch={ARCH}", "-fPIC", "-std=c++17", "-I", INCLUDE, "-I", CSRC,
         # packed fp32 VALU ops stay off on this target
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-Wno-unused-variable", "-Wno-unused-command-line-argument"]


def _run(cmd: list[str]) -> None:
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr).strip()
    # hipcc's host pass does not know the packed-fp32 target feature; that warning is noise
    lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l and "not a recognized feature" not in l]
    if r.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + "\n".join(lines))


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []

    def compile_one(src: str) -> str:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        _run([HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose:
            print("compiled", src, flush=True)
        return obj

    with ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-o", tmp, *objs, "-L", os.path.join(ROCM, "lib"),
          "-lhipblaslt", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"])
    # the bf16 softmax and the merged dK/dV backward write their MFMAs as inline asm:
    # check the wait states around them, and that no compiler-generated code uses M0 in
    # the sources whose LDS copies write it from inline asm.  The library is installed
    # only when the check passes; on failure the previous one is removed as well, so that
    # nothing loads a library built from other sources.
    from .asm_check import check
    problems = check()
    if problems:
        for f in (tmp, LIB):
            if os.path.exists(f):
                os.remove(f)
        raise RuntimeError("static check of the compiled kernels failed:\n" + "\n".join(problems))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
