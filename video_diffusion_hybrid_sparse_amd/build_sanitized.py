"""Host AddressSanitizer + UndefinedBehaviorSanitizer build of the C ABI.

The C ABI's host code (api.hip: argument and configuration checks, workspace layout,
error strings, the library-held buffers) is compiled with -fsanitize=address and
-fsanitize=undefined for the host pass only (GPU code is not built with sanitizers);
the kernel sources are the regular objects of build().  The result,
_build/libvdn_hybrid_attn_san.so, leaves the sanitizer symbols to the runtime that the
process preloads (sanitizer_env()), so any Python process can load it.

Usage: python -m video_diffusion_hybrid_sparse_amd.build_sanitized
"""
from __future__ import annotations

import glob
import os
import sys

from . import build as B

SAN_LIB = os.path.join(B.BUILD, "libvdn_hybrid_attn_san.so")
# each sanitizer flag applies to the host pass only
SAN_FLAGS = ["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def runtime() -> str:
    """The AddressSanitizer runtime of hipcc's clang (it carries the UBSan handlers too)."""
    found = sorted(glob.glob(os.path.join(B.ROCM, "lib", "llvm", "lib", "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    found += sorted(glob.glob(os.path.join(B.ROCM, "llvm", "lib", "clang", "*", "lib", "linux",
                                           "libclang_rt.asan-x86_64.so")))
    if not found:
        raise FileNotFoundError("libclang_rt.asan-x86_64.so not found under " + B.ROCM)
    return found[-1]


def sanitizer_env(env: dict | None = None) -> dict:
    """Environment for a child process that loads the sanitized library: the runtime
    first in LD_PRELOAD (anything already there is kept after it), leaks not checked
    (the interpreter keeps allocations until exit), every report fatal."""
    env = dict(os.environ if env is None else env)
    pre = env.get("LD_PRELOAD", "").strip()
    env["LD_PRELOAD"] = runtime() + (" " + pre if pre else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


def build_sanitized() -> str:
    os.makedirs(B.BUILD, exist_ok=True)
    objs = [os.path.join(B.BUILD, os.path.splitext(s)[0] + ".o") for s in B.SOURCES if s != "api.hip"]
    if not all(os.path.exists(o) for o in objs):
        B.build()
    api = os.path.join(B.BUILD, "api_san.o")
    B._run([B.HIPCC, *B.FLAGS, *SAN_FLAGS, "-c", os.path.join(B.CSRC, "api.hip"), "-o", api])
    tmp = SAN_LIB + ".tmp"
    B._run([B.HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-o", tmp, api, *objs, "-L", os.path.join(B.ROCM, "lib"),
            "-lhipblaslt", f"-Wl,-rpath,{os.path.join(B.ROCM, 'lib')}"])
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    print(build_sanitized())
    sys.exit(0)
