"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The CPU tests of the ABI (tests/test_abi.py: configuration and argument checks, the
workspace layouts, error strings, entry points that must reject their arguments before
launching anything) run in a child process against a build of api.hip whose host pass
has both sanitizers on (build_sanitized.py), with the sanitizer runtime preloaded; a
report of either sanitizer aborts the child and fails this test.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or (os.path.exists("/opt/rocm/bin/hipcc") and "/opt/rocm/bin/hipcc")

CHILD = """
import ctypes, sys
import pytest
from video_diffusion_hybrid_sparse_amd import binding
binding.LIB_PATH = sys.argv[1]
# the sanitizer runtime is in the process (preloaded), and the sanitized library is the one loaded
assert hasattr(ctypes.CDLL(None), "__asan_init"), "AddressSanitizer runtime not loaded"
assert binding.lib()._name == sys.argv[1]
rc = pytest.main(["-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu", "tests/test_abi.py"])
print("child pytest exit", int(rc), flush=True)
sys.exit(int(rc))
"""


@pytest.mark.skipif(not HIPCC, reason="hipcc not installed")
def test_abi_checks_clean_under_asan_and_ubsan():
    from video_diffusion_hybrid_sparse_amd import build_sanitized as bs

    lib = bs.build_sanitized()
    r = subprocess.run([sys.executable, "-c", CHILD, lib], cwd=ROOT, env=bs.sanitizer_env(), capture_output=True,
                       text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-6000:]
    assert "runtime error:" not in out, out[-6000:]
    assert r.returncode == 0 and "child pytest exit 0" in out, out[-6000:]
