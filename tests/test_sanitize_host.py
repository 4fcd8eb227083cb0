"""The host side of the C ABI under AddressSanitizer, on the CPU.

build.py --asan compiles the host code of liblce (argument checks, workspace
plans, launch sequences) with AddressSanitizer; the device code is built as
usual.  This test builds that library into a temporary directory and runs the
host ABI tests against it in a child process that preloads the sanitizer
runtime, so an out-of-bounds or use-after-free access in the host code ends
the child with a sanitizer report.  No GPU is used: without a device every
entry point stops at its argument checks or at the device query.
"""
import os
import subprocess
import sys

import pytest

from linear_cross_entropy_lse_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import ctypes, os, sys
import pytest
proc = ctypes.CDLL(None)
assert hasattr(proc, "__asan_init"), "sanitizer runtime not preloaded"
from linear_cross_entropy_lse_amd import _lib
lib = _lib.load()
assert lib._name == os.environ["LCE_LIB"], lib._name
sys.exit(pytest.main(["-x", "-q", "-p", "no:cacheprovider", sys.argv[1]]))
"""


@pytest.mark.slow
def test_host_abi_under_address_sanitizer(tmp_path):
    try:
        runtime = B.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = B.build(out=str(tmp_path / "liblce_asan.so"), asan=True, bdir=str(tmp_path / "obj"))
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report_load8" in nm, "host code was not instrumented"
    env = dict(os.environ)
    env.update(LD_PRELOAD=runtime, LCE_LIB=lib, PYTHONPATH=ROOT,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=86")
    res = subprocess.run([sys.executable, "-c", CHILD, os.path.join(ROOT, "tests", "test_abi_host.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out, out[-4000:]
