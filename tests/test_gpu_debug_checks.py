"""The row kernels' index checks on the GPU.

build.py --debug-checks builds liblce_debug.so, whose row kernels check every
row, label and column index they take from their inputs (labels, sorted keys,
dominant columns) before using it and print the check that fails.  This test
runs a set of the parity tests against that build in a child process and
requires that they pass and that no check fires.  It is skipped when the
debug build is absent or older than the sources (build it with
`python -m linear_cross_entropy_lse_amd.build --debug-checks`).
"""
import glob
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEBUG_LIB = os.path.join(ROOT, "linear_cross_entropy_lse_amd", "liblce_debug.so")


def _fresh():
    if not os.path.exists(DEBUG_LIB):
        return False
    srcs = glob.glob(os.path.join(ROOT, "linear_cross_entropy_lse_amd", "csrc", "*")) + \
        glob.glob(os.path.join(ROOT, "include", "*.h"))
    return os.path.getmtime(DEBUG_LIB) >= max(os.path.getmtime(s) for s in srcs)


def test_parity_under_index_checks():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not _fresh():
        pytest.skip("liblce_debug.so is absent or older than the sources")
    env = dict(os.environ, LCE_LIB=DEBUG_LIB, PYTHONPATH=ROOT)
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p", "no:cacheprovider",
           "--timeout", "200", "--timeout-method", "thread",
           os.path.join(ROOT, "tests", "test_gpu_parity.py") + "::test_irregular_shapes",
           os.path.join(ROOT, "tests", "test_gpu_confident.py") + "::test_shared_rows",
           os.path.join(ROOT, "tests", "test_gpu_precise.py") + "::test_precise_sorted_and_shard"]
    print("[debug-checks] running parity cases against liblce_debug.so", flush=True)
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert "lce check failed" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out, out[-4000:]
