"""Host-side checks of the product's contract, no GPU needed:

- the benchmark measures one GPU and refuses any other count, before it
  touches torch or the GPU;
- the binding has no fallback: a missing library raises, and host tensors are
  rejected before any call into the library;
- the package (Python and HIP sources) never imports, includes or loads the
  CPU oracle, which is test infrastructure only.
"""
import os
import re
import subprocess
import sys

import pytest

from linear_cross_entropy_lse_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "linear_cross_entropy_lse_amd")


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_bench_refuses_more_than_one_gpu(argv, env):
    e = dict(os.environ)
    e.update(env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv, cwd=ROOT, env=e,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""   # no JSON line for a refused run


def test_missing_library_raises(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        _lib.load(str(tmp_path / "liblce.so"))


def test_host_tensors_are_rejected():
    import torch
    X = torch.zeros(4, 8, dtype=torch.bfloat16)
    W = torch.zeros(16, 8, dtype=torch.bfloat16)
    y = torch.zeros(4, dtype=torch.int64)
    with pytest.raises(ValueError, match="device"):
        _lib._prep(X, W, y)


def _package_sources():
    for d, _, files in os.walk(PKG):
        if "_build" in d or "__pycache__" in d:
            continue
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                yield os.path.join(d, f)


def test_package_never_reaches_the_oracle():
    paths = list(_package_sources())
    assert any(p.endswith(".hip") for p in paths) and any(p.endswith(".py") for p in paths)
    pat = re.compile(r"^\s*(from\s+oracle|import\s+oracle|#\s*include\s*[<\"][^>\"]*oracle)"
                     r"|oracle/|liboracle", re.M)
    hits = [p for p in paths if pat.search(open(p, encoding="utf-8").read())]
    assert hits == []
