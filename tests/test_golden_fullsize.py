"""The stored full-size expected values still belong to the seeded inputs.

tests/golden/fullsize_<workload>.npz hold oracle values the GPU parity test
compares against.  Here, on the CPU, each file's input fingerprint is checked
against freshly generated inputs and a few of its rows are recomputed with the
oracle, so a change to the input generator or the oracle cannot leave stale
expected values behind unnoticed.
"""
import os

import numpy as np
import pytest

import lce_inputs as L
from oracle import lce_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.slow
@pytest.mark.parametrize("name", ["liger", "llama3_8b", "gemma2_2b", "qwen25_long"])
def test_golden_matches_inputs_and_oracle(name):
    gold = np.load(os.path.join(HERE, "golden", f"fullsize_{name}.npz"))
    w = L.WORKLOADS[name]
    X, W, y = L.make_inputs(w)
    assert L.fingerprint(X, W, y) == str(gold["fingerprint"])
    y64 = y.numpy()
    n_valid = int((y64 != L.IGNORE_INDEX).sum())
    assert n_valid == int(gold["n_valid"])
    rows = np.array([0, w.N // 2, w.N - 1])
    W64 = L.to_f64(W)
    f = O.forward(L.to_f64(X[rows]), W64, y64[rows], L.IGNORE_INDEX, w.softcap,
                  n_valid_total=n_valid)
    np.testing.assert_allclose(f["lse"], gold["lse"][rows], rtol=0, atol=1e-9)
    np.testing.assert_allclose(f["loss"], gold["loss"][rows], rtol=0, atol=1e-9)
    assert gold["dX"].shape == (len(gold["dx_rows"]), w.H)
    assert gold["dW"].shape == (len(gold["dw_rows"]), w.H)
