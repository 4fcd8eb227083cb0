#!/usr/bin/env python3
"""Write the full-size expected values the GPU parity tests compare against.

    python tests/golden/make_fullsize.py [workload ...]

For each large workload this evaluates the CPU oracle (float64) on the seeded
inputs and stores, in tests/golden/fullsize_<workload>.npz:
  * lse, loss           every row (the oracle's forward, row block by row block)
  * mean, n_valid       the mean over valid targets and its denominator
  * dx_rows, dX         dX on a seeded sample of token rows
  * dw_rows, dW         dW on sampled vocabulary rows: the most frequent labels,
                        a seeded sample, and the last row
  * fingerprint         sha256 of the input bytes (X, W, labels), so a test can
                        confirm it regenerated exactly the same inputs
Only the oracle and the seeded input generator are used.
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import lce_inputs as L  # noqa: E402
from oracle import lce_oracle as O  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
LARGE = ["liger", "llama3_8b", "gemma2_2b", "qwen25_long"]
ROW_BLOCK = 256
N_DX_ROWS = 12
N_DW_RANDOM = 8


def golden_path(name: str) -> str:
    return os.path.join(HERE, f"fullsize_{name}.npz")


def make(name: str) -> None:
    w = L.WORKLOADS[name]
    t0 = time.time()
    X, W, y = L.make_inputs(w)
    fp = L.fingerprint(X, W, y)
    X64, W64, y64 = L.to_f64(X), L.to_f64(W), y.numpy()
    del X, W
    n_valid = int((y64 != L.IGNORE_INDEX).sum())
    lse = np.empty(w.N)
    loss = np.empty(w.N)
    for a in range(0, w.N, ROW_BLOCK):
        b = min(a + ROW_BLOCK, w.N)
        f = O.forward(X64[a:b], W64, y64[a:b], L.IGNORE_INDEX, w.softcap, n_valid_total=n_valid)
        lse[a:b] = f["lse"]
        loss[a:b] = f["loss"]
        if a // ROW_BLOCK % 8 == 0:
            print(f"  {name}: rows {b}/{w.N} ({time.time() - t0:.0f} s)", flush=True)
    mean = float(loss.sum() / n_valid)
    dx_rows = L.row_sample(w.N, N_DX_ROWS, seed=w.seed + 101)
    dX = O.dX_rows(X64[dx_rows], W64, y64[dx_rows], lse[dx_rows], n_valid, 1.0,
                   L.IGNORE_INDEX, w.softcap)
    valid = y64[y64 != L.IGNORE_INDEX]
    counts = np.bincount(valid, minlength=w.V)
    top = np.argsort(-counts, kind="stable")[:4]
    rng = np.random.default_rng(w.seed + 202)
    dw_rows = np.unique(np.concatenate([top, rng.choice(w.V, N_DW_RANDOM, replace=False),
                                        [w.V - 1]])).astype(np.int64)
    dW = O.dW_vocab_rows(X64, W64, y64, lse, n_valid, dw_rows, 1.0, L.IGNORE_INDEX, w.softcap)
    np.savez_compressed(golden_path(name), lse=lse, loss=loss, mean=mean, n_valid=n_valid,
                        dx_rows=dx_rows, dX=dX.astype(np.float32), dw_rows=dw_rows,
                        dW=dW.astype(np.float32), fingerprint=fp,
                        source="tests/golden/make_fullsize.py (CPU oracle, float64)")
    print(f"  {name}: wrote {golden_path(name)} in {time.time() - t0:.0f} s", flush=True)


if __name__ == "__main__":
    for n in (sys.argv[1:] or LARGE):
        make(n)
