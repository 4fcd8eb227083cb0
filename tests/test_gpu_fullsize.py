"""Parity at the full workload sizes, in the same launch configuration the
benchmark times (float32 dX and dW, dloss = 1, ignore_index = -100).

The float64 oracle cannot run inside a test at these sizes, so its values come
from tests/golden/fullsize_<workload>.npz, written by make_fullsize.py next to
them (which calls only the oracle and the seeded input generator):
  * LSE and loss of every row                     abs err ≤ 2e-3
  * the mean over valid targets                   rel err ≤ 1e-4; n_valid exact
  * dX on sampled token rows, dW on sampled
    vocabulary rows (incl. the most frequent
    labels and the last vocabulary row)           rel L2 ≤ 1e-3 per sample set
and, from the oracle at test time (tests/fullsize_samples.py), 1024+ dX rows
and dW rows from every vocabulary chunk, its boundaries, tile boundaries and
offsets past 2^31 bytes, checked twice: whole (rel L2 ≤ 1e-3) and as their
dense part alone, the output minus the oracle's exact one-hot term against the
oracle's softmax term (rel L2 ≤ 1e-2, the bar of a value that passes through
bf16 by design), the label-free dW rows as their own set.
Properties that hold at any size are checked on the whole output: ignored rows
have loss 0 and dX 0, every LSE is finite, no bad label is flagged, and the
peak device memory stays far below one N x V logit matrix.
"""
import os

import numpy as np
import pytest
import torch

import lce_inputs as L
from tests import fullsize_samples as FS

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
LSE_ATOL = 2e-3
MEAN_RTOL = 1e-4
GRAD_RTOL_F32 = 1e-3
DENSE_RTOL = 1e-2
FULL = ["liger", "llama3_8b", "gemma2_2b", "qwen25_long"]


@pytest.fixture(scope="module")
def lce():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_cross_entropy_lse_amd as P
    P.load()
    return P


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (den if den > 0 else 1.0)


@pytest.mark.parametrize("name", FULL)
def test_fullsize_against_oracle(lce, name):
    path = os.path.join(HERE, "golden", f"fullsize_{name}.npz")
    gold = np.load(path)
    w = L.WORKLOADS[name]
    print(f"[fullsize] {name}: N={w.N} H={w.H} V={w.V} softcap={w.softcap} seed={w.seed}",
          flush=True)
    X, W, y = L.make_inputs(w)
    assert L.fingerprint(X, W, y) == str(gold["fingerprint"]), "seeded inputs changed"
    dev = "cuda"
    Xd, Wd, yd = X.to(dev), W.to(dev), y.to(dev)
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    out = lce.lce_forward(Xd, Wd, yd, L.IGNORE_INDEX, w.softcap)
    dX, dW = lce.lce_backward(Xd, Wd, yd, out["lse"], torch.ones((), device=dev),
                              L.IGNORE_INDEX, w.softcap)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    print(f"[fullsize] {name}: GPU done, peak extra {peak / 2**20:.0f} MiB", flush=True)

    lse = out["lse"].cpu().numpy()
    loss = out["loss"].cpu().numpy()
    assert int(out["n_valid"]) == int(gold["n_valid"])
    assert int(out["bad_label"]) == 0
    assert np.isfinite(lse).all()
    e_lse = np.abs(lse - gold["lse"]).max()
    e_loss = np.abs(loss - gold["loss"]).max()
    mean, gmean = float(out["mean"]), float(gold["mean"])
    ign = (y == L.IGNORE_INDEX).numpy()
    assert (loss[ign] == 0).all()
    dx_rows = torch.from_numpy(gold["dx_rows"])
    dw_rows = torch.from_numpy(gold["dw_rows"])
    e_dx = rel_l2(dX[dx_rows.to(dev)].float().cpu(), gold["dX"])
    e_dw = rel_l2(dW[dw_rows.to(dev)].float().cpu(), gold["dW"])
    dx_ign_zero = bool((dX[torch.from_numpy(ign).to(dev)] == 0).all())
    print(f"[fullsize] {name}: lse max err {e_lse:.2e} loss max err {e_loss:.2e} "
          f"mean rel {abs(mean - gmean) / abs(gmean):.2e} dX rel {e_dx:.2e} dW rel {e_dw:.2e}",
          flush=True)
    assert e_lse <= LSE_ATOL and e_loss <= LSE_ATOL
    assert abs(mean - gmean) <= MEAN_RTOL * abs(gmean)
    assert e_dx <= GRAD_RTOL_F32 and e_dw <= GRAD_RTOL_F32
    assert dx_ign_zero
    S = FS.samples(name, X, W, y, dict(softcap=w.softcap))
    FS.check(f"fullsize {name}", dX, dW, S, GRAD_RTOL_F32, DENSE_RTOL,
             log=lambda m: print(m, flush=True))
    # Outputs (dX, dW in float32, five per-row vectors) plus the library's
    # workspace, and nothing the size of the logits.
    ws = lce.lce_backward_workspace_bytes(w.N, w.H, w.V)
    outputs = w.N * w.H * 4 + w.V * w.H * 4 + 5 * w.N * 4
    # (slack for the caching allocator's rounding of each allocation)
    assert peak <= ws + outputs + (8 << 20), (peak, ws, outputs)
    # The workspace is O(N·H + V·H): one bf16 gradient chunk no larger than W
    # and the float32 dX accumulator.
    assert ws <= 2 * w.V * w.H + 4 * w.N * w.H + (64 << 20), ws
    assert ws < w.N * w.V * 2
