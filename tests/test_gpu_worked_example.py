"""The pages' worked example, through the GPU kernels, against its closed form.

AI-infra KB page M011 works one row of logits z = [0, ln2, ln3, ln4] with
target 2: the loss is ln(10/3) ≈ 1.203973 (§03), and §05 splits the row into
two vocabulary tiles A = [0, ln2] (exp-sum 3) and B = [ln3, ln4] (exp-sum 7),
warning that normalising by the target's tile alone gives the wrong
ln(7/3) ≈ 0.847298 (tests/golden/worked_example.txt).

Here the same logits are planted in a Gemma-sized vocabulary (V = 256128):
row i of X is the unit vector e_i, so its logits are column i of W; the four
values sit at vocabulary rows in different 256-row tiles, forward splits and
backward chunks, and every other entry of that column is −100.  For the rows
that mirror §05, tile A's two values share one forward split and tile B's two
values another, far away, so a merge that normalised per split would give the
wrong value.  Expected values are the closed form in float64 on the bf16-rounded
values (no oracle call): LSE = log(Σ e^{w}), loss = LSE − w_target, and the
gradient of the mean loss at the four planted entries, dW[v, i] =
(p_v − [v = y_i]) / n_valid.
"""
import math

import numpy as np
import pytest
import torch

from tests.conftest import read_golden

pytestmark = pytest.mark.gpu

V, H = 256128, 64
# (positions of 0, ln2, ln3, ln4) per row; the target is the ln3 entry.
PLACES = [
    (0, 300, 200000, 200100),          # tile A in split 0, tile B in one split near the end
    (10, 1000, 129000, 130000),        # A early, B straddling a backward chunk region
    (255, 256, 64255, 64256),          # tile and backward-chunk edges
    (256127, 128512, 1, 99999),        # last vocabulary row holds the 0
    (5000, 5001, 5002, 5003),          # all four in one tile
    (70000, 180000, 250000, 30000),    # four different splits
]


@pytest.fixture(scope="module")
def lce():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_cross_entropy_lse_amd as P
    P.load()
    return P


def planted(softcap):
    vals = torch.tensor([0.0, math.log(2), math.log(3), math.log(4)]).to(torch.bfloat16)
    n = len(PLACES) + 1                       # one more row, ignored
    X = torch.zeros(n, H, dtype=torch.bfloat16)
    W = torch.zeros(V, H, dtype=torch.bfloat16)
    y = torch.full((n,), -100, dtype=torch.int64)
    for i, pos in enumerate(PLACES):
        X[i, i] = 1.0
        W[:, i] = -100.0
        for v, val in zip(pos, vals):
            W[v, i] = val
        y[i] = pos[2]
    X[n - 1, n - 1] = 1.0
    W[:, n - 1] = -100.0
    return X, W, y, vals.double().numpy()


def closed_form(vals, softcap):
    """Per planted row: LSE, loss and p of the four planted entries, float64."""
    w = np.array(vals, dtype=np.float64)
    rest = np.full(1, -100.0)
    if softcap > 0:
        w = softcap * np.tanh(w / softcap)
        rest = softcap * np.tanh(rest / softcap)
    m = w.max()
    total = np.exp(w - m).sum() + (V - 4) * np.exp(rest[0] - m)
    lse = m + math.log(total)
    return lse, lse - w[2], np.exp(w - lse)


@pytest.mark.parametrize("softcap", [0.0, 30.0])
def test_worked_example_through_the_kernels(lce, softcap):
    g = read_golden("worked_example.txt")
    X, W, y, vals = planted(softcap)
    print(f"[worked] softcap={softcap}: {len(PLACES)} planted rows in V={V}", flush=True)
    Xd, Wd, yd = X.cuda(), W.cuda(), y.cuda()
    out = lce.lce_forward(Xd, Wd, yd, -100, softcap)
    dX, dW = lce.lce_backward(Xd, Wd, yd, out["lse"], 1.0, -100, softcap)
    torch.cuda.synchronize()
    lse_e, loss_e, p = closed_form(vals, softcap)
    lse = out["lse"].cpu().numpy()
    loss = out["loss"].cpu().numpy()
    n_valid = len(PLACES)
    print(f"[worked] closed form: lse {lse_e:.7f} loss {loss_e:.7f}", flush=True)
    for i in range(len(PLACES) + 1):
        print(f"[worked] row {i}: lse {lse[i]:.7f} loss {loss[i]:.7f}", flush=True)
    assert int(out["n_valid"]) == n_valid and int(out["bad_label"]) == 0
    assert abs(float(out["mean"]) - loss_e) <= 1e-4 * loss_e
    if softcap == 0.0:
        # The page's numbers (printed to 6 decimals; the bf16 rounding of ln2,
        # ln3, ln4 moves the loss by less than 1e-2).
        assert abs(loss_e - float(g["loss"])) < 1e-2
    for i in range(n_valid):
        assert abs(lse[i] - lse_e) <= 1e-5, (i, lse[i], lse_e)
        assert abs(loss[i] - loss_e) <= 1e-5, (i, loss[i], loss_e)
        # Partial-denominator mistake of §05 rejected through the split merge.
        assert abs(loss[i] - float(g["wrong_target_tile_only"])) > 0.3
    assert loss[n_valid] == 0.0 and not dX[n_valid].any()
    # Gradient at the planted entries: (p − onehot) / n_valid, times the
    # softcap derivative; bf16 rounding of the dense part bounds the error.
    d = np.ones(4)
    if softcap > 0:
        d = 1.0 - np.tanh(vals / softcap) ** 2
    dWn = dW.cpu().numpy()
    for i, pos in enumerate(PLACES):
        expect = (p - np.array([0, 0, 1, 0])) * d / n_valid
        got = dWn[list(pos), i]
        assert np.all(np.abs(got - expect) <= 2.0 ** -8 * p * d / n_valid + 1e-7), (i, got, expect)
