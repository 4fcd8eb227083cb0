"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test ties the oracle to something it does not compute itself: the pages'
worked example, the textbook softmax definition, torch's own cross-entropy
and autograd (a library routine, float64 on the CPU), central finite
differences, closed forms and invariants.  A dropped term, a wrong sign or
index, a transposed operand, a wrong normaliser or a missing softcap
derivative each fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

from oracle import lce_oracle as O
from tests.conftest import read_golden


def _rand_problem(N, H, V, seed, n_ignore=0, scale=1.0):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((N, H)) * scale
    W = rng.standard_normal((V, H)) * scale
    y = rng.integers(0, V, size=N)
    if n_ignore:
        y[rng.choice(N, size=n_ignore, replace=False)] = O.IGNORE_INDEX
    return X, W, y


# --------------------------------------------------------------------------- #
# The pages' worked example (M011 §03 and §05)
# --------------------------------------------------------------------------- #
def _worked_example_inputs():
    # A one-dimensional hidden state x = [1] and W's single column equal to the
    # example's logits make z = X·Wᵀ exactly the page's row.
    z = np.array([0.0, math.log(2), math.log(3), math.log(4)])
    return np.array([[1.0]]), z[:, None].copy(), np.array([2]), z


def test_worked_example_loss_matches_page():
    g = read_golden("worked_example.txt")
    X, W, y, _ = _worked_example_inputs()
    out = O.forward(X, W, y)
    dec = int(g["printed_decimals"])
    assert round(float(out["loss"][0]), dec) == pytest.approx(float(g["loss"]), abs=0.5 * 10 ** -dec)
    assert round(float(out["mean"]), dec) == pytest.approx(float(g["loss"]), abs=0.5 * 10 ** -dec)
    assert out["n_valid"] == 1
    # the page's denominator is 10: LSE = ln 10 exactly
    assert out["lse"][0] == pytest.approx(math.log(10.0), abs=1e-14)


def test_worked_example_two_tile_merge_and_wrong_value_rejected():
    g = read_golden("worked_example.txt")
    _, _, y, z = _worked_example_inputs()
    lse = O.logsumexp_by_vocab_tiles(z, [0, 2, 4])
    loss = lse - z[int(g["target"])]
    dec = int(g["printed_decimals"])
    assert round(loss, dec) == pytest.approx(float(g["loss"]), abs=0.5 * 10 ** -dec)
    assert math.exp(lse) == pytest.approx(float(g["tile_mass_A"]) + float(g["tile_mass_B"]), rel=1e-14)
    # The single-tile masses of the page.
    assert math.exp(O.logsumexp_by_vocab_tiles(z, [0, 2])) == pytest.approx(float(g["tile_mass_A"]), rel=1e-14)
    assert math.exp(O.logsumexp_by_vocab_tiles(z, [2, 4])) == pytest.approx(float(g["tile_mass_B"]), rel=1e-14)
    # The target-tile-only normalisation gives the page's wrong value, which the
    # oracle must not produce.
    wrong = O.logsumexp_by_vocab_tiles(z[2:], [0, 2]) - z[2]
    assert round(wrong, dec) == pytest.approx(float(g["wrong_target_tile_only"]), abs=0.5 * 10 ** -dec)
    X, W, y, _ = _worked_example_inputs()
    assert abs(O.forward(X, W, y)["loss"][0] - float(g["wrong_target_tile_only"])) > 0.3


def test_worked_example_gradient_is_softmax_minus_onehot():
    # Probabilities of the example are [1, 2, 3, 4] / 10; the target is 2.
    X, W, y, _ = _worked_example_inputs()
    out = O.forward(X, W, y)
    dZ = O.logit_gradient(X, W, y, out["lse"], out["n_valid"])
    np.testing.assert_allclose(dZ[0], [0.1, 0.2, 0.3 - 1.0, 0.4], atol=1e-15)


# --------------------------------------------------------------------------- #
# Blocking of the vocabulary does not change the LSE (M011 §05, §08 checklist)
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_partition_independence(seed):
    rng = np.random.default_rng(seed)
    V = 1003
    z = rng.standard_normal(V) * 3.0
    direct = O.row_logsumexp(z[None, :])[0]
    for _ in range(5):
        k = int(rng.integers(1, 40))
        inner = np.sort(rng.choice(np.arange(1, V), size=k, replace=False))
        bounds = [0] + inner.tolist() + [V]
        assert O.logsumexp_by_vocab_tiles(z, bounds) == pytest.approx(direct, abs=1e-12)
    assert O.logsumexp_by_vocab_tiles(z, list(range(V + 1))) == pytest.approx(direct, abs=1e-12)


# --------------------------------------------------------------------------- #
# Textbook definition: loss = −log softmax(z)[y] (CCE blog §三), pure Python
# --------------------------------------------------------------------------- #
def test_textbook_softmax_definition_bruteforce():
    X, W, y = _rand_problem(6, 5, 9, seed=3, n_ignore=1, scale=0.7)
    out = O.forward(X, W, y)
    losses = []
    for i in range(X.shape[0]):
        if y[i] == O.IGNORE_INDEX:
            losses.append(0.0)
            continue
        zi = [math.fsum(X[i, h] * W[v, h] for h in range(X.shape[1])) for v in range(W.shape[0])]
        prob = math.exp(zi[y[i]]) / math.fsum(math.exp(t) for t in zi)
        losses.append(-math.log(prob))
    np.testing.assert_allclose(out["loss"], losses, rtol=0, atol=1e-12)
    n_valid = sum(1 for t in y if t != O.IGNORE_INDEX)
    assert out["n_valid"] == n_valid
    assert out["mean"] == pytest.approx(math.fsum(losses) / n_valid, abs=1e-12)


# --------------------------------------------------------------------------- #
# Library routine: torch's float64 cross-entropy + autograd on the CPU
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("softcap", [0.0, 2.5])
def test_matches_torch_cross_entropy_and_autograd(softcap):
    X, W, y = _rand_problem(37, 11, 53, seed=5, n_ignore=6, scale=1.3)
    Xt = torch.tensor(X, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    z = Xt @ Wt.T
    if softcap > 0:
        z = softcap * torch.tanh(z / softcap)
    loss = torch.nn.functional.cross_entropy(z, torch.tensor(y), ignore_index=-100,
                                             reduction="mean")
    per_row = torch.nn.functional.cross_entropy(z.detach(), torch.tensor(y), ignore_index=-100,
                                                reduction="none")
    loss.backward()
    out = O.forward(X, W, y, softcap=softcap)
    dX, dW = O.backward(X, W, y, softcap=softcap)
    assert out["mean"] == pytest.approx(loss.item(), rel=1e-13, abs=1e-13)
    np.testing.assert_allclose(out["loss"], per_row.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dX, Xt.grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(dW, Wt.grad.numpy(), rtol=1e-11, atol=1e-13)


def test_dloss_scales_gradient_like_autograd():
    X, W, y = _rand_problem(9, 4, 13, seed=8, n_ignore=2)
    Xt = torch.tensor(X, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    loss = torch.nn.functional.cross_entropy(Xt @ Wt.T, torch.tensor(y), ignore_index=-100)
    (loss * 0.37).backward()
    dX, dW = O.backward(X, W, y, dloss=0.37)
    np.testing.assert_allclose(dX, Xt.grad.numpy(), rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(dW, Wt.grad.numpy(), rtol=1e-11, atol=1e-14)


# --------------------------------------------------------------------------- #
# Central finite differences of the mean loss (M011 §08 checklist)
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("softcap", [0.0, 0.9])
def test_finite_differences(softcap):
    X, W, y = _rand_problem(5, 3, 7, seed=11, n_ignore=1)
    dX, dW = O.backward(X, W, y, softcap=softcap)
    eps = 1e-6

    def f(Xv, Wv):
        return O.mean_loss_value(Xv, Wv, y, softcap=softcap)

    num_dX = np.zeros_like(X)
    for idx in np.ndindex(*X.shape):
        Xp, Xm = X.copy(), X.copy()
        Xp[idx] += eps
        Xm[idx] -= eps
        num_dX[idx] = (f(Xp, W) - f(Xm, W)) / (2 * eps)
    num_dW = np.zeros_like(W)
    for idx in np.ndindex(*W.shape):
        Wp, Wm = W.copy(), W.copy()
        Wp[idx] += eps
        Wm[idx] -= eps
        num_dW[idx] = (f(X, Wp) - f(X, Wm)) / (2 * eps)
    for a, n in ((dX, num_dX), (dW, num_dW)):
        rel = np.linalg.norm(a - n) / np.linalg.norm(n)
        assert rel < 1e-7, rel


# --------------------------------------------------------------------------- #
# ignore_index, the all-ignored convention, bad labels
# --------------------------------------------------------------------------- #
def test_ignored_rows_contribute_nothing():
    X, W, y = _rand_problem(12, 6, 20, seed=2)
    y_ign = y.copy()
    y_ign[[1, 4, 7]] = O.IGNORE_INDEX
    out = O.forward(X, W, y_ign)
    assert out["n_valid"] == 9
    assert np.all(out["loss"][[1, 4, 7]] == 0.0)
    # the LSE of an ignored row is still its row's LSE (reading R3)
    np.testing.assert_allclose(out["lse"], O.forward(X, W, y)["lse"], rtol=0, atol=0)
    keep = np.setdiff1d(np.arange(12), [1, 4, 7])
    sub = O.forward(X[keep], W, y[keep])
    assert out["mean"] == pytest.approx(sub["mean"], rel=1e-14)
    dX, dW = O.backward(X, W, y_ign)
    assert np.all(dX[[1, 4, 7]] == 0.0)
    dXs, dWs = O.backward(X[keep], W, y[keep])
    np.testing.assert_allclose(dX[keep], dXs, rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(dW, dWs, rtol=1e-12, atol=1e-16)


def test_all_rows_ignored_convention():
    X, W, _ = _rand_problem(4, 3, 5, seed=4)
    y = np.full(4, O.IGNORE_INDEX)
    out = O.forward(X, W, y)
    assert out["n_valid"] == 0 and out["mean"] == 0.0
    dX, dW = O.backward(X, W, y)
    assert np.all(dX == 0) and np.all(dW == 0)


def test_bad_label_gives_nan_row():
    X, W, y = _rand_problem(4, 3, 5, seed=6)
    y[2] = 5                     # == V: out of range
    out = O.forward(X, W, y)
    assert np.isnan(out["loss"][2]) and np.isnan(out["mean"])
    assert np.all(np.isfinite(out["loss"][[0, 1, 3]]))


# --------------------------------------------------------------------------- #
# Closed forms and invariants
# --------------------------------------------------------------------------- #
def test_zero_weight_closed_form():
    # W = 0: every logit is 0, p = 1/V, LSE = ln V, loss = ln V, dX = 0 and
    # dW[v] = (dloss/n_valid) Σ_valid (1/V − [y_i = v]) x_i.
    rng = np.random.default_rng(9)
    N, H, V = 10, 4, 6
    X = rng.standard_normal((N, H))
    W = np.zeros((V, H))
    y = rng.integers(0, V, size=N)
    y[3] = O.IGNORE_INDEX
    out = O.forward(X, W, y)
    np.testing.assert_allclose(out["lse"], np.log(V), atol=1e-15)
    valid = y != O.IGNORE_INDEX
    np.testing.assert_allclose(out["loss"][valid], np.log(V), atol=1e-15)
    dX, dW = O.backward(X, W, y, dloss=2.0)
    assert np.all(dX == 0)
    s = 2.0 / valid.sum()
    expect = np.zeros((V, H))
    for i in range(N):
        if not valid[i]:
            continue
        for v in range(V):
            expect[v] += s * ((1.0 / V) - (1.0 if y[i] == v else 0.0)) * X[i]
    np.testing.assert_allclose(dW, expect, atol=1e-14)


def test_bounds_nonnegativity_and_gradient_row_sums():
    X, W, y = _rand_problem(30, 8, 41, seed=12)
    out = O.forward(X, W, y)
    zmax = (X @ W.T).max(axis=1)
    assert np.all(out["lse"] >= zmax - 1e-12)
    assert np.all(out["lse"] <= zmax + math.log(41) + 1e-12)
    assert np.all(out["loss"] >= 0)
    dZ = O.logit_gradient(X, W, y, out["lse"], out["n_valid"])
    np.testing.assert_allclose(dZ.sum(axis=1), 0.0, atol=1e-15)
    _, dW = O.backward(X, W, y)
    np.testing.assert_allclose(dW.sum(axis=0), 0.0, atol=1e-14)


def test_shift_equivariance():
    # Appending a ones column to X and a constant column c to W adds c to every
    # logit: the LSE moves by c, the loss and dX[:, :H] do not change.
    X, W, y = _rand_problem(8, 5, 12, seed=13, n_ignore=2)
    c = 1.75
    X2 = np.hstack([X, np.ones((8, 1))])
    W2 = np.hstack([W, np.full((12, 1), c)])
    a, b = O.forward(X, W, y), O.forward(X2, W2, y)
    np.testing.assert_allclose(b["lse"], a["lse"] + c, atol=1e-13)
    np.testing.assert_allclose(b["loss"], a["loss"], atol=1e-13)
    dX, _ = O.backward(X, W, y)
    dX2, _ = O.backward(X2, W2, y)
    np.testing.assert_allclose(dX2[:, :5], dX, atol=1e-14)


def test_vocab_permutation_equivariance():
    X, W, y = _rand_problem(9, 4, 15, seed=14, n_ignore=1)
    perm = np.random.default_rng(0).permutation(15)
    inv = np.argsort(perm)
    Wp = W[perm]
    yp = np.where(y == O.IGNORE_INDEX, y, inv[np.maximum(y, 0)])
    a, b = O.forward(X, W, y), O.forward(X, Wp, yp)
    np.testing.assert_allclose(b["loss"], a["loss"], atol=1e-13)
    dX, dW = O.backward(X, W, y)
    dXp, dWp = O.backward(X, Wp, yp)
    np.testing.assert_allclose(dXp, dX, atol=1e-14)
    np.testing.assert_allclose(dWp, dW[perm], atol=1e-14)


def test_softcap_large_cap_reduces_to_plain():
    X, W, y = _rand_problem(7, 4, 9, seed=15)
    a = O.forward(X, W, y)
    b = O.forward(X, W, y, softcap=1e7)
    np.testing.assert_allclose(b["loss"], a["loss"], atol=1e-9)
    dXa, dWa = O.backward(X, W, y)
    dXb, dWb = O.backward(X, W, y, softcap=1e7)
    np.testing.assert_allclose(dXb, dXa, atol=1e-9)
    np.testing.assert_allclose(dWb, dWa, atol=1e-9)


def test_softcap_bounds_logits():
    X, W, y = _rand_problem(5, 3, 6, seed=16, scale=10.0)
    c = 2.0
    out = O.forward(X, W, y, softcap=c)
    assert np.all(out["lse"] < c + math.log(6) + 1e-12)
    assert np.all(out["lse"] > -c)


# --------------------------------------------------------------------------- #
# Row / vocabulary subsets used at full sizes agree with the full evaluation
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("softcap", [0.0, 3.0])
def test_subset_evaluations_agree(softcap):
    X, W, y = _rand_problem(23, 7, 31, seed=17, n_ignore=4)
    full = O.forward(X, W, y, softcap=softcap)
    dX, dW = O.backward(X, W, y, dloss=1.5, softcap=softcap)
    rows = np.array([0, 5, 22])
    sub = O.forward(X[rows], W, y[rows], softcap=softcap, n_valid_total=full["n_valid"])
    np.testing.assert_allclose(sub["lse"], full["lse"][rows], atol=1e-14)
    dXr = O.dX_rows(X[rows], W, y[rows], full["lse"][rows], full["n_valid"], 1.5,
                    softcap=softcap)
    np.testing.assert_allclose(dXr, dX[rows], atol=1e-14)
    # dW shares of a row partition add up to the full dW
    parts = [np.arange(0, 9), np.arange(9, 23)]
    dW_sum = sum(O.backward_rows(X[r], W, y[r], full["lse"][r], full["n_valid"], 1.5,
                                 softcap=softcap)[1] for r in parts)
    np.testing.assert_allclose(dW_sum, dW, atol=1e-14)
    dXb, _ = O.backward_rows(X[rows], W, y[rows], full["lse"][rows], full["n_valid"], 1.5,
                             softcap=softcap)
    np.testing.assert_allclose(dXb, dX[rows], atol=1e-14)
    vrows = np.array([1, 7, 30])
    dWr = O.dW_vocab_rows(X, W, y, full["lse"], full["n_valid"], vrows, 1.5,
                          softcap=softcap)
    np.testing.assert_allclose(dWr, dW[vrows], atol=1e-14)
