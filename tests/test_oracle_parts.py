"""Pins of the oracle's gradient split into its softmax ("dense") and target
("one-hot") terms (logit_gradient_parts, dX_rows_parts, dW_vocab_rows_parts).

The split follows from the loss itself: with z the (scaled, capped) logits,
  loss_i = LSE_i + l·LSE_i² − (e/V)·Σ_v z_iv − (1 − e)·z_{i,y_i},
the first three terms give the dense part of the gradient and the last one the
one-hot part.  Each part is checked against torch autograd (a library routine)
of its own terms, in float64, with every option on; the two parts must add up
to the oracle's full gradient, and rows with a bad label are NaN in both.
"""
import numpy as np
import pytest
import torch

from oracle import lce_oracle as O


def small(seed, N=7, H=6, V=11, ignore=(2,)):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((N, H))
    W = rng.standard_normal((V, H)) * 0.8
    y = rng.integers(0, V, N)
    for i in ignore:
        y[i] = -100
    return X, W, y


def autograd_parts(X, W, y, opts, scale):
    """Gradients of Σ_i s_i·(dense terms) and of Σ_i s_i·(target term) w.r.t. X, W."""
    a, c = float(opts["logit_scale"]), float(opts["softcap"])
    e, lam = float(opts["label_smoothing"]), float(opts["z_loss"])
    V = W.shape[0]
    out = []
    for part in ("dense", "onehot"):
        Xt = torch.tensor(X, dtype=torch.float64, requires_grad=True)
        Wt = torch.tensor(W, dtype=torch.float64, requires_grad=True)
        z = a * (Xt @ Wt.T)
        if c > 0:
            z = c * torch.tanh(z / c)
        s = torch.tensor(scale, dtype=torch.float64)
        valid = torch.tensor(y != -100)
        if part == "dense":
            lse = torch.logsumexp(z, dim=1)
            term = lse + lam * lse * lse - (e / V) * z.sum(dim=1)
        else:
            yy = torch.tensor(np.where(y == -100, 0, y))
            term = -(1.0 - e) * z.gather(1, yy[:, None])[:, 0]
        (torch.where(valid, s * term, torch.zeros_like(term))).sum().backward()
        out.append((Xt.grad.numpy(), Wt.grad.numpy()))
    return out


CASES = [
    dict(),
    dict(softcap=2.0),
    dict(softcap=1.5, logit_scale=0.7, z_loss=0.05),
    dict(label_smoothing=0.2, logit_scale=1.3),
    dict(softcap=3.0, label_smoothing=0.1, z_loss=0.02, reduction="sum"),
    dict(softcap=2.5, z_loss=0.01, reduction="none"),
]


@pytest.mark.parametrize("kw", CASES)
def test_parts_match_autograd_of_their_terms(kw):
    X, W, y = small(seed=11)
    opts = O.options(**kw)
    f = O.forward_ex(X, W, y, opts)
    dloss = (np.random.default_rng(4).standard_normal(len(y)) if opts["reduction"] == "none"
             else 0.8)
    scale = O.row_scale(y, dloss, f["n_valid"], opts)
    (gXd, gWd), (gXo, gWo) = autograd_parts(X, W, y, opts, scale)
    rows = np.arange(len(y))
    dXd, dXo = O.dX_rows_parts(X[rows], W, y[rows], f["lse"][rows], scale[rows], opts)
    np.testing.assert_allclose(dXd, gXd, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dXo, gXo, rtol=1e-10, atol=1e-12)
    vrows = np.array([0, 3, 4, 10])
    dWd, dWo = O.dW_vocab_rows_parts(X, W, y, f["lse"], scale, vrows, opts)
    np.testing.assert_allclose(dWd, gWd[vrows], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dWo, gWo[vrows], rtol=1e-10, atol=1e-12)
    # The two parts add up to the full gradient (torch's gradient of the loss).
    dX, dW = O.backward_ex(X, W, y, dloss, opts)
    np.testing.assert_allclose(dXd + dXo, dX, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dWd + dWo, dW[vrows], rtol=1e-10, atol=1e-12)


def test_parts_of_a_subset_of_rows_and_bad_labels():
    X, W, y = small(seed=5, N=9)
    y[4] = 11                       # out of range: a bad label
    opts = O.options(softcap=2.0)
    f = O.forward_ex(X, W, y, opts)
    scale = O.row_scale(y, 1.0, f["n_valid"], opts)
    rows = np.array([1, 4, 7])
    dXd, dXo = O.dX_rows_parts(X[rows], W, y[rows], f["lse"][rows], scale[rows], opts)
    assert np.isnan(dXd[1]).all() and np.isnan(dXo[1]).all()
    assert not np.isnan(dXd[[0, 2]]).any() and not np.isnan(dXo[[0, 2]]).any()
    # An ignored row has zero in both parts; the one-hot part of a row is
    # −s·d_y·w_y (one W row), the target term alone.
    X2, W2, y2 = small(seed=6)
    f2 = O.forward_ex(X2, W2, y2, opts)
    s2 = O.row_scale(y2, 1.0, f2["n_valid"], opts)
    dXd2, dXo2 = O.dX_rows_parts(X2, W2, y2, f2["lse"], s2, opts)
    assert not dXd2[2].any() and not dXo2[2].any()
    i = 0
    z = X2[i] @ W2[y2[i]]
    d = 1.0 - np.tanh(z / 2.0) ** 2
    np.testing.assert_allclose(dXo2[i], -s2[i] * d * W2[y2[i]], rtol=1e-12, atol=1e-15)
