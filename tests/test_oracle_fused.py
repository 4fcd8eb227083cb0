"""Pins of the oracle's row-chunked forward-with-gradient
(forward_backward_chunked):

* torch.nn.functional.cross_entropy in float64 and its autograd (a library
  routine) give the same loss and gradients;
* for every chunk size (one row, ragged, the whole batch, more than the
  batch) it equals forward_ex followed by backward_ex, with every option;
* the loss, the gradients and n_valid do not depend on the chunk size.
"""
import numpy as np
import pytest
import torch

from oracle import lce_oracle as O


def small(seed, N=11, H=6, V=17):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((N, H))
    W = rng.standard_normal((V, H)) * 0.7
    y = rng.integers(0, V, N)
    y[3] = -100
    return X, W, y


@pytest.mark.parametrize("softcap", [0.0, 2.5])
def test_matches_torch_autograd(softcap):
    X, W, y = small(1)
    Xt = torch.tensor(X, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    z = Xt @ Wt.T
    if softcap > 0:
        z = softcap * torch.tanh(z / softcap)
    loss = torch.nn.functional.cross_entropy(z, torch.tensor(y), ignore_index=-100)
    (0.9 * loss).backward()
    f, dX, dW = O.forward_backward_chunked(X, W, y, 0.9, O.options(softcap=softcap), 4)
    assert abs(f["reduced"] - loss.item()) < 1e-12
    np.testing.assert_allclose(dX, Xt.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(dW, Wt.grad.numpy(), rtol=1e-10, atol=1e-13)


OPTS = [dict(), dict(softcap=3.0, logit_scale=0.8, z_loss=0.02),
        dict(label_smoothing=0.15, reduction="sum"), dict(softcap=1.5, reduction="none"),
        dict(label_smoothing=0.05, z_loss=0.01, logit_scale=1.4, reduction="none")]


@pytest.mark.parametrize("opts", OPTS)
@pytest.mark.parametrize("chunk", [1, 4, 11, 40])
def test_equals_forward_then_backward(opts, chunk):
    X, W, y = small(2 + chunk)
    o = O.options(**opts)
    rng = np.random.default_rng(chunk)
    dloss = rng.standard_normal(len(y)) if o["reduction"] == "none" else 1.3
    f, dX, dW = O.forward_backward_chunked(X, W, y, dloss, o, chunk)
    g = O.forward_ex(X, W, y, o)
    rX, rW = O.backward_ex(X, W, y, dloss, o)
    np.testing.assert_allclose(f["lse"], g["lse"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(f["loss"], g["loss"], rtol=0, atol=1e-13)
    assert f["n_valid"] == g["n_valid"] and abs(f["reduced"] - g["reduced"]) < 1e-12
    np.testing.assert_allclose(dX, rX, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dW, rW, rtol=0, atol=1e-13)


def test_out_of_range_label_gives_nan_row_and_nan_dw():
    X, W, y = small(5)
    y[6] = 99
    f, dX, dW = O.forward_backward_chunked(X, W, y, 1.0, O.options(), 3)
    assert np.isnan(f["loss"][6]) and np.isnan(f["reduced"])
    assert np.isnan(dX[6]).all() and not np.isnan(np.delete(dX, 6, axis=0)).any()
    assert np.isnan(dW).all()
