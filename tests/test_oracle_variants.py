"""Pins of the oracle's loss variants (logit scale, label smoothing, Z-loss,
reduction), each against something other than the oracle's own formula:

* torch.nn.functional.cross_entropy in float64 (a library routine) for label
  smoothing and the three reductions, and its autograd for the gradients;
* closed forms at W = 0, where every logit is 0 and p = 1/V exactly;
* central finite differences of the reduced loss, all options on at once;
* invariances: a logit scale a on W is the same as a on the product;
  "none" with a uniform upstream gradient is "sum"; "sum" is "mean" · n_valid.
"""
import math

import numpy as np
import pytest
import torch

from oracle import lce_oracle as O


def small(seed=0, N=6, H=5, V=9, ignore=(2,)):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((N, H))
    W = rng.standard_normal((V, H)) * 0.7
    y = rng.integers(0, V, N)
    for i in ignore:
        y[i] = -100
    return X, W, y


def torch_loss(X, W, y, softcap, scale, eps, reduction):
    Xt = torch.tensor(X, dtype=torch.float64, requires_grad=True)
    Wt = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    z = scale * (Xt @ Wt.T)
    if softcap > 0:
        z = softcap * torch.tanh(z / softcap)
    loss = torch.nn.functional.cross_entropy(z, torch.tensor(y), ignore_index=-100,
                                             label_smoothing=eps, reduction=reduction)
    return loss, Xt, Wt


@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
@pytest.mark.parametrize("softcap,scale,eps", [(0.0, 1.0, 0.1), (2.0, 0.5, 0.3), (0.0, 1.7, 0.0)])
def test_label_smoothing_and_reduction_match_torch(reduction, softcap, scale, eps):
    X, W, y = small(seed=3)
    opts = O.options(softcap=softcap, logit_scale=scale, label_smoothing=eps, reduction=reduction)
    f = O.forward_ex(X, W, y, opts)
    loss, Xt, Wt = torch_loss(X, W, y, softcap, scale, eps, reduction)
    if reduction == "none":
        np.testing.assert_allclose(f["loss"], loss.detach().numpy(), rtol=1e-12, atol=1e-12)
        dloss = np.random.default_rng(5).standard_normal(len(y))
        loss.backward(torch.tensor(dloss))
    else:
        assert abs(f["reduced"] - loss.item()) < 1e-12
        dloss = 0.73
        (loss * dloss).backward()
    dX, dW = O.backward_ex(X, W, y, dloss, opts)
    np.testing.assert_allclose(dX, Xt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dW, Wt.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_zero_weight_closed_forms():
    # W = 0: z = 0, LSE = ln V, p = 1/V; the smoothing and Z-loss terms are
    # then plain numbers.
    N, H, V = 7, 4, 11
    rng = np.random.default_rng(1)
    X = rng.standard_normal((N, H))
    W = np.zeros((V, H))
    y = rng.integers(0, V, N)
    y[3] = -100
    eps, lam, dl = 0.2, 0.05, 1.3
    opts = O.options(label_smoothing=eps, z_loss=lam, reduction="sum", logit_scale=2.0)
    f = O.forward_ex(X, W, y, opts)
    valid = y != -100
    lnV = math.log(V)
    np.testing.assert_allclose(f["loss"][valid], lnV + lam * lnV * lnV, rtol=1e-14)
    assert f["loss"][3] == 0.0
    # dL/dz_v = (1 + 2 lam lnV)/V - (1 - eps)[v = y] - eps/V, times a = 2.
    dX, dW = O.backward_ex(X, W, y, dl, opts)
    assert np.all(dX == 0)
    expect = np.zeros((V, H))
    for i in np.nonzero(valid)[0]:
        g = np.full(V, (1 + 2 * lam * lnV) / V - eps / V)
        g[y[i]] -= (1 - eps)
        expect += 2.0 * dl * np.outer(g, X[i])
    np.testing.assert_allclose(dW, expect, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_finite_differences_all_options(reduction):
    X, W, y = small(seed=7, N=5, H=4, V=6, ignore=(1,))
    opts = O.options(softcap=1.5, logit_scale=0.8, label_smoothing=0.25, z_loss=0.07,
                     reduction=reduction)
    rng = np.random.default_rng(11)
    dloss = rng.standard_normal(len(y)) if reduction == "none" else 0.9

    def L(Xv, Wv):
        f = O.forward_ex(Xv, Wv, y, opts)
        if reduction == "none":
            return float(np.dot(dloss, f["loss"]))
        return dloss * f["reduced"]

    dX, dW = O.backward_ex(X, W, y, dloss, opts)
    h = 1e-6
    for (A, G) in ((X, dX), (W, dW)):
        num = np.zeros_like(A)
        for idx in np.ndindex(A.shape):
            Ap, Am = A.copy(), A.copy()
            Ap[idx] += h
            Am[idx] -= h
            if A is X:
                num[idx] = (L(Ap, W) - L(Am, W)) / (2 * h)
            else:
                num[idx] = (L(X, Ap) - L(X, Am)) / (2 * h)
        np.testing.assert_allclose(G, num, rtol=1e-6, atol=1e-8)


def test_logit_scale_is_a_scale_of_W():
    X, W, y = small(seed=9)
    a = 1.9
    f1 = O.forward_ex(X, W, y, O.options(logit_scale=a, softcap=3.0, label_smoothing=0.1))
    f2 = O.forward_ex(X, a * W, y, O.options(softcap=3.0, label_smoothing=0.1))
    np.testing.assert_allclose(f1["loss"], f2["loss"], rtol=1e-13)
    dX1, dW1 = O.backward_ex(X, W, y, 1.0, O.options(logit_scale=a, softcap=3.0, label_smoothing=0.1))
    dX2, dW2 = O.backward_ex(X, a * W, y, 1.0, O.options(softcap=3.0, label_smoothing=0.1))
    np.testing.assert_allclose(dX1, dX2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dW1, a * dW2, rtol=1e-12, atol=1e-14)


def test_reduction_relations():
    X, W, y = small(seed=13)
    base = dict(softcap=2.0, label_smoothing=0.2, z_loss=0.03)
    fm = O.forward_ex(X, W, y, O.options(reduction="mean", **base))
    fs = O.forward_ex(X, W, y, O.options(reduction="sum", **base))
    assert abs(fs["reduced"] - fm["reduced"] * fm["n_valid"]) < 1e-12
    dXs, dWs = O.backward_ex(X, W, y, 0.4, O.options(reduction="sum", **base))
    dXn, dWn = O.backward_ex(X, W, y, np.full(len(y), 0.4), O.options(reduction="none", **base))
    np.testing.assert_allclose(dXs, dXn, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(dWs, dWn, rtol=1e-13, atol=1e-15)
    dXm, _ = O.backward_ex(X, W, y, 0.4 * fm["n_valid"], O.options(reduction="mean", **base))
    np.testing.assert_allclose(dXs, dXm, rtol=1e-12, atol=1e-15)


def test_defaults_reduce_to_the_plain_path():
    X, W, y = small(seed=17)
    f = O.forward_ex(X, W, y, O.options(softcap=1.2))
    g = O.forward(X, W, y, softcap=1.2)
    np.testing.assert_allclose(f["loss"], g["loss"], rtol=1e-14)
    assert abs(f["reduced"] - g["mean"]) < 1e-14
    dX1, dW1 = O.backward_ex(X, W, y, 0.6, O.options(softcap=1.2))
    dX2, dW2 = O.backward(X, W, y, 0.6, softcap=1.2)
    np.testing.assert_allclose(dX1, dX2, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(dW1, dW2, rtol=1e-13, atol=1e-15)
