"""Pins of the oracle's gradient filter (backward_filtered):

* eps = 0 keeps every block: the result is backward_ex (pinned elsewhere);
* eps above every value removes the whole dense part: dX and dW are then the
  one-hot term alone, a closed form;
* with tiny blocks (tile = 2) a brute-force reimplementation from the
  definition (block maxima by explicit loops) agrees, and a block holding a
  single value above eps is kept while its neighbours are dropped;
* a row with an out-of-range label still gives a NaN dX row and a NaN dW.
"""
import math

import numpy as np
import pytest

from oracle import lce_oracle as O


def small(seed, N=9, H=4, V=11):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((N, H))
    W = rng.standard_normal((V, H)) * 0.9
    y = rng.integers(0, V, N)
    y[2] = -100
    return X, W, y


@pytest.mark.parametrize("opts", [dict(), dict(softcap=2.0, z_loss=0.03, reduction="sum")])
def test_eps_zero_is_exact(opts):
    X, W, y = small(1)
    o = O.options(**opts)
    dX, dW = O.backward_filtered(X, W, y, 0.7, o, 0.0, tile=2)
    rX, rW = O.backward_ex(X, W, y, 0.7, o)
    np.testing.assert_allclose(dX, rX, rtol=0, atol=1e-14)
    np.testing.assert_allclose(dW, rW, rtol=0, atol=1e-14)


def test_everything_filtered_leaves_the_onehot_term():
    X, W, y = small(2)
    o = O.options(softcap=3.0)
    dX, dW = O.backward_filtered(X, W, y, 1.0, o, 2.0, tile=3)
    n = int((y != -100).sum())
    Z = X @ W.T
    eX = np.zeros_like(X)
    eW = np.zeros_like(W)
    for i, t in enumerate(y):
        if t == -100:
            continue
        d = 1.0 - math.tanh(Z[i, t] / 3.0) ** 2
        eX[i] = -d * W[t] / n
        eW[t] -= d * X[i] / n
    np.testing.assert_allclose(dX, eX, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(dW, eW, rtol=1e-12, atol=1e-15)


def test_bruteforce_blocks_and_single_kept_block():
    X, W, y = small(3, N=6, H=3, V=8)
    W[5] *= 6.0                                   # one column with large probabilities
    o = O.options()
    f = O.forward_ex(X, W, y, o)
    P = np.exp(X @ W.T - f["lse"][:, None])
    eps = 0.5 * P[:, 5][y != -100].max()
    dX, dW = O.backward_filtered(X, W, y, 1.0, o, eps, tile=2)
    # Brute force from the definition.
    G = P.copy()
    for bi in range(3):
        for bj in range(4):
            rows = [i for i in range(2 * bi, 2 * bi + 2) if y[i] != -100]
            vals = [P[i, v] for i in rows for v in range(2 * bj, 2 * bj + 2)]
            if not vals or max(vals) < eps:
                G[2 * bi:2 * bi + 2, 2 * bj:2 * bj + 2] = 0.0
    n = int((y != -100).sum())
    for i, t in enumerate(y):
        if t == -100:
            G[i] = 0.0
        else:
            G[i, t] -= 1.0
    G /= n
    np.testing.assert_allclose(dX, G @ W, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(dW, G.T @ X, rtol=1e-12, atol=1e-15)
    kept = O.filter_block_max(X, W, y, f["lse"], o, tile=2) >= eps
    assert kept[:, 2].any() and not kept.all()


def test_out_of_range_label_still_gives_nan():
    X, W, y = small(4)
    y[4] = 50
    dX, dW = O.backward_filtered(X, W, y, 1.0, O.options(), 10.0, tile=3)
    assert np.isnan(dX[4]).all() and np.isnan(dW).all()
    assert not np.isnan(np.delete(dX, 4, axis=0)).any()


def test_smoothing_refused():
    X, W, y = small(5)
    with pytest.raises(ValueError):
        O.backward_filtered(X, W, y, 1.0, O.options(label_smoothing=0.1), 1e-3)
