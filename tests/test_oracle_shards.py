"""Pins of the oracle's vocabulary-shard functions (forward_shard,
merge_shards, backward_shard), each against something other than their own
formulas:

* the worked example of the AI-infra KB page M011 (§05: two blocks of the row
  z = [0, ln2, ln3, ln4] with masses 3 and 7, target in the second block; the
  correct denominator is 10, and ln(7/3) is the mistake of using one block);
* partition independence: any split of the vocabulary into shards, merged,
  gives the full-vocabulary forward_ex / backward_ex (themselves pinned by
  torch and finite differences), for every option;
* central finite differences of the merged loss with respect to one shard's
  weights and to X, summed over the shards' dX shares.
"""
import math

import numpy as np
import pytest

from oracle import lce_oracle as O


def shards_of(W, edges):
    return [(a, W[a:b]) for a, b in zip(edges[:-1], edges[1:])]


def test_worked_example_split_in_two_shards():
    # H = 1, x = 1: the logits are the weights themselves.
    X = np.array([[1.0]])
    W = np.array([[0.0], [math.log(2)], [math.log(3)], [math.log(4)]])
    y = np.array([2])
    o = O.options()
    a = O.forward_shard(X, W[:2], y, 0, 4, o)
    b = O.forward_shard(X, W[2:], y, 2, 4, o)
    assert abs(math.exp(a["lse_part"][0]) - 3.0) < 1e-12      # mass of block A
    assert abs(math.exp(b["lse_part"][0]) - 7.0) < 1e-12      # mass of block B
    assert a["target_part"][0] == 0.0 and abs(b["target_part"][0] - math.log(3)) < 1e-15
    m = O.merge_shards([a, b], y, 4, o)
    assert abs(m["lse"][0] - math.log(10)) < 1e-12
    assert abs(m["loss"][0] - 1.203973) < 1e-6
    wrong = b["lse_part"][0] - b["target_part"][0]            # block B alone
    assert abs(wrong - 0.847298) < 1e-6
    assert abs(m["loss"][0] - wrong) > 0.3


OPTION_SETS = [
    dict(),
    dict(softcap=2.0),
    dict(softcap=1.5, logit_scale=0.7, label_smoothing=0.2, z_loss=0.05, reduction="sum"),
    dict(label_smoothing=0.1, reduction="none"),
]


@pytest.mark.parametrize("opts", OPTION_SETS)
@pytest.mark.parametrize("edges", [[0, 4, 5, 13], [0, 13], [0, 1, 2, 3, 13], [0, 6, 12, 13]])
def test_partition_independence(opts, edges):
    rng = np.random.default_rng(len(edges) * 7 + len(opts))
    N, H, V = 9, 5, 13
    X = rng.standard_normal((N, H))
    W = rng.standard_normal((V, H)) * 0.8
    y = rng.integers(0, V, N)
    y[1] = -100
    y[4] = V + 3            # bad label: NaN row on both sides
    o = O.options(**opts)
    parts = [O.forward_shard(X, Ws, y, lo, V, o) for lo, Ws in shards_of(W, edges)]
    m = O.merge_shards(parts, y, V, o)
    f = O.forward_ex(X, W, y, o)
    np.testing.assert_allclose(m["lse"], f["lse"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(m["loss"], f["loss"], rtol=0, atol=1e-13)   # NaN rows match
    assert m["n_valid"] == f["n_valid"]
    dloss = rng.standard_normal(N) if o["reduction"] == "none" else 0.8
    dX, dWs = 0.0, []
    for lo, Ws in shards_of(W, edges):
        gx, gw = O.backward_shard(X, Ws, y, m["lse"], dloss, lo, V, o)
        dX = dX + gx
        dWs.append(gw)
    rX, rW = O.backward_ex(X, W, y, dloss, o)
    np.testing.assert_allclose(dX, rX, rtol=0, atol=1e-13)
    np.testing.assert_allclose(np.concatenate(dWs), rW, rtol=0, atol=1e-13)


@pytest.mark.parametrize("reduction", ["mean", "none"])
def test_finite_differences_through_the_merge(reduction):
    rng = np.random.default_rng(21)
    N, H, V = 4, 3, 7
    X = rng.standard_normal((N, H))
    W = rng.standard_normal((V, H)) * 0.7
    y = np.array([0, 5, -100, 3])
    edges = [0, 3, 7]
    o = O.options(softcap=1.7, logit_scale=1.2, label_smoothing=0.15, z_loss=0.04,
                  reduction=reduction)
    dloss = rng.standard_normal(N) if reduction == "none" else 1.1

    def objective(Xv, Wv):
        parts = [O.forward_shard(Xv, Wv[a:b], y, a, V, o) for a, b in zip(edges[:-1], edges[1:])]
        m = O.merge_shards(parts, y, V, o)
        return float(np.dot(dloss, m["loss"])) if reduction == "none" else dloss * m["reduced"]

    lse = O.merge_shards([O.forward_shard(X, W[a:b], y, a, V, o)
                          for a, b in zip(edges[:-1], edges[1:])], y, V, o)["lse"]
    grads = [O.backward_shard(X, W[a:b], y, lse, dloss, a, V, o)
             for a, b in zip(edges[:-1], edges[1:])]
    dX = sum(g[0] for g in grads)
    dW = np.concatenate([g[1] for g in grads])
    h = 1e-6
    for A, G, is_x in ((X, dX, True), (W, dW, False)):
        num = np.zeros_like(A)
        for idx in np.ndindex(A.shape):
            Ap, Am = A.copy(), A.copy()
            Ap[idx] += h
            Am[idx] -= h
            fp = objective(Ap, W) if is_x else objective(X, Ap)
            fm = objective(Am, W) if is_x else objective(X, Am)
            num[idx] = (fp - fm) / (2 * h)
        np.testing.assert_allclose(G, num, rtol=1e-6, atol=1e-8)
