"""Pins of the oracle's vocabulary order (vocab_mean_logit, vocab_order) and
of the backward on a reordered vocabulary (backward_sorted):

* the average logit agrees with explicit loops over rows and columns, and
  with the closed form W·x̄ (linearity of the logit in x), and is 0 when no
  row has a target;
* the order is checked element by element: a permutation, averages never
  increasing, equal averages by increasing index, NaN first;
* without the filter, any order gives the unordered gradients (the loss does
  not depend on how the vocabulary is numbered); with the identity order the
  filtered gradients are backward_filtered's;
* with tiny blocks a brute-force version from the definition (blocks cut in
  positions, dense part dropped where a block's values all lie below eps)
  agrees;
* on a vocabulary whose large logits sit on a few scattered entries, the
  order puts them together and the filter then keeps fewer blocks, which is
  what the reordering is for.
"""
import numpy as np
import pytest

from oracle import lce_oracle as O


def small(seed, N=9, H=4, V=11):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((N, H))
    W = rng.standard_normal((V, H)) * 0.9
    y = rng.integers(0, V, N)
    y[2] = -100
    y[5] = -100
    return X, W, y


def test_mean_logit_by_loops():
    X, W, y = small(1)
    got = O.vocab_mean_logit(X, W, y)
    rows = [i for i in range(len(y)) if y[i] != -100]
    for v in range(W.shape[0]):
        tot = 0.0
        for i in rows:
            tot += sum(X[i, h] * W[v, h] for h in range(X.shape[1]))
        assert abs(got[v] - tot / len(rows)) <= 1e-12


def test_mean_logit_is_w_times_mean_row():
    X, W, y = small(2, N=40, H=7, V=30)
    xbar = X[y != -100].mean(axis=0)
    np.testing.assert_allclose(O.vocab_mean_logit(X, W, y), W @ xbar, rtol=1e-12, atol=1e-13)


def test_mean_logit_without_targets_is_zero():
    X, W, y = small(3)
    y[:] = -100
    assert np.array_equal(O.vocab_mean_logit(X, W, y), np.zeros(W.shape[0]))


def check_order(key, order):
    V = len(key)
    assert sorted(order.tolist()) == list(range(V))
    for j in range(V - 1):
        a, b = order[j], order[j + 1]
        ka, kb = key[a], key[b]
        if np.isnan(kb):
            assert np.isnan(ka) and a < b
        elif np.isnan(ka):
            continue
        else:
            assert ka > kb or (ka == kb and a < b)


def test_order_elementwise():
    key = np.array([0.5, 2.0, -1.0, 2.0, np.nan, 0.0, -0.0, 0.5, np.nan, -3.0])
    order = O.vocab_order(key)
    check_order(key, order)
    assert order.tolist() == [4, 8, 1, 3, 0, 7, 5, 6, 2, 9]


def test_order_of_duplicate_entries():
    X, W, y = small(4, N=12, H=5, V=9)
    W[6] = W[2]
    W[8] = W[2]
    key = O.vocab_mean_logit(X, W, y)
    order = O.vocab_order(key)
    check_order(key, order)
    pos = {int(v): j for j, v in enumerate(order)}
    assert pos[2] + 1 == pos[6] and pos[6] + 1 == pos[8]


@pytest.mark.parametrize("opts", [dict(), dict(softcap=2.5, z_loss=0.02),
                                  dict(label_smoothing=0.1, reduction="sum"),
                                  dict(ignore_index=3, logit_scale=0.7)])
def test_any_order_without_filter_is_the_plain_backward(opts):
    X, W, y = small(5, N=10, H=4, V=13)
    if opts.get("ignore_index") == 3:
        y[y == -100] = 3
    o = O.options(**opts)
    order = np.random.default_rng(9).permutation(W.shape[0])
    dX, dW = O.backward_sorted(X, W, y, 0.8, o, order)
    rX, rW = O.backward_ex(X, W, y, 0.8, o)
    np.testing.assert_allclose(dX, rX, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dW, rW, rtol=1e-12, atol=1e-14)


def test_identity_order_is_the_filtered_backward():
    X, W, y = small(6, N=10, H=4, V=13)
    o = O.options(softcap=3.0)
    f = O.forward_ex(X, W, y, o)
    bm = O.filter_block_max(X, W, y, f["lse"], o, tile=3)
    eps = float(np.median(bm[np.isfinite(bm)]))
    dX, dW = O.backward_sorted(X, W, y, 1.0, o, np.arange(13), eps, tile=3)
    rX, rW = O.backward_filtered(X, W, y, 1.0, o, eps, tile=3)
    assert np.array_equal(dX, rX) and np.array_equal(dW, rW)


def test_bruteforce_blocks_in_positions():
    X, W, y = small(7, N=6, H=3, V=8)
    W[[1, 6]] *= 5.0                              # two entries with large probabilities
    order = np.array([6, 1, 0, 2, 3, 4, 5, 7])   # ... moved into positions 0 and 1
    t, eps = 2, 0.02
    N, V = X.shape[0], W.shape[0]
    Z = X @ W.T
    lse = np.log(np.exp(Z).sum(axis=1))
    P = np.exp(Z - lse[:, None])
    valid = y != -100
    n = int(valid.sum())
    pos = np.empty(V, dtype=int)
    pos[order] = np.arange(V)
    G = np.zeros((N, V))
    for i in range(N):
        if not valid[i]:
            continue
        for v in range(V):
            bi, bj = i // t, pos[v] // t
            blk = [P[r, order[c]] for r in range(bi * t, min(N, bi * t + t)) if valid[r]
                   for c in range(bj * t, bj * t + t)]
            keep = max(blk) >= eps
            G[i, v] = ((P[i, v] if keep else 0.0) - (1.0 if v == y[i] else 0.0)) / n
    dX, dW = O.backward_sorted(X, W, y, 1.0, O.options(), order, eps, tile=t)
    np.testing.assert_allclose(dX, G @ W, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(dW, G.T @ X, rtol=1e-12, atol=1e-15)
    # The dropped part is not empty and not everything.
    full = O.backward_ex(X, W, y, 1.0, O.options())
    assert not np.allclose(dW, full[1]) and np.abs(dW).max() > 0


def test_order_gathers_hot_entries_and_the_filter_keeps_fewer_blocks():
    rng = np.random.default_rng(11)
    N, H, V, tile = 512, 16, 2048, 256
    u = np.zeros(H)
    u[0] = 1.0
    X = rng.standard_normal((N, H)) + 2.0 * u
    W = rng.standard_normal((V, H)) * 0.3
    hot = rng.choice(V, 96, replace=False)        # scattered over every block
    W[hot] += 2.5 * u
    y = rng.integers(0, V, N)
    o = O.options()
    order = O.vocab_order(O.vocab_mean_logit(X, W, y))
    assert set(order[:96].tolist()) == set(hot.tolist())
    pos = np.empty(V, dtype=int)
    pos[order] = np.arange(V)
    lse = O.forward_ex(X, W, y, o)["lse"]
    natural = O.filter_block_max(X, W, y, lse, o, tile)
    moved = O.filter_block_max(X, W[order], pos[y], lse, o, tile)
    # With 2048 entries the probabilities are large; this threshold lies above
    # every cold block once the hot entries have been gathered, and below every
    # block of the natural order.
    eps = 2.0 ** -4
    kept_nat, kept_sorted = int((natural >= eps).sum()), int((moved >= eps).sum())
    assert kept_nat == natural.size and kept_sorted <= natural.size // 2
