"""The vocabulary order (lce_vocab_order) and the backward on a reordered
vocabulary (lce_backward_sorted) against the oracle.

* Averages: within 3e-5 of Σ_h |w_vh|·mean|x_h| (float32 column sums and dot
  products against float64).  The order has several valid answers where
  averages are closer than that, so it is checked for what is unique: it is a
  permutation, the GPU's own averages never increase along it and equal ones
  come by increasing index, and the oracle's averages never increase along
  it beyond the two tolerances.
* The sorted backward takes its order from the oracle (vocab_order of
  vocab_mean_logit), so both sides cut the same filter blocks; the threshold
  is put in the widest gap of the oracle's block maxima (hot entries against
  the rest), so no block lies near it; rel-L2 <= 1e-3 against
  backward_sorted.  Without the filter a random order
  must give the plain gradients (backward_ex), and the identity order the
  plain GPU path bit for bit.
* At the Gemma-2 head size: averages on sampled entries, the order's validity,
  and the sorted backward with that order against the stored oracle samples
  of the plain backward (an order does not change the exact gradients).
"""
import os

import numpy as np
import pytest
import torch

import lce_inputs as L
from tests import fullsize_samples as FS
from oracle import lce_oracle as O

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
GRAD_RTOL = 1e-3
KEY_RTOL = 3e-5


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


def pick_threshold(bm):
    """A threshold in the widest log gap between block maxima (on these inputs:
    between the blocks holding hot entries and the rest), at least 1% away
    from every block maximum."""
    v = np.sort(bm[np.isfinite(bm) & (bm > 0)].ravel())
    gaps = np.log(v[1:]) - np.log(v[:-1])
    k = int(np.argmax(gaps))
    eps = float(np.sqrt(v[k] * v[k + 1]))
    assert np.all(np.abs(v / eps - 1.0) > 0.01), "no clear threshold in this case"
    return eps


def hot_inputs(N, H, V, n_hot, seed, labels="zipf"):
    """Seeded inputs whose large logits sit on n_hot scattered entries: the
    rows share a mean direction (hidden unit 0) and the hot entries' weights
    point along it."""
    w = L.Workload("sorted", N=N, H=H, V=V, labels=labels, ignore_frac=0.1, seed=seed)
    X, W, y = L.make_inputs(w)
    g = torch.Generator().manual_seed(seed + 1)
    hot = torch.randperm(V, generator=g)[:n_hot]
    Xf, Wf = X.float(), W.float()
    Xf[:, 0] += 2.0
    Wf[hot, 0] += 2.5
    return Xf.to(torch.bfloat16), Wf.to(torch.bfloat16), y


def key_tolerance(X64, W64, y, ignore_index=L.IGNORE_INDEX):
    rows = y != ignore_index
    m = np.abs(X64[rows]).mean(axis=0) if rows.any() else np.zeros(X64.shape[1])
    return KEY_RTOL * (np.abs(W64) @ m) + 1e-7


def check_order(key_gpu, order, key_ref, tol):
    V = len(order)
    assert np.array_equal(np.sort(order), np.arange(V)), "not a permutation"
    kg = key_gpu[order].astype(np.float64)
    d = kg[:-1] - kg[1:]
    assert (d >= 0).all(), "the GPU's averages increase along its order"
    eq = d == 0
    assert (order[:-1][eq] < order[1:][eq]).all(), "equal averages out of index order"
    kr, t = key_ref[order], tol[order]
    worst = float((kr[1:] - kr[:-1] - t[:-1] - t[1:]).max())
    assert worst <= 0, f"oracle averages increase along the order by {worst:.3e}"


ORDER_CASES = [
    # N, H, V, hot entries (0: plain inputs)
    (256, 64, 1000, 0),
    (700, 72, 3000, 40),
    (100, 8, 40, 0),
    (2048, 64, 40000, 64),
]


@pytest.mark.parametrize("N,H,V,n_hot", ORDER_CASES)
def test_order_against_oracle(lce, N, H, V, n_hot):
    print(f"[order] N={N} H={H} V={V} hot={n_hot}", flush=True)
    if n_hot:
        X, W, y = hot_inputs(N, H, V, n_hot, seed=8100 + N)
    else:
        X, W, y = L.make_inputs(L.Workload("order", N=N, H=H, V=V, labels="uniform",
                                           ignore_frac=0.1, seed=8000 + N))
    key, order = lce.lce_vocab_order(X.cuda(), W.cuda(), y.cuda())
    torch.cuda.synchronize()
    X64, W64, y64 = L.to_f64(X), L.to_f64(W), y.numpy()
    ref = O.vocab_mean_logit(X64, W64, y64)
    tol = key_tolerance(X64, W64, y64)
    kg = key.cpu().numpy()
    err = np.abs(kg - ref) / tol * KEY_RTOL
    print(f"[order] average max err / scale {err.max():.2e}", flush=True)
    assert (np.abs(kg - ref) <= tol).all()
    check_order(kg, order.cpu().numpy(), ref, tol)


def test_order_ties_and_no_targets(lce):
    X, W, y = L.make_inputs(L.Workload("order", N=300, H=16, V=700, labels="uniform",
                                       ignore_frac=0.1, seed=8200))
    W[6] = W[2]
    W[8] = W[2]
    W[699] = W[2]
    key, order = lce.lce_vocab_order(X.cuda(), W.cuda(), y.cuda())
    o = order.cpu().numpy()
    pos = np.empty_like(o)
    pos[o] = np.arange(len(o))
    assert pos[2] + 1 == pos[6] and pos[6] + 1 == pos[8] and pos[8] + 1 == pos[699]
    assert torch.equal(key[2], key[699])
    # No row with a target: every average is 0 and the order is the identity.
    y_none = torch.full_like(y, L.IGNORE_INDEX)
    key, order = lce.lce_vocab_order(X.cuda(), W.cuda(), y_none.cuda())
    assert (key.cpu() == 0).all() and torch.equal(order.cpu(), torch.arange(700, dtype=torch.int32))
    # No rows at all.
    key, order = lce.lce_vocab_order(X[:0].cuda(), W.cuda(), y[:0].cuda())
    torch.cuda.synchronize()
    assert (key.cpu() == 0).all() and torch.equal(order.cpu(), torch.arange(700, dtype=torch.int32))


@pytest.mark.parametrize("dW_dtype", [torch.float32, torch.bfloat16])
def test_identity_order_is_the_plain_backward(lce, dW_dtype):
    """Identity order: the gathered W chunk equals the slice and the dW rows go
    back where they came from, so every operation and its order match."""
    X, W, y = hot_inputs(2048, 64, 40000, 64, seed=8300)
    Xd, Wd, yd = X.cuda(), W.cuda(), y.cuda()
    lse = lce.lce_forward_ex(Xd, Wd, yd, softcap=30.0)["lse"]
    ident = torch.arange(40000, dtype=torch.int32, device="cuda")
    for eps in (0.0, 2.0 ** -12):
        a = lce.lce_backward_ex(Xd, Wd, yd, lse, 0.9, softcap=30.0, dW_dtype=dW_dtype,
                                filter_eps=eps)
        b = lce.lce_backward_sorted(Xd, Wd, yd, lse, 0.9, ident, softcap=30.0,
                                    dW_dtype=dW_dtype, filter_eps=eps)
        torch.cuda.synchronize()
        print(f"[sorted] identity order, eps={eps}, dW {dW_dtype}", flush=True)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


SORTED_CASES = [
    # N, H, V, hot entries, options, filter, dW dtype
    (2048, 64, 40000, 64, dict(), True, torch.float32),
    (700, 64, 3000, 40, dict(softcap=30.0, z_loss=1e-3, reduction="sum"), True, torch.bfloat16),
    (600, 72, 2600, 0, dict(softcap=4.0), False, torch.float32),
    (520, 64, 2100, 30, dict(ignore_index=3, logit_scale=0.8), True, torch.float32),
]


@pytest.mark.parametrize("N,H,V,n_hot,opts,filt,dW_dtype", SORTED_CASES)
def test_sorted_backward_against_oracle(lce, N, H, V, n_hot, opts, filt, dW_dtype):
    if n_hot:
        X, W, y = hot_inputs(N, H, V, n_hot, seed=8400 + N)
    else:
        X, W, y = L.make_inputs(L.Workload("sorted", N=N, H=H, V=V, labels="zipf",
                                           ignore_frac=0.1, seed=8400 + N))
    if "ignore_index" in opts:
        y = torch.where(y == L.IGNORE_INDEX, torch.full_like(y, opts["ignore_index"]), y)
    o = O.options(**opts)
    X64, W64, y64 = L.to_f64(X), L.to_f64(W), y.numpy()
    if filt:
        order = O.vocab_order(O.vocab_mean_logit(X64, W64, y64, int(o["ignore_index"])))
    else:
        order = np.random.default_rng(N).permutation(V)
    eps = 0.0
    if filt:
        pos = np.empty(V, dtype=np.int64)
        pos[order] = np.arange(V)
        ignored = y64 == int(o["ignore_index"])
        moved = ~ignored & (y64 >= 0) & (y64 < V)
        y_pos = y64.copy()
        y_pos[moved] = pos[y64[moved]]
        y_pos[ignored] = -1000          # a marker no position takes
        f = O.forward_ex(X64, W64, y64, o)
        bm_pos = O.filter_block_max(X64, W64[order], y_pos, f["lse"], dict(o, ignore_index=-1000))
        eps = pick_threshold(bm_pos)
        bm_nat = O.filter_block_max(X64, W64, y64, f["lse"], o)
        kept_pos, kept_nat = int((bm_pos >= eps).sum()), int((bm_nat >= eps).sum())
        print(f"[sorted] eps={eps:.3e}: blocks kept {kept_pos} of {bm_pos.size} in order, "
              f"{kept_nat} unordered", flush=True)
        assert 0 < kept_pos < kept_nat
    print(f"[sorted] N={N} H={H} V={V} hot={n_hot} {opts} filter={filt} dW {dW_dtype}",
          flush=True)
    Xd, Wd, yd = X.cuda(), W.cuda(), y.cuda()
    fw = {k: v for k, v in opts.items()}
    lse = lce.lce_forward_ex(Xd, Wd, yd, **fw)["lse"]
    od = torch.from_numpy(order.astype(np.int32)).cuda()
    dX, dW = lce.lce_backward_sorted(Xd, Wd, yd, lse, 0.9, od, dW_dtype=dW_dtype,
                                     filter_eps=eps, **fw)
    torch.cuda.synchronize()
    rX, rW = O.backward_sorted(X64, W64, y64, 0.9, o, order, eps)
    e_dx, e_dw = rel_l2(dX.float().cpu(), rX), rel_l2(dW.float().cpu(), rW)
    print(f"[sorted] dX {e_dx:.2e} dW {e_dw:.2e}", flush=True)
    bar = 1e-2 if dW_dtype == torch.bfloat16 else GRAD_RTOL
    assert e_dx <= GRAD_RTOL and e_dw <= bar
    if not filt:
        eX, eW = O.backward_ex(X64, W64, y64, 0.9, o)
        assert rel_l2(dX.cpu(), eX) <= GRAD_RTOL and rel_l2(dW.float().cpu(), eW) <= bar


def test_fullsize_gemma_order_and_sorted_backward(lce):
    name = "gemma2_2b"
    gold = np.load(os.path.join(HERE, "golden", f"fullsize_{name}.npz"))
    w = L.WORKLOADS[name]
    print(f"[sorted] {name} full size: N={w.N} H={w.H} V={w.V} softcap={w.softcap}", flush=True)
    X, W, y = L.make_inputs(w)
    assert L.fingerprint(X, W, y) == str(gold["fingerprint"]), "seeded inputs changed"
    Xd, Wd, yd = X.cuda(), W.cuda(), y.cuda()
    key, order = lce.lce_vocab_order(Xd, Wd, yd)
    lse = lce.lce_forward(Xd, Wd, yd, L.IGNORE_INDEX, w.softcap)["lse"]
    dX, dW = lce.lce_backward_sorted(Xd, Wd, yd, lse, 1.0, order, softcap=w.softcap)
    torch.cuda.synchronize()
    print(f"[sorted] {name}: GPU done", flush=True)
    # Averages on sampled entries (the first and last of the order among them).
    kg, og = key.cpu().numpy(), order.cpu().numpy()
    rng = np.random.default_rng(5)
    sample = np.unique(np.concatenate([rng.choice(w.V, 60, replace=False), og[:2], og[-2:]]))
    X64, W64, y64 = L.to_f64(X), L.to_f64(W[torch.from_numpy(sample)]), y.numpy()
    ref = O.vocab_mean_logit(X64, W64, y64)
    tol = key_tolerance(X64, W64, y64)
    assert (np.abs(kg[sample] - ref) <= tol).all()
    # The order itself, on the GPU's own averages.
    assert np.array_equal(np.sort(og), np.arange(w.V))
    ks = kg[og].astype(np.float64)
    d = ks[:-1] - ks[1:]
    assert (d >= 0).all() and (og[:-1][d == 0] < og[1:][d == 0]).all()
    # The exact gradients do not depend on the order.
    dx_rows = torch.from_numpy(gold["dx_rows"]).cuda()
    dw_rows = torch.from_numpy(gold["dw_rows"]).cuda()
    e_dx = rel_l2(dX[dx_rows].cpu(), gold["dX"])
    e_dw = rel_l2(dW[dw_rows].cpu(), gold["dW"])
    print(f"[sorted] {name}: dX rel {e_dx:.2e} dW rel {e_dw:.2e}", flush=True)
    assert e_dx <= GRAD_RTOL and e_dw <= GRAD_RTOL
    S = FS.samples(name, X, W, y, dict(softcap=w.softcap))
    FS.check(f"sorted {name}", dX, dW, S, GRAD_RTOL, 1e-2, log=lambda m: print(m, flush=True))
