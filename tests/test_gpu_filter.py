"""The opt-in gradient filter (filter_eps > 0 in lce_backward_ex and
lce_shard_backward) against the oracle's backward_filtered.

Which 256 x 256 blocks are skipped is decided by comparing a value with the
threshold; the GPU compares float32 values, the oracle float64 ones.  To keep
that decision unique, each case puts the threshold in the middle of the
widest gap (in log scale) between the oracle's block maxima near their
median and checks that no block maximum lies within 1% of it; the gradients
must then match the oracle's filtered gradients to the usual bars (rel-L2
<= 1e-3).  Also: a threshold below every value reproduces the exact path (dW
bit for bit; dX up to the order of its sums, since the exact path may split a
dX tile's vocabulary range into parts summed at the end and the filtered one
does not), one above every value leaves the one-hot term alone, and the
filter is refused with label smoothing.
"""
import numpy as np
import pytest
import torch

import lce_inputs as L
from oracle import lce_oracle as O

pytestmark = pytest.mark.gpu

GRAD_RTOL = 1e-3


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
    """A threshold in the widest log gap between block maxima around the
    median, at least 1% away from every block maximum."""
    v = np.sort(bm[np.isfinite(bm) & (bm > 0)].ravel())
    lo, hi = len(v) // 4, 3 * len(v) // 4
    gaps = np.log(v[lo + 1:hi + 1]) - np.log(v[lo:hi])
    k = lo + int(np.argmax(gaps))
    eps = float(np.sqrt(v[k] * v[k + 1]))
    assert np.all(np.abs(v / eps - 1.0) > 0.01), "no clear threshold in this case"
    return eps


CASES = [
    # N, H, V, W scale, options
    (700, 64, 3000, 6.0, dict()),
    (520, 72, 2600, 5.0, dict(softcap=4.0)),
    (600, 64, 2100, 6.0, dict(softcap=30.0, z_loss=1e-3, reduction="sum")),
]


@pytest.mark.parametrize("N,H,V,ws,opts", CASES)
def test_filter_against_oracle(lce, N, H, V, ws, opts):
    w = L.Workload("filter", N=N, H=H, V=V, labels="zipf", ignore_frac=0.1, seed=7000 + N)
    X, W, y = L.make_inputs(w)
    W = (W.float() * ws).to(torch.bfloat16)
    o = O.options(**opts)
    X64, W64, y64 = L.to_f64(X), L.to_f64(W), y.numpy()
    f = O.forward_ex(X64, W64, y64, o)
    bm = O.filter_block_max(X64, W64, y64, f["lse"], o)
    eps = pick_threshold(bm)
    kept = int((bm >= eps).sum())
    print(f"[filter] N={N} V={V} {opts} eps={eps:.3e} kept {kept} of {bm.size} blocks",
          flush=True)
    assert 0 < kept < bm.size
    dev = "cuda"
    Xd, Wd, yd = X.to(dev), W.to(dev), y.to(dev)
    out = lce.lce_forward_ex(Xd, Wd, yd, **opts)
    dX, dW = lce.lce_backward_ex(Xd, Wd, yd, out["lse"], 0.9, filter_eps=eps, **opts)
    torch.cuda.synchronize()
    rX, rW = O.backward_filtered(X64, W64, y64, 0.9, o, eps)
    eX, eW = O.backward_ex(X64, W64, y64, 0.9, o)
    e_dx, e_dw = rel_l2(dX.cpu(), rX), rel_l2(dW.cpu(), rW)
    print(f"[filter] vs filtered oracle: dX {e_dx:.2e} dW {e_dw:.2e}; filtered oracle vs "
          f"exact: dX {rel_l2(rX, eX):.2e} dW {rel_l2(rW, eW):.2e}", flush=True)
    assert e_dx <= GRAD_RTOL and e_dw <= GRAD_RTOL


def test_tiny_threshold_is_the_exact_path(lce):
    w = L.Workload("filter", N=600, H=128, V=3000, labels="zipf", ignore_frac=0.1, seed=71)
    X, W, y = (t.cuda() for t in L.make_inputs(w))
    out = lce.lce_forward_ex(X, W, y, softcap=30.0)
    a = lce.lce_backward_ex(X, W, y, out["lse"], 1.0, softcap=30.0)
    b = lce.lce_backward_ex(X, W, y, out["lse"], 1.0, softcap=30.0, filter_eps=1e-37)
    torch.cuda.synchronize()
    assert torch.equal(a[1], b[1])
    e = float(torch.linalg.vector_norm(a[0] - b[0]) / torch.linalg.vector_norm(a[0]))
    print(f"[filter] tiny threshold: dX {e:.1e} from the exact path, dW equal", flush=True)
    assert e <= 1e-6


def test_huge_threshold_leaves_the_onehot_term(lce):
    w = L.Workload("filter", N=530, H=64, V=1100, labels="uniform", ignore_frac=0.1, seed=72)
    X, W, y = L.make_inputs(w)
    out = lce.lce_forward_ex(X.cuda(), W.cuda(), y.cuda(), softcap=3.0)
    dX, dW = lce.lce_backward_ex(X.cuda(), W.cuda(), y.cuda(), out["lse"], 1.0, softcap=3.0,
                                 filter_eps=10.0)
    torch.cuda.synchronize()
    rX, rW = O.backward_filtered(L.to_f64(X), L.to_f64(W), y.numpy(), 1.0,
                                 O.options(softcap=3.0), 10.0)
    assert rel_l2(dX.cpu(), rX) <= GRAD_RTOL and rel_l2(dW.cpu(), rW) <= GRAD_RTOL


def test_filter_refused_with_smoothing(lce):
    X, W, y = (t.cuda() for t in L.make_inputs(L.Workload("v", N=8, H=8, V=10)))
    lse = lce.lce_forward_ex(X, W, y)["lse"]
    with pytest.raises(lce.LceError):
        lce.lce_backward_ex(X, W, y, lse, 1.0, label_smoothing=0.1, filter_eps=1e-3)


def test_filter_with_vocabulary_shards(lce):
    """Shards cut at multiples of 256 keep the filter blocks intact, so the
    filtered shard gradients add up to the filtered whole-vocabulary ones."""
    w = L.Workload("filter", N=700, H=64, V=3000, labels="zipf", ignore_frac=0.1, seed=7700)
    X, W, y = L.make_inputs(w)
    W = (W.float() * 6.0).to(torch.bfloat16)
    o = O.options()
    X64, W64, y64 = L.to_f64(X), L.to_f64(W), y.numpy()
    f = O.forward_ex(X64, W64, y64, o)
    eps = pick_threshold(O.filter_block_max(X64, W64, y64, f["lse"], o))
    dev = "cuda"
    Xd, Wd, yd = X.to(dev), W.to(dev), y.to(dev)
    lse = lce.lce_forward_ex(Xd, Wd, yd)["lse"]
    edges = [0, 1024, 2048, 3000]
    dX, dWs = None, []
    for a, b in zip(edges[:-1], edges[1:]):
        gx, gw = lce.lce_shard_backward(Xd, Wd[a:b], yd, lse, 1.0, a, 3000, filter_eps=eps)
        dX = gx if dX is None else dX + gx
        dWs.append(gw)
    torch.cuda.synchronize()
    rX, rW = O.backward_filtered(X64, W64, y64, 1.0, o, eps)
    assert rel_l2(dX.cpu(), rX) <= GRAD_RTOL
    assert rel_l2(torch.cat(dWs).cpu(), rW) <= GRAD_RTOL
