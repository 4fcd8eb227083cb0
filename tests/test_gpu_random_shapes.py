"""Seeded random shapes and options against the oracle.

The grids depend on the shape in several ways: forward launches of 32 token
tiles, logit-gradient rounds past 32 token tiles, K parts of the dX tiles
with few token tiles, the chunk width (bound by W's size, a floor set by H,
a cap of 2^21 columns), ragged rows, vocabulary and K.  Fixed cases cover
each rule on its own; these draw (N, H, V, softcap, loss options) from a
seeded generator over ranges where the rules meet in combinations nobody
picked by hand, with the oracle cost bounded (N·V ≤ 4e7, N·V·H ≤ 4e9).

Bars: per-row LSE and loss abs ≤ 2e-3, reduced loss rel ≤ 1e-4, dX and dW
rel-L2 ≤ 1e-3 (float32 outputs), n_valid exact.  The rel-L2 denominators
are floored at 1e-2 of the one-hot terms' norm (grad_floors): with one class
the exact gradient is zero.  The reduced loss also gets
an absolute allowance of 2^-20 times the mean (or, for the sum, the sum) of
|LSE|: each row's loss is LSE − z formed in float32, so it carries a few ulps
of LSE whatever its own size, and where the loss is mostly cancellation (one
class: LSE = z and only the Z-loss term is left) a purely relative bar on a
value near zero asks for more than float32 holds.
"""
import math

import numpy as np
import pytest
import torch

import lce_inputs as L
from oracle import lce_oracle as O

pytestmark = pytest.mark.gpu

N_CASES = 48


def log_uniform(rng, lo, hi):
    return int(round(math.exp(rng.uniform(math.log(lo), math.log(hi)))))


def draw(k):
    """Case k: three regimes in turn, (a) any N up to 3000 with vocabularies
    up to 70000 (several chunks, few token tiles), (b) 33 to 80 token tiles
    with small vocabularies (forward groups, gradient rounds), (c) H from 512
    to 1024 with mid-size N and V (chunk-width floor, dX parts, dealing)."""
    rng = np.random.default_rng(90_000 + k)
    regime = k % 3
    while True:
        if regime == 0:
            N, H, V = log_uniform(rng, 1, 3000), 8 * int(rng.integers(1, 65)), log_uniform(rng, 1, 70000)
        elif regime == 1:
            N, H, V = int(rng.integers(8193, 20481)), 8 * int(rng.integers(1, 33)), log_uniform(rng, 100, 3000)
        else:
            N, H, V = log_uniform(rng, 256, 4096), 8 * int(rng.integers(64, 129)), log_uniform(rng, 1000, 20000)
        if N * V <= 4e7 and N * V * H <= 4e9:
            break
    softcap = float(rng.choice([0.0, 0.0, 30.0, 2.5]))
    opts = {}
    if rng.random() < 0.5:
        kind = int(rng.integers(0, 4))
        if kind == 0:
            opts = dict(label_smoothing=0.1)
        elif kind == 1:
            opts = dict(z_loss=1e-3, reduction="sum")
        elif kind == 2:
            opts = dict(logit_scale=0.7, reduction="none")
        else:
            opts = dict(label_smoothing=0.05, z_loss=1e-3)
    labels = "zipf" if rng.random() < 0.5 else "uniform"
    return N, H, V, softcap, opts, labels


@pytest.fixture(scope="module")
def lce():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_cross_entropy_lse_amd as P
    P.load()
    return P


def rel_l2(a, b, floor=1e-300):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), floor))


def grad_floors(X, W, y, dloss, red, softcap, opts):
    """Floors for the denominators of the gradient errors: 1e-2 of the norms of
    the one-hot terms s_i·w_{y_i} (dX) and Σ_{y_i = v} s_i·x_i (dW).  With one
    class and no Z-loss the exact gradient is zero (softmax 1 minus target 1)
    and its float64 value is rounding noise; a relative error against it means
    nothing, and the floor turns it into an error relative to the size the
    gradient's terms have.  The float32 softmax value there is 1 within a few
    ulps of its base-2 exponent arithmetic (logit scale, softcap), about 1e-6,
    so the floor sits a decade above that times the 1e-3 bar.  Wherever the
    gradient is not nearly zero its norm is far above the floor."""
    o = O.options(softcap=softcap, **opts)
    y64 = y.numpy()
    X64, W64 = L.to_f64(X), L.to_f64(W)
    valid = y64 != L.IGNORE_INDEX
    n_valid = int(valid.sum())
    s = O.row_scale(y64, dloss.astype(np.float64) if red == "none" else 0.9, n_valid, o)
    yv = np.where(valid, y64, 0)
    dx_oh = s[:, None] * W64[yv]
    dw_oh = np.zeros_like(W64)
    np.add.at(dw_oh, yv[valid], s[valid, None] * X64[valid])
    return 1e-2 * np.linalg.norm(dx_oh), 1e-2 * np.linalg.norm(dw_oh)


@pytest.mark.parametrize("k", range(N_CASES))
def test_random_shape(lce, k):
    N, H, V, softcap, opts, labels = draw(k)
    print(f"[random] case {k}: N={N} H={H} V={V} softcap={softcap} {opts} {labels}", flush=True)
    w = L.Workload("random", N=N, H=H, V=V, labels=labels, ignore_frac=0.1, softcap=softcap,
                   seed=91_000 + k)
    X, W, y = L.make_inputs(w)
    W = (W.float() * 4.0).to(torch.bfloat16)
    red = opts.get("reduction", "mean")
    rng = np.random.default_rng(92_000 + k)
    dloss = rng.standard_normal(N).astype(np.float32) if red == "none" else np.float32(0.9)
    dev = "cuda"
    Xd, Wd, yd = X.to(dev), W.to(dev), y.to(dev)
    out = lce.lce_forward_ex(Xd, Wd, yd, softcap=softcap, **opts)
    dX, dW = lce.lce_backward_ex(Xd, Wd, yd, out["lse"],
                                 torch.from_numpy(np.atleast_1d(dloss)).to(dev),
                                 softcap=softcap, **opts)
    torch.cuda.synchronize()
    o = O.options(softcap=softcap, **opts)
    X64, W64, y64 = L.to_f64(X), L.to_f64(W), y.numpy()
    f = O.forward_ex(X64, W64, y64, o)
    rdX, rdW = O.backward_ex(X64, W64, y64, dloss.astype(np.float64) if red == "none" else 0.9, o)
    assert int(out["n_valid"]) == f["n_valid"]
    np.testing.assert_allclose(out["lse"].cpu().numpy(), f["lse"], rtol=0, atol=2e-3)
    np.testing.assert_allclose(out["loss"].cpu().numpy(), f["loss"], rtol=0, atol=2e-3)
    if red != "none" and f["n_valid"] > 0:
        valid = y64 != L.IGNORE_INDEX
        lse_mass = np.abs(f["lse"][valid]).sum() / (f["n_valid"] if red == "mean" else 1)
        tol = 1e-4 * abs(f["reduced"]) + 2.0 ** -20 * lse_mass
        assert abs(float(out["reduced"]) - f["reduced"]) <= tol
    fx, fw = grad_floors(X, W, y, dloss, red, softcap, opts)
    e = (rel_l2(dX.cpu(), rdX, fx), rel_l2(dW.cpu(), rdW, fw))
    print(f"[random] case {k}: dX {e[0]:.2e} dW {e[1]:.2e}", flush=True)
    assert max(e) <= 1e-3, e


N_FUSED = 24


@pytest.mark.parametrize("k", range(N_FUSED))
def test_random_shape_fused_call(lce, k):
    """The row-chunked fused call (its own grids: even row chunks of whole
    256-row tiles, split-K dX per chunk, accumulating dW) on the same kind of draws,
    against the oracle's forward_backward_chunked.  The call takes label
    smoothing only without a softcap, so a draw with both drops the smoothing."""
    N, H, V, softcap, opts, labels = draw(1000 + k)
    if softcap > 0 and "label_smoothing" in opts:
        opts = {a: b for a, b in opts.items() if a != "label_smoothing"}
    print(f"[random fused] case {k}: N={N} H={H} V={V} softcap={softcap} {opts} {labels}",
          flush=True)
    w = L.Workload("random", N=N, H=H, V=V, labels=labels, ignore_frac=0.1, softcap=softcap,
                   seed=93_000 + k)
    X, W, y = L.make_inputs(w)
    W = (W.float() * 4.0).to(torch.bfloat16)
    red = opts.get("reduction", "mean")
    rng = np.random.default_rng(94_000 + k)
    dloss = rng.standard_normal(N).astype(np.float32) if red == "none" else np.float32(0.9)
    dev = "cuda"
    out, dX, dW = lce.lce_forward_backward(X.to(dev), W.to(dev), y.to(dev),
                                           torch.from_numpy(np.atleast_1d(dloss)).to(dev),
                                           softcap=softcap, **opts)
    torch.cuda.synchronize()
    o = O.options(softcap=softcap, **opts)
    y64 = y.numpy()
    f, rdX, rdW = O.forward_backward_chunked(L.to_f64(X), L.to_f64(W), y64,
                                             dloss.astype(np.float64) if red == "none" else 0.9,
                                             o, 256)
    assert int(out["n_valid"]) == f["n_valid"]
    np.testing.assert_allclose(out["lse"].cpu().numpy(), f["lse"], rtol=0, atol=2e-3)
    np.testing.assert_allclose(out["loss"].cpu().numpy(), f["loss"], rtol=0, atol=2e-3)
    if red != "none" and f["n_valid"] > 0:
        valid = y64 != L.IGNORE_INDEX
        lse_mass = np.abs(f["lse"][valid]).sum() / (f["n_valid"] if red == "mean" else 1)
        tol = 1e-4 * abs(f["reduced"]) + 2.0 ** -20 * lse_mass
        assert abs(float(out["reduced"]) - f["reduced"]) <= tol
    fx, fw = grad_floors(X, W, y, dloss, red, softcap, opts)
    e = (rel_l2(dX.cpu(), rdX, fx), rel_l2(dW.cpu(), rdW, fw))
    print(f"[random fused] case {k}: dX {e[0]:.2e} dW {e[1]:.2e}", flush=True)
    assert max(e) <= 1e-3, e


def oracle_grads(X, W, y, dloss, red, softcap, opts):
    o = O.options(softcap=softcap, **opts)
    return O.backward_ex(L.to_f64(X), L.to_f64(W), y.numpy(),
                         dloss.astype(np.float64) if red == "none" else 0.9, o)


def inputs_for(k, base):
    N, H, V, softcap, opts, labels = draw(base + k)
    w = L.Workload("random", N=N, H=H, V=V, labels=labels, ignore_frac=0.1, softcap=softcap,
                   seed=95_000 + base + k)
    X, W, y = L.make_inputs(w)
    W = (W.float() * 4.0).to(torch.bfloat16)
    red = opts.get("reduction", "mean")
    rng = np.random.default_rng(96_000 + base + k)
    dloss = rng.standard_normal(N).astype(np.float32) if red == "none" else np.float32(0.9)
    return N, H, V, softcap, opts, X, W, y, red, dloss, rng


N_OTHER = 16


@pytest.mark.parametrize("k", range(N_OTHER))
def test_random_shape_sorted_backward(lce, k):
    """lce_backward_sorted with a seeded random vocabulary order (its chunks
    gather W rows in that order and scatter the dW rows back)."""
    N, H, V, softcap, opts, X, W, y, red, dloss, rng = inputs_for(k, 2000)
    print(f"[random sorted] case {k}: N={N} H={H} V={V} softcap={softcap} {opts}", flush=True)
    dev = "cuda"
    Xd, Wd, yd = X.to(dev), W.to(dev), y.to(dev)
    lse = lce.lce_forward_ex(Xd, Wd, yd, softcap=softcap, **opts)["lse"]
    order = torch.from_numpy(rng.permutation(V).astype(np.int32)).to(dev)
    dX, dW = lce.lce_backward_sorted(Xd, Wd, yd, lse, torch.from_numpy(np.atleast_1d(dloss)).to(dev),
                                     order, softcap=softcap, **opts)
    torch.cuda.synchronize()
    rdX, rdW = oracle_grads(X, W, y, dloss, red, softcap, opts)
    fx, fw = grad_floors(X, W, y, dloss, red, softcap, opts)
    e = (rel_l2(dX.cpu(), rdX, fx), rel_l2(dW.cpu(), rdW, fw))
    print(f"[random sorted] case {k}: dX {e[0]:.2e} dW {e[1]:.2e}", flush=True)
    assert max(e) <= 1e-3, e


@pytest.mark.parametrize("k", range(N_OTHER))
def test_random_shape_shards(lce, k):
    """The vocabulary cut into 1 to 4 seeded shards of random sizes: shard
    forwards, the merge, shard backwards, dX shares added in shard order."""
    N, H, V, softcap, opts, X, W, y, red, dloss, rng = inputs_for(k, 3000)
    n_sh = int(min(V, rng.integers(1, 5)))
    cuts = sorted(rng.choice(np.arange(1, V), size=n_sh - 1, replace=False).tolist()) if n_sh > 1 else []
    edges = [0] + cuts + [V]
    print(f"[random shards] case {k}: N={N} H={H} V={V} softcap={softcap} {opts} edges={edges}",
          flush=True)
    dev = "cuda"
    Xd, Wd, yd = X.to(dev), W.to(dev), y.to(dev)
    smoothing = opts.get("label_smoothing", 0.0) > 0
    fwd = {a: b for a, b in opts.items() if a == "logit_scale"}
    merge = {a: b for a, b in opts.items() if a in ("label_smoothing", "z_loss", "reduction")}
    parts = [lce.lce_shard_forward(Xd, Wd[a:b], yd, a, V, softcap=softcap, with_zsum=smoothing, **fwd)
             for a, b in zip(edges[:-1], edges[1:])]
    stack = lambda key: torch.stack([p[key] for p in parts])  # noqa: E731
    out = lce.lce_shard_merge(stack("lse_part"), stack("target_part"), yd, V,
                              zsum_parts=stack("zsum_part") if smoothing else None, **merge)
    dl = torch.from_numpy(np.atleast_1d(dloss)).to(dev)
    dX, dWs = None, []
    for a, b in zip(edges[:-1], edges[1:]):
        gx, gw = lce.lce_shard_backward(Xd, Wd[a:b], yd, out["lse"], dl, a, V, softcap=softcap, **opts)
        dX = gx if dX is None else dX + gx
        dWs.append(gw)
    dW = torch.cat(dWs)
    torch.cuda.synchronize()
    o = O.options(softcap=softcap, **opts)
    f = O.forward_ex(L.to_f64(X), L.to_f64(W), y.numpy(), o)
    np.testing.assert_allclose(out["lse"].cpu().numpy(), f["lse"], rtol=0, atol=2e-3)
    np.testing.assert_allclose(out["loss"].cpu().numpy(), f["loss"], rtol=0, atol=2e-3)
    rdX, rdW = oracle_grads(X, W, y, dloss, red, softcap, opts)
    fx, fw = grad_floors(X, W, y, dloss, red, softcap, opts)
    e = (rel_l2(dX.cpu(), rdX, fx), rel_l2(dW.cpu(), rdW, fw))
    print(f"[random shards] case {k}: dX {e[0]:.2e} dW {e[1]:.2e}", flush=True)
    assert max(e) <= 1e-3, e


@pytest.mark.parametrize("k", range(N_OTHER))
def test_random_shape_precise(lce, k):
    """The precise gradient (two bf16 parts, chunks half as wide): within the
    float32 bar, and where the default path is above 1e-4, ten times closer.
    With one class and no label smoothing the second check does not apply:
    the label's entry is then the whole gradient, which both paths take
    exactly in float32, so both carry the same float32 error (the forward's
    logit against the backward's own, p − 1 of a few ulps against a Z-loss
    term of about 2l·LSE) and nothing is rounded to bf16 for the precise path
    to remove.  With label smoothing the label's slot still holds its −e/V
    term in bf16 on the default path, which the precise path's second part
    carries, so the check applies."""
    N, H, V, softcap, opts, X, W, y, red, dloss, rng = inputs_for(k, 4000)
    print(f"[random precise] case {k}: N={N} H={H} V={V} softcap={softcap} {opts}", flush=True)
    dev = "cuda"
    Xd, Wd, yd = X.to(dev), W.to(dev), y.to(dev)
    lse = lce.lce_forward_ex(Xd, Wd, yd, softcap=softcap, **opts)["lse"]
    dl = torch.from_numpy(np.atleast_1d(dloss)).to(dev)
    pX, pW = lce.lce_backward_ex(Xd, Wd, yd, lse, dl, softcap=softcap, precise=True, **opts)
    qX, qW = lce.lce_backward_ex(Xd, Wd, yd, lse, dl, softcap=softcap, **opts)
    torch.cuda.synchronize()
    rdX, rdW = oracle_grads(X, W, y, dloss, red, softcap, opts)
    fx, fw = grad_floors(X, W, y, dloss, red, softcap, opts)
    p = (rel_l2(pX.cpu(), rdX, fx), rel_l2(pW.cpu(), rdW, fw))
    q = (rel_l2(qX.cpu(), rdX, fx), rel_l2(qW.cpu(), rdW, fw))
    print(f"[random precise] case {k}: default dX {q[0]:.2e} dW {q[1]:.2e} | precise dX {p[0]:.2e} "
          f"dW {p[1]:.2e}", flush=True)
    assert max(p) <= 1e-3, p
    if V == 1 and "label_smoothing" not in opts:
        return
    for a, b in zip(q, p):
        if a > 1e-4:
            assert b <= 0.1 * a, (a, b)


@pytest.mark.parametrize("k", range(N_OTHER))
def test_random_shape_bf16_outputs(lce, k):
    """dX and dW emitted in bf16 (bar 1e-2), from the separate calls and the
    fused call."""
    N, H, V, softcap, opts, X, W, y, red, dloss, rng = inputs_for(k, 5000)
    fused = bool(k % 2)
    if fused and softcap > 0 and "label_smoothing" in opts:
        opts = {a: b for a, b in opts.items() if a != "label_smoothing"}
    print(f"[random bf16] case {k}: N={N} H={H} V={V} softcap={softcap} {opts} fused={fused}",
          flush=True)
    dev = "cuda"
    Xd, Wd, yd = X.to(dev), W.to(dev), y.to(dev)
    dl = torch.from_numpy(np.atleast_1d(dloss)).to(dev)
    if fused:
        _, dX, dW = lce.lce_forward_backward(Xd, Wd, yd, dl, softcap=softcap, dX_dtype=torch.bfloat16,
                                             dW_dtype=torch.bfloat16, **opts)
    else:
        lse = lce.lce_forward_ex(Xd, Wd, yd, softcap=softcap, **opts)["lse"]
        dX, dW = lce.lce_backward_ex(Xd, Wd, yd, lse, dl, softcap=softcap, dX_dtype=torch.bfloat16,
                                     dW_dtype=torch.bfloat16, **opts)
    torch.cuda.synchronize()
    assert dX.dtype == torch.bfloat16 and dW.dtype == torch.bfloat16
    rdX, rdW = oracle_grads(X, W, y, dloss, red, softcap, opts)
    fx, fw = grad_floors(X, W, y, dloss, red, softcap, opts)
    e = (rel_l2(dX.float().cpu(), rdX, fx), rel_l2(dW.float().cpu(), rdW, fw))
    print(f"[random bf16] case {k}: dX {e[0]:.2e} dW {e[1]:.2e}", flush=True)
    assert max(e) <= 1e-2, e


def filter_case(k):
    """Seeded shape, options and threshold for the gradient filter: several
    256 x 256 blocks in both directions, no label smoothing (refused with the
    filter), and a threshold in the widest log gap between the oracle's block
    maxima near their median, at least 1 % from every block maximum, so the
    float32 skip decisions match the oracle's; a draw without such a gap is
    drawn again."""
    for t in range(20):
        rng = np.random.default_rng(97_000 + 100 * k + t)
        N = int(rng.integers(300, 3001))
        H = 8 * int(rng.integers(1, 33))
        V = log_uniform(rng, 600, 20000)
        softcap = float(rng.choice([0.0, 30.0, 4.0]))
        opts = [dict(), dict(z_loss=1e-3, reduction="sum"), dict(logit_scale=1.3)][int(rng.integers(0, 3))]
        w = L.Workload("random", N=N, H=H, V=V, labels="zipf", ignore_frac=0.1, softcap=softcap,
                       seed=98_000 + 100 * k + t)
        X, W, y = L.make_inputs(w)
        W = (W.float() * float(rng.uniform(4.0, 7.0))).to(torch.bfloat16)
        o = O.options(softcap=softcap, **opts)
        X64, W64, y64 = L.to_f64(X), L.to_f64(W), y.numpy()
        f = O.forward_ex(X64, W64, y64, o)
        bm = O.filter_block_max(X64, W64, y64, f["lse"], o)
        v = np.sort(bm[np.isfinite(bm) & (bm > 0)].ravel())
        if len(v) < 8:
            continue
        lo, hi = len(v) // 4, 3 * len(v) // 4
        gaps = np.log(v[lo + 1:hi + 1]) - np.log(v[lo:hi])
        j = lo + int(np.argmax(gaps))
        eps = float(np.sqrt(v[j] * v[j + 1]))
        if np.all(np.abs(v / eps - 1.0) > 0.01):
            return N, H, V, softcap, opts, X, W, y, o, eps, bm
    pytest.skip("no draw with a clear threshold")


@pytest.mark.parametrize("k", range(12))
def test_random_shape_filter(lce, k):
    N, H, V, softcap, opts, X, W, y, o, eps, bm = filter_case(k)
    kept = int((bm >= eps).sum())
    print(f"[random filter] case {k}: N={N} H={H} V={V} softcap={softcap} {opts} eps={eps:.3e} "
          f"kept {kept} of {bm.size}", flush=True)
    dev = "cuda"
    Xd, Wd, yd = X.to(dev), W.to(dev), y.to(dev)
    lse = lce.lce_forward_ex(Xd, Wd, yd, softcap=softcap, **opts)["lse"]
    dX, dW = lce.lce_backward_ex(Xd, Wd, yd, lse, 0.9, softcap=softcap, filter_eps=eps, **opts)
    torch.cuda.synchronize()
    rX, rW = O.backward_filtered(L.to_f64(X), L.to_f64(W), y.numpy(), 0.9, o, eps)
    fx, fw = grad_floors(X, W, y, np.float32(0.9), opts.get("reduction", "mean"), softcap, opts)
    e = (rel_l2(dX.cpu(), rX, fx), rel_l2(dW.cpu(), rW, fw))
    print(f"[random filter] case {k}: dX {e[0]:.2e} dW {e[1]:.2e}", flush=True)
    assert max(e) <= 1e-3, e


@pytest.mark.parametrize("k", range(12))
def test_random_shape_vocab_order(lce, k):
    """lce_vocab_order on seeded shapes (a third of them with hot entries):
    the averages against the oracle's vocab_mean_logit within the tolerance of
    tests/test_gpu_sorted.py, and the order valid (a permutation, the GPU's
    averages never increasing along it, ties by index, the oracle's never
    increasing beyond tolerance)."""
    from tests import test_gpu_sorted as S
    rng = np.random.default_rng(99_000 + k)
    N, H, V = log_uniform(rng, 1, 6000), 8 * int(rng.integers(1, 65)), log_uniform(rng, 2, 60000)
    print(f"[random order] case {k}: N={N} H={H} V={V}", flush=True)
    if k % 3 == 0 and V >= 16:
        X, W, y = S.hot_inputs(N, H, V, max(1, V // 50), seed=99_500 + k)
    else:
        X, W, y = L.make_inputs(L.Workload("random", N=N, H=H, V=V, labels="zipf", ignore_frac=0.1,
                                           seed=99_500 + k))
    key, order = lce.lce_vocab_order(X.cuda(), W.cuda(), y.cuda())
    torch.cuda.synchronize()
    X64, W64, y64 = L.to_f64(X), L.to_f64(W), y.numpy()
    ref = O.vocab_mean_logit(X64, W64, y64)
    tol = S.key_tolerance(X64, W64, y64)
    kg = key.cpu().numpy()
    assert (np.abs(kg - ref) <= tol).all()
    S.check_order(kg, order.cpu().numpy(), ref, tol)


@pytest.mark.parametrize("k", range(12))
def test_random_shape_bad_labels_and_ignore_index(lce, k):
    """Seeded shapes with a custom ignore index and a few labels out of range:
    the bad-label flag, a NaN loss on exactly the bad rows (and a NaN reduced
    loss), the other rows' losses and LSE against the oracle, finite dX rows
    for every row that is not bad; with no bad row, the gradients against the
    oracle under the custom ignore index."""
    rng = np.random.default_rng(99_800 + k)
    N, H, V = log_uniform(rng, 2, 4000), 8 * int(rng.integers(1, 65)), log_uniform(rng, 4, 30000)
    softcap = float(rng.choice([0.0, 30.0]))
    ignore = int(rng.integers(0, V))                  # a real class index used as the ignore index
    w = L.Workload("random", N=N, H=H, V=V, labels="uniform", ignore_frac=0.0, softcap=softcap,
                   seed=99_900 + k)
    X, W, y = L.make_inputs(w)
    W = (W.float() * 4.0).to(torch.bfloat16)
    y = y.clone()
    y[torch.from_numpy(rng.random(N) < 0.1)] = ignore
    n_bad = 0 if k % 3 == 0 else int(rng.integers(1, max(2, N // 50) + 1))
    bad_rows = rng.choice(N, size=min(n_bad, N), replace=False) if n_bad else np.array([], dtype=np.int64)
    for r in bad_rows:
        y[int(r)] = int(V + rng.integers(0, 1000)) if rng.random() < 0.5 else -int(rng.integers(1, 1000))
        if int(y[int(r)]) == ignore:
            y[int(r)] = V
    bad = np.zeros(N, dtype=bool)
    bad[bad_rows] = True
    print(f"[random labels] case {k}: N={N} H={H} V={V} softcap={softcap} ignore={ignore} "
          f"bad={int(bad.sum())}", flush=True)
    dev = "cuda"
    Xd, Wd, yd = X.to(dev), W.to(dev), y.to(dev)
    out = lce.lce_forward(Xd, Wd, yd, ignore, softcap)
    dX, dW = lce.lce_backward(Xd, Wd, yd, out["lse"], 0.9, ignore, softcap)
    torch.cuda.synchronize()
    loss = out["loss"].cpu().numpy()
    assert int(out["bad_label"]) == (1 if bad.any() else 0)
    assert np.isnan(loss[bad]).all() and np.isfinite(loss[~bad]).all()
    assert np.isfinite(dX.cpu().numpy()[~bad]).all()
    y_ok = y.clone()
    y_ok[torch.from_numpy(bad)] = ignore                # the oracle's rows without the bad ones
    X64, W64 = L.to_f64(X), L.to_f64(W)
    f = O.forward(X64, W64, y_ok.numpy(), ignore, softcap)
    valid = (y_ok.numpy() != ignore)
    np.testing.assert_allclose(out["lse"].cpu().numpy()[~bad], f["lse"][~bad], rtol=0, atol=2e-3)
    np.testing.assert_allclose(loss[~bad], f["loss"][~bad], rtol=0, atol=2e-3)
    if bad.any():
        assert math.isnan(float(out["mean"]))
        return
    assert int(out["n_valid"]) == int(valid.sum())
    if valid.any():
        assert abs(float(out["mean"]) - f["mean"]) <= 1e-4 * abs(f["mean"]) + 2.0 ** -20 * np.abs(f["lse"][valid]).mean()
    rdX, rdW = O.backward(X64, W64, y.numpy(), 0.9, ignore, softcap)
    fx, fw = grad_floors(X, W, y, np.float32(0.9), "mean", softcap, dict(ignore_index=ignore))
    e = (rel_l2(dX.cpu(), rdX, fx), rel_l2(dW.cpu(), rdW, fw))
    print(f"[random labels] case {k}: dX {e[0]:.2e} dW {e[1]:.2e}", flush=True)
    assert max(e) <= 1e-3, e


@pytest.mark.parametrize("k", range(16))
def test_random_shape_combinations(lce, k):
    """Options that meet in one call: the sorted backward or a vocabulary
    shard's backward, each with the precise gradient or with bf16 dW (bars
    1e-3 and 1e-2)."""
    N, H, V, softcap, opts, X, W, y, red, dloss, rng = inputs_for(k, 6000)
    combo = ["sorted+precise", "shard+precise", "sorted+bf16", "shard+bf16"][k % 4]
    print(f"[random combo] case {k}: {combo} N={N} H={H} V={V} softcap={softcap} {opts}", flush=True)
    dev = "cuda"
    Xd, Wd, yd = X.to(dev), W.to(dev), y.to(dev)
    lse = lce.lce_forward_ex(Xd, Wd, yd, softcap=softcap, **opts)["lse"]
    dl = torch.from_numpy(np.atleast_1d(dloss)).to(dev)
    extra = dict(precise=True) if combo.endswith("precise") else dict(dW_dtype=torch.bfloat16)
    if combo.startswith("sorted"):
        order = torch.from_numpy(rng.permutation(V).astype(np.int32)).to(dev)
        dX, dW = lce.lce_backward_sorted(Xd, Wd, yd, lse, dl, order, softcap=softcap, **opts, **extra)
    else:
        a = int(rng.integers(0, V))
        b = int(rng.integers(a + 1, V + 1))
        gx, gw = lce.lce_shard_backward(Xd, Wd[a:b], yd, lse, dl, a, V, softcap=softcap, **opts, **extra)
        rest = [(0, a), (b, V)]
        parts = {a: gw}
        for lo, hi in rest:
            if hi > lo:
                hx, hw = lce.lce_shard_backward(Xd, Wd[lo:hi], yd, lse, dl, lo, V, softcap=softcap,
                                                **opts, **extra)
                gx = gx + hx
                parts[lo] = hw
        dX, dW = gx, torch.cat([parts[s] for s in sorted(parts)])
    torch.cuda.synchronize()
    rdX, rdW = oracle_grads(X, W, y, dloss, red, softcap, opts)
    fx, fw = grad_floors(X, W, y, dloss, red, softcap, opts)
    e = (rel_l2(dX.float().cpu(), rdX, fx), rel_l2(dW.float().cpu(), rdW, fw))
    bar = 1e-3 if combo.endswith("precise") else 1e-2
    print(f"[random combo] case {k}: dX {e[0]:.2e} dW {e[1]:.2e}", flush=True)
    assert max(e) <= bar, e


def sorted_filter_case(k):
    """Seeded hot-entry inputs, the oracle's vocabulary order, and a filter
    threshold in a wide gap of the block maxima taken in that order (the
    procedure of tests/test_gpu_sorted.py); drawn again without such a gap."""
    from tests import test_gpu_sorted as S
    for t in range(20):
        rng = np.random.default_rng(99_600 + 100 * k + t)
        N = int(rng.integers(300, 3001))
        H = 8 * int(rng.integers(1, 33))
        V = log_uniform(rng, 600, 30000)
        opts = [dict(), dict(softcap=30.0), dict(softcap=4.0, z_loss=1e-3, reduction="sum")][k % 3]
        X, W, y = S.hot_inputs(N, H, V, max(2, V // 60), seed=99_700 + 100 * k + t)
        o = O.options(**opts)
        X64, W64, y64 = L.to_f64(X), L.to_f64(W), y.numpy()
        order = O.vocab_order(O.vocab_mean_logit(X64, W64, y64, int(o["ignore_index"])))
        pos = np.empty(V, dtype=np.int64)
        pos[order] = np.arange(V)
        ignored = y64 == int(o["ignore_index"])
        y_pos = y64.copy()
        y_pos[~ignored] = pos[y64[~ignored]]
        y_pos[ignored] = -1000
        f = O.forward_ex(X64, W64, y64, o)
        bm = O.filter_block_max(X64, W64[order], y_pos, f["lse"], dict(o, ignore_index=-1000))
        v = np.sort(bm[np.isfinite(bm) & (bm > 0)].ravel())
        if len(v) < 8:
            continue
        lo, hi = len(v) // 4, 3 * len(v) // 4
        gaps = np.log(v[lo + 1:hi + 1]) - np.log(v[lo:hi])
        j = lo + int(np.argmax(gaps))
        eps = float(np.sqrt(v[j] * v[j + 1]))
        if np.all(np.abs(v / eps - 1.0) > 0.01):
            return N, H, V, opts, X, W, y, o, order, eps
    pytest.skip("no draw with a clear threshold")


@pytest.mark.parametrize("k", range(9))
def test_random_shape_sorted_filter(lce, k):
    N, H, V, opts, X, W, y, o, order, eps = sorted_filter_case(k)
    print(f"[random sorted filter] case {k}: N={N} H={H} V={V} {opts} eps={eps:.3e}", flush=True)
    Xd, Wd, yd = X.cuda(), W.cuda(), y.cuda()
    lse = lce.lce_forward_ex(Xd, Wd, yd, **opts)["lse"]
    od = torch.from_numpy(order.astype(np.int32)).cuda()
    dX, dW = lce.lce_backward_sorted(Xd, Wd, yd, lse, 0.9, od, filter_eps=eps, **opts)
    torch.cuda.synchronize()
    rX, rW = O.backward_sorted(L.to_f64(X), L.to_f64(W), y.numpy(), 0.9, o, order, eps)
    fx, fw = grad_floors(X, W, y, np.float32(0.9), opts.get("reduction", "mean"),
                         opts.get("softcap", 0.0), {a: b for a, b in opts.items() if a != "softcap"})
    e = (rel_l2(dX.cpu(), rX, fx), rel_l2(dW.cpu(), rW, fw))
    print(f"[random sorted filter] case {k}: dX {e[0]:.2e} dW {e[1]:.2e}", flush=True)
    assert max(e) <= 1e-3, e


@pytest.mark.parametrize("k", range(12))
def test_random_shape_autograd(lce, k):
    """The autograd wrapper on seeded shapes and options: the loss it returns
    (reduced, or per row with reduction "none" and a random upstream gradient
    through loss.backward) and X.grad, W.grad (bf16, as the inputs) against
    the oracle (bar 1e-2)."""
    N, H, V, softcap, opts, X, W, y, red, dloss, rng = inputs_for(k, 7000)
    print(f"[random autograd] case {k}: N={N} H={H} V={V} softcap={softcap} {opts}", flush=True)
    Xp = X.cuda().requires_grad_(True)
    Wp = W.cuda().requires_grad_(True)
    loss = lce.linear_cross_entropy(Xp, Wp, y.cuda(), softcap=softcap, **opts)
    if red == "none":
        loss.backward(torch.from_numpy(dloss).cuda())
    else:
        (loss * 0.9).backward()
    torch.cuda.synchronize()
    o = O.options(softcap=softcap, **opts)
    f = O.forward_ex(L.to_f64(X), L.to_f64(W), y.numpy(), o)
    if red == "none":
        np.testing.assert_allclose(loss.detach().cpu().numpy(), f["loss"], rtol=0, atol=2e-3)
    elif f["n_valid"] > 0:
        valid = y.numpy() != L.IGNORE_INDEX
        lse_mass = np.abs(f["lse"][valid]).sum() / (f["n_valid"] if red == "mean" else 1)
        assert abs(float(loss.detach()) - f["reduced"]) <= 1e-4 * abs(f["reduced"]) + 2.0 ** -20 * lse_mass
    assert Xp.grad.dtype == torch.bfloat16 and Wp.grad.dtype == torch.bfloat16
    rdX, rdW = oracle_grads(X, W, y, dloss, red, softcap, opts)
    fx, fw = grad_floors(X, W, y, dloss, red, softcap, opts)
    e = (rel_l2(Xp.grad.float().cpu(), rdX, fx), rel_l2(Wp.grad.float().cpu(), rdW, fw))
    print(f"[random autograd] case {k}: dX {e[0]:.2e} dW {e[1]:.2e}", flush=True)
    assert max(e) <= 1e-2, e
