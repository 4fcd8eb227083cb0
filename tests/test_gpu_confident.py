"""Confident rows: gradients of rows whose softmax has one large entry.

When a row predicts its label with p_y near 1, the label's softmax term p_y·d
nearly cancels its one-hot term d, and the true entry d·(p_y − 1) is far
smaller than the bf16 rounding of p_y·d; when a row is confident about an
entry other than its label, that entry alone carries a large share of the
row's gradient.  The backward takes both entries out of the bf16 gradient
chunk and applies them in fp32 (the softmax − onehot gradient of the blog on
Liger Kernel and Cut Cross-Entropy, section two, and AI-infra KB M011 section
06; the softcap derivative of the Unsloth fused cross-entropy chapter, section
4).  These cases hold every row in that regime and must meet the float32 bar
of the whole path, dX and dW relative L2 <= 1e-3 against the float64 oracle.

Logits are set directly: with N < H rows of X drawn N(0, 1), W is solved so
that X·Wᵀ hits the target logits, then rounded to bf16 (the oracle sees the
same bf16 W).
"""
import numpy as np
import pytest
import torch

import lce_inputs as L
from oracle import lce_oracle as O

pytestmark = pytest.mark.gpu

LSE_ATOL = 2e-3
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
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def inputs_with_logits(Z, seed, ignore=()):
    """bf16 X [N, H] and W [V, H] with X·Wᵀ ≈ Z (N < H)."""
    N, V = Z.shape
    H = 384
    rng = np.random.default_rng(seed)
    X = torch.from_numpy(rng.standard_normal((N, H)).astype(np.float32)).to(torch.bfloat16)
    Xf = X.double().numpy()
    Wt = np.linalg.lstsq(Xf, Z, rcond=None)[0]          # H x V with Xf·Wt = Z
    W = torch.from_numpy(Wt.T.astype(np.float32)).to(torch.bfloat16)
    return X, W


def confident_case(kind, seed):
    """Target logits of one confident regime (see the parametrisation)."""
    N, V = 300, 20000
    rng = np.random.default_rng(seed)
    if kind == "softcap_wrong_label":
        # Top logit 25 at a random entry, the others N(0, 9), labels random
        # (almost never the top entry); softcap 30.
        Z = rng.standard_normal((N, V)) * 3.0
        Z[np.arange(N), rng.integers(0, V, N)] = 25.0
        y = rng.integers(0, V, N)
        return Z, y, 30.0
    if kind.startswith("label_is_top"):
        # The label is the top entry, boosted so p_y is 0.9 ... 0.999.
        Z = rng.standard_normal((N, V))
        y = rng.integers(0, V, N)
        Z[np.arange(N), y] = rng.uniform(12.0, 17.0, N)
        return Z, y, (30.0 if kind.endswith("softcap") else 0.0)
    raise ValueError(kind)


SEEDS = {"softcap_wrong_label": 11, "label_is_top": 12, "label_is_top_softcap": 13}


def shared_case(kind, seed):
    """Rows whose softmax mass is shared by two or three large entries
    (logit 14 each, the others N(0, 1), V = 20000: p ≈ 0.49 each for two,
    0.33 for three), with the label one of them or none."""
    N, V = 300, 20000
    rng = np.random.default_rng(seed)
    Z = rng.standard_normal((N, V))
    k = 3 if kind.startswith("three") else 2
    tops = np.stack([rng.permutation(V)[:k] for _ in range(N)])
    for j in range(k):
        Z[np.arange(N), tops[:, j]] = 14.0
    y = tops[:, 0].copy() if "label" in kind else rng.integers(0, V, N)
    return Z, y, (30.0 if kind.endswith("softcap") else 0.0)


SHARED = {"two_label": 21, "two_label_softcap": 22, "two_other_softcap": 23,
          "three_label": 24, "three_label_softcap": 25}


# Rows whose gradient is carried by a few mid-sized entries show the bf16
# rounding of the chunk at about 1e-3 relative: the label's entry is exact,
# the others are rounded to 2^-9 of themselves.  That stays within this bound
# on the default path; the precise gradient (two bf16 parts) meets the float32
# bar on them.
SHARED_DEFAULT_BOUND = 2e-3


@pytest.mark.parametrize("kind", sorted(SHARED))
def test_shared_rows(lce, kind):
    """Two or three entries share each row's mass (at most one of them the
    label): the default path within SHARED_DEFAULT_BOUND, the precise
    gradient within the float32 bar."""
    Z, y, c = shared_case(kind, seed=SHARED[kind])
    X, W = inputs_with_logits(Z, seed=9)
    y[::13] = -100
    yt = torch.from_numpy(y.astype(np.int64))
    dev = "cuda"
    out = lce.lce_forward(X.to(dev), W.to(dev), yt.to(dev), -100, c)
    dX, dW = lce.lce_backward(X.to(dev), W.to(dev), yt.to(dev), out["lse"], 1.0, -100, c)
    N = len(y)
    o2, dX2, dW2 = lce.lce_forward_backward(X.to(dev), W.to(dev), yt.to(dev),
                                            torch.ones(1, device=dev), softcap=c)
    dX3, dW3 = lce.lce_backward_ex(X.to(dev), W.to(dev), yt.to(dev), out["lse"], 1.0, softcap=c,
                                   precise=True)
    torch.cuda.synchronize()
    X64, W64 = L.to_f64(X), L.to_f64(W)
    f = O.forward(X64, W64, y, -100, c)
    rdX, rdW = O.backward(X64, W64, y, 1.0, -100, c)
    p = np.exp(O.apply_softcap(X64 @ W64.T, c) - f["lse"][:, None])
    p_top = np.sort(p, axis=1)[:, ::-1][:, :3].mean(0)
    e = [rel_l2(dX.cpu(), rdX), rel_l2(dW.cpu(), rdW), rel_l2(dX2.cpu(), rdX), rel_l2(dW2.cpu(), rdW)]
    ep = [rel_l2(dX3.cpu(), rdX), rel_l2(dW3.cpu(), rdW)]
    print(f"[shared] {kind}: mean top-3 p {p_top.round(3)} recompute dX {e[0]:.2e} dW {e[1]:.2e} "
          f"fused dX {e[2]:.2e} dW {e[3]:.2e} precise dX {ep[0]:.2e} dW {ep[1]:.2e}", flush=True)
    assert max(e) <= SHARED_DEFAULT_BOUND
    assert max(ep) <= GRAD_RTOL


@pytest.mark.parametrize("kind", sorted(SEEDS))
def test_confident_rows(lce, kind):
    Z, y, c = confident_case(kind, seed=SEEDS[kind])
    X, W = inputs_with_logits(Z, seed=7)
    y[::17] = -100                                       # a few ignored rows
    yt = torch.from_numpy(y.astype(np.int64))
    dev = "cuda"
    out = lce.lce_forward(X.to(dev), W.to(dev), yt.to(dev), -100, c)
    dX, dW = lce.lce_backward(X.to(dev), W.to(dev), yt.to(dev), out["lse"], 1.0, -100, c)
    torch.cuda.synchronize()
    X64, W64 = L.to_f64(X), L.to_f64(W)
    f = O.forward(X64, W64, y, -100, c)
    rdX, rdW = O.backward(X64, W64, y, 1.0, -100, c)
    p_top = np.exp(O.apply_softcap(X64 @ W64.T, c).max(1) - f["lse"])
    valid = y != -100
    p_y = np.exp(f["target_logit"][valid] - f["lse"][valid])
    e_lse = float(np.abs(out["lse"].cpu().numpy() - f["lse"]).max())
    e_dx, e_dw = rel_l2(dX.cpu(), rdX), rel_l2(dW.cpu(), rdW)
    print(f"[confident] {kind}: mean top p {p_top.mean():.4f} mean p_y {p_y.mean():.4f} "
          f"lse {e_lse:.1e} dX {e_dx:.2e} dW {e_dw:.2e}", flush=True)
    assert p_top.mean() > 0.9
    assert e_lse <= LSE_ATOL
    assert e_dx <= GRAD_RTOL and e_dw <= GRAD_RTOL


@pytest.mark.parametrize("opts", [
    dict(softcap=30.0, z_loss=1e-3, reduction="none"),
    dict(z_loss=1e-3),
    dict(reduction="none", label_smoothing=0.05),
])
def test_confident_rows_variants(lce, opts):
    """Per-row factors (Z-loss, per-row upstream gradients) and label
    smoothing with peaked logits, half the rows predicting their label."""
    N, V = 300, 20000
    rng = np.random.default_rng(31)
    Z = rng.standard_normal((N, V)) * 3.0
    top = rng.integers(0, V, N)
    Z[np.arange(N), top] = 25.0
    y = np.where(np.arange(N) % 2 == 0, top, rng.integers(0, V, N))
    X, W = inputs_with_logits(Z, seed=8)
    y[5] = -100
    yt = torch.from_numpy(y.astype(np.int64))
    red = opts.get("reduction", "mean")
    dloss = rng.standard_normal(N).astype(np.float32) if red == "none" else np.float32(0.7)
    dev = "cuda"
    out = lce.lce_forward_ex(X.to(dev), W.to(dev), yt.to(dev), **opts)
    dX, dW = lce.lce_backward_ex(X.to(dev), W.to(dev), yt.to(dev), out["lse"],
                                 torch.from_numpy(np.atleast_1d(dloss)).to(dev), **opts)
    torch.cuda.synchronize()
    o = O.options(**opts)
    rdX, rdW = O.backward_ex(L.to_f64(X), L.to_f64(W), y, dloss.astype(np.float64), o)
    e_dx, e_dw = rel_l2(dX.cpu(), rdX), rel_l2(dW.cpu(), rdW)
    print(f"[confident] {opts}: dX {e_dx:.2e} dW {e_dw:.2e}", flush=True)
    assert e_dx <= GRAD_RTOL and e_dw <= GRAD_RTOL


@pytest.mark.parametrize("kind,opts", [
    ("softcap_wrong_label", dict()),                        # fixed reference (softcap 30)
    ("label_is_top", dict()),                               # no softcap: running reference
    ("label_is_top_softcap", dict(z_loss=1e-3)),            # fixed reference, per-row factor
    ("label_is_top", dict(reduction="none")),               # per-row upstream gradients
])
def test_confident_rows_fused(lce, kind, opts):
    """The row-chunked fused call (two row chunks here) on the same regimes."""
    Z, y, c = confident_case(kind, seed=SEEDS[kind])
    X, W = inputs_with_logits(Z, seed=7)
    y[::17] = -100
    yt = torch.from_numpy(y.astype(np.int64))
    N = len(y)
    red = opts.get("reduction", "mean")
    dloss = (np.random.default_rng(5).standard_normal(N).astype(np.float32) if red == "none"
             else np.float32(1.0))
    dev = "cuda"
    out, dX, dW = lce.lce_forward_backward(X.to(dev), W.to(dev), yt.to(dev),
                                           torch.from_numpy(np.atleast_1d(dloss)).to(dev),
                                           softcap=c, **opts)
    torch.cuda.synchronize()
    o = O.options(softcap=c, **opts)
    X64, W64 = L.to_f64(X), L.to_f64(W)
    f = O.forward_ex(X64, W64, y, o)
    rdX, rdW = O.backward_ex(X64, W64, y, dloss.astype(np.float64), o)
    e_lse = float(np.abs(out["lse"].cpu().numpy() - f["lse"]).max())
    e_dx, e_dw = rel_l2(dX.cpu(), rdX), rel_l2(dW.cpu(), rdW)
    print(f"[confident fused] {kind} {opts}: lse {e_lse:.1e} dX {e_dx:.2e} dW {e_dw:.2e}",
          flush=True)
    assert e_lse <= LSE_ATOL
    assert e_dx <= GRAD_RTOL and e_dw <= GRAD_RTOL
