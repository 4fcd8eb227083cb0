"""Parity of the loss variants (lce_forward_ex / lce_backward_ex: logit scale,
label smoothing, Z-loss, sum / none reductions) with the CPU oracle.

Same bars as the plain path: per-row LSE and loss abs err <= 2e-3, the
reduced loss rel err <= 1e-4, dX and dW rel-L2 err <= 1e-3 in float32,
n_valid exact.  The full-size case (Gemma-2 2B head) compares sampled rows.
"""
import os

import numpy as np
import pytest
import torch

import lce_inputs as L
from tests import fullsize_samples as FS
from oracle import lce_oracle as O

pytestmark = pytest.mark.gpu

LSE_ATOL = 2e-3
RED_RTOL = 1e-4
GRAD_RTOL = 1e-3
HERE = os.path.dirname(os.path.abspath(__file__))


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


CASES = [
    # N, H, V, options
    (257, 72, 1003, dict(logit_scale=1.5, label_smoothing=0.1)),
    (513, 136, 2100, dict(softcap=3.0, logit_scale=0.7, label_smoothing=0.2, z_loss=1e-3,
                          reduction="sum")),
    (600, 200, 1500, dict(z_loss=1e-2, reduction="none")),
    (300, 64, 40000, dict(softcap=30.0, label_smoothing=0.05, reduction="none")),
    (700, 48, 20000, dict(softcap=4.0, logit_scale=2.0, reduction="sum")),
    (96, 64, 300, dict(softcap=80.0, label_smoothing=0.3, z_loss=5e-3)),   # general softcap path
    # 36 token tiles: the forward's last 4 tiles run in a launch of their own,
    # whose partials and logit sums (label smoothing) form a block of their own.
    (9100, 64, 2500, dict(label_smoothing=0.1, z_loss=1e-3)),
]


@pytest.mark.parametrize("N,H,V,opts", CASES)
def test_variants_against_oracle(lce, N, H, V, opts):
    w = L.Workload("variant", N=N, H=H, V=V, labels="uniform", ignore_frac=0.1, seed=4000 + N + V)
    X, W, y = L.make_inputs(w)
    W = (W.float() * 4.0).to(torch.bfloat16)
    red = opts.get("reduction", "mean")
    print(f"[variants] N={N} H={H} V={V} {opts}", flush=True)
    dev = "cuda"
    Xd, Wd, yd = X.to(dev), W.to(dev), y.to(dev)
    out = lce.lce_forward_ex(Xd, Wd, yd, **opts)
    rng = np.random.default_rng(N)
    dloss = rng.standard_normal(N).astype(np.float32) if red == "none" else np.float32(0.61)
    dl_dev = torch.from_numpy(np.atleast_1d(dloss)).to(dev)
    dX, dW = lce.lce_backward_ex(Xd, Wd, yd, out["lse"], dl_dev, **opts)
    torch.cuda.synchronize()

    o = O.options(**opts)
    X64, W64, y64 = L.to_f64(X), L.to_f64(W), y.numpy()
    f = O.forward_ex(X64, W64, y64, o)
    rdX, rdW = O.backward_ex(X64, W64, y64, dloss.astype(np.float64) if red == "none" else 0.61, o)
    assert int(out["n_valid"]) == f["n_valid"]
    np.testing.assert_allclose(out["lse"].cpu().numpy(), f["lse"], rtol=0, atol=LSE_ATOL)
    np.testing.assert_allclose(out["loss"].cpu().numpy(), f["loss"], rtol=0, atol=LSE_ATOL)
    assert abs(float(out["reduced"]) - f["reduced"]) <= RED_RTOL * abs(f["reduced"])
    e_dx, e_dw = rel_l2(dX.cpu(), rdX), rel_l2(dW.cpu(), rdW)
    print(f"[variants] dX rel {e_dx:.2e} dW rel {e_dw:.2e}", flush=True)
    assert e_dx <= GRAD_RTOL and e_dw <= GRAD_RTOL


# Logits in the hundreds, so each row's softmax is dominated by one entry
# near 1.  With one scale for every row (mean or sum, no Z-loss) the general
# form keeps that scale out of the bf16 gradient chunk, as the plain form
# does, so the dominant value rounds to the exactly representable 1.
@pytest.mark.parametrize("opts", [
    dict(label_smoothing=0.1),
    dict(label_smoothing=0.1, logit_scale=0.8, reduction="sum"),
    dict(softcap=100.0, label_smoothing=0.05),
])
def test_variants_large_logits(lce, opts):
    N, H, V = 1100, 72, 20000
    w = L.Workload("variant", N=N, H=H, V=V, labels="uniform", ignore_frac=0.1, seed=4500)
    X, W, y = L.make_inputs(w)
    W = (W.float() * 200.0 * torch.linspace(0.25, 1.5, V).unsqueeze(1)).to(torch.bfloat16)
    print(f"[variants] large logits {opts}", flush=True)
    Xd, Wd, yd = X.cuda(), W.cuda(), y.cuda()
    out = lce.lce_forward_ex(Xd, Wd, yd, **opts)
    dX, dW = lce.lce_backward_ex(Xd, Wd, yd, out["lse"], 0.61, **opts)
    torch.cuda.synchronize()
    o = O.options(**opts)
    X64, W64, y64 = L.to_f64(X), L.to_f64(W), y.numpy()
    f = O.forward_ex(X64, W64, y64, o)
    rdX, rdW = O.backward_ex(X64, W64, y64, 0.61, o)
    np.testing.assert_allclose(out["lse"].cpu().numpy(), f["lse"], rtol=0, atol=LSE_ATOL)
    np.testing.assert_allclose(out["loss"].cpu().numpy(), f["loss"], rtol=0, atol=LSE_ATOL)
    assert abs(float(out["reduced"]) - f["reduced"]) <= RED_RTOL * abs(f["reduced"])
    e_dx, e_dw = rel_l2(dX.cpu(), rdX), rel_l2(dW.cpu(), rdW)
    print(f"[variants] dX rel {e_dx:.2e} dW rel {e_dw:.2e}", flush=True)
    assert e_dx <= GRAD_RTOL and e_dw <= GRAD_RTOL


def test_mean_and_sum_differ_by_the_valid_count(lce):
    # One scale shared by every row is applied after the contractions, so the
    # sum reduction's gradients are the mean's times n_valid, up to the float
    # rounding of that scalar (not the bf16 rounding of the gradient chunk).
    w = L.Workload("variant", N=700, H=72, V=3000, labels="uniform", ignore_frac=0.1, seed=4600)
    X, W, y = (t.cuda() for t in L.make_inputs(w))
    W = (W.float() * 4.0).to(torch.bfloat16)
    for opts in (dict(label_smoothing=0.1), dict(softcap=80.0), dict()):
        fm = lce.lce_forward_ex(X, W, y, **opts)
        dXm, dWm = lce.lce_backward_ex(X, W, y, fm["lse"], 1.0, **opts)
        dXs, dWs = lce.lce_backward_ex(X, W, y, fm["lse"], 1.0, reduction="sum", **opts)
        torch.cuda.synchronize()
        n = int(fm["n_valid"])
        assert rel_l2(dXs.cpu(), dXm.cpu() * n) <= 1e-6, opts
        assert rel_l2(dWs.cpu(), dWm.cpu() * n) <= 1e-6, opts


def test_defaults_match_plain_entry_points_bitwise(lce):
    w = L.Workload("v", N=400, H=128, V=3000, labels="uniform", ignore_frac=0.1, seed=77)
    X, W, y = (t.cuda() for t in L.make_inputs(w))
    a = lce.lce_forward(X, W, y, -100, 5.0)
    b = lce.lce_forward_ex(X, W, y, softcap=5.0)
    for k in ("loss", "lse"):
        assert torch.equal(a[k], b[k])
    assert torch.equal(a["mean"], b["reduced"])
    dXa, dWa = lce.lce_backward(X, W, y, a["lse"], 0.8, -100, 5.0)
    dXb, dWb = lce.lce_backward_ex(X, W, y, a["lse"], 0.8, softcap=5.0)
    assert torch.equal(dXa, dXb) and torch.equal(dWa, dWb)


def test_invalid_options_rejected(lce):
    X, W, y = (t.cuda() for t in L.make_inputs(L.Workload("v", N=8, H=8, V=10)))
    for bad in (dict(logit_scale=0.0), dict(logit_scale=float("nan")), dict(label_smoothing=1.5),
                dict(label_smoothing=-0.1), dict(z_loss=-1.0)):
        with pytest.raises(lce.LceError):
            lce.lce_forward_ex(X, W, y, **bad)
    with pytest.raises(ValueError):
        lce.lce_forward_ex(X, W, y, reduction="max")


def test_autograd_with_options(lce):
    w = L.Workload("v", N=300, H=64, V=1000, labels="uniform", ignore_frac=0.1, seed=78)
    X, W, y = L.make_inputs(w)
    Xd = X.cuda().requires_grad_(True)
    Wd = W.cuda().requires_grad_(True)
    loss = lce.linear_cross_entropy(Xd, Wd, y.cuda(), softcap=2.0, label_smoothing=0.1,
                                    z_loss=1e-3, reduction="none")
    g = torch.linspace(-1, 1, 300, device="cuda")
    (loss * g).sum().backward()
    o = O.options(softcap=2.0, label_smoothing=0.1, z_loss=1e-3, reduction="none")
    f = O.forward_ex(L.to_f64(X), L.to_f64(W), y.numpy(), o)
    np.testing.assert_allclose(loss.detach().cpu().numpy(), f["loss"], atol=LSE_ATOL)
    rdX, rdW = O.backward_ex(L.to_f64(X), L.to_f64(W), y.numpy(), g.cpu().double().numpy(), o)
    assert rel_l2(Xd.grad.float().cpu(), rdX) <= 1e-2      # bf16 gradients
    assert rel_l2(Wd.grad.float().cpu(), rdW) <= 1e-2


def test_gemma_fullsize_variant_sampled(lce):
    """Gemma-2 2B head with label smoothing, Z-loss and per-row upstream
    gradients, checked on sampled rows (the LSE of every row comes from the
    stored oracle values: the variants do not change it at logit scale 1)."""
    gold = np.load(os.path.join(HERE, "golden", "fullsize_gemma2_2b.npz"))
    w = L.WORKLOADS["gemma2_2b"]
    X, W, y = L.make_inputs(w)
    assert L.fingerprint(X, W, y) == str(gold["fingerprint"])
    opts = dict(softcap=w.softcap, label_smoothing=0.1, z_loss=1e-4, reduction="none")
    print(f"[variants] gemma2_2b full size {opts}", flush=True)
    dev = "cuda"
    Xd, Wd, yd = X.to(dev), W.to(dev), y.to(dev)
    out = lce.lce_forward_ex(Xd, Wd, yd, **opts)
    dloss = np.random.default_rng(3).standard_normal(w.N).astype(np.float32)
    dX, dW = lce.lce_backward_ex(Xd, Wd, yd, out["lse"], torch.from_numpy(dloss).to(dev), **opts)
    torch.cuda.synchronize()
    o = O.options(**opts)
    X64, W64, y64 = L.to_f64(X), L.to_f64(W), y.numpy()
    lse_all = gold["lse"]
    np.testing.assert_allclose(out["lse"].cpu().numpy(), lse_all, atol=LSE_ATOL)
    rows = gold["dx_rows"]
    f = O.forward_ex(X64[rows], W64, y64[rows], o)
    np.testing.assert_allclose(out["loss"].cpu().numpy()[rows], f["loss"], atol=LSE_ATOL)
    scale = O.row_scale(y64, dloss.astype(np.float64), int(gold["n_valid"]), o)
    gx = O.logit_gradient_ex(X64[rows], W64, y64[rows], lse_all[rows], scale[rows], o)
    e_dx = rel_l2(dX[torch.from_numpy(rows).to(dev)].cpu(), gx @ W64)
    vrows = gold["dw_rows"]
    gw = O.logit_gradient_ex(X64, W64, y64, lse_all, scale, o, vocab_rows=vrows)
    e_dw = rel_l2(dW[torch.from_numpy(vrows).to(dev)].cpu(), gw.T @ X64)
    print(f"[variants] gemma full size: dX rel {e_dx:.2e} dW rel {e_dw:.2e}", flush=True)
    assert e_dx <= GRAD_RTOL and e_dw <= GRAD_RTOL
    S = FS.samples("gemma2_2b", X, W, y, opts, dloss.astype(np.float64))
    FS.check("variants gemma2_2b", dX, dW, S, GRAD_RTOL, 1e-2, log=lambda m: print(m, flush=True))
