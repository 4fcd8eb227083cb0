"""Parity of the row-chunked forward-and-backward call (lce_forward_backward)
with the CPU oracle's forward_backward_chunked.

Bars as for the separate calls: per-row LSE and loss abs err <= 2e-3, the
reduced loss rel err <= 1e-4, dX and dW rel-L2 err <= 1e-3 in float32 and
<= 1e-2 in bf16, n_valid exact.  The small cases take H = 64 or 72, so the
chunks hold 256 rows and every case runs several chunks with a ragged last
one; they cover the three ways the stored logits are referenced (no
softcap, a softcap small enough for the fixed reference, a large one) and
every option the call takes.  The full-size cases run the four large
workloads (Liger example, Llama-3 8B, Gemma-2 2B, long Qwen2.5) against the
stored oracle values.
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
    (700, 64, 3001, dict()),
    (600, 72, 2100, dict(softcap=3.0)),                            # fixed reference
    (530, 64, 1500, dict(softcap=80.0, z_loss=1e-3)),              # running reference
    (800, 64, 5003, dict(softcap=30.0, logit_scale=1.3, reduction="none")),
    (513, 72, 900, dict(label_smoothing=0.1, z_loss=1e-2, reduction="sum")),
    (300, 64, 777, dict(logit_scale=0.6, reduction="none", label_smoothing=0.05)),
    (100, 64, 300, dict(softcap=20.0)),                            # N < 256, one partial tile
    (257, 8, 40, dict(z_loss=1e-2)),                               # tiny H and V
    (64, 64, 700, dict()),                                         # one-step dW tiles (K = 64 rows)
    (128, 192, 640, dict(softcap=30.0)),                           # two-step dW, three-step logits
    (300, 64, 150000, dict()),                                     # one-step logit tiles, 2-3 per split
    (200, 32, 90000, dict(softcap=30.0)),                          # the same with the fixed reference
    (513, 64, 5, dict()),                                          # a handful of classes
    (600, 64, 3, dict(softcap=30.0, z_loss=1e-3)),
    # Label smoothing with a handful of classes: e/V is large, so the slot of
    # an exactly taken entry must come out of the in-place rescale as −gs·e/V.
    (300, 64, 2, dict(label_smoothing=0.1)),
    (400, 376, 5, dict(label_smoothing=0.2, reduction="sum")),
    # Uneven row chunks with their own dX K parts: 1536 + 1536 + 1025 rows,
    # 6, 6 and 7 parts (the last chunk's part stride is its 1025 rows); and
    # 1536 + 1064 rows, 6 and 7 parts.
    (4097, 1024, 6000, dict(softcap=30.0)),
    (2600, 1024, 4000, dict(z_loss=1e-3, reduction="none")),
]


@pytest.mark.parametrize("N,H,V,opts", CASES)
def test_fused_against_oracle(lce, N, H, V, opts):
    w = L.Workload("fused", N=N, H=H, V=V, labels="uniform", ignore_frac=0.1, seed=6000 + N + V)
    X, W, y = L.make_inputs(w)
    W = (W.float() * 4.0).to(torch.bfloat16)
    red = opts.get("reduction", "mean")
    print(f"[fused] N={N} H={H} V={V} {opts}", flush=True)
    rng = np.random.default_rng(N)
    dloss = rng.standard_normal(N).astype(np.float32) if red == "none" else np.float32(0.8)
    dev = "cuda"
    out, dX, dW = lce.lce_forward_backward(X.to(dev), W.to(dev), y.to(dev),
                                           torch.from_numpy(np.atleast_1d(dloss)).to(dev), **opts)
    torch.cuda.synchronize()
    o = O.options(**opts)
    f, rdX, rdW = O.forward_backward_chunked(L.to_f64(X), L.to_f64(W), y.numpy(),
                                             dloss.astype(np.float64) if red == "none" else 0.8,
                                             o, 256)
    assert int(out["n_valid"]) == f["n_valid"] and int(out["bad_label"]) == 0
    np.testing.assert_allclose(out["lse"].cpu().numpy(), f["lse"], rtol=0, atol=LSE_ATOL)
    np.testing.assert_allclose(out["loss"].cpu().numpy(), f["loss"], rtol=0, atol=LSE_ATOL)
    assert abs(float(out["reduced"]) - f["reduced"]) <= RED_RTOL * abs(f["reduced"])
    e_dx, e_dw = rel_l2(dX.cpu(), rdX), rel_l2(dW.cpu(), rdW)
    print(f"[fused] dX rel {e_dx:.2e} dW rel {e_dw:.2e}", flush=True)
    assert e_dx <= GRAD_RTOL and e_dw <= GRAD_RTOL


# Logits in the hundreds, largest in the last vocabulary tiles: the stored
# block's per-block reference (running maximum) rises across the sweep and
# every block is rescaled by its own 2^(ref − lse).  Five row chunks.
@pytest.mark.parametrize("softcap", [0.0, 100.0, 30.0])
def test_fused_large_logits(lce, softcap):
    N, H, V = 1100, 72, 20000
    w = L.Workload("fused", N=N, H=H, V=V, labels="uniform", ignore_frac=0.1,
                   seed=6500 + int(softcap))
    X, W, y = L.make_inputs(w)
    W = (W.float() * 200.0 * torch.linspace(0.25, 1.5, V).unsqueeze(1)).to(torch.bfloat16)
    print(f"[fused] large logits c={softcap}", flush=True)
    out, dX, dW = lce.lce_forward_backward(X.cuda(), W.cuda(), y.cuda(), 1.0, softcap=softcap)
    torch.cuda.synchronize()
    f, rdX, rdW = O.forward_backward_chunked(L.to_f64(X), L.to_f64(W), y.numpy(), 1.0,
                                             O.options(softcap=softcap), 256)
    assert int(out["n_valid"]) == f["n_valid"]
    np.testing.assert_allclose(out["lse"].cpu().numpy(), f["lse"], rtol=0, atol=LSE_ATOL)
    np.testing.assert_allclose(out["loss"].cpu().numpy(), f["loss"], rtol=0, atol=LSE_ATOL)
    assert abs(float(out["reduced"]) - f["reduced"]) <= RED_RTOL * abs(f["reduced"])
    e_dx, e_dw = rel_l2(dX.cpu(), rdX), rel_l2(dW.cpu(), rdW)
    print(f"[fused] dX rel {e_dx:.2e} dW rel {e_dw:.2e}", flush=True)
    assert e_dx <= GRAD_RTOL and e_dw <= GRAD_RTOL


def test_fused_matches_separate_calls(lce):
    """Same inputs through lce_forward_ex + lce_backward_ex: equal within rounding."""
    w = L.Workload("fused", N=1100, H=128, V=4000, labels="zipf", ignore_frac=0.1, seed=61)
    X, W, y = (t.cuda() for t in L.make_inputs(w))
    for opts in (dict(softcap=30.0), dict(), dict(softcap=50.0, z_loss=1e-4)):
        out, dX, dW = lce.lce_forward_backward(X, W, y, 1.0, **opts)
        ref = lce.lce_forward_ex(X, W, y, **opts)
        rX, rW = lce.lce_backward_ex(X, W, y, ref["lse"], 1.0, **opts)
        torch.cuda.synchronize()
        assert torch.allclose(out["lse"], ref["lse"], atol=1e-5, rtol=0)
        assert abs(float(out["reduced"]) - float(ref["reduced"])) <= 1e-6 * abs(float(ref["reduced"]))
        assert rel_l2(dX.cpu(), rX.cpu()) <= 2e-3 and rel_l2(dW.cpu(), rW.cpu()) <= 2e-3


def test_fused_bf16_outputs_and_bad_label(lce):
    w = L.Workload("fused", N=520, H=64, V=1000, labels="uniform", ignore_frac=0.1, seed=62)
    X, W, y = L.make_inputs(w)
    y[9] = 1000
    out, dX, dW = lce.lce_forward_backward(X.cuda(), W.cuda(), y.cuda(), 1.0, softcap=5.0,
                                           dX_dtype=torch.bfloat16, dW_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    f, rdX, rdW = O.forward_backward_chunked(L.to_f64(X), L.to_f64(W), y.numpy(), 1.0,
                                             O.options(softcap=5.0), 256)
    assert int(out["bad_label"]) == 1 and np.isnan(float(out["reduced"]))
    loss = out["loss"].cpu().numpy()
    ok = np.arange(520) != 9
    assert np.isnan(loss[9])
    np.testing.assert_allclose(loss[ok], f["loss"][ok], rtol=0, atol=LSE_ATOL)
    dXn = dX.float().cpu().numpy()
    assert np.isnan(dXn[9]).all() and not np.isnan(dXn[ok]).any()
    assert np.isnan(dW.float().cpu().numpy()).all() and np.isnan(rdW).all()
    # Without the bad row, bf16 outputs against the oracle.
    y2 = y.clone()
    y2[9] = 3
    out, dX, dW = lce.lce_forward_backward(X.cuda(), W.cuda(), y2.cuda(), 1.0, softcap=5.0,
                                           dX_dtype=torch.bfloat16, dW_dtype=torch.bfloat16)
    f, rdX, rdW = O.forward_backward_chunked(L.to_f64(X), L.to_f64(W), y2.numpy(), 1.0,
                                             O.options(softcap=5.0), 256)
    assert rel_l2(dX.float().cpu(), rdX) <= 1e-2 and rel_l2(dW.float().cpu(), rdW) <= 1e-2


def test_fused_rejects_smoothing_with_softcap(lce):
    X, W, y = (t.cuda() for t in L.make_inputs(L.Workload("v", N=8, H=8, V=10)))
    with pytest.raises(lce.LceError):
        lce.lce_forward_backward(X, W, y, 1.0, softcap=30.0, label_smoothing=0.1)


@pytest.mark.parametrize("name", ["gemma2_2b", "llama3_8b", "liger", "qwen25_long"])
def test_fused_fullsize(lce, name):
    """Each large workload in one fused call against the stored oracle values
    (every row's LSE and loss, sampled dX and dW rows)."""
    gold = np.load(os.path.join(HERE, "golden", f"fullsize_{name}.npz"))
    w = L.WORKLOADS[name]
    X, W, y = L.make_inputs(w)
    assert L.fingerprint(X, W, y) == str(gold["fingerprint"])
    print(f"[fused] {name} full size: N={w.N} H={w.H} V={w.V} softcap={w.softcap}", flush=True)
    dev = "cuda"
    out, dX, dW = lce.lce_forward_backward(X.to(dev), W.to(dev), y.to(dev), 1.0,
                                           softcap=w.softcap)
    torch.cuda.synchronize()
    assert int(out["n_valid"]) == int(gold["n_valid"]) and int(out["bad_label"]) == 0
    e_lse = np.abs(out["lse"].cpu().numpy() - gold["lse"]).max()
    e_loss = np.abs(out["loss"].cpu().numpy() - gold["loss"]).max()
    mean, gmean = float(out["reduced"]), float(gold["mean"])
    e_dx = rel_l2(dX[torch.from_numpy(gold["dx_rows"]).to(dev)].cpu(), gold["dX"])
    e_dw = rel_l2(dW[torch.from_numpy(gold["dw_rows"]).to(dev)].cpu(), gold["dW"])
    print(f"[fused] {name}: lse {e_lse:.2e} loss {e_loss:.2e} mean rel "
          f"{abs(mean - gmean) / abs(gmean):.2e} dX {e_dx:.2e} dW {e_dw:.2e}", flush=True)
    assert e_lse <= LSE_ATOL and e_loss <= LSE_ATOL
    assert abs(mean - gmean) <= RED_RTOL * abs(gmean)
    assert e_dx <= GRAD_RTOL and e_dw <= GRAD_RTOL
    S = FS.samples(name, X, W, y, dict(softcap=w.softcap))
    FS.check(f"fused {name}", dX, dW, S, GRAD_RTOL, 1e-2, log=lambda m: print(m, flush=True))
