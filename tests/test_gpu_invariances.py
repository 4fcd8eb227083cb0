"""Closed-form properties of the kernels' results that need no oracle.

Shift (no softcap): with a column of ones appended to X and a column of a
bf16-exact constant c appended to W (seven zero columns after each keep H a
multiple of 8), every logit x·w_v becomes x·w_v + c.  The softmax and so the
loss, dX and dW restricted to the original columns are unchanged, and every
LSE moves by exactly c (the shift-invariance of log-sum-exp behind the
running-max merge: blog "最贵的一层：深入浅出 Liger Kernel 与 Cut Cross-Entropy",
§二; AI-infra KB M011 §05).

Permutation (with and without softcap): with the rows of W permuted by π and
every label relabelled so that it names the same W row, the per-row LSE and
loss are unchanged and dW comes out permuted the same way, dX unchanged.

Both sides run on the GPU; only the order of floating-point sums differs
(where the constant enters the K sum, which tiles and splits a row's terms
fall in), so LSE and loss agree to 1e-5 and the gradients to 1e-4 relative L2
(a bf16 rounding of the gradient chunk may flip for entries a few ulps from a
rounding boundary).
"""
import numpy as np
import pytest
import torch

import lce_inputs as L

pytestmark = pytest.mark.gpu

ATOL = 1e-5
GRAD_RTOL = 1e-4


@pytest.fixture(scope="module")
def lce():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_cross_entropy_lse_amd as P
    P.load()
    return P


def inputs(N, H, V, seed, softcap):
    w = L.Workload("invariance", N=N, H=H, V=V, labels="uniform", ignore_frac=0.1,
                   softcap=softcap, seed=seed)
    X, W, y = L.make_inputs(w)
    W = (W.float() * 4.0).to(torch.bfloat16)
    return X.cuda(), W.cuda(), y.cuda()


def step(lce, X, W, y, softcap):
    out = lce.lce_forward(X, W, y, -100, softcap)
    dX, dW = lce.lce_backward(X, W, y, out["lse"], 1.0, -100, softcap)
    torch.cuda.synchronize()
    return out, dX, dW


def rel_l2(a, b):
    return float(torch.linalg.vector_norm((a - b).double()) / torch.linalg.vector_norm(b.double()))


@pytest.mark.parametrize("N,H,V,c", [
    (700, 64, 3001, 3.0),      # H + 8 = 72: a K tail appears
    (300, 256, 20000, -5.5),   # several vocabulary chunks
])
def test_shift_moves_lse_by_the_constant(lce, N, H, V, c):
    X, W, y = inputs(N, H, V, 7100 + N, 0.0)
    pad_x = torch.zeros(N, 8, dtype=torch.bfloat16, device="cuda")
    pad_x[:, 0] = 1.0
    pad_w = torch.zeros(V, 8, dtype=torch.bfloat16, device="cuda")
    pad_w[:, 0] = c
    Xs, Ws = torch.cat([X, pad_x], 1).contiguous(), torch.cat([W, pad_w], 1).contiguous()
    print(f"[invariance] shift N={N} H={H}->{H + 8} V={V} c={c}", flush=True)
    a, dX, dW = step(lce, X, W, y, 0.0)
    b, dXs, dWs = step(lce, Xs, Ws, y, 0.0)
    e_lse = float((b["lse"] - a["lse"] - c).abs().max())
    e_loss = float((b["loss"] - a["loss"]).abs().max())
    e_dx, e_dw = rel_l2(dXs[:, :H], dX), rel_l2(dWs[:, :H], dW)
    print(f"[invariance] shift: LSE - c {e_lse:.2e} loss {e_loss:.2e} dX {e_dx:.2e} dW {e_dw:.2e}",
          flush=True)
    assert int(a["n_valid"]) == int(b["n_valid"])
    assert e_lse <= ATOL and e_loss <= ATOL
    assert abs(float(b["mean"]) - float(a["mean"])) <= ATOL
    assert e_dx <= GRAD_RTOL and e_dw <= GRAD_RTOL
    # Zero columns of W and X give exactly zero dX and dW columns.
    assert torch.count_nonzero(dXs[:, H + 1:]).item() == 0
    assert torch.count_nonzero(dWs[:, H + 1:]).item() == 0


@pytest.mark.parametrize("N,H,V,softcap", [
    (600, 136, 5000, 30.0),
    (513, 64, 40000, 0.0),     # several vocabulary chunks
])
def test_vocabulary_permutation(lce, N, H, V, softcap):
    X, W, y = inputs(N, H, V, 7200 + N, softcap)
    perm = torch.from_numpy(np.random.default_rng(N).permutation(V)).cuda()   # row v of Wp is W[perm[v]]
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(V, device="cuda")
    Wp = W[perm].contiguous()
    yp = torch.where(y == -100, y, inv[y.clamp(min=0)])
    print(f"[invariance] permutation N={N} H={H} V={V} softcap={softcap}", flush=True)
    a, dX, dW = step(lce, X, W, y, softcap)
    b, dXp, dWp = step(lce, X, Wp, yp, softcap)
    e_lse = float((b["lse"] - a["lse"]).abs().max())
    e_loss = float((b["loss"] - a["loss"]).abs().max())
    e_dx, e_dw = rel_l2(dXp, dX), rel_l2(dWp, dW[perm])
    print(f"[invariance] permutation: LSE {e_lse:.2e} loss {e_loss:.2e} dX {e_dx:.2e} dW {e_dw:.2e}",
          flush=True)
    assert e_lse <= ATOL and e_loss <= ATOL
    assert e_dx <= GRAD_RTOL and e_dw <= GRAD_RTOL


def test_noncontiguous_inputs_match_contiguous(lce):
    """Strided and transposed views (a contiguity class of wrong results the
    Liger Kernel paper page lists among its test cases) give bitwise the
    results of contiguous copies: the binding passes the kernels, which
    address memory directly, contiguous tensors."""
    N, H, V, softcap = 300, 72, 2000, 30.0
    X, W, y = inputs(N, H, V, 7300, softcap)
    Xv = X.t().contiguous().t()                                   # column-major view
    Wbig = torch.zeros(2 * V, H, dtype=torch.bfloat16, device="cuda")
    Wbig[::2] = W
    Wv = Wbig[::2]                                                # row stride 2H
    ybig = torch.full((2 * N,), -7, dtype=torch.int64, device="cuda")
    ybig[1::2] = y
    yv = ybig[1::2]                                               # element stride 2
    assert not (Xv.is_contiguous() or Wv.is_contiguous() or yv.is_contiguous())
    print(f"[invariance] non-contiguous views N={N} H={H} V={V}", flush=True)
    a, dX, dW = step(lce, X, W, y, softcap)
    b, dXv, dWv = step(lce, Xv, Wv, yv, softcap)
    for k in ("loss", "lse", "mean", "n_valid"):
        assert torch.equal(a[k], b[k]), k
    assert torch.equal(dX, dXv) and torch.equal(dW, dWv)
