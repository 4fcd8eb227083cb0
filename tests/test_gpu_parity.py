"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Tolerances (stated for this method): per-row LSE and loss absolute error
≤ 2e-3, mean-loss relative error ≤ 1e-4, dX and dW relative L2 error ≤ 1e-3
when emitted in float32 and ≤ 1e-2 when emitted in bfloat16.  Integer outputs
(n_valid, the bad-label flag) must match exactly.
"""
import math

import numpy as np
import pytest
import torch

import lce_inputs as L
from oracle import lce_oracle as O

pytestmark = pytest.mark.gpu

LSE_ATOL = 2e-3
MEAN_RTOL = 1e-4
GRAD_RTOL_F32 = 1e-3
GRAD_RTOL_BF16 = 1e-2


@pytest.fixture(scope="module")
def lce():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_cross_entropy_lse_amd as P
    P.load()          # raises if liblce.so is missing: no fallback path exists
    return P


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (den if den > 0 else 1.0)


def run_gpu(lce, X, W, y, softcap=0.0, ignore_index=-100, dloss=1.0, dX_dtype=torch.float32,
            dW_dtype=torch.float32):
    dev = "cuda"
    Xd, Wd, yd = X.to(dev), W.to(dev), y.to(dev)
    out = lce.lce_forward(Xd, Wd, yd, ignore_index, softcap)
    dX, dW = lce.lce_backward(Xd, Wd, yd, out["lse"], torch.tensor(dloss, device=dev),
                              ignore_index, softcap, dX_dtype=dX_dtype, dW_dtype=dW_dtype)
    torch.cuda.synchronize()
    res = {k: v.cpu() for k, v in out.items()}
    res["dX"] = dX.float().cpu()
    res["dW"] = dW.float().cpu()
    return res


def oracle_all(X, W, y, softcap=0.0, ignore_index=-100, dloss=1.0):
    X64, W64, y64 = L.to_f64(X), L.to_f64(W), y.numpy()
    f = O.forward(X64, W64, y64, ignore_index, softcap)
    dX, dW = O.backward(X64, W64, y64, dloss, ignore_index, softcap)
    return f, dX, dW


def check(g, f, dX, dW, grad_rtol=GRAD_RTOL_F32, what=""):
    print(f"[parity] {what}", flush=True)
    assert int(g["n_valid"]) == f["n_valid"]
    np.testing.assert_allclose(g["lse"].numpy(), f["lse"], rtol=0, atol=LSE_ATOL)
    np.testing.assert_allclose(g["loss"].numpy(), f["loss"], rtol=0, atol=LSE_ATOL)
    if f["n_valid"] > 0:
        assert abs(float(g["mean"]) - f["mean"]) <= MEAN_RTOL * max(abs(f["mean"]), 1e-30)
    else:
        assert float(g["mean"]) == 0.0
    e_dx, e_dw = rel_l2(g["dX"], dX), rel_l2(g["dW"], dW)
    print(f"[parity] {what}: lse max err {np.abs(g['lse'].numpy() - f['lse']).max():.2e} "
          f"dX rel {e_dx:.2e} dW rel {e_dw:.2e}", flush=True)
    assert e_dx <= grad_rtol, e_dx
    assert e_dw <= grad_rtol, e_dw


def synth(N, H, V, seed, softcap=0.0, ignore_frac=0.1, labels="uniform"):
    w = L.Workload("synthetic", N=N, H=H, V=V, labels=labels, ignore_frac=ignore_frac,
                   softcap=softcap, seed=seed)
    return L.make_inputs(w)


# --------------------------------------------------------------------------- #
def test_tiny_config(lce):
    w = L.WORKLOADS["tiny"]
    X, W, y = L.make_inputs(w)
    g = run_gpu(lce, X, W, y, w.softcap)
    check(g, *oracle_all(X, W, y, w.softcap), what="tiny")
    assert int(g["bad_label"]) == 0


@pytest.mark.parametrize("N,H,V,softcap", [
    (257, 72, 1003, 0.0),       # ragged rows, K tail (72 = 64 + 8), ragged vocab
    (600, 200, 1500, 0.0),      # 3 token tiles, 6 vocab tiles, 4 K-steps with a tail
    (513, 136, 2100, 1.5),      # softcap that actually bends the logits
    (96, 64, 300, 30.0),        # a single partial tile in both dimensions
    (1, 8, 1, 0.0),             # degenerate: one row, one class
    (300, 64, 40000, 0.0),      # several backward vocabulary chunks, split-K for dX
    (700, 48, 20000, 4.0),      # several chunks with softcap and a short K
    # A handful of classes: the softmax part is most of each gradient row.
    (513, 64, 5, 0.0),
    (513, 64, 3, 30.0),
    (300, 72, 2, 0.0),
])
def test_irregular_shapes(lce, N, H, V, softcap):
    X, W, y = synth(N, H, V, seed=1000 + N + V, softcap=softcap)
    # Logits of a useful size so the softmax is neither flat nor one-hot.
    W = (W.float() * 4.0).to(torch.bfloat16)
    g = run_gpu(lce, X, W, y, softcap)
    check(g, *oracle_all(X, W, y, softcap), what=f"N={N} H={H} V={V} c={softcap}")


# The pipelined tile loop has separate code for tiles of one, two and three
# or more 64-deep K-steps (its last two steps load nothing unless a sweep
# runs on into the next tile), and for a K that is not a multiple of 64.
# K is H in the forward and the logit-gradient pass, N in the dW contraction
# and the chunk's vocabulary in the dX contraction (one chunk at these sizes).
@pytest.mark.parametrize("N,H,V,softcap", [
    (64, 64, 64, 0.0),          # one step in every contraction
    (128, 128, 128, 0.0),       # two steps
    (192, 192, 192, 30.0),      # three steps, fixed-reference softcap
    (256, 256, 256, 0.0),       # four steps
    (320, 264, 200, 0.0),       # five steps with a K tail (264 = 4·64 + 8); ragged vocabulary
    (64, 128, 3000, 1.5),       # sweeps over 12 vocabulary tiles with one-step dW tiles
    (192, 64, 130, 0.0),        # one-step forward, three-step dW, three-step dX (130 = 2·64 + 2)
    # One-step tiles (H <= 64) in sweeps of several vocabulary tiles per split
    # (one token tile: 256 splits, V / 65536 tiles and more per split): each
    # tile of such a sweep loads its own first step.
    (100, 64, 150000, 0.0),
    (300, 32, 90000, 30.0),
    (64, 8, 70000, 1.5),
])
def test_pipeline_step_counts(lce, N, H, V, softcap):
    X, W, y = synth(N, H, V, seed=3000 + N + H + V, softcap=softcap)
    W = (W.float() * 4.0).to(torch.bfloat16)
    g = run_gpu(lce, X, W, y, softcap)
    check(g, *oracle_all(X, W, y, softcap), what=f"steps N={N} H={H} V={V} c={softcap}")


# Few token tiles: the dX tiles of a chunk are too few to spread over the
# workgroups, so their vocabulary range is split into K parts summed at the
# end.  (N, H, V): 2 chunks of 16128 columns in 9 parts each; 4 chunks of
# 12544 columns in 16 parts, the last one (12368 columns) in 15, with
# softcap; one chunk in 2 parts at H = 2304 (K tail, 9 hidden tiles).
@pytest.mark.parametrize("N,H,V,softcap", [
    (4096, 256, 32000, 0.0),
    (1100, 64, 50000, 30.0),
    (2000, 2304, 6000, 30.0),
])
def test_split_dx_parts(lce, N, H, V, softcap):
    X, W, y = synth(N, H, V, seed=3500 + N, softcap=softcap)
    W = (W.float() * 4.0).to(torch.bfloat16)
    g = run_gpu(lce, X, W, y, softcap)
    check(g, *oracle_all(X, W, y, softcap), what=f"dX parts N={N} H={H} V={V} c={softcap}")


# More than 32 token tiles: the forward runs in launches of 32 token tiles x
# 8 splits and the tiles left over in a launch of their own with more splits;
# the logit-gradient grid runs in full rounds of 256 / S token tiles x S
# splits, then the tiles left over in a launch of their own.  (N, H, V):
#   * 36 token tiles, one chunk of 12 vocabulary tiles: one round of 32 x 8,
#     then 4 tiles x 12 splits (forward: 32 x 8, then 4 x 12);
#   * 79 token tiles, one chunk of 20 vocabulary tiles, a K tail and softcap:
#     one round of 64 x 4, then 15 x 17 (forward: two launches of 32 x 8, then
#     15 x 17);
#   * 33 token tiles, the last holding one row: 32 x 8, then 1 x 8 (8
#     vocabulary tiles) in both;
#   * 36 token tiles and 4 vocabulary tiles: no full round fits, one gradient
#     launch of 36 x 4 (forward: 32 x 4, then 4 x 4).
@pytest.mark.parametrize("N,H,V,softcap", [
    (9000, 64, 3000, 0.0),
    (20000, 72, 5000, 30.0),
    (8193, 64, 2000, 0.0),
    (9000, 64, 1000, 30.0),
])
def test_many_token_tiles(lce, N, H, V, softcap):
    X, W, y = synth(N, H, V, seed=3700 + N, softcap=softcap)
    W = (W.float() * 4.0).to(torch.bfloat16)
    g = run_gpu(lce, X, W, y, softcap)
    check(g, *oracle_all(X, W, y, softcap), what=f"token tiles N={N} H={H} V={V} c={softcap}")


# Logits in the hundreds: e^z overflows a float from z ≈ 88.7, so the forward
# must keep its running maximum, rescale its running sums when the maximum
# rises in a later vocabulary tile (the ramp puts the largest logits in the
# last tiles), and merge split partials whose maxima differ by hundreds.
# V = 20000 gives 79 vocabulary tiles, 2–3 per split, a partial last tile and
# ~30 backward vocabulary chunks; H = 72 has a K tail.  Softcap 100 takes the
# general path (max pass on the raw logits), 30 the fixed reference with the
# tanh saturated.
@pytest.mark.parametrize("softcap,ramp", [
    (0.0, False),
    (0.0, True),
    (100.0, False),
    (100.0, True),
    (30.0, True),
])
def test_large_logits(lce, softcap, ramp):
    N, H, V = 2300, 72, 20000
    X, W, y = synth(N, H, V, seed=4100 + int(softcap) + int(ramp), softcap=softcap)
    Wf = W.float() * 200.0      # logit std ≈ 34, extremes ≈ ±200 (±260 with the ramp)
    if ramp:
        Wf *= torch.linspace(0.25, 1.5, V).unsqueeze(1)
    W = Wf.to(torch.bfloat16)
    g = run_gpu(lce, X, W, y, softcap)
    check(g, *oracle_all(X, W, y, softcap), what=f"large logits c={softcap} ramp={ramp}")
    assert bool(torch.isfinite(g["lse"]).all())


def test_bf16_gradients(lce):
    X, W, y = synth(400, 128, 3000, seed=7, softcap=2.0)
    W = (W.float() * 4.0).to(torch.bfloat16)
    g = run_gpu(lce, X, W, y, 2.0, dX_dtype=torch.bfloat16, dW_dtype=torch.bfloat16)
    check(g, *oracle_all(X, W, y, 2.0), grad_rtol=GRAD_RTOL_BF16, what="bf16 grads")


def test_dloss_and_ignore_index(lce):
    X, W, y = synth(300, 64, 700, seed=8)
    y = y.clone()
    y[y == -100] = 7            # the ignore marker is -100 no longer...
    y[::5] = 3                  # ...every 5th row now carries the custom marker 3
    g = run_gpu(lce, X, W, y, ignore_index=3, dloss=0.37)
    check(g, *oracle_all(X, W, y, ignore_index=3, dloss=0.37), what="ignore_index=3 dloss=0.37")


def test_all_rows_ignored(lce):
    X, W, y = synth(100, 64, 500, seed=9)
    y = torch.full_like(y, -100)
    g = run_gpu(lce, X, W, y)
    assert int(g["n_valid"]) == 0 and float(g["mean"]) == 0.0
    assert torch.all(g["loss"] == 0) and torch.all(g["dX"] == 0) and torch.all(g["dW"] == 0)
    f = O.forward(L.to_f64(X), L.to_f64(W), y.numpy())
    np.testing.assert_allclose(g["lse"].numpy(), f["lse"], atol=LSE_ATOL)


def test_bad_label_flag(lce):
    X, W, y = synth(64, 64, 100, seed=10)
    y = y.clone()
    y[5] = 100                  # == V: out of range
    g = run_gpu(lce, X, W, y)
    assert int(g["bad_label"]) == 1
    assert math.isnan(float(g["loss"][5])) and math.isnan(float(g["mean"]))
    ok = torch.ones(64, dtype=torch.bool)
    ok[5] = False
    f = O.forward(L.to_f64(X), L.to_f64(W), y.numpy())
    np.testing.assert_allclose(g["loss"].numpy()[ok.numpy()], f["loss"][ok.numpy()], atol=LSE_ATOL)


def test_empty_batch(lce):
    X = torch.zeros(0, 64, dtype=torch.bfloat16)
    W = L.make_w(L.Workload("e", N=0, H=64, V=50))
    y = torch.zeros(0, dtype=torch.int64)
    g = run_gpu(lce, X, W, y)
    assert int(g["n_valid"]) == 0 and float(g["mean"]) == 0.0
    assert g["dX"].shape == (0, 64) and torch.all(g["dW"] == 0)


def test_zero_weight_closed_form(lce):
    # W = 0: every logit is 0, so LSE = ln V exactly, dX = 0 and
    # dW_v = s · Σ_valid (1/V − [y_i = v]) x_i — needs no oracle.
    N, H, V = 300, 64, 777
    X, _, y = synth(N, H, V, seed=11)
    W = torch.zeros(V, H, dtype=torch.bfloat16)
    g = run_gpu(lce, X, W, y, dloss=2.0)
    np.testing.assert_allclose(g["lse"].numpy(), math.log(V), rtol=0, atol=1e-5)
    assert torch.all(g["dX"] == 0)
    valid = (y != -100).numpy()
    s = 2.0 / valid.sum()
    X64 = L.to_f64(X)
    expect = np.zeros((V, H))
    expect += s * (X64[valid].sum(axis=0) / V)[None, :]
    np.add.at(expect, y.numpy()[valid], -s * X64[valid])
    assert rel_l2(g["dW"], expect) < 1e-3


@pytest.mark.parametrize("N,H,V", [
    (600, 200, 1500),
    (8300, 64, 3000),    # 33 token tiles: the forward's and the gradient's tail launches
])
def test_deterministic_bitwise(lce, N, H, V):
    X, W, y = synth(N, H, V, seed=12, softcap=5.0)
    a = run_gpu(lce, X, W, y, 5.0)
    b = run_gpu(lce, X, W, y, 5.0)
    for k in ("loss", "lse", "mean", "dX", "dW"):
        assert torch.equal(a[k].view(torch.int32), b[k].view(torch.int32)), k


def test_fused_deterministic_bitwise(lce):
    """The fused call twice on uneven row chunks (1536 + 1064 rows, their own
    dX parts): bitwise the same outputs."""
    X, W, y = synth(2600, 1024, 4000, seed=14, softcap=0.0)
    Xd, Wd, yd = X.cuda(), W.cuda(), y.cuda()
    a = lce.lce_forward_backward(Xd, Wd, yd, 1.0)
    b = lce.lce_forward_backward(Xd, Wd, yd, 1.0)
    torch.cuda.synchronize()
    for k in ("loss", "lse", "reduced"):
        assert torch.equal(a[0][k], b[0][k]), k
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])


def test_autograd_wrapper(lce):
    X, W, y = synth(300, 64, 1000, seed=13)
    Xd = X.cuda().requires_grad_(True)
    Wd = W.cuda().requires_grad_(True)
    loss = lce.linear_cross_entropy(Xd, Wd, y.cuda())
    (loss * 1.5).backward()
    f, dX, dW = oracle_all(X, W, y, dloss=1.5)
    assert abs(loss.item() - f["mean"]) <= MEAN_RTOL * abs(f["mean"])
    assert rel_l2(Xd.grad.float().cpu(), dX) <= GRAD_RTOL_BF16
    assert rel_l2(Wd.grad.float().cpu(), dW) <= GRAD_RTOL_BF16


def test_no_logit_sized_allocation(lce):
    # Peak extra memory of forward + backward stays O(N·H + V·H), far below the
    # N·V·2 bytes a bf16 logit matrix would need.
    X, W, y = synth(4096, 256, 32000, seed=14)
    dev = "cuda"
    Xd, Wd, yd = X.to(dev), W.to(dev), y.to(dev)
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    out = lce.lce_forward(Xd, Wd, yd)
    dX, dW = lce.lce_backward(Xd, Wd, yd, out["lse"], 1.0)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    N, H, V = 4096, 256, 32000
    ws = lce.lce_backward_workspace_bytes(N, H, V)
    outputs = N * H * 4 + V * H * 4 + 5 * N * 4
    assert peak <= ws + outputs + (1 << 20), (peak, ws, outputs)
    assert ws < N * V * 2
