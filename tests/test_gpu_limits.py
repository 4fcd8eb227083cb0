"""Large-vocabulary limits of the backward's chunking, against the oracle.

The bf16 gradient chunk is at most 2^21 columns wide: a 256-row block of it
then spans less than 2^31 bytes, the range of the 32-bit buffer offsets the
gradient kernels use.  With few rows and a vocabulary past 2^21 entries that
cap is what sets the chunks (N·Vc ≤ V·H would allow wider ones), so these cases
run chunks at or near the cap, a forward with one token tile split over every
compute unit, and a dW of V rows past the 2^31-byte mark.

Checked: every row's LSE and loss (abs ≤ 2e-3), the mean (rel ≤ 1e-4),
n_valid, dX and dW in float32 (rel-L2 ≤ 1e-3), and dW on the rows no label hits
on its own (only the bf16 chunk and the MFMA contraction form them; bf16 bar
1e-2).
"""
import numpy as np
import pytest
import torch

import lce_inputs as L
from oracle import lce_oracle as O

pytestmark = pytest.mark.gpu

CASES = [
    # N, H, V, softcap
    (40, 64, (1 << 21) + 100003, 30.0),     # the cap sets two chunks of 1 098 752 columns
    (260, 200, (1 << 21) + 256 * 7, 0.0),   # N·Vc ≤ V·H sets two of 1 049 600; K tail, two token tiles
]


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


@pytest.mark.parametrize("N,H,V,softcap", CASES)
def test_vocabulary_past_the_chunk_cap(lce, N, H, V, softcap):
    print(f"[limits] N={N} H={H} V={V} softcap={softcap}", flush=True)
    w = L.Workload("limits", N=N, H=H, V=V, labels="uniform", ignore_frac=0.1, softcap=softcap,
                   seed=7700 + N)
    X, W, y = L.make_inputs(w)
    W = (W.float() * 4.0).to(torch.bfloat16)
    dev = "cuda"
    Xd, Wd, yd = X.to(dev), W.to(dev), y.to(dev)
    out = lce.lce_forward(Xd, Wd, yd, -100, softcap)
    dX, dW = lce.lce_backward(Xd, Wd, yd, out["lse"], 1.0, -100, softcap)
    torch.cuda.synchronize()
    g = {k: v.cpu() for k, v in out.items()}
    dX, dW = dX.cpu().numpy(), dW.cpu().numpy()
    del Xd, Wd, out
    torch.cuda.empty_cache()
    print("[limits] GPU done; oracle", flush=True)
    X64, W64, y64 = L.to_f64(X), L.to_f64(W), y.numpy()
    f = O.forward(X64, W64, y64, -100, softcap)
    rdX, rdW = O.backward(X64, W64, y64, 1.0, -100, softcap)
    assert int(g["n_valid"]) == f["n_valid"]
    np.testing.assert_allclose(g["lse"].numpy(), f["lse"], rtol=0, atol=2e-3)
    np.testing.assert_allclose(g["loss"].numpy(), f["loss"], rtol=0, atol=2e-3)
    assert abs(float(g["mean"]) - f["mean"]) <= 1e-4 * abs(f["mean"])
    free = np.ones(V, dtype=bool)
    free[y64[y64 != -100]] = False
    e = [rel_l2(dX, rdX), rel_l2(dW, rdW), rel_l2(dW[free], rdW[free])]
    print(f"[limits] lse max err {np.abs(g['lse'].numpy() - f['lse']).max():.2e} dX {e[0]:.2e} "
          f"dW {e[1]:.2e} label-free dW rows {e[2]:.2e}", flush=True)
    assert e[0] <= 1e-3 and e[1] <= 1e-3
    assert e[2] <= 1e-2


@pytest.mark.parametrize("mode", ["sorted", "precise", "shards"])
def test_past_the_chunk_cap_other_paths(lce, mode):
    """The same 2^21-column chunks through the sorted backward (a seeded random
    order: the gathered W chunk and the scattered dW rows span past 2^31
    bytes), the precise gradient (three chunks of 732 416 columns, two parts
    each) and two vocabulary shards of uneven size."""
    N, H, V, softcap = 40, 64, (1 << 21) + 100003, 30.0
    print(f"[limits] {mode}: N={N} H={H} V={V} softcap={softcap}", flush=True)
    w = L.Workload("limits", N=N, H=H, V=V, labels="uniform", ignore_frac=0.1, softcap=softcap,
                   seed=7800)
    X, W, y = L.make_inputs(w)
    W = (W.float() * 4.0).to(torch.bfloat16)
    Xd, Wd, yd = X.cuda(), W.cuda(), y.cuda()
    lse = lce.lce_forward(Xd, Wd, yd, -100, softcap)["lse"]
    if mode == "sorted":
        order = torch.from_numpy(np.random.default_rng(5).permutation(V).astype(np.int32)).cuda()
        dX, dW = lce.lce_backward_sorted(Xd, Wd, yd, lse, 1.0, order, softcap=softcap)
    elif mode == "precise":
        dX, dW = lce.lce_backward_ex(Xd, Wd, yd, lse, 1.0, softcap=softcap, precise=True)
    else:
        cut = 700001
        ax, aw = lce.lce_shard_backward(Xd, Wd[:cut], yd, lse, 1.0, 0, V, softcap=softcap)
        bx, bw = lce.lce_shard_backward(Xd, Wd[cut:], yd, lse, 1.0, cut, V, softcap=softcap)
        dX, dW = ax + bx, torch.cat([aw, bw])
    torch.cuda.synchronize()
    dX, dW = dX.cpu().numpy(), dW.cpu().numpy()
    del Xd, Wd
    torch.cuda.empty_cache()
    X64, W64, y64 = L.to_f64(X), L.to_f64(W), y.numpy()
    rdX, rdW = O.backward(X64, W64, y64, 1.0, -100, softcap)
    free = np.ones(V, dtype=bool)
    free[y64[y64 != -100]] = False
    e = [rel_l2(dX, rdX), rel_l2(dW, rdW), rel_l2(dW[free], rdW[free])]
    print(f"[limits] {mode}: dX {e[0]:.2e} dW {e[1]:.2e} label-free dW rows {e[2]:.2e}", flush=True)
    assert e[0] <= 1e-3 and e[1] <= 1e-3
    assert e[2] <= (1e-4 if mode == "precise" else 1e-2)
