"""Parity of the vocabulary-shard calls (lce_shard_forward, lce_shard_merge,
lce_shard_backward) with the CPU oracle.

W is cut into contiguous shards; each shard's partials go into row k of
[n_shards, N] buffers (standing in for the all-gather between ranks), the
merge gives the loss, and the shards' dX shares are added in shard order
(standing in for the all-reduce).  Bars as for the whole-vocabulary path:
LSE and loss abs err <= 2e-3, the reduced loss rel err <= 1e-4, dX and dW
rel-L2 err <= 1e-3 (float32), n_valid exact.  The full-size case runs the
Gemma-2 2B head as 8 shards of 32016 rows, the shape one rank holds at a
vocabulary-parallel degree of 8.
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


def run_shards(lce, Xd, Wd, yd, edges, opts, dloss):
    """Forward of every shard, merge, backward of every shard."""
    V = Wd.shape[0]
    fwd_opts = {k: opts[k] for k in ("ignore_index", "softcap", "logit_scale") if k in opts}
    merge_opts = {k: opts[k] for k in ("ignore_index", "label_smoothing", "z_loss", "reduction")
                  if k in opts}
    smoothing = opts.get("label_smoothing", 0.0) > 0
    parts = [lce.lce_shard_forward(Xd, Wd[a:b], yd, a, V, with_zsum=smoothing, **fwd_opts)
             for a, b in zip(edges[:-1], edges[1:])]
    stack = lambda k: torch.stack([p[k] for p in parts])  # noqa: E731
    out = lce.lce_shard_merge(stack("lse_part"), stack("target_part"), yd, V,
                              zsum_parts=stack("zsum_part") if smoothing else None, **merge_opts)
    dX, dWs = None, []
    for a, b in zip(edges[:-1], edges[1:]):
        gx, gw = lce.lce_shard_backward(Xd, Wd[a:b], yd, out["lse"], dloss, a, V, **opts)
        dX = gx if dX is None else dX + gx
        dWs.append(gw)
    return parts, out, dX, torch.cat(dWs)


CASES = [
    # N, H, V, shard edges (fractions of V), options
    (257, 72, 1003, [0, 0.3, 0.31, 1.0], dict()),
    (513, 136, 2100, [0, 0.25, 0.5, 0.75, 1.0], dict(softcap=3.0, reduction="sum")),
    (300, 64, 40000, [0, 0.5, 1.0], dict(softcap=30.0, label_smoothing=0.1, z_loss=1e-3,
                                         logit_scale=1.3, reduction="none")),
    (96, 48, 700, [0, 0.1, 0.9, 1.0], dict(label_smoothing=0.2)),
    # 33 token tiles: each shard's forward runs a launch of 32 token tiles and
    # one of the last tile, whose partials and per-row logit sums (label
    # smoothing) sit in a block of their own.
    (8400, 64, 3000, [0, 0.4, 1.0], dict(label_smoothing=0.1, softcap=30.0)),
]


@pytest.mark.parametrize("N,H,V,fr,opts", CASES)
def test_shards_against_oracle(lce, N, H, V, fr, opts):
    w = L.Workload("shards", N=N, H=H, V=V, labels="uniform", ignore_frac=0.1,
                   seed=5000 + N + V)
    X, W, y = L.make_inputs(w)
    W = (W.float() * 4.0).to(torch.bfloat16)
    edges = sorted(set([0, V] + [int(round(f * V)) for f in fr]))
    print(f"[shards] N={N} H={H} V={V} edges={edges} {opts}", flush=True)
    red = opts.get("reduction", "mean")
    rng = np.random.default_rng(N)
    dloss = rng.standard_normal(N).astype(np.float32) if red == "none" else np.float32(0.7)
    dev = "cuda"
    Xd, Wd, yd = X.to(dev), W.to(dev), y.to(dev)
    dl = torch.from_numpy(np.atleast_1d(dloss)).to(dev)
    parts, out, dX, dW = run_shards(lce, Xd, Wd, yd, edges, opts, dl)
    torch.cuda.synchronize()

    o = O.options(**opts)
    X64, W64, y64 = L.to_f64(X), L.to_f64(W), y.numpy()
    # Each shard's partials against the oracle's shard function.
    for k, (a, b) in enumerate(zip(edges[:-1], edges[1:])):
        ref = O.forward_shard(X64, W64[a:b], y64, a, V, o)
        np.testing.assert_allclose(parts[k]["lse_part"].cpu().numpy(), ref["lse_part"],
                                   rtol=0, atol=LSE_ATOL)
        np.testing.assert_allclose(parts[k]["target_part"].cpu().numpy(), ref["target_part"],
                                   rtol=0, atol=LSE_ATOL)
        if "zsum_part" in parts[k]:
            zs = parts[k]["zsum_part"].cpu().numpy()
            assert np.abs(zs - ref["zsum_part"]).max() <= 1e-4 * np.abs(ref["zsum_part"]).max() + 1e-3
    f = O.forward_ex(X64, W64, y64, o)
    assert int(out["n_valid"]) == f["n_valid"] and int(out["bad_label"]) == 0
    np.testing.assert_allclose(out["lse"].cpu().numpy(), f["lse"], rtol=0, atol=LSE_ATOL)
    np.testing.assert_allclose(out["loss"].cpu().numpy(), f["loss"], rtol=0, atol=LSE_ATOL)
    assert abs(float(out["reduced"]) - f["reduced"]) <= RED_RTOL * abs(f["reduced"])
    rdX, rdW = O.backward_ex(X64, W64, y64, dloss.astype(np.float64) if red == "none" else 0.7, o)
    e_dx = rel_l2(dX.cpu(), rdX)
    e_dw = rel_l2(dW.cpu(), rdW)
    print(f"[shards] dX rel {e_dx:.2e} dW rel {e_dw:.2e}", flush=True)
    assert e_dx <= GRAD_RTOL and e_dw <= GRAD_RTOL


def test_merge_flags_out_of_range_label(lce):
    """A label outside [0, vocab_total) gives a NaN loss for its row, a NaN
    reduced loss and the bad-label flag; the other rows are unaffected."""
    w = L.Workload("shards", N=200, H=64, V=900, labels="uniform", ignore_frac=0.1, seed=93)
    X, W, y = L.make_inputs(w)
    y[7] = 900
    Xd, Wd, yd = X.cuda(), W.cuda(), y.cuda()
    parts = [lce.lce_shard_forward(Xd, Wd[a:b], yd, a, 900) for a, b in ((0, 300), (300, 900))]
    out = lce.lce_shard_merge(torch.stack([p["lse_part"] for p in parts]),
                              torch.stack([p["target_part"] for p in parts]), yd, 900)
    torch.cuda.synchronize()
    f = O.forward_ex(L.to_f64(X), L.to_f64(W), y.numpy(), O.options())
    loss = out["loss"].cpu().numpy()
    assert int(out["bad_label"]) == 1 and np.isnan(float(out["reduced"]))
    assert np.isnan(loss[7]) and np.isnan(f["loss"][7])
    ok = np.arange(200) != 7
    np.testing.assert_allclose(loss[ok], f["loss"][ok], rtol=0, atol=LSE_ATOL)
    assert int(out["n_valid"]) == f["n_valid"]


def test_merge_matches_whole_vocabulary_call(lce):
    """Without bad labels the merged loss equals the whole-vocabulary call's
    within rounding, and the reduced value is finite."""
    w = L.Workload("shards", N=640, H=128, V=5000, labels="zipf", ignore_frac=0.1, seed=91)
    X, W, y = (t.cuda() for t in L.make_inputs(w))
    full = lce.lce_forward_ex(X, W, y, softcap=20.0)
    _, out, dX, dW = run_shards(lce, X, W, y, [0, 1250, 2500, 3750, 5000], dict(softcap=20.0),
                                torch.ones(1, device="cuda"))
    dXf, dWf = lce.lce_backward_ex(X, W, y, full["lse"], 1.0, softcap=20.0)
    torch.cuda.synchronize()
    assert int(out["n_valid"]) == int(full["n_valid"])
    assert torch.allclose(out["lse"], full["lse"], atol=1e-5, rtol=0)
    assert abs(float(out["reduced"]) - float(full["reduced"])) <= 1e-5 * abs(float(full["reduced"]))
    assert rel_l2(dX.cpu(), dXf.cpu()) <= 1e-5 and rel_l2(dW.cpu(), dWf.cpu()) <= 1e-5


def test_gemma_eight_shards_fullsize(lce):
    """Gemma-2 2B head as 8 shards of V/8 = 32016 rows against the stored
    oracle values (every row's LSE and loss, sampled dX and dW rows)."""
    gold = np.load(os.path.join(HERE, "golden", "fullsize_gemma2_2b.npz"))
    w = L.WORKLOADS["gemma2_2b"]
    X, W, y = L.make_inputs(w)
    assert L.fingerprint(X, W, y) == str(gold["fingerprint"])
    g = 8
    assert w.V % g == 0
    edges = [k * (w.V // g) for k in range(g + 1)]
    print(f"[shards] gemma2_2b full size, {g} shards of {w.V // g}", flush=True)
    dev = "cuda"
    Xd, Wd, yd = X.to(dev), W.to(dev), y.to(dev)
    _, out, dX, dW = run_shards(lce, Xd, Wd, yd, edges, dict(softcap=w.softcap),
                                torch.ones(1, device=dev))
    torch.cuda.synchronize()
    assert int(out["n_valid"]) == int(gold["n_valid"]) and int(out["bad_label"]) == 0
    e_lse = np.abs(out["lse"].cpu().numpy() - gold["lse"]).max()
    e_loss = np.abs(out["loss"].cpu().numpy() - gold["loss"]).max()
    mean, gmean = float(out["reduced"]), float(gold["mean"])
    e_dx = rel_l2(dX[torch.from_numpy(gold["dx_rows"]).to(dev)].cpu(), gold["dX"])
    e_dw = rel_l2(dW[torch.from_numpy(gold["dw_rows"]).to(dev)].cpu(), gold["dW"])
    print(f"[shards] gemma: lse {e_lse:.2e} loss {e_loss:.2e} mean rel "
          f"{abs(mean - gmean) / abs(gmean):.2e} dX {e_dx:.2e} dW {e_dw:.2e}", flush=True)
    assert e_lse <= LSE_ATOL and e_loss <= LSE_ATOL
    assert abs(mean - gmean) <= RED_RTOL * abs(gmean)
    assert e_dx <= GRAD_RTOL and e_dw <= GRAD_RTOL
    S = FS.samples("gemma2_2b", X, W, y, dict(softcap=w.softcap))
    FS.check("shards gemma2_2b", dX, dW, S, GRAD_RTOL, 1e-2, log=lambda m: print(m, flush=True))
