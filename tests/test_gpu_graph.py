"""The training step, the row-chunked fused call, and the vocabulary shards
with the vocabulary order and the sorted backward, captured in a HIP graph.

Every entry point of the step only enqueues kernels on the caller's stream (no
allocation, copy, memset or synchronisation inside the library), so a
forward + backward can be captured once and replayed.  The binding allocates
its outputs and workspace from torch, which serves them from the graph's own
pool during capture.  The upstream gradient is passed as a device tensor made
before the capture (a host scalar would be a host-to-device copy inside it).

The graph is replayed several times, with eager work and synchronisations
between the replays and new inputs copied into the captured input buffers,
and every replay must equal, bitwise, the eager step on the same inputs.
"""
import pytest
import torch

import lce_inputs as L

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lce():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_cross_entropy_lse_amd as P
    P.load()
    return P


def inputs(N, H, V, seed, softcap):
    w = L.Workload("graph", N=N, H=H, V=V, labels="uniform", ignore_frac=0.1,
                   softcap=softcap, seed=seed)
    X, W, y = L.make_inputs(w)
    W = (W.float() * 4.0).to(torch.bfloat16)
    return X.cuda(), W.cuda(), y.cuda()


def step(lce, X, W, y, dloss, softcap, precise=False):
    out = lce.lce_forward(X, W, y, -100, softcap)
    dX, dW = lce.lce_backward_ex(X, W, y, out["lse"], dloss, -100, softcap, precise=precise)
    return [out["loss"], out["lse"], out["mean"], out["n_valid"], dX, dW]


@pytest.mark.parametrize("N,H,V,softcap,precise", [
    (600, 136, 40000, 30.0, False),    # several chunks, K tail, ragged rows and vocabulary
    (256, 64, 1000, 0.0, False),       # the tiny workload's shape
    (300, 64, 2000, 30.0, True),       # the precise gradient (two contractions per chunk)
    (8300, 64, 3000, 30.0, False),     # 33 token tiles: the forward's and the gradient's tail launches
])
def test_graph_replays_match_eager(lce, N, H, V, softcap, precise):
    seeds = [21, 22, 23]
    sets = [inputs(N, H, V, s, softcap) for s in seeds]
    dloss = torch.tensor(0.7, dtype=torch.float32, device="cuda")
    print(f"[graph] N={N} H={H} V={V} softcap={softcap} precise={precise}: eager", flush=True)
    eager = [step(lce, X, W, y, dloss, softcap, precise) for X, W, y in sets]
    torch.cuda.synchronize()
    Xb, Wb, yb = (t.clone() for t in sets[0])
    g = torch.cuda.CUDAGraph()
    print("[graph] capture", flush=True)
    with torch.cuda.graph(g):
        outs = step(lce, Xb, Wb, yb, dloss, softcap, precise)
    for rep, k in enumerate([0, 1, 2, 1, 0]):
        X, W, y = sets[k]
        Xb.copy_(X)
        Wb.copy_(W)
        yb.copy_(y)
        g.replay()
        torch.cuda.synchronize()
        print(f"[graph] replay {rep} on input set {k}", flush=True)
        for a, b in zip(eager[k], outs):
            assert torch.equal(a, b)
        # eager work between replays
        step(lce, *sets[(k + 1) % 3], dloss, softcap, precise)
        torch.cuda.synchronize()


def fused_step(lce, X, W, y, dloss, softcap):
    out, dX, dW = lce.lce_forward_backward(X, W, y, dloss, softcap=softcap)
    return [out["loss"], out["lse"], out["reduced"], out["n_valid"], dX, dW]


@pytest.mark.parametrize("N,H,V,softcap", [
    (600, 136, 40000, 30.0),     # two row chunks, fixed reference
    (2600, 1024, 4000, 0.0),     # uneven chunks (1536 + 1064 rows, 6 and 7 dX parts), running reference
])
def test_fused_graph_replays_match_eager(lce, N, H, V, softcap):
    """The row-chunked fused call captured once and replayed, as above."""
    seeds = [31, 32, 33]
    sets = [inputs(N, H, V, s, softcap) for s in seeds]
    dloss = torch.tensor(0.7, dtype=torch.float32, device="cuda")
    print(f"[graph] fused N={N} H={H} V={V} softcap={softcap}: eager", flush=True)
    eager = [fused_step(lce, X, W, y, dloss, softcap) for X, W, y in sets]
    torch.cuda.synchronize()
    Xb, Wb, yb = (t.clone() for t in sets[0])
    g = torch.cuda.CUDAGraph()
    print("[graph] fused capture", flush=True)
    with torch.cuda.graph(g):
        outs = fused_step(lce, Xb, Wb, yb, dloss, softcap)
    for rep, k in enumerate([0, 1, 2, 1, 0]):
        X, W, y = sets[k]
        Xb.copy_(X)
        Wb.copy_(W)
        yb.copy_(y)
        g.replay()
        torch.cuda.synchronize()
        print(f"[graph] fused replay {rep} on input set {k}", flush=True)
        for a, b in zip(eager[k], outs):
            assert torch.equal(a, b)
        fused_step(lce, *sets[(k + 1) % 3], dloss, softcap)
        torch.cuda.synchronize()


def shard_and_sorted_step(lce, X, W, y, dloss, softcap):
    from tests.test_gpu_shards import run_shards
    V = W.shape[0]
    _, out, dX, dW = run_shards(lce, X, W, y, [0, V // 3, V], dict(softcap=softcap), dloss)
    mean_logit, order = lce.lce_vocab_order(X, W, y)
    lse = lce.lce_forward(X, W, y, -100, softcap)["lse"]
    sX, sW = lce.lce_backward_sorted(X, W, y, lse, dloss, order, softcap=softcap)
    return [out["loss"], out["lse"], out["reduced"], dX, dW, mean_logit, order, sX, sW]


def test_shard_and_sorted_graph_replays_match_eager(lce):
    """Two vocabulary shards (forwards, merge, backwards), the vocabulary
    order and the backward on it, captured once and replayed, as above."""
    N, H, V, softcap = 700, 72, 6000, 30.0
    sets = [inputs(N, H, V, s, softcap) for s in (41, 42, 43)]
    dloss = torch.tensor(0.7, dtype=torch.float32, device="cuda")
    print(f"[graph] shards + sorted N={N} H={H} V={V}: eager", flush=True)
    eager = [shard_and_sorted_step(lce, X, W, y, dloss, softcap) for X, W, y in sets]
    torch.cuda.synchronize()
    Xb, Wb, yb = (t.clone() for t in sets[0])
    g = torch.cuda.CUDAGraph()
    print("[graph] shards + sorted capture", flush=True)
    with torch.cuda.graph(g):
        outs = shard_and_sorted_step(lce, Xb, Wb, yb, dloss, softcap)
    for rep, k in enumerate([0, 1, 2, 1]):
        X, W, y = sets[k]
        Xb.copy_(X)
        Wb.copy_(W)
        yb.copy_(y)
        g.replay()
        torch.cuda.synchronize()
        print(f"[graph] shards + sorted replay {rep} on input set {k}", flush=True)
        for a, b in zip(eager[k], outs):
            assert torch.equal(a, b)
        shard_and_sorted_step(lce, *sets[(k + 1) % 3], dloss, softcap)
        torch.cuda.synchronize()
