"""Stream semantics of the C ABI: every launch goes on the stream the caller
passes, and calls share no state.

include/lce.h states that calls are asynchronous on their stream, stateless and
re-entrant, and that concurrent calls need workspaces of their own.  Checked
here through the binding (which passes torch's current stream):
  * two different problems enqueued on two side streams at once give bitwise
    the results of the same calls run one after the other on the default
    stream (results are deterministic for a fixed shape and device);
  * a call enqueued on a side stream right behind a slow producer of its input
    on that stream reads the produced input, not what the buffer held before.
Side streams are created at the default priority.
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


def problem(N, H, V, seed, softcap):
    w = L.Workload("streams", N=N, H=H, V=V, labels="uniform", ignore_frac=0.1,
                   softcap=softcap, seed=seed)
    X, W, y = L.make_inputs(w)
    W = (W.float() * 4.0).to(torch.bfloat16)
    return X.cuda(), W.cuda(), y.cuda(), softcap


def step(lce, X, W, y, softcap):
    out = lce.lce_forward(X, W, y, -100, softcap)
    dX, dW = lce.lce_backward(X, W, y, out["lse"], 0.7, -100, softcap)
    return [out["loss"], out["lse"], out["mean"], out["n_valid"], dX, dW]


def test_concurrent_streams_match_sequential(lce):
    probs = [problem(1100, 136, 3000, 11, 30.0), problem(700, 64, 9000, 12, 0.0)]
    print("[streams] sequential on the default stream", flush=True)
    ref = [step(lce, *p) for p in probs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    got = [None, None]
    for rep in range(3):
        print(f"[streams] concurrent, repetition {rep}", flush=True)
        for i, (p, s) in enumerate(zip(probs, streams)):
            with torch.cuda.stream(s):
                got[i] = step(lce, *p)
        torch.cuda.synchronize()
        for r, g in zip(ref, got):
            for a, b in zip(r, g):
                assert torch.equal(a, b)


def test_call_follows_producer_on_its_stream(lce):
    X, W, y, softcap = problem(2048, 256, 5000, 13, 30.0)
    ref = step(lce, X, W, y, softcap)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    a = torch.randn(4096, 4096, device="cuda")
    Xs = torch.zeros_like(X)
    with torch.cuda.stream(s):
        print("[streams] slow producer, then the call, on one side stream", flush=True)
        big = a
        for _ in range(8):
            big = big @ a * (1.0 / 64.0)
        # The input equals X exactly (a finite value times 0 added to bf16 X),
        # written only after the products above have run on this stream.
        Xs.copy_((X.float() + 0.0 * big[: X.shape[0], : X.shape[1]].clamp(-1, 1)).to(torch.bfloat16))
        got = step(lce, Xs, W, y, softcap)
    torch.cuda.synchronize()
    assert torch.equal(Xs, X)
    for a_, b_ in zip(ref, got):
        assert torch.equal(a_, b_)
