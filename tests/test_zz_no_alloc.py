"""lce_forward_noalloc (the forward for callers that cannot allocate) against
lce_forward, through the C ABI.

Both calls run the same kernels on the same inputs, so every output must be
equal bit for bit.  Two calls in a row on one device, the second with a
smaller shape, check that the library's scratch array carries nothing from
one call to the next.  The call must not allocate: the caching allocator's
count of allocated bytes is the same before and after it.
"""
import ctypes

import pytest
import torch

import lce_inputs as L

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_cross_entropy_lse_amd import _lib
    return _lib.load()


def forward_with_workspace(lib, X, W, y, softcap):
    from linear_cross_entropy_lse_amd import _lib
    N, H = X.shape
    V = W.shape[0]
    out = {"loss": torch.empty(N, device="cuda"), "lse": torch.empty(N, device="cuda"),
           "mean": torch.empty(1, device="cuda"),
           "n_valid": torch.empty(1, dtype=torch.int32, device="cuda"),
           "bad": torch.empty(1, dtype=torch.int32, device="cuda")}
    ws_n = lib.lce_forward_workspace_bytes(N, H, V)
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    st = lib.lce_forward(X.data_ptr(), W.data_ptr(), y.data_ptr(), N, H, V, -100,
                         ctypes.c_float(softcap), out["loss"].data_ptr(), out["lse"].data_ptr(),
                         out["mean"].data_ptr(), out["n_valid"].data_ptr(), out["bad"].data_ptr(),
                         ws.data_ptr(), ws_n, torch.cuda.current_stream().cuda_stream)
    assert st == _lib.LCE_OK, _lib.status_string(st)
    return out


def forward_noalloc(lib, X, W, y, softcap):
    from linear_cross_entropy_lse_amd import _lib
    N, H = X.shape
    V = W.shape[0]
    # Output buffers are the caller's; filled with a pattern the call must overwrite.
    out = {"loss": torch.full((N,), 7.0, device="cuda"), "lse": torch.full((N,), 7.0, device="cuda"),
           "mean": torch.full((1,), 7.0, device="cuda"),
           "n_valid": torch.full((1,), -7, dtype=torch.int32, device="cuda"),
           "bad": torch.full((1,), -7, dtype=torch.int32, device="cuda")}
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    st = lib.lce_forward_noalloc(X.data_ptr(), W.data_ptr(), y.data_ptr(), N, H, V, -100,
                                 ctypes.c_float(softcap), out["loss"].data_ptr(),
                                 out["lse"].data_ptr(), out["mean"].data_ptr(),
                                 out["n_valid"].data_ptr(), out["bad"].data_ptr(),
                                 torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == _lib.LCE_OK, _lib.status_string(st)
    assert torch.cuda.memory_allocated() == before
    return out


def inputs(N, H, V, softcap, seed):
    w = L.Workload("noalloc", N, H, V, labels="uniform", ignore_frac=0.1, softcap=softcap,
                   seed=seed)
    X, W, y = L.make_inputs(w)
    return X.cuda(), W.cuda(), y.cuda()


def test_noalloc_matches_forward_twice_shrinking(lib):
    # Calls of decreasing size: more than 32 token tiles (the forward in two
    # launches of token tiles), several token tiles with a ragged vocabulary,
    # then a smaller one.
    for (N, H, V, c, seed) in [(9000, 64, 3000, 30.0, 10), (1100, 136, 5003, 30.0, 11),
                               (300, 64, 1000, 0.0, 12)]:
        print(f"[noalloc] N={N} H={H} V={V} softcap={c}", flush=True)
        X, W, y = inputs(N, H, V, c, seed)
        ref = forward_with_workspace(lib, X, W, y, c)
        got = forward_noalloc(lib, X, W, y, c)
        for k in ref:
            assert torch.equal(ref[k], got[k]), k
        assert int(got["n_valid"]) == int((y != -100).sum())


def test_noalloc_limit_and_empty(lib):
    from linear_cross_entropy_lse_amd import _lib
    cap = lib.lce_forward_noalloc_max_bytes()
    assert cap == 64 << 20
    # A shape whose forward workspace exceeds the scratch is refused before any launch.
    N = 1 << 22
    assert lib.lce_forward_workspace_bytes(N, 64, 1000) > cap
    X, W, y = inputs(8, 64, 1000, 0.0, 13)
    st = lib.lce_forward_noalloc(X.data_ptr(), W.data_ptr(), y.data_ptr(), N, 64, 1000, -100,
                                 ctypes.c_float(0.0), X.data_ptr(), X.data_ptr(), X.data_ptr(),
                                 X.data_ptr(), None, torch.cuda.current_stream().cuda_stream)
    assert st == _lib.LCE_ERR_SCRATCH_LIMIT
    # N = 0: the reduction outputs are written, nothing else is touched.
    mean = torch.full((1,), 7.0, device="cuda")
    nv = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    st = lib.lce_forward_noalloc(None, None, None, 0, 64, 1000, -100, ctypes.c_float(0.0),
                                 None, None, mean.data_ptr(), nv.data_ptr(), None,
                                 torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == _lib.LCE_OK
    assert float(mean) == 0.0 and int(nv) == 0


def test_noalloc_under_graph_capture(lib):
    """The use the variant exists for: the call captured into a HIP graph
    (nothing is allocated inside the capture) and replayed on new inputs
    copied into the captured buffers, with eager calls between the replays;
    every replay equals lce_forward on the same inputs bit for bit.  The
    first call on the device (which looks up the scratch address) runs
    before the capture."""
    from linear_cross_entropy_lse_amd import _lib
    N, H, V, c = 9000, 64, 3000, 30.0
    sets = [inputs(N, H, V, c, 20 + k) for k in range(3)]
    refs = [forward_with_workspace(lib, *s, c) for s in sets]
    torch.cuda.synchronize()
    Xb, Wb, yb = (t.clone() for t in sets[0])
    forward_noalloc(lib, Xb, Wb, yb, c)
    out = {"loss": torch.empty(N, device="cuda"), "lse": torch.empty(N, device="cuda"),
           "mean": torch.empty(1, device="cuda"),
           "n_valid": torch.empty(1, dtype=torch.int32, device="cuda"),
           "bad": torch.empty(1, dtype=torch.int32, device="cuda")}
    g = torch.cuda.CUDAGraph()
    print(f"[noalloc] capture N={N} H={H} V={V} softcap={c}", flush=True)
    with torch.cuda.graph(g):
        st = lib.lce_forward_noalloc(Xb.data_ptr(), Wb.data_ptr(), yb.data_ptr(), N, H, V, -100,
                                     ctypes.c_float(c), out["loss"].data_ptr(),
                                     out["lse"].data_ptr(), out["mean"].data_ptr(),
                                     out["n_valid"].data_ptr(), out["bad"].data_ptr(),
                                     torch.cuda.current_stream().cuda_stream)
    assert st == _lib.LCE_OK, _lib.status_string(st)
    for rep, k in enumerate([1, 2, 0, 1]):
        X, W, y = sets[k]
        Xb.copy_(X)
        Wb.copy_(W)
        yb.copy_(y)
        g.replay()
        torch.cuda.synchronize()
        print(f"[noalloc] replay {rep} on input set {k}", flush=True)
        for key in out:
            assert torch.equal(out[key], refs[k][key]), key
        forward_noalloc(lib, *sets[(k + 2) % 3], c)   # eager use of the same scratch between replays
