"""The seeded workload generator: reproducible, with the stated shapes and laws."""
import numpy as np
import torch

import lce_inputs as L


def test_tiny_is_reproducible_and_shaped():
    w = L.WORKLOADS["tiny"]
    a = L.make_inputs(w)
    b = L.make_inputs(w)
    assert L.fingerprint(*a) == L.fingerprint(*b)
    X, W, y = a
    assert X.shape == (256, 64) and X.dtype == torch.bfloat16
    assert W.shape == (1000, 64) and W.dtype == torch.bfloat16
    assert y.shape == (256,) and y.dtype == torch.int64
    assert int((y == L.IGNORE_INDEX).sum()) == 25           # floor(0.1 * 256)
    v = y[y != L.IGNORE_INDEX]
    assert int(v.min()) >= 0 and int(v.max()) < 1000
    # bf16 rounding is round-to-nearest-even of an fp32 N(0, 0.02^2) draw
    assert 0.015 < float(W.float().std()) < 0.025
    assert 0.9 < float(X.float().std()) < 1.1


def test_to_f64_is_exact():
    X = L.make_x(L.WORKLOADS["tiny"])
    x64 = L.to_f64(X)
    assert x64.dtype == np.float64
    back = torch.from_numpy(x64).to(torch.bfloat16)
    assert torch.equal(back.view(torch.int16), X.view(torch.int16))


def test_label_laws_of_large_configs():
    for name in ("liger", "llama3_8b", "gemma2_2b", "qwen25_long"):
        w = L.WORKLOADS[name]
        y = L.make_labels(w)
        assert y.shape == (w.N,)
        ign = y == L.IGNORE_INDEX
        if w.ignore_frac:
            assert int(ign.sum()) == int(np.floor(w.ignore_frac * w.N))
        if w.ignore_period:
            pos = torch.arange(w.N)
            assert torch.equal(ign, (pos % w.ignore_period) == w.ignore_period - 1)
        v = y[~ign]
        assert int(v.min()) >= 0 and int(v.max()) < w.V
        if w.labels == "zipf":
            # rank 1 (token 0) has probability 1 / sum_k k^-1.1 over V ranks
            k = np.arange(1, w.V + 1, dtype=np.float64)
            p0 = 1.0 / np.sum(k ** -1.1)
            frac = float((v == 0).float().mean())
            assert abs(frac - p0) < 5 * np.sqrt(p0 * (1 - p0) / v.numel())


def test_row_sample():
    r = L.row_sample(1000, 17, seed=3)
    assert r[0] == 0 and r[-1] == 999 and len(set(r.tolist())) == len(r) == 17
