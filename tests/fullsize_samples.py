"""Oracle values of sampled outputs at the full workload sizes, computed when
a test asks for them and kept for the rest of the test session.

The float64 oracle cannot form a whole N x V gradient at these sizes, but it
can compute chosen rows: a dX row needs its own logit row only, and a dW row
needs one logit column over every token row plus each row's LSE, which
tests/golden/fullsize_<workload>.npz holds (written by make_fullsize.py, oracle
only).  Each sample is returned as its two terms, the softmax ("dense") part
and the target ("one-hot") part, so a test can weigh the part that passes
through the bf16 gradient chunk on its own (logit_gradient_parts).

Samples:
  dX rows  1024 seeded rows, plus both sides of every row-chunk boundary of
           the row-chunked fused call (chunks of Nc rows) and the first and
           last rows;
  dW rows  both sides of every vocabulary-chunk boundary of the backward,
           seeded label-free rows inside every chunk, both sides of seeded
           256-row tile boundaries, the most frequent labels, seeded rows past
           the 2^31-byte offset of an fp32 dW (where there are any) and the
           last row.
"""
from __future__ import annotations

import os

import numpy as np

import lce_inputs as L
from oracle import lce_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))
N_DX_ROWS = 1024
FREE_PER_CHUNK = 24
TILE_EDGES = 16
ROW_BLOCK = 128


def backward_chunk_columns(N: int, H: int, V: int) -> int:
    """Vocabulary columns per chunk of the backward's bf16 gradient chunk:
    the fewest chunks with N·Vc <= V·H before the width is rounded up to a
    multiple of 256 (ceil(N/H) chunks; widths of at least max(4096,
    32768 / ceil(H/256)) columns in whole tiles, that floor at most 16384, and
    at most 2^21 columns), evened out over the chunks."""
    Nc = max(N, 1)
    nt_h = -(-H // 256)
    floor_cols = max(4096, min(16384, -(-(-(-32768 // nt_h)) // 256) * 256))
    if V * H < floor_cols * Nc:
        n = -(-V // floor_cols)
    elif V * H > (1 << 21) * Nc:
        n = -(-V // (1 << 21))
    else:
        n = -(-Nc // H)
    per = -(-V // max(n, 1))
    return -(-per // 256) * 256


def fused_chunk_rows(N: int, H: int, V: int) -> int:
    """Rows per chunk of the row-chunked fused call (every chunk but the last).

    Whole 256-row tiles, at most 2H rows and, from two tiles on, at most half
    of the tiles rounded up.  Among the fewest chunks that meet this and up to
    three more, each count with chunks as even as whole tiles allow, the one
    with the least estimated time: per chunk ceil(n_vt / S) for its logits
    pass (S = min(256 // tiles, n_vt), at least 1), plus V / 16384 for each
    chunk after the first (a further pass over the fp32 dW)."""
    T = -(-max(N, 1) // 256)
    nvt = -(-V // 256)
    half = -(-T // 2) if T >= 2 else 1
    lim = max(1, min(2 * H // 256, half))
    n_min = -(-T // lim)

    def waves(t):
        return -(-nvt // max(1, min(256 // t, nvt)))

    best, best_cost = -(-T // n_min), None
    for n in range(n_min, min(n_min + 3, T) + 1):
        t = -(-T // n)
        last = T - (n - 1) * t
        if last <= 0:
            continue
        cost = float(n - 1) * waves(t) + float(waves(last)) + float(n - 1) * (V / 16384.0)
        if best_cost is None or cost < best_cost:
            best, best_cost = t, cost
    return best * 256


def sample_rows(w: L.Workload, y: np.ndarray):
    """(dx_rows, dw_rows, dw_free): the sampled token rows, the sampled
    vocabulary rows, and the mask of those vocabulary rows no label hits."""
    N, H, V = w.N, w.H, w.V
    rng = np.random.default_rng(w.seed + 303)
    nc = fused_chunk_rows(N, H, V)
    edges = [r for k in range(1, -(-N // nc)) for r in (k * nc - 1, k * nc)]
    dx = np.unique(np.concatenate([L.row_sample(N, N_DX_ROWS, seed=w.seed + 301),
                                   np.array(edges, dtype=np.int64), [0, N - 1]]))
    valid = y[y != L.IGNORE_INDEX]
    counts = np.bincount(valid, minlength=V)
    vc = backward_chunk_columns(N, H, V)
    pick = []
    for b in range(0, V, vc):
        e = min(b + vc, V)
        pick += [b, e - 1]
        free = np.nonzero(counts[b:e] == 0)[0] + b
        if len(free):
            pick += rng.choice(free, size=min(FREE_PER_CHUNK, len(free)), replace=False).tolist()
    nt = -(-V // 256)
    for k in rng.choice(np.arange(1, nt), size=min(TILE_EDGES, nt - 1), replace=False):
        pick += [256 * int(k) - 1, min(256 * int(k), V - 1)]
    pick += np.argsort(-counts, kind="stable")[:4].tolist()
    past = -(-(1 << 31) // (4 * H))          # first row whose fp32 dW starts past 2^31 bytes
    if past < V:
        pick += rng.choice(np.arange(past, V), size=min(8, V - past), replace=False).tolist()
    pick.append(V - 1)
    dw = np.unique(np.array(pick, dtype=np.int64))
    return dx, dw, counts[dw] == 0


def _compute(name, opts_items, X, W, y, dloss):
    w = L.WORKLOADS[name]
    gold = np.load(os.path.join(HERE, "golden", f"fullsize_{name}.npz"))
    opts = O.options(**dict(opts_items))
    X64, W64, y64 = L.to_f64(X), L.to_f64(W), y.numpy()
    n_valid = int(gold["n_valid"])
    lse = gold["lse"]              # every row's LSE (the options used keep it: logit scale 1)
    scale = O.row_scale(y64, dloss, n_valid, opts)
    dx_rows, dw_rows, free = sample_rows(w, y64)
    dxd = np.empty((len(dx_rows), w.H))
    dxo = np.empty((len(dx_rows), w.H))
    for a in range(0, len(dx_rows), ROW_BLOCK):
        r = dx_rows[a:a + ROW_BLOCK]
        dxd[a:a + len(r)], dxo[a:a + len(r)] = O.dX_rows_parts(X64[r], W64, y64[r], lse[r],
                                                                scale[r], opts)
    dwd, dwo = O.dW_vocab_rows_parts(X64, W64, y64, lse, scale, dw_rows, opts)
    return {"dx_rows": dx_rows, "dx_dense": dxd, "dx_onehot": dxo,
            "dw_rows": dw_rows, "dw_dense": dwd, "dw_onehot": dwo, "dw_free": free}


_CACHE = {}


def samples(name: str, X, W, y, opts: dict | None = None, dloss=1.0):
    """Oracle dense and one-hot parts of the sampled dX and dW rows of the
    workload `name` (inputs X, W, y as generated for it), for the loss options
    `opts` (keyword arguments of O.options) and upstream gradient `dloss` (a
    scalar, or one value per row for reduction "none").  Cached per session."""
    opts_items = tuple(sorted((opts or {}).items()))
    d = np.asarray(dloss, dtype=np.float64)
    key = (name, opts_items, d.tobytes() if d.ndim else float(d))
    if key not in _CACHE:
        _CACHE[key] = _compute(name, opts_items, X, W, y, d if d.ndim else float(d))
    return _CACHE[key]


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def check(tag, dX_dev, dW_dev, S, total_tol, dense_tol, log=print):
    """Compare sampled device gradients with the oracle samples S.

    total: rel-L2 of the rows against dense + one-hot (the stated bar for the
    output dtype); dense: rel-L2 after taking the oracle's one-hot term off
    the GPU rows, against the oracle's dense term (the part the bf16 gradient
    chunk carries; bar 1e-2); free: the label-free dW rows, whose whole value
    is the dense term.  Returns the errors."""
    import torch
    dev = dX_dev.device
    gx = dX_dev[torch.from_numpy(S["dx_rows"]).to(dev)].double().cpu().numpy()
    gw = dW_dev[torch.from_numpy(S["dw_rows"]).to(dev)].double().cpu().numpy()
    tx = S["dx_dense"] + S["dx_onehot"]
    tw = S["dw_dense"] + S["dw_onehot"]
    free = S["dw_free"]
    e = {"dx": rel_l2(gx, tx), "dw": rel_l2(gw, tw),
         "dx_dense": rel_l2(gx - S["dx_onehot"], S["dx_dense"]),
         "dw_dense": rel_l2(gw - S["dw_onehot"], S["dw_dense"]),
         "dw_free": rel_l2(gw[free], S["dw_dense"][free]) if free.any() else 0.0,
         "dx_dense_share": float(np.linalg.norm(S["dx_dense"]) / max(np.linalg.norm(tx), 1e-300)),
         "dw_dense_share": float(np.linalg.norm(S["dw_dense"]) / max(np.linalg.norm(tw), 1e-300)),
         "n_dx": len(S["dx_rows"]), "n_dw": len(S["dw_rows"]), "n_free": int(free.sum())}
    log(f"[{tag}] sampled {e['n_dx']} dX rows, {e['n_dw']} dW rows ({e['n_free']} label-free): "
        f"dX {e['dx']:.2e} dW {e['dw']:.2e} | dense part: dX {e['dx_dense']:.2e} "
        f"(share {e['dx_dense_share']:.3f}) dW {e['dw_dense']:.2e} "
        f"(share {e['dw_dense_share']:.2e}) label-free dW {e['dw_free']:.2e}")
    assert np.isfinite(gx).all() and np.isfinite(gw).all()
    assert e["dx"] <= total_tol and e["dw"] <= total_tol, e
    assert e["dx_dense"] <= dense_tol and e["dw_dense"] <= dense_tol and \
        e["dw_free"] <= dense_tol, e
    return e
