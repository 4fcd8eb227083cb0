"""CPU oracle for the fused LM-head linear + cross-entropy (linear-LSE).

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously correct reference
the HIP path is checked against.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the product path never does.  It
shares no code with the HIP path: it reads nothing from the package
`linear_cross_entropy_lse_amd` and the package reads nothing from here.

Everything is float64 numpy.  Inputs are the bf16 bits of X and W widened
exactly to float64, so the oracle sees the same numbers the GPU sees.

Sources (web pages, cited by title and section):
  [CCE-blog]  "最贵的一层：深入浅出 Liger Kernel 与 Cut Cross-Entropy"
              (blog.jiaqiguo.xyz), §二 (gradient softmax − onehot), §三 (loss as
              LSE minus the indexed target logit; running max / sum-exp merge;
              backward by recomputation).
  [M011]      AI-infra knowledge base, page M011 (fused Linear + loss), §01 (W[V,D],
              Z = H·Wᵀ), §03 (stable per-row form and the worked example),
              §04 (sum per block, divide once by the valid-target count), §05
              (tile merge, first tile initialises), §06 (backward: p − onehot,
              scaled by normalisation and upstream gradient, dH += dZ·W,
              dW += dZᵀ·H), §07 (ignore_index, softcap needs its own definition,
              all-ignored convention must be stated).
  [Unsloth]   "03 · 融合交叉熵：让 logits 从不存在" (Unsloth fused cross-entropy
              chapter), §4 (optional in-kernel softcap scaling; label −100 gives
              loss 0; backward multiplies the softcap derivative 1 − tanh²;
              final division by n_items = count of labels ≠ −100).

Readings where the pages leave a step open (each restated where it is used;
R7 - R12 concern the GPU path's interface and are listed with its design):
  R1 softcap: z = c·tanh(z_raw / c) is applied to every logit, the target
     included, before the LSE; its derivative is 1 − tanh²(z_raw / c); c <= 0
     means no softcap.
  R2 no intermediate rounding of logits: they are exact float64 products of
     the bf16 inputs.
  R3 the LSE of an ignored row is still reported (it depends on X and W only);
     its loss is 0 and it is excluded from the valid count.
  R4 the mean divides by the number of valid targets; when that count is 0
     the mean is 0 and both gradients are 0.
  R5 `dloss` is the scalar upstream gradient of the mean loss.
  R6 a label outside [0, V) that is not ignore_index gives a NaN loss for its
     row (and therefore a NaN mean); its gradient row is NaN.

Loss variants (forward_ex / backward_ex).  [M011] §07 lists label smoothing,
Z-loss and the reduction mode as terms that need their own definition, and
[Unsloth] §4 an optional logit scaling (Cohere's logit_scale) next to the
softcap; the pages give no formulas, so the plainest standard readings are
taken:
  R13 logit_scale a: z = a·(x·w), applied before the softcap.
  R14 label smoothing e: the target distribution is (1 − e)·onehot(y) + e/V,
     so loss_i = LSE_i − (1 − e)·z_{i,y} − (e/V)·Σ_v z_{i,v} (the definition
     of PyTorch's CrossEntropyLoss, which [M011] §07 cites for its semantics).
  R15 Z-loss l: each valid row adds l·LSE_i².
  R16 reduction: "mean" divides the sum of the row losses by n_valid (R4),
     "sum" does not divide, "none" keeps the row losses; the backward of
     "none" takes one upstream gradient per row.
  Gradient of a valid row: dL_i/dz_v = (1 + 2l·LSE_i)·p_v − (1 − e)·[v = y_i]
  − e/V, times the softcap derivative, times a, times the row's upstream
  scale (dloss / n_valid, dloss, or dloss_i).
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np

IGNORE_INDEX = -100


# --------------------------------------------------------------------------- #
# Building blocks
# --------------------------------------------------------------------------- #
def logits(X: np.ndarray, W: np.ndarray) -> np.ndarray:
    """Z = X · Wᵀ with W stored [V, H] ([M011] §01)."""
    return X @ W.T


def apply_softcap(Z: np.ndarray, softcap: float) -> np.ndarray:
    """Reading R1: c·tanh(Z/c) when c > 0, else Z unchanged ([Unsloth] §4)."""
    if softcap > 0:
        return softcap * np.tanh(Z / softcap)
    return Z


def softcap_derivative(Z: np.ndarray, softcap: float) -> np.ndarray:
    """d(c·tanh(z/c))/dz = 1 − tanh²(z/c) ([Unsloth] §4 backward); 1 if off."""
    if softcap > 0:
        t = np.tanh(Z / softcap)
        return 1.0 - t * t
    return np.ones_like(Z)


def row_logsumexp(Zc: np.ndarray) -> np.ndarray:
    """Per-row log Σ_v exp(z_v) in the stable form m + log Σ exp(z − m),
    m = max_v z ([M011] §03)."""
    m = Zc.max(axis=1)
    return m + np.log(np.exp(Zc - m[:, None]).sum(axis=1))


def logsumexp_by_vocab_tiles(z: Sequence[float], bounds: Sequence[int]) -> float:
    """LSE of one logit row visited tile by tile with the running merge.

    `bounds` are the tile edges over the vocabulary (0 = b0 < b1 < ... = V).
    Each tile yields its own max m_b and its own Σ exp(z − m_b); they are folded
    into (m, s) with m' = max(m, m_b), s' = s·e^(m − m') + s_b·e^(m_b − m'),
    and the result is m + log s ([CCE-blog] §三; [M011] §05).  The first tile
    initialises (m, s) directly so no −inf − (−inf) is ever formed.
    Plain Python floats: used by the pins on tiny rows.
    """
    m = None
    s = 0.0
    for a, b in zip(bounds[:-1], bounds[1:]):
        tile = [float(v) for v in z[a:b]]
        m_b = max(tile)
        s_b = math.fsum(math.exp(v - m_b) for v in tile)
        if m is None:
            m, s = m_b, s_b
            continue
        m_new = max(m, m_b)
        s = s * math.exp(m - m_new) + s_b * math.exp(m_b - m_new)
        m = m_new
    return m + math.log(s)


def valid_mask(labels: np.ndarray, ignore_index: int = IGNORE_INDEX) -> np.ndarray:
    """Rows that carry a target: label ≠ ignore_index ([M011] §07; [Unsloth] §4)."""
    return labels != ignore_index


def bad_mask(labels: np.ndarray, V: int, ignore_index: int = IGNORE_INDEX) -> np.ndarray:
    """Reading R6: labels neither ignored nor in [0, V)."""
    return (labels != ignore_index) & ((labels < 0) | (labels >= V))


# --------------------------------------------------------------------------- #
# Forward
# --------------------------------------------------------------------------- #
def forward(X: np.ndarray, W: np.ndarray, labels: np.ndarray,
            ignore_index: int = IGNORE_INDEX, softcap: float = 0.0,
            n_valid_total: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Per-row LSE and loss, valid count and mean over valid targets.

    loss_i = LSE(z_i) − z_{i, y_i} ([CCE-blog] §三; [M011] §03), 0 for ignored
    rows ([Unsloth] §4).  mean = Σ_i loss_i / n_valid ([M011] §04; [Unsloth] §4).
    `n_valid_total` lets a caller evaluate a subset of rows while dividing by
    the count of the whole batch (the definition is row-separable).
    """
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64)
    V = W.shape[0]
    Z = logits(X, W)
    Zc = apply_softcap(Z, softcap)
    lse = row_logsumexp(Zc)
    valid = valid_mask(labels, ignore_index)
    bad = bad_mask(labels, V, ignore_index)
    ok = valid & ~bad
    target = np.zeros(X.shape[0])
    rows = np.nonzero(ok)[0]
    target[rows] = Zc[rows, labels[rows]]
    loss = np.where(valid, lse - target, 0.0)
    loss[bad] = np.nan
    n_valid = int(valid.sum()) if n_valid_total is None else int(n_valid_total)
    total = loss.sum()
    mean = total / n_valid if n_valid > 0 else 0.0      # reading R4
    return {"lse": lse, "loss": loss, "n_valid": n_valid, "mean": mean,
            "loss_sum": total, "target_logit": target}


# --------------------------------------------------------------------------- #
# Backward
# --------------------------------------------------------------------------- #
def logit_gradient(X: np.ndarray, W: np.ndarray, labels: np.ndarray,
                   lse: np.ndarray, n_valid: int, dloss: float = 1.0,
                   ignore_index: int = IGNORE_INDEX, softcap: float = 0.0,
                   vocab_rows: Optional[np.ndarray] = None) -> np.ndarray:
    """dL/dz_raw for the rows of X (all vocabulary columns, or `vocab_rows`).

    The logits are recomputed, p = exp(z − LSE) ([CCE-blog] §三; [M011] §06),
    dZ = p − onehot(y) ([CCE-blog] §二; [M011] §06), multiplied by the softcap
    derivative ([Unsloth] §4) and by dloss / n_valid ([M011] §06, §04).
    Ignored rows have zero gradient.
    """
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64)
    V = W.shape[0]
    cols = np.arange(V) if vocab_rows is None else np.asarray(vocab_rows)
    Z = logits(X, W[cols])
    Zc = apply_softcap(Z, softcap)
    P = np.exp(Zc - lse[:, None])
    onehot = (labels[:, None] == cols[None, :]).astype(np.float64)
    dZ = (P - onehot) * softcap_derivative(Z, softcap)
    valid = valid_mask(labels, ignore_index)
    scale = (dloss / n_valid) if n_valid > 0 else 0.0      # reading R4
    dZ = dZ * (scale * valid)[:, None]
    bad = bad_mask(labels, V, ignore_index)
    dZ[bad] = np.nan
    return dZ


def backward(X: np.ndarray, W: np.ndarray, labels: np.ndarray,
             dloss: float = 1.0, ignore_index: int = IGNORE_INDEX,
             softcap: float = 0.0, lse: Optional[np.ndarray] = None):
    """(dX, dW) of the mean loss: dX = dZ · W and dW = dZᵀ · X ([M011] §06;
    the same two contractions appear in [CCE-blog] §二 for the row-chunked
    variant).  `lse` defaults to the oracle's own forward."""
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64)
    fwd = forward(X, W, labels, ignore_index, softcap)
    if lse is None:
        lse = fwd["lse"]
    dZ = logit_gradient(X, W, labels, lse, fwd["n_valid"], dloss,
                        ignore_index, softcap)
    return dZ @ W, dZ.T @ X


def dX_rows(X_rows: np.ndarray, W: np.ndarray, labels_rows: np.ndarray,
            lse_rows: np.ndarray, n_valid: int, dloss: float = 1.0,
            ignore_index: int = IGNORE_INDEX, softcap: float = 0.0) -> np.ndarray:
    """dX for a subset of rows: each row of dX depends on its own row only."""
    dZ = logit_gradient(X_rows, W, labels_rows, lse_rows, n_valid, dloss,
                        ignore_index, softcap)
    return dZ @ np.asarray(W, dtype=np.float64)


def dW_vocab_rows(X: np.ndarray, W: np.ndarray, labels: np.ndarray,
                  lse: np.ndarray, n_valid: int, vocab_rows: np.ndarray,
                  dloss: float = 1.0, ignore_index: int = IGNORE_INDEX,
                  softcap: float = 0.0) -> np.ndarray:
    """dW[v] for selected vocabulary rows v: dW[v] = Σ_i dZ[i, v] · x_i over
    every token row i (needs the LSE of every row)."""
    dZ = logit_gradient(X, W, labels, lse, n_valid, dloss, ignore_index,
                        softcap, vocab_rows=vocab_rows)
    return dZ.T @ np.asarray(X, dtype=np.float64)


def mean_loss_value(X, W, labels, ignore_index=IGNORE_INDEX, softcap=0.0):
    """Scalar mean loss (used by the finite-difference pins)."""
    return float(forward(X, W, labels, ignore_index, softcap)["mean"])


def backward_rows(X_rows: np.ndarray, W: np.ndarray, labels_rows: np.ndarray,
                  lse_rows: np.ndarray, n_valid: int, dloss: float = 1.0,
                  ignore_index: int = IGNORE_INDEX, softcap: float = 0.0):
    """Contribution of a subset of token rows to the backward: their dX rows
    and their share Σ_{i in subset} dZ[i, :]ᵀ x_i of dW ([M011] §06: dH += dZ·W,
    dW accumulates dZᵀ·H over the token rows).  Summing the dW shares of a
    partition of the rows gives the full dW."""
    X_rows = np.asarray(X_rows, dtype=np.float64)
    dZ = logit_gradient(X_rows, W, labels_rows, lse_rows, n_valid, dloss,
                        ignore_index, softcap)
    return dZ @ np.asarray(W, dtype=np.float64), dZ.T @ X_rows


# --------------------------------------------------------------------------- #
# Loss variants (readings R13 - R16)
# --------------------------------------------------------------------------- #
DEFAULT_OPTIONS = {"softcap": 0.0, "logit_scale": 1.0, "label_smoothing": 0.0,
                   "z_loss": 0.0, "reduction": "mean", "ignore_index": IGNORE_INDEX}


def options(**kw) -> Dict[str, object]:
    o = dict(DEFAULT_OPTIONS)
    o.update(kw)
    return o


def forward_ex(X: np.ndarray, W: np.ndarray, labels: np.ndarray, opts: Dict[str, object],
               n_valid_total: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Per-row LSE and loss with logit scale (R13), label smoothing (R14) and
    Z-loss (R15); `reduced` is the mean, the sum, or (for "none") the sum of
    the row losses (R16)."""
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64)
    V = W.shape[0]
    a, e, lam = float(opts["logit_scale"]), float(opts["label_smoothing"]), float(opts["z_loss"])
    ignore_index = int(opts["ignore_index"])
    Z = a * logits(X, W)
    Zc = apply_softcap(Z, float(opts["softcap"]))
    lse = row_logsumexp(Zc)
    valid = valid_mask(labels, ignore_index)
    bad = bad_mask(labels, V, ignore_index)
    ok = valid & ~bad
    target = np.zeros(X.shape[0])
    rows = np.nonzero(ok)[0]
    target[rows] = Zc[rows, labels[rows]]
    zsum = Zc.sum(axis=1)
    row_loss = lse - (1.0 - e) * target - (e / V) * zsum + lam * lse * lse
    loss = np.where(valid, row_loss, 0.0)
    loss[bad] = np.nan
    n_valid = int(valid.sum()) if n_valid_total is None else int(n_valid_total)
    total = loss.sum()
    if opts["reduction"] == "mean":
        reduced = total / n_valid if n_valid > 0 else 0.0
    else:
        reduced = total
    return {"lse": lse, "loss": loss, "n_valid": n_valid, "reduced": reduced,
            "loss_sum": total, "target_logit": target, "logit_sum": zsum}


def row_scale(labels: np.ndarray, dloss, n_valid: int, opts: Dict[str, object]) -> np.ndarray:
    """Upstream scale of each row's gradient (R16): dloss / n_valid ("mean",
    0 when n_valid = 0), dloss ("sum"), or the row's own dloss_i ("none");
    zero for ignored rows."""
    labels = np.asarray(labels, dtype=np.int64)
    valid = valid_mask(labels, int(opts["ignore_index"]))
    if opts["reduction"] == "none":
        s = np.asarray(dloss, dtype=np.float64).reshape(-1)
    elif opts["reduction"] == "sum":
        s = np.full(labels.shape[0], float(dloss))
    else:
        s = np.full(labels.shape[0], float(dloss) / n_valid if n_valid > 0 else 0.0)
    return s * valid


def logit_gradient_ex(X: np.ndarray, W: np.ndarray, labels: np.ndarray, lse: np.ndarray,
                      scale: np.ndarray, opts: Dict[str, object],
                      vocab_rows: Optional[np.ndarray] = None) -> np.ndarray:
    """dL/d(x·w) for the rows of X: ((1 + 2l·LSE)·p − (1 − e)·onehot − e/V)
    · softcap derivative · a · scale_i (gradient of R13 - R15)."""
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64)
    V = W.shape[0]
    a, e, lam = float(opts["logit_scale"]), float(opts["label_smoothing"]), float(opts["z_loss"])
    c = float(opts["softcap"])
    cols = np.arange(V) if vocab_rows is None else np.asarray(vocab_rows)
    Z = a * logits(X, W[cols])
    Zc = apply_softcap(Z, c)
    P = np.exp(Zc - lse[:, None])
    onehot = (labels[:, None] == cols[None, :]).astype(np.float64)
    dZ = (1.0 + 2.0 * lam * lse)[:, None] * P - (1.0 - e) * onehot - e / V
    dZ = dZ * softcap_derivative(Z, c) * a * np.asarray(scale, dtype=np.float64)[:, None]
    bad = bad_mask(labels, V, int(opts["ignore_index"]))
    dZ[bad] = np.nan
    return dZ


def backward_ex(X: np.ndarray, W: np.ndarray, labels: np.ndarray, dloss,
                opts: Dict[str, object], lse: Optional[np.ndarray] = None):
    """(dX, dW) of the reduced loss with the variant options."""
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    fwd = forward_ex(X, W, labels, opts)
    if lse is None:
        lse = fwd["lse"]
    scale = row_scale(labels, dloss, fwd["n_valid"], opts)
    dZ = logit_gradient_ex(X, W, labels, lse, scale, opts)
    return dZ @ W, dZ.T @ X



def logit_gradient_parts(X: np.ndarray, W: np.ndarray, labels: np.ndarray, lse: np.ndarray,
                         scale: np.ndarray, opts: Dict[str, object],
                         vocab_rows: Optional[np.ndarray] = None):
    """The gradient of logit_gradient_ex as its two terms, (dense, onehot):
    the softmax term s_i·a·((1 + 2l·LSE_i)·p_v − e/V)·d and the target term
    −s_i·a·(1 − e)·[v = y_i]·d ([CCE-blog] §二 and [M011] §06: dZ = p −
    onehot; the variant terms as in logit_gradient_ex).  Their sum is the
    gradient.  Rows with a bad label are NaN in both.  A method that applies
    the target term apart from the rest (exactly, or through another path)
    can be checked term by term with these."""
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64)
    V = W.shape[0]
    a, e, lam = float(opts["logit_scale"]), float(opts["label_smoothing"]), float(opts["z_loss"])
    c = float(opts["softcap"])
    cols = np.arange(V) if vocab_rows is None else np.asarray(vocab_rows)
    Z = a * logits(X, W[cols])
    Zc = apply_softcap(Z, c)
    P = np.exp(Zc - lse[:, None])
    factor = softcap_derivative(Z, c) * a * np.asarray(scale, dtype=np.float64)[:, None]
    dense = ((1.0 + 2.0 * lam * lse)[:, None] * P - e / V) * factor
    onehot = -(1.0 - e) * (labels[:, None] == cols[None, :]) * factor
    bad = bad_mask(labels, V, int(opts["ignore_index"]))
    dense[bad] = np.nan
    onehot[bad] = np.nan
    return dense, onehot


def dX_rows_parts(X_rows: np.ndarray, W: np.ndarray, labels_rows: np.ndarray,
                  lse_rows: np.ndarray, scale_rows: np.ndarray, opts: Dict[str, object]):
    """(dense, onehot) parts of dX for a subset of rows: each term of the
    row's logit gradient contracted with W ([M011] §06: dH = dZ·W)."""
    W = np.asarray(W, dtype=np.float64)
    dense, onehot = logit_gradient_parts(X_rows, W, labels_rows, lse_rows, scale_rows, opts)
    # The target term has at most one non-zero per row (all NaN for a bad
    # row): only the columns holding one enter its product.
    cols = np.nonzero((onehot != 0).any(axis=0))[0]
    return dense @ W, onehot[:, cols] @ W[cols]


def dW_vocab_rows_parts(X: np.ndarray, W: np.ndarray, labels: np.ndarray, lse: np.ndarray,
                        scale: np.ndarray, vocab_rows: np.ndarray, opts: Dict[str, object]):
    """(dense, onehot) parts of dW[v] for selected vocabulary rows, summed
    over every token row ([M011] §06: dW = dZᵀ·H); needs every row's LSE."""
    X = np.asarray(X, dtype=np.float64)
    dense, onehot = logit_gradient_parts(X, W, labels, lse, scale, opts, vocab_rows=vocab_rows)
    return dense.T @ X, onehot.T @ X


# --------------------------------------------------------------------------- #
# Vocabulary shards (reading R17)
# --------------------------------------------------------------------------- #
# [M011] §07 places the vocabulary columns on several ranks: the per-row max,
# exp-sum and target score have to be made global before the loss is formed,
# the hidden-state gradient is a sum of per-shard contributions, and averaging
# a per-shard cross-entropy gives a wrong loss.  The news-site article on GPU
# acceleration of the loss function (§4.3, sharded softmax) describes the same
# split of the class dimension with an all-reduce of the global denominator.
#   R17 a shard owns the contiguous vocabulary rows [v_lo, v_lo + V_shard) of
#       W.  Per shard and row it reports log Σ_{v in shard} exp(z_v), the
#       target logit when the label lies in the shard (else 0) and Σ_{v in
#       shard} z_v.  The merge takes the log-sum-exp of the shard values in
#       shard order (the §05 merge with one block per shard), sums the target
#       and logit-sum parts, and forms the loss of R14 - R16 with the full
#       vocabulary size.  The backward of a shard uses the merged LSE, applies
#       the one-hot term only on the shard that owns the label, and returns
#       its share of dX (the shares add up to dX) and its rows of dW.
def forward_shard(X: np.ndarray, W_shard: np.ndarray, labels: np.ndarray, v_lo: int,
                  V_total: int, opts: Dict[str, object]) -> Dict[str, np.ndarray]:
    """Per-row partials of one vocabulary shard (R17)."""
    X = np.asarray(X, dtype=np.float64)
    W_shard = np.asarray(W_shard, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64)
    a, c = float(opts["logit_scale"]), float(opts["softcap"])
    Zc = apply_softcap(a * logits(X, W_shard), c)
    ok = valid_mask(labels, int(opts["ignore_index"])) & \
        ~bad_mask(labels, V_total, int(opts["ignore_index"]))
    owned = ok & (labels >= v_lo) & (labels < v_lo + W_shard.shape[0])
    target = np.zeros(X.shape[0])
    rows = np.nonzero(owned)[0]
    target[rows] = Zc[rows, labels[rows] - v_lo]
    return {"lse_part": row_logsumexp(Zc), "target_part": target,
            "zsum_part": Zc.sum(axis=1)}


def merge_shards(parts: Sequence[Dict[str, np.ndarray]], labels: np.ndarray, V_total: int,
                 opts: Dict[str, object]) -> Dict[str, np.ndarray]:
    """Global LSE, row losses and the reduced loss from the shard partials,
    taken in shard order (R17)."""
    labels = np.asarray(labels, dtype=np.int64)
    L = np.stack([p["lse_part"] for p in parts])
    m = L.max(axis=0)
    lse = m + np.log(np.exp(L - m[None, :]).sum(axis=0))
    target = np.sum([p["target_part"] for p in parts], axis=0)
    zsum = np.sum([p["zsum_part"] for p in parts], axis=0)
    e, lam = float(opts["label_smoothing"]), float(opts["z_loss"])
    ignore_index = int(opts["ignore_index"])
    valid = valid_mask(labels, ignore_index)
    bad = bad_mask(labels, V_total, ignore_index)
    row_loss = lse - (1.0 - e) * target - (e / V_total) * zsum + lam * lse * lse
    loss = np.where(valid, row_loss, 0.0)
    loss[bad] = np.nan
    n_valid = int(valid.sum())
    total = loss.sum()
    if opts["reduction"] == "mean":
        reduced = total / n_valid if n_valid > 0 else 0.0
    else:
        reduced = total
    return {"lse": lse, "loss": loss, "n_valid": n_valid, "reduced": reduced}


def backward_shard(X: np.ndarray, W_shard: np.ndarray, labels: np.ndarray, lse: np.ndarray,
                   dloss, v_lo: int, V_total: int, opts: Dict[str, object]):
    """(dX share, dW rows) of one vocabulary shard given the merged LSE (R17)."""
    X = np.asarray(X, dtype=np.float64)
    W_shard = np.asarray(W_shard, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64)
    ignore_index = int(opts["ignore_index"])
    n_valid = int(valid_mask(labels, ignore_index).sum())
    scale = row_scale(labels, dloss, n_valid, opts)
    a, c = float(opts["logit_scale"]), float(opts["softcap"])
    e, lam = float(opts["label_smoothing"]), float(opts["z_loss"])
    Z = a * logits(X, W_shard)
    Zc = apply_softcap(Z, c)
    P = np.exp(Zc - lse[:, None])
    cols = v_lo + np.arange(W_shard.shape[0])
    onehot = (labels[:, None] == cols[None, :]).astype(np.float64)
    dZ = (1.0 + 2.0 * lam * lse)[:, None] * P - (1.0 - e) * onehot - e / V_total
    dZ = dZ * softcap_derivative(Z, c) * a * scale[:, None]
    dZ[bad_mask(labels, V_total, ignore_index)] = np.nan
    return dZ @ W_shard, dZ.T @ X


# --------------------------------------------------------------------------- #
# Row-chunked forward with the gradient formed in the same pass (reading R18)
# --------------------------------------------------------------------------- #
# [CCE-blog] §二 (the FLCE pipeline of Liger, also [Liger] §3.2): the rows are
# cut into chunks; for each chunk the logits block is formed, its loss is
# computed and the logit gradient is written in place of the logits, then
# projected back at once (dX rows = dZ_chunk · W, dW accumulated over the
# chunks) before the next chunk starts.  The gradient needs the upstream
# scalar, which the pages apply in the real backward.
#   R18 the upstream gradient (scalar, or one value per row for "none") is an
#       input of the fused call, so dX and dW come out fully scaled; the
#       result equals forward_ex followed by backward_ex for every chunk
#       size (the chunking only changes the schedule).
def forward_backward_chunked(X: np.ndarray, W: np.ndarray, labels: np.ndarray, dloss,
                             opts: Dict[str, object], chunk_rows: int):
    """(forward dict, dX, dW) computed chunk by chunk of `chunk_rows` rows."""
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64)
    N, V = X.shape[0], W.shape[0]
    ignore_index = int(opts["ignore_index"])
    a, c = float(opts["logit_scale"]), float(opts["softcap"])
    e, lam = float(opts["label_smoothing"]), float(opts["z_loss"])
    valid = valid_mask(labels, ignore_index)
    bad = bad_mask(labels, V, ignore_index)
    n_valid = int(valid.sum())          # known before the first chunk (R4)
    scale = row_scale(labels, dloss, n_valid, opts)
    lse = np.zeros(N)
    loss = np.zeros(N)
    dX = np.zeros_like(X)
    dW = np.zeros_like(W)
    for r0 in range(0, N, max(1, int(chunk_rows))):
        r1 = min(N, r0 + max(1, int(chunk_rows)))
        Xb, yb = X[r0:r1], labels[r0:r1]
        Z = a * logits(Xb, W)                        # the chunk's logits block
        Zc = apply_softcap(Z, c)
        lse_b = row_logsumexp(Zc)
        ok = valid[r0:r1] & ~bad[r0:r1]
        t = np.zeros(r1 - r0)
        t[ok] = Zc[np.nonzero(ok)[0], yb[ok]]
        l_b = lse_b - (1.0 - e) * t - (e / V) * Zc.sum(axis=1) + lam * lse_b * lse_b
        l_b = np.where(valid[r0:r1], l_b, 0.0)
        l_b[bad[r0:r1]] = np.nan
        lse[r0:r1], loss[r0:r1] = lse_b, l_b
        # The gradient takes the place of the logits block.
        onehot = (yb[:, None] == np.arange(V)[None, :]).astype(np.float64)
        G = (1.0 + 2.0 * lam * lse_b)[:, None] * np.exp(Zc - lse_b[:, None]) \
            - (1.0 - e) * onehot - e / V
        G = G * softcap_derivative(Z, c) * a * scale[r0:r1, None]
        G[bad[r0:r1]] = np.nan
        dX[r0:r1] = G @ W
        dW += G.T @ Xb
    total = loss.sum()
    if opts["reduction"] == "mean":
        reduced = total / n_valid if n_valid > 0 else 0.0
    else:
        reduced = total
    return {"lse": lse, "loss": loss, "n_valid": n_valid, "reduced": reduced}, dX, dW


# --------------------------------------------------------------------------- #
# Gradient filtering (reading R19; opt-in, not exact)
# --------------------------------------------------------------------------- #
# [CCE-blog] §三: in bf16 training a softmax entry below 2^-12 is lost to
# rounding once it is accumulated into the gradient, and only a tiny share of
# a row's entries is above it, so CCE skips every tile of the backward whose
# entries all lie below the threshold.  [M011] §06 keeps this apart from the
# memory idea: filtering drops gradient terms, and an unfiltered reference is
# kept for comparison.
#   R19 the tile is a block of 256 token rows by 256 vocabulary columns
#       (aligned to multiples of 256 in both indices); the value compared is
#       the dense positive part of the logit gradient, (1 + 2l·LSE_i)·p_iv,
#       over the block's rows that have a target (NaN counts as above); a
#       block whose values are all below eps loses that dense part in both
#       contractions, while the one-hot term is always kept.  Label smoothing
#       (whose −e/V term is not small relative to the threshold in sum) is
#       not combined with filtering.
def filter_block_max(X: np.ndarray, W: np.ndarray, labels: np.ndarray, lse: np.ndarray,
                     opts: Dict[str, object], tile: int = 256) -> np.ndarray:
    """Per (token block, vocabulary block): max over rows with a target of
    (1 + 2l·LSE)·p (NaN if any such value is NaN), −inf for blocks without
    such rows."""
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64)
    N, V = X.shape[0], W.shape[0]
    a, c, lam = float(opts["logit_scale"]), float(opts["softcap"]), float(opts["z_loss"])
    Zc = apply_softcap(a * logits(X, W), c)
    P = (1.0 + 2.0 * lam * lse)[:, None] * np.exp(Zc - lse[:, None])
    P[~valid_mask(labels, int(opts["ignore_index"]))] = -np.inf
    nb_r, nb_c = -(-N // tile), -(-V // tile)
    out = np.full((nb_r, nb_c), -np.inf)
    for bi in range(nb_r):
        for bj in range(nb_c):
            blk = P[bi * tile:(bi + 1) * tile, bj * tile:(bj + 1) * tile]
            out[bi, bj] = np.nan if np.isnan(blk).any() else blk.max()
    return out


def backward_filtered(X: np.ndarray, W: np.ndarray, labels: np.ndarray, dloss,
                      opts: Dict[str, object], eps: float, tile: int = 256):
    """(dX, dW) with the dense gradient part of every block whose values all
    lie below eps removed (R19)."""
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64)
    if float(opts["label_smoothing"]) > 0:
        raise ValueError("gradient filtering is not combined with label smoothing (R19)")
    N, V = X.shape[0], W.shape[0]
    fwd = forward_ex(X, W, labels, opts)
    lse = fwd["lse"]
    scale = row_scale(labels, dloss, fwd["n_valid"], opts)
    a, c, lam = float(opts["logit_scale"]), float(opts["softcap"]), float(opts["z_loss"])
    Z = a * logits(X, W)
    Zc = apply_softcap(Z, c)
    dense = (1.0 + 2.0 * lam * lse)[:, None] * np.exp(Zc - lse[:, None])
    bm = filter_block_max(X, W, labels, lse, opts, tile)
    for bi in range(bm.shape[0]):
        for bj in range(bm.shape[1]):
            if bm[bi, bj] < eps:                     # NaN compares False: kept
                dense[bi * tile:(bi + 1) * tile, bj * tile:(bj + 1) * tile] = 0.0
    onehot = (labels[:, None] == np.arange(V)[None, :]).astype(np.float64)
    G = (dense - onehot) * softcap_derivative(Z, c) * a * scale[:, None]
    G[bad_mask(labels, V, int(opts["ignore_index"]))] = np.nan
    return G @ W, G.T @ X


# --------------------------------------------------------------------------- #
# Vocabulary order for the gradient filter (reading R20)
# --------------------------------------------------------------------------- #
# [CCE-blog] §三: alongside the filter, the forward records every vocabulary
# entry's average logit and the backward moves the frequently large ("hot")
# entries next to each other, so that the blocks it skips are whole ones more
# often.
#   R20 the average is over the rows whose label is not the ignore index, of
#       the plain logit x_i·w_v (before logit scale and softcap, both of which
#       are increasing); with no such row every average is 0.  Entries are
#       ordered by decreasing average, equal averages by increasing index, a
#       NaN average before every number.  The backward with an order is the
#       backward of the vocabulary relabelled by it: position j holds entry
#       order[j], a label y becomes the position of y, filter blocks are cut
#       in positions, and each dW row is returned to its entry.
def vocab_mean_logit(X: np.ndarray, W: np.ndarray, labels: np.ndarray,
                     ignore_index: int = IGNORE_INDEX) -> np.ndarray:
    """Average logit of every vocabulary entry over the rows with a target."""
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    rows = valid_mask(np.asarray(labels, dtype=np.int64), ignore_index)
    n = int(rows.sum())
    if n == 0:
        return np.zeros(W.shape[0])
    return logits(X[rows], W).sum(axis=0) / n


def vocab_order(mean_logit: np.ndarray) -> np.ndarray:
    """Entries by decreasing average logit; ties by index; NaN first."""
    m = np.asarray(mean_logit, dtype=np.float64)
    idx = np.arange(m.shape[0])
    nan = np.isnan(m)
    # lexsort: last key is the primary one.
    return np.lexsort((idx, -np.where(nan, 0.0, m), ~nan)).astype(np.int64)


def backward_sorted(X: np.ndarray, W: np.ndarray, labels: np.ndarray, dloss,
                    opts: Dict[str, object], order: np.ndarray, eps: float = 0.0,
                    tile: int = 256):
    """(dX, dW) of the backward on the vocabulary relabelled by `order`
    (R20), filtered with threshold eps when eps > 0 (R19)."""
    W = np.asarray(W, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64)
    order = np.asarray(order, dtype=np.int64)
    V = W.shape[0]
    if not np.array_equal(np.sort(order), np.arange(V)):
        raise ValueError("order must be a permutation of the vocabulary")
    position = np.empty(V, dtype=np.int64)
    position[order] = np.arange(V)
    ign = int(opts["ignore_index"])
    ignored = labels == ign
    moved = ~ignored & (labels >= 0) & (labels < V)
    lab = labels.copy()
    lab[moved] = position[labels[moved]]
    # A position may equal a non-negative ignore index: the relabelled problem
    # marks its ignored rows with a value no label or position takes.
    ign_pos = min(int(labels.min(initial=0)), 0) - 1
    lab[ignored] = ign_pos
    o_pos = dict(opts, ignore_index=ign_pos)
    W_pos = W[order]
    if eps > 0:
        dX, dW_pos = backward_filtered(X, W_pos, lab, dloss, o_pos, eps, tile)
    else:
        dX, dW_pos = backward_ex(X, W_pos, lab, dloss, o_pos)
    dW = np.empty_like(dW_pos)
    dW[order] = dW_pos
    return dX, dW
