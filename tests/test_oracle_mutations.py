"""Plant plausible mistakes in the oracle (CPU only) and check the pins notice.

Each mutation replaces one oracle building block by a subtly wrong one; the
pin suite must then fail at least one of its checks.  This guards the pins
themselves: a pin set that passes a wrong oracle pins nothing.
"""
import numpy as np
import pytest

from oracle import lce_oracle as O
from tests import test_oracle_pins as P

PINS = [
    P.test_worked_example_loss_matches_page,
    P.test_worked_example_two_tile_merge_and_wrong_value_rejected,
    P.test_worked_example_gradient_is_softmax_minus_onehot,
    P.test_textbook_softmax_definition_bruteforce,
    lambda: P.test_matches_torch_cross_entropy_and_autograd(0.0),
    lambda: P.test_matches_torch_cross_entropy_and_autograd(2.5),
    lambda: P.test_finite_differences(0.0),
    lambda: P.test_finite_differences(0.9),
    P.test_ignored_rows_contribute_nothing,
    P.test_zero_weight_closed_form,
    P.test_bounds_nonnegativity_and_gradient_row_sums,
]

_orig_forward = O.forward
_orig_logit_gradient = O.logit_gradient


def _forward_mean_over_all_rows(X, W, labels, ignore_index=-100, softcap=0.0, n_valid_total=None):
    out = _orig_forward(X, W, labels, ignore_index, softcap, n_valid_total)
    out["n_valid"] = len(labels)
    out["mean"] = out["loss_sum"] / len(labels)
    return out


def _forward_target_off_by_one(X, W, labels, ignore_index=-100, softcap=0.0, n_valid_total=None):
    out = _orig_forward(X, W, labels, ignore_index, softcap, n_valid_total)
    Zc = O.apply_softcap(O.logits(np.asarray(X, float), np.asarray(W, float)), softcap)
    V = Zc.shape[1]
    t = np.array([Zc[i, (y + 1) % V] if y != ignore_index else 0.0 for i, y in enumerate(labels)])
    out["loss"] = np.where(labels != ignore_index, out["lse"] - t, 0.0)
    out["mean"] = out["loss"].sum() / max(out["n_valid"], 1)
    return out


def _forward_uncapped_target(X, W, labels, ignore_index=-100, softcap=0.0, n_valid_total=None):
    out = _orig_forward(X, W, labels, ignore_index, softcap, n_valid_total)
    Z = O.logits(np.asarray(X, float), np.asarray(W, float))
    t = np.array([Z[i, y] if y != ignore_index else 0.0 for i, y in enumerate(labels)])
    out["loss"] = np.where(labels != ignore_index, out["lse"] - t, 0.0)
    out["mean"] = out["loss"].sum() / max(out["n_valid"], 1)
    return out


def _grad_without_onehot(X, W, labels, lse, n_valid, dloss=1.0, ignore_index=-100,
                         softcap=0.0, vocab_rows=None):
    g = _orig_logit_gradient(X, W, labels, lse, n_valid, dloss, ignore_index, softcap, vocab_rows)
    V = np.asarray(W).shape[0]
    cols = np.arange(V) if vocab_rows is None else np.asarray(vocab_rows)
    onehot = (np.asarray(labels)[:, None] == cols[None, :])
    valid = (np.asarray(labels) != ignore_index)[:, None]
    s = dloss / n_valid if n_valid else 0.0
    d = O.softcap_derivative(O.logits(np.asarray(X, float), np.asarray(W, float)[cols]), softcap)
    return g + s * onehot * valid * d


def _grad_wrong_sign(X, W, labels, lse, n_valid, dloss=1.0, ignore_index=-100,
                     softcap=0.0, vocab_rows=None):
    return -_orig_logit_gradient(X, W, labels, lse, n_valid, dloss, ignore_index, softcap, vocab_rows)


def _bad_softcap_derivative(Z, softcap):
    if softcap > 0:
        t = np.tanh(Z / softcap)
        return 1.0 + t * t
    return np.ones_like(Z)


def _no_softcap_derivative(Z, softcap):
    return np.ones_like(Z)


def _transposed_logits(X, W):
    # uses the weight as if it were stored [H, V] (the orientation conflict
    # between the pages): only differs for square/compatible shapes, else raises
    return X @ np.asarray(W).reshape(np.asarray(W).shape[::-1])


def _lse_without_log(Zc):
    m = Zc.max(axis=1)
    return m + np.exp(Zc - m[:, None]).sum(axis=1) - 1.0


MUTATIONS = {
    "mean_over_all_rows": ("forward", _forward_mean_over_all_rows),
    "target_off_by_one": ("forward", _forward_target_off_by_one),
    "uncapped_target": ("forward", _forward_uncapped_target),
    "gradient_without_onehot": ("logit_gradient", _grad_without_onehot),
    "gradient_wrong_sign": ("logit_gradient", _grad_wrong_sign),
    "softcap_derivative_sign": ("softcap_derivative", _bad_softcap_derivative),
    "softcap_derivative_dropped": ("softcap_derivative", _no_softcap_derivative),
    "weight_transposed": ("logits", _transposed_logits),
    "lse_missing_log": ("row_logsumexp", _lse_without_log),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    failures = 0
    for pin in PINS:
        try:
            pin()
        except Exception:       # AssertionError or a shape error: both are catches
            failures += 1
    assert failures > 0, f"no pin caught mutation {name}"


# --------------------------------------------------------------------------- #
# Loss variants: mistakes planted in forward_ex / logit_gradient_ex must be
# caught by the variant pins.
# --------------------------------------------------------------------------- #
from tests import test_oracle_variants as PV  # noqa: E402

VARIANT_PINS = [
    lambda: PV.test_label_smoothing_and_reduction_match_torch("mean", 0.0, 1.0, 0.1),
    lambda: PV.test_label_smoothing_and_reduction_match_torch("none", 2.0, 0.5, 0.3),
    lambda: PV.test_label_smoothing_and_reduction_match_torch("sum", 0.0, 1.7, 0.0),
    PV.test_zero_weight_closed_forms,
    lambda: PV.test_finite_differences_all_options("mean"),
    lambda: PV.test_finite_differences_all_options("none"),
    PV.test_logit_scale_is_a_scale_of_W,
    PV.test_reduction_relations,
]

_orig_forward_ex = O.forward_ex
_orig_grad_ex = O.logit_gradient_ex
_orig_row_scale = O.row_scale


def _fx_smoothing_over_v_minus_1(X, W, labels, opts, n_valid_total=None):
    out = _orig_forward_ex(X, W, labels, opts, n_valid_total)
    V = np.asarray(W).shape[0]
    e = float(opts["label_smoothing"])
    valid = np.asarray(labels) != int(opts["ignore_index"])
    out["loss"] = out["loss"] + valid * (e / V - e / (V - 1)) * out["logit_sum"]
    out["reduced"] = out["loss"].sum() / (out["n_valid"] if opts["reduction"] == "mean" else 1)
    return out


def _fx_zloss_not_squared(X, W, labels, opts, n_valid_total=None):
    out = _orig_forward_ex(X, W, labels, opts, n_valid_total)
    lam = float(opts["z_loss"])
    valid = np.asarray(labels) != int(opts["ignore_index"])
    out["loss"] = out["loss"] + valid * lam * (out["lse"] - out["lse"] ** 2)
    out["reduced"] = out["loss"].sum() / (out["n_valid"] if opts["reduction"] == "mean" else 1)
    return out


def _fx_scale_after_softcap(X, W, labels, opts, n_valid_total=None):
    # a · c·tanh(z / c) (scale applied after the cap) equals a softcap of a·c
    # applied to a·z; without a softcap the order does not matter, so the
    # mutant then drops the scale instead.
    o = dict(opts)
    if float(o["softcap"]) > 0:
        o["softcap"] = float(o["softcap"]) * float(o["logit_scale"])
    else:
        o["logit_scale"] = 1.0
    return _orig_forward_ex(X, W, labels, o, n_valid_total)


def _gx_onehot_not_smoothed(X, W, labels, lse, scale, opts, vocab_rows=None):
    g = _orig_grad_ex(X, W, labels, lse, scale, opts, vocab_rows)
    V = np.asarray(W).shape[0]
    cols = np.arange(V) if vocab_rows is None else np.asarray(vocab_rows)
    e, a = float(opts["label_smoothing"]), float(opts["logit_scale"])
    onehot = (np.asarray(labels)[:, None] == cols[None, :])
    Z = a * O.logits(np.asarray(X, float), np.asarray(W, float)[cols])
    d = O.softcap_derivative(Z, float(opts["softcap"]))
    return g - e * onehot * d * a * np.asarray(scale)[:, None]


def _gx_zloss_factor_one(X, W, labels, lse, scale, opts, vocab_rows=None):
    o = dict(opts)
    o["z_loss"] = float(opts["z_loss"]) / 2.0      # (1 + l·LSE) instead of (1 + 2l·LSE)
    return _orig_grad_ex(X, W, labels, lse, scale, o, vocab_rows)


def _rs_none_uses_mean(labels, dloss, n_valid, opts):
    if opts["reduction"] == "none":
        s = np.asarray(dloss, dtype=np.float64).reshape(-1) / max(n_valid, 1)
        return s * (np.asarray(labels) != int(opts["ignore_index"]))
    return _orig_row_scale(labels, dloss, n_valid, opts)


VARIANT_MUTATIONS = {
    "smoothing_over_V_minus_1": ("forward_ex", _fx_smoothing_over_v_minus_1),
    "zloss_not_squared": ("forward_ex", _fx_zloss_not_squared),
    "scale_after_softcap": ("forward_ex", _fx_scale_after_softcap),
    "onehot_not_smoothed": ("logit_gradient_ex", _gx_onehot_not_smoothed),
    "zloss_gradient_factor": ("logit_gradient_ex", _gx_zloss_factor_one),
    "none_reduction_divides": ("row_scale", _rs_none_uses_mean),
}


@pytest.mark.parametrize("name", sorted(VARIANT_MUTATIONS))
def test_variant_pins_catch_mutation(name, monkeypatch):
    attr, fn = VARIANT_MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    failures = 0
    for pin in VARIANT_PINS:
        try:
            pin()
        except Exception:
            failures += 1
    assert failures > 0, f"no pin caught mutation {name}"


# --------------------------------------------------------------------------- #
# Vocabulary shards: mistakes planted in forward_shard / merge_shards /
# backward_shard must be caught by the shard pins.
# --------------------------------------------------------------------------- #
from tests import test_oracle_shards as PS  # noqa: E402

SHARD_PINS = [
    PS.test_worked_example_split_in_two_shards,
    lambda: PS.test_partition_independence(PS.OPTION_SETS[2], [0, 4, 5, 13]),
    lambda: PS.test_partition_independence(PS.OPTION_SETS[0], [0, 6, 12, 13]),
    lambda: PS.test_finite_differences_through_the_merge("mean"),
]

_orig_forward_shard = O.forward_shard
_orig_merge_shards = O.merge_shards
_orig_backward_shard = O.backward_shard


def _ms_max_of_shards(parts, labels, V_total, opts):
    # Keeps only the largest shard's mass instead of adding all of them.
    out = _orig_merge_shards(parts, labels, V_total, opts)
    L = np.stack([p["lse_part"] for p in parts]).max(axis=0)
    delta = L - out["lse"]
    valid = np.asarray(labels) != int(opts["ignore_index"])
    out["lse"] = L
    out["loss"] = out["loss"] + valid * delta
    return out


def _fs_target_on_every_shard(X, W_shard, labels, v_lo, V_total, opts):
    out = _orig_forward_shard(X, W_shard, labels, v_lo, V_total, opts)
    Vs = np.asarray(W_shard).shape[0]
    Zc = O.apply_softcap(float(opts["logit_scale"]) * O.logits(np.asarray(X, float),
                                                               np.asarray(W_shard, float)),
                         float(opts["softcap"]))
    lab = np.asarray(labels)
    ok = (lab != int(opts["ignore_index"])) & (lab >= 0) & (lab < V_total)
    rows = np.nonzero(ok)[0]
    out["target_part"] = np.zeros(len(lab))
    out["target_part"][rows] = Zc[rows, (lab[rows] - v_lo) % Vs]
    return out


def _bs_local_lse(X, W_shard, labels, lse, dloss, v_lo, V_total, opts):
    local = _orig_forward_shard(X, W_shard, labels, v_lo, V_total, opts)["lse_part"]
    return _orig_backward_shard(X, W_shard, labels, local, dloss, v_lo, V_total, opts)


SHARD_MUTATIONS = {
    "merge_keeps_max_shard": ("merge_shards", _ms_max_of_shards),
    "target_on_every_shard": ("forward_shard", _fs_target_on_every_shard),
    "backward_with_shard_lse": ("backward_shard", _bs_local_lse),
}


@pytest.mark.parametrize("name", sorted(SHARD_MUTATIONS))
def test_shard_pins_catch_mutation(name, monkeypatch):
    attr, fn = SHARD_MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    failures = 0
    for pin in SHARD_PINS:
        try:
            pin()
        except Exception:
            failures += 1
    assert failures > 0, f"no pin caught mutation {name}"


# --------------------------------------------------------------------------- #
# Row-chunked forward with gradient: planted mistakes must be caught by its
# pins.
# --------------------------------------------------------------------------- #
from tests import test_oracle_fused as PF  # noqa: E402

FUSED_PINS = [
    lambda: PF.test_matches_torch_autograd(0.0),
    lambda: PF.test_equals_forward_then_backward(PF.OPTS[1], 4),
    lambda: PF.test_equals_forward_then_backward(PF.OPTS[0], 11),
]

_orig_fused = O.forward_backward_chunked


def _fused_dw_overwritten(X, W, labels, dloss, opts, chunk_rows):
    # dW keeps only the last chunk's contribution.
    N = len(labels)
    last0 = (N - 1) // chunk_rows * chunk_rows
    f, dX, _ = _orig_fused(X, W, labels, dloss, opts, chunk_rows)
    _, _, dW_last = _orig_fused(np.asarray(X)[last0:], W, np.asarray(labels)[last0:],
                                dloss, opts, chunk_rows)
    return f, dX, dW_last


def _fused_mean_per_chunk(X, W, labels, dloss, opts, chunk_rows):
    # Each chunk normalised by its own valid count instead of the batch's.
    labels = np.asarray(labels)
    outs = []
    for r0 in range(0, len(labels), chunk_rows):
        outs.append(_orig_fused(np.asarray(X)[r0:r0 + chunk_rows], W, labels[r0:r0 + chunk_rows],
                                dloss, opts, chunk_rows))
    f = _orig_fused(X, W, labels, dloss, opts, chunk_rows)[0]
    dX = np.concatenate([o[1] for o in outs])
    dW = sum(o[2] for o in outs)
    return f, dX, dW


FUSED_MUTATIONS = {
    "dw_not_accumulated": ("forward_backward_chunked", _fused_dw_overwritten),
    "mean_per_chunk": ("forward_backward_chunked", _fused_mean_per_chunk),
}


@pytest.mark.parametrize("name", sorted(FUSED_MUTATIONS))
def test_fused_pins_catch_mutation(name, monkeypatch):
    attr, fn = FUSED_MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    failures = 0
    for pin in FUSED_PINS:
        try:
            pin()
        except Exception:
            failures += 1
    assert failures > 0, f"no pin caught mutation {name}"


# --------------------------------------------------------------------------- #
# Vocabulary order: planted mistakes must be caught by its pins.
# --------------------------------------------------------------------------- #
from tests import test_oracle_sorting as PO  # noqa: E402

ORDER_PINS = [
    PO.test_mean_logit_by_loops,
    PO.test_order_elementwise,
    PO.test_order_of_duplicate_entries,
    lambda: PO.test_any_order_without_filter_is_the_plain_backward(dict(softcap=2.5, z_loss=0.02)),
    PO.test_bruteforce_blocks_in_positions,
]

_orig_mean_logit = O.vocab_mean_logit
_orig_order = O.vocab_order
_orig_sorted = O.backward_sorted


def _ml_all_rows(X, W, labels, ignore_index=-100):
    # Averages over every row, ignored ones included.
    return _orig_mean_logit(X, W, np.zeros_like(np.asarray(labels)), ignore_index)


def _order_ascending(mean_logit):
    return _orig_order(-np.asarray(mean_logit))


def _order_ties_reversed(mean_logit):
    m = np.asarray(mean_logit)
    idx = np.arange(len(m))
    return np.lexsort((-idx, -m)).astype(np.int64)


def _sorted_dw_in_positions(X, W, labels, dloss, opts, order, eps=0.0, tile=256):
    # dW rows left in positions instead of returned to their entries.
    dX, dW = _orig_sorted(X, W, labels, dloss, opts, order, eps, tile)
    return dX, dW[np.asarray(order)]


def _sorted_labels_not_moved(X, W, labels, dloss, opts, order, eps=0.0, tile=256):
    # The reordered W is used with the original labels.
    W = np.asarray(W, dtype=np.float64)
    dX, dW_pos = _orig_sorted(X, W[np.asarray(order)], labels, dloss, opts,
                              np.arange(W.shape[0]), eps, tile)
    dW = np.empty_like(dW_pos)
    dW[np.asarray(order)] = dW_pos
    return dX, dW


ORDER_MUTATIONS = {
    "mean_over_all_rows": ("vocab_mean_logit", _ml_all_rows),
    "ascending": ("vocab_order", _order_ascending),
    "ties_reversed": ("vocab_order", _order_ties_reversed),
    "dw_left_in_positions": ("backward_sorted", _sorted_dw_in_positions),
    "labels_not_moved": ("backward_sorted", _sorted_labels_not_moved),
}


@pytest.mark.parametrize("name", sorted(ORDER_MUTATIONS))
def test_order_pins_catch_mutation(name, monkeypatch):
    attr, fn = ORDER_MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    failures = 0
    for pin in ORDER_PINS:
        try:
            pin()
        except Exception:
            failures += 1
    assert failures > 0, f"no pin caught mutation {name}"


# --------------------------------------------------------------------------- #
# Gradient split into its softmax and target terms: planted mistakes must be
# caught by its pins.
# --------------------------------------------------------------------------- #
from tests import test_oracle_parts as PP  # noqa: E402

PARTS_PINS = [lambda kw=kw: PP.test_parts_match_autograd_of_their_terms(kw) for kw in PP.CASES]
PARTS_PINS.append(PP.test_parts_of_a_subset_of_rows_and_bad_labels)

_orig_parts = O.logit_gradient_parts


def _parts_smoothing_in_onehot(X, W, labels, lse, scale, opts, vocab_rows=None):
    # The uniform −e/V term moved from the dense part into the one-hot part.
    dense, onehot = _orig_parts(X, W, labels, lse, scale, opts, vocab_rows)
    e = float(opts["label_smoothing"])
    a = float(opts["logit_scale"])
    V = np.asarray(W).shape[0]
    cols = np.arange(V) if vocab_rows is None else np.asarray(vocab_rows)
    Z = a * O.logits(np.asarray(X, float), np.asarray(W, float)[cols])
    shift = (e / V) * O.softcap_derivative(Z, float(opts["softcap"])) * a * \
        np.asarray(scale, float)[:, None]
    return dense + shift, onehot - shift


def _parts_onehot_without_derivative(X, W, labels, lse, scale, opts, vocab_rows=None):
    # The target term without the softcap derivative at the target.
    dense, _ = _orig_parts(X, W, labels, lse, scale, opts, vocab_rows)
    e, a = float(opts["label_smoothing"]), float(opts["logit_scale"])
    V = np.asarray(W).shape[0]
    cols = np.arange(V) if vocab_rows is None else np.asarray(vocab_rows)
    onehot = -(1.0 - e) * (np.asarray(labels)[:, None] == cols[None, :]) * a * \
        np.asarray(scale, float)[:, None]
    return dense, onehot


def _parts_zloss_factor_dropped(X, W, labels, lse, scale, opts, vocab_rows=None):
    # The dense term without the Z-loss factor 1 + 2l·LSE.
    o = dict(opts)
    o["z_loss"] = 0.0
    return _orig_parts(X, W, labels, lse, scale, o, vocab_rows)


PARTS_MUTATIONS = {
    "smoothing_in_onehot": ("logit_gradient_parts", _parts_smoothing_in_onehot),
    "onehot_without_derivative": ("logit_gradient_parts", _parts_onehot_without_derivative),
    "zloss_factor_dropped": ("logit_gradient_parts", _parts_zloss_factor_dropped),
}


@pytest.mark.parametrize("name", sorted(PARTS_MUTATIONS))
def test_parts_pins_catch_mutation(name, monkeypatch):
    attr, fn = PARTS_MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    failures = 0
    for pin in PARTS_PINS:
        try:
            pin()
        except Exception:
            failures += 1
    assert failures > 0, f"no pin caught mutation {name}"
