"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments with the documented status before
touching the GPU (no compute call is made)."""
import ctypes
import os
import re

import pytest

from linear_cross_entropy_lse_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("liblce.so not built")
    return _lib.load()


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "lce.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lce_[a-z_]+)\s*\(", text)))


def test_header_declares_exactly_the_binding_symbols():
    assert declared_symbols() == sorted(_lib.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.lce_version() >= 100
    for st in range(7):
        assert len(lib.lce_status_string(st)) > 0


def test_workspace_queries(lib):
    assert lib.lce_forward_workspace_bytes(256, 64, 1000) > 0
    assert lib.lce_forward_workspace_bytes(256, 63, 1000) == 0        # H % 8
    assert lib.lce_forward_workspace_bytes(-1, 64, 1000) == 0
    assert lib.lce_backward_workspace_bytes(256, 64, 0, 0) == 0
    assert lib.lce_backward_workspace_bytes(256, 64, 1000, 7) == 0    # bad dtype enum
    # The backward workspace never holds the whole N x V logit matrix.
    for (N, H, V) in [(8192, 2304, 256128), (32768, 3584, 152064), (16384, 4096, 32000),
                      (8192, 4096, 128256)]:
        ws = lib.lce_backward_workspace_bytes(N, H, V, 0)
        assert 0 < ws < N * V * 2
        assert lib.lce_backward_workspace_bytes(N, H, V, 1) > ws      # + fp32 dW chunk
        assert lib.lce_forward_workspace_bytes(N, H, V) < 64 * N * 8 + (1 << 20)


def test_forward_workspace_holds_the_split_partials(lib):
    """The forward workspace is the row state and target (8 bytes a row), the
    split partials m, s and the logit sums (12 bytes a row and split) and the
    per-block sums (24 bytes a block of 256 rows), each region aligned to 256
    bytes.  Up to 32 token tiles every row has S = min(256 / T, vocabulary
    tiles) splits; past that the rows of the full groups of 32 tiles have 8
    and the r tiles after them min(256 / r, vocabulary tiles), so the tail's
    block adds at most 256·256 partials, 768 KiB, over 8 a row."""
    import random

    def parts(N, V):
        T, nvt = max(1, -(-N // 256)), -(-V // 256)
        S = max(1, min(256 // min(T, 32), nvt))
        tail = T % 32 if T > 32 else 0
        if not tail:
            return S * N, 0
        main = (T - tail) * 256
        s_tail = max(1, min(256 // tail, nvt))
        return S * main + s_tail * (N - main), s_tail * (N - main)

    rng = random.Random(13)
    shapes = [(8192, 256128), (8193, 256128), (8448, 256128), (16640, 32000), (16383, 5), (1, 1),
              (32 * 256 + 1, 1000), (63 * 256, 128256), (640000, 2048)]
    shapes += [(rng.randint(1, 200000), rng.randint(1, 300000)) for _ in range(300)]
    for N, V in shapes:
        total, tail = parts(N, V)
        lo = 8 * N + 12 * total + 24 * -(-N // 256)
        ws = lib.lce_forward_workspace_bytes(N, 64, V)
        assert lo <= ws <= lo + 6 * 256, (N, V, ws, lo)
        assert 12 * tail <= 768 << 10


FAKE = 1 << 20  # a 256-byte-aligned non-NULL address: never dereferenced on these paths


def fwd(lib, X=FAKE, W=FAKE, y=FAKE, N=4, H=8, V=5, loss=FAKE, lse=FAKE, mean=FAKE,
        nv=FAKE, bad=0, ws=FAKE, wsb=None):
    if wsb is None:
        wsb = lib.lce_forward_workspace_bytes(max(N, 0), H, V)
    return lib.lce_forward(X, W, y, N, H, V, -100, 0.0, loss, lse, mean, nv, bad, ws, wsb, None)


def bwd(lib, X=FAKE, W=FAKE, y=FAKE, lse=FAKE, dl=FAKE, N=4, H=8, V=5, dX=FAKE, dXt=0,
        dW=FAKE, dWt=0, ws=FAKE, wsb=None):
    if wsb is None:
        wsb = lib.lce_backward_workspace_bytes(max(N, 0), H, V, dWt if dWt in (0, 1) else 0)
    return lib.lce_backward(X, W, y, lse, dl, N, H, V, -100, 0.0, dX, dXt, dW, dWt, ws, wsb,
                            None)


def test_shape_limits(lib):
    """The limits of include/lce.h, on both sides of each bound: H < 2^20,
    V < 2^31 - 1, N < 2^31 - 1 (workspace queries return 0 for a refused shape)."""
    big = (1 << 31) - 2
    for q in (lambda N, H, V: lib.lce_forward_workspace_bytes(N, H, V),
              lambda N, H, V: lib.lce_backward_workspace_bytes(N, H, V, 0),
              lambda N, H, V: lib.lce_backward_workspace_bytes(N, H, V, 1)):
        assert q(4, (1 << 20) - 8, 5) > 0
        assert q(4, 1 << 20, 5) == 0
        assert q(4, 8, big) > 0
        assert q(4, 8, big + 1) == 0
        assert q(big, 8, 5) > 0
        assert q(big + 1, 8, 5) == 0
    assert fwd(lib, H=1 << 20) == _lib.LCE_ERR_SHAPE
    assert fwd(lib, V=big + 1) == _lib.LCE_ERR_SHAPE
    assert fwd(lib, N=big + 1) == _lib.LCE_ERR_SHAPE
    assert bwd(lib, H=1 << 20) == _lib.LCE_ERR_SHAPE
    assert bwd(lib, V=big + 1) == _lib.LCE_ERR_SHAPE


def test_fused_plan_matches_the_sampling_mirror(lib):
    """The fused call's row chunking (lce_fused_plan) equals the mirror the
    full-size tests use to sample both sides of every chunk boundary, and
    meets its stated bounds: whole tiles, at most 2H rows (one tile at least)
    and, from two tiles on, at most half the tiles rounded up; chunks as even
    as whole tiles allow; the last chunk holds at least one row; the dX parts
    of a full chunk follow dx_parts of its tiles."""
    import random
    from tests import fullsize_samples as FS

    def dx_parts(steps, T, nt_h):
        avg = max(1, 2 * T * nt_h * steps // 256)
        ks = min(max(1, -(-steps // avg)), 16)
        return -(-steps // -(-steps // ks))

    rng = random.Random(12)
    shapes = [(8192, 2304, 256128), (16384, 4096, 32000), (8192, 4096, 128256), (32768, 3584, 152064),
              (256, 64, 1000), (8448, 2304, 256128), (4352, 2304, 256128), (1, 8, 1), (0, 64, 100)]
    shapes += [(rng.randint(1, 70000), 8 * rng.randint(1, 1024), rng.randint(1, 300000)) for _ in range(300)]
    rows, nch, parts = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32()
    for N, H, V in shapes:
        assert lib.lce_fused_plan(N, H, V, ctypes.byref(rows), ctypes.byref(nch),
                                  ctypes.byref(parts)) == _lib.LCE_OK
        nc = FS.fused_chunk_rows(N, H, V)
        assert rows.value == nc, (N, H, V, rows.value, nc)
        T, t = -(-max(N, 1) // 256), nc // 256
        assert nc % 256 == 0 and t >= 1
        assert t == 1 or nc <= 2 * H
        assert T == 1 or t <= -(-T // 2)
        assert nch.value == -(-max(N, 1) // nc) and max(N, 1) - (nch.value - 1) * nc >= 1
        assert t == -(-T // nch.value), (N, H, V)
        assert parts.value == dx_parts(-(-V // 64), t, -(-H // 256)), (N, H, V)
    for N, H, V, n_expect in [(8192, 2304, 256128, 2), (8448, 2304, 256128, 2), (4352, 2304, 256128, 2)]:
        assert lib.lce_fused_plan(N, H, V, ctypes.byref(rows), ctypes.byref(nch),
                                  ctypes.byref(parts)) == _lib.LCE_OK
        assert nch.value == n_expect, (N, nch.value)
    assert lib.lce_fused_plan(8, 12, 5, ctypes.byref(rows), ctypes.byref(nch),
                              ctypes.byref(parts)) == _lib.LCE_ERR_SHAPE
    assert lib.lce_fused_plan(8, 16, 5, None, ctypes.byref(nch), ctypes.byref(parts)) == _lib.LCE_ERR_INVALID_ARG


def test_backward_plan_matches_the_sampling_mirror(lib):
    """The chunking the library reports (lce_backward_plan) equals the mirror
    the full-size tests use to place their samples at chunk boundaries
    (tests/fullsize_samples.py), and its dX parts follow the rule written
    out here: split a dX tile's K range until one part is no longer than the
    average work per workgroup, 2·T·nt_h·steps / 256 K steps, at most 16
    parts, every part holding a step."""
    import random
    from tests import fullsize_samples as FS

    def dx_parts(steps, T, nt_h):
        avg = max(1, 2 * T * nt_h * steps // 256)
        ks = min(max(1, -(-steps // avg)), 16)
        return -(-steps // -(-steps // ks))

    rng = random.Random(11)
    shapes = [(8192, 2304, 256128), (16384, 4096, 32000), (8192, 4096, 128256), (32768, 3584, 152064),
              (256, 64, 1000), (1024, 2304, 256128), (16384, 768, 50257), (40, 64, (1 << 21) + 100003)]
    shapes += [(rng.randint(1, 70000), 8 * rng.randint(1, 1024), rng.randint(1, 300000)) for _ in range(300)]
    cols, nch, parts = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32()
    for N, H, V in shapes:
        assert lib.lce_backward_plan(N, H, V, 0, ctypes.byref(cols), ctypes.byref(nch),
                                     ctypes.byref(parts)) == _lib.LCE_OK
        vc = FS.backward_chunk_columns(N, H, V)
        assert cols.value == vc, (N, H, V, cols.value, vc)
        assert nch.value == -(-V // vc)
        steps0 = -(-min(vc, V) // 64)
        assert parts.value == dx_parts(steps0, -(-max(N, 1) // 256), -(-H // 256)), (N, H, V)
        assert lib.lce_backward_plan(N, H, V, 1, ctypes.byref(cols), ctypes.byref(nch),
                                     ctypes.byref(parts)) == _lib.LCE_OK
        assert cols.value % 256 == 0 and cols.value <= vc
    assert lib.lce_backward_plan(4, 12, 5, 0, ctypes.byref(cols), ctypes.byref(nch),
                                 ctypes.byref(parts)) == _lib.LCE_ERR_SHAPE
    assert lib.lce_backward_plan(4, 16, 5, 2, ctypes.byref(cols), ctypes.byref(nch),
                                 ctypes.byref(parts)) == _lib.LCE_ERR_INVALID_ARG
    assert lib.lce_backward_plan(4, 16, 5, 0, None, ctypes.byref(nch),
                                 ctypes.byref(parts)) == _lib.LCE_ERR_INVALID_ARG


def test_forward_error_paths(lib):
    assert fwd(lib, H=12) == _lib.LCE_ERR_SHAPE
    assert fwd(lib, H=0) == _lib.LCE_ERR_SHAPE
    assert fwd(lib, V=0) == _lib.LCE_ERR_SHAPE
    assert fwd(lib, N=-1) == _lib.LCE_ERR_SHAPE
    assert fwd(lib, X=0) == _lib.LCE_ERR_INVALID_ARG
    assert fwd(lib, mean=0) == _lib.LCE_ERR_INVALID_ARG
    assert fwd(lib, ws=0) == _lib.LCE_ERR_INVALID_ARG
    assert fwd(lib, X=FAKE + 8) == _lib.LCE_ERR_ALIGNMENT
    assert fwd(lib, y=FAKE + 4) == _lib.LCE_ERR_ALIGNMENT
    assert fwd(lib, ws=FAKE + 16) == _lib.LCE_ERR_ALIGNMENT
    assert fwd(lib, wsb=16) == _lib.LCE_ERR_WORKSPACE


def test_backward_error_paths(lib):
    assert bwd(lib, H=20) == _lib.LCE_ERR_SHAPE
    assert bwd(lib, dXt=3) == _lib.LCE_ERR_INVALID_ARG
    assert bwd(lib, dWt=-1) == _lib.LCE_ERR_INVALID_ARG
    assert bwd(lib, dW=0) == _lib.LCE_ERR_INVALID_ARG
    assert bwd(lib, lse=0) == _lib.LCE_ERR_INVALID_ARG
    assert bwd(lib, dl=0) == _lib.LCE_ERR_INVALID_ARG
    assert bwd(lib, dX=FAKE + 4) == _lib.LCE_ERR_ALIGNMENT
    assert bwd(lib, dW=FAKE + 8) == _lib.LCE_ERR_ALIGNMENT
    assert bwd(lib, wsb=255) == _lib.LCE_ERR_WORKSPACE


def opts(**kw):
    o = _lib.Options()
    _lib.load().lce_options_default(ctypes.byref(o))
    for k, v in kw.items():
        setattr(o, k, v)
    return o


def test_options_default(lib):
    o = opts()
    assert (o.ignore_index, o.softcap, o.logit_scale, o.label_smoothing, o.z_loss,
            o.reduction) == (-100, 0.0, 1.0, 0.0, 0.0, _lib.LCE_REDUCE_MEAN)


def fwd_ex(lib, o, N=4, H=8, V=5):
    wsb = lib.lce_forward_workspace_bytes(N, H, V)
    return lib.lce_forward_ex(FAKE, FAKE, FAKE, N, H, V, o, FAKE, FAKE, FAKE, FAKE, 0, FAKE,
                              wsb, None)


def bwd_ex(lib, o, N=4, H=8, V=5):
    wsb = lib.lce_backward_workspace_bytes(N, H, V, 0)
    return lib.lce_backward_ex(FAKE, FAKE, FAKE, FAKE, FAKE, N, H, V, o, FAKE, 0, FAKE, 0, FAKE,
                               wsb, None)


@pytest.mark.parametrize("bad", [dict(logit_scale=0.0), dict(logit_scale=-1.0),
                                 dict(logit_scale=float("inf")), dict(label_smoothing=1.01),
                                 dict(label_smoothing=-0.5), dict(z_loss=-1e-3),
                                 dict(z_loss=float("nan")), dict(softcap=float("nan")),
                                 dict(reduction=3), dict(reduction=-1)])
def test_ex_rejects_bad_options(lib, bad):
    o = opts(**bad)
    assert fwd_ex(lib, ctypes.byref(o)) == _lib.LCE_ERR_INVALID_ARG
    assert bwd_ex(lib, ctypes.byref(o)) == _lib.LCE_ERR_INVALID_ARG


def test_ex_null_options_and_shapes(lib):
    assert fwd_ex(lib, None) == _lib.LCE_ERR_INVALID_ARG
    assert bwd_ex(lib, None) == _lib.LCE_ERR_INVALID_ARG
    o = opts()
    assert fwd_ex(lib, ctypes.byref(o), H=12) == _lib.LCE_ERR_SHAPE
    assert bwd_ex(lib, ctypes.byref(o), V=0) == _lib.LCE_ERR_SHAPE


# Vocabulary-shard calls: argument checks that return before any launch.


def shard_fwd(lib, o, N=8, H=16, Vs=10, off=0, total=40, lse=FAKE, tgt=FAKE, zs=None):
    return lib.lce_shard_forward(FAKE, FAKE, FAKE, N, H, Vs, off, total, o, lse, tgt, zs,
                                 FAKE, 1 << 20, None)


def shard_bwd(lib, o, N=8, H=16, Vs=10, off=0, total=40):
    return lib.lce_shard_backward(FAKE, FAKE, FAKE, FAKE, FAKE, N, H, Vs, off, total, o, FAKE,
                                  _lib.LCE_F32, FAKE, _lib.LCE_F32, FAKE, 1 << 30, None)


def shard_merge(lib, o, g=2, N=8, total=40, zs=None):
    return lib.lce_shard_merge(FAKE, FAKE, zs, g, FAKE, N, total, o, FAKE, FAKE, FAKE, FAKE,
                               FAKE, FAKE, 1 << 20, None)


@pytest.mark.parametrize("off,Vs,total", [(-1, 10, 40), (31, 10, 40), (0, 10, 9),
                                          (0, 10, 1 << 31)])
def test_shard_calls_reject_bad_vocabulary_ranges(lib, off, Vs, total):
    o = opts()
    assert shard_fwd(lib, ctypes.byref(o), Vs=Vs, off=off, total=total) == _lib.LCE_ERR_SHAPE
    assert shard_bwd(lib, ctypes.byref(o), Vs=Vs, off=off, total=total) == _lib.LCE_ERR_SHAPE


def test_shard_calls_argument_checks(lib):
    o = opts()
    assert shard_fwd(lib, None) == _lib.LCE_ERR_INVALID_ARG
    assert shard_fwd(lib, ctypes.byref(o), lse=None) == _lib.LCE_ERR_INVALID_ARG
    assert shard_fwd(lib, ctypes.byref(o), tgt=FAKE + 2) == _lib.LCE_ERR_ALIGNMENT
    assert shard_fwd(lib, ctypes.byref(o), N=0, lse=None, tgt=None) == _lib.LCE_OK
    assert shard_bwd(lib, None) == _lib.LCE_ERR_INVALID_ARG
    assert shard_merge(lib, ctypes.byref(o), g=0) == _lib.LCE_ERR_INVALID_ARG
    assert shard_merge(lib, ctypes.byref(o), total=0) == _lib.LCE_ERR_SHAPE
    smooth = opts(label_smoothing=0.1)
    assert shard_merge(lib, ctypes.byref(smooth)) == _lib.LCE_ERR_INVALID_ARG   # no Σz parts
    assert lib.lce_shard_merge_workspace_bytes(-1) == 0
    assert lib.lce_shard_merge_workspace_bytes(1 << 20) >= 4096 * 24


# Fused forward + backward: argument checks that return before any launch.
def fused(lib, o, N=8, H=16, V=40, dW=_lib.LCE_F32):
    wsb = lib.lce_fused_workspace_bytes(N, H, V, dW)
    return lib.lce_forward_backward(FAKE, FAKE, FAKE, FAKE, N, H, V, o, FAKE, FAKE, FAKE, FAKE, 0,
                                    FAKE, _lib.LCE_F32, FAKE, dW, FAKE, max(wsb, 256), None)


def test_fused_argument_checks(lib):
    o = opts()
    assert fused(lib, None) == _lib.LCE_ERR_INVALID_ARG
    assert fused(lib, ctypes.byref(o), H=12) == _lib.LCE_ERR_SHAPE
    assert fused(lib, ctypes.byref(o), V=(1 << 21) + 1) == _lib.LCE_ERR_SHAPE
    assert fused(lib, ctypes.byref(o), dW=7) == _lib.LCE_ERR_INVALID_ARG
    both = opts(softcap=30.0, label_smoothing=0.1)
    assert fused(lib, ctypes.byref(both)) == _lib.LCE_ERR_INVALID_ARG
    assert lib.lce_fused_workspace_bytes(8, 12, 40, 0) == 0
    assert lib.lce_fused_workspace_bytes(8, 16, (1 << 21) + 1, 0) == 0


@pytest.mark.parametrize("N,H,V", [(8192, 2304, 256128), (8192, 4096, 128256),
                                   (32768, 3584, 152064), (16384, 4096, 32000)])
def test_fused_workspace_is_one_logits_block(lib, N, H, V):
    # One bf16 block of at most 2H rows and at most half the rows by V
    # columns (at most twice the size of W), dX partials and O(N) row data:
    # below the N x V logits.
    ws = lib.lce_fused_workspace_bytes(N, H, V, _lib.LCE_F32)
    extra = 16 * 4 * H * H + 64 * N + (64 << 20)
    assert 0 < ws < N * V * 2
    assert ws <= 2 * (2 * H) * V + extra
    assert ws <= (N // 2) * V * 2 + extra


def test_filter_option_checks(lib):
    for bad in (dict(filter_eps=-1e-3), dict(filter_eps=float("nan")), dict(filter_eps=float("inf"))):
        o = opts(**bad)
        assert fwd_ex(lib, ctypes.byref(o)) == _lib.LCE_ERR_INVALID_ARG
        assert bwd_ex(lib, ctypes.byref(o)) == _lib.LCE_ERR_INVALID_ARG
    both = opts(filter_eps=2.0 ** -12, label_smoothing=0.1)
    assert bwd_ex(lib, ctypes.byref(both)) == _lib.LCE_ERR_INVALID_ARG
    assert fused(lib, ctypes.byref(opts(filter_eps=2.0 ** -12))) == _lib.LCE_ERR_INVALID_ARG
    assert opts().filter_eps == 0.0


def test_precise_option_checks(lib):
    assert opts().precise == 0
    for bad in (2, -1):
        o = opts(precise=bad)
        assert fwd_ex(lib, ctypes.byref(o)) == _lib.LCE_ERR_INVALID_ARG
        assert bwd_ex(lib, ctypes.byref(o)) == _lib.LCE_ERR_INVALID_ARG
    # Not with the gradient filter, and not in the fused call.
    both = opts(precise=1, filter_eps=2.0 ** -12)
    assert bwd_ex(lib, ctypes.byref(both)) == _lib.LCE_ERR_INVALID_ARG
    assert fused(lib, ctypes.byref(opts(precise=1))) == _lib.LCE_ERR_INVALID_ARG
    # The workspace the query returns holds the two-part chunk too: the
    # precise backward gets past its workspace check and stops at the device
    # (no GPU here), like the plain one.
    o = opts(precise=1)
    assert bwd_ex(lib, ctypes.byref(o)) == bwd_ex(lib, ctypes.byref(opts()))


def order_call(lib, X=FAKE, W=FAKE, y=FAKE, N=4, H=8, V=5, mean=FAKE, order=FAKE, ws=FAKE,
               wsb=None):
    if wsb is None:
        wsb = lib.lce_vocab_order_workspace_bytes(max(N, 0), H, V)
    return lib.lce_vocab_order(X, W, y, N, H, V, -100, mean, order, ws, wsb, None)


def sorted_bwd(lib, o, X=FAKE, W=FAKE, y=FAKE, lse=FAKE, dl=FAKE, N=4, H=8, V=5, order=FAKE,
               dX=FAKE, dXt=0, dW=FAKE, dWt=0, ws=FAKE, wsb=None):
    if wsb is None:
        wsb = lib.lce_backward_sorted_workspace_bytes(max(N, 0), H, V, dWt if dWt in (0, 1) else 0)
    return lib.lce_backward_sorted(X, W, y, lse, dl, N, H, V, o, order, dX, dXt, dW, dWt, ws, wsb,
                                   None)


def test_vocab_order_workspace_and_argument_checks(lib):
    assert lib.lce_vocab_order_workspace_bytes(256, 64, 1000) > 0
    assert lib.lce_vocab_order_workspace_bytes(256, 12, 1000) == 0
    assert lib.lce_vocab_order_workspace_bytes(256, 64, 0) == 0
    # Sort buffers for V keys plus O(N·H / 256 + V) floats: far below W itself.
    N, H, V = 8192, 2304, 256128
    assert lib.lce_vocab_order_workspace_bytes(N, H, V) < 32 * V + 4 * (N // 256 + 2) * H + 8192
    assert order_call(lib, H=12) == _lib.LCE_ERR_SHAPE
    assert order_call(lib, V=0) == _lib.LCE_ERR_SHAPE
    assert order_call(lib, W=0) == _lib.LCE_ERR_INVALID_ARG
    assert order_call(lib, order=0) == _lib.LCE_ERR_INVALID_ARG
    assert order_call(lib, X=0) == _lib.LCE_ERR_INVALID_ARG
    assert order_call(lib, y=0) == _lib.LCE_ERR_INVALID_ARG
    assert order_call(lib, ws=0) == _lib.LCE_ERR_INVALID_ARG
    assert order_call(lib, X=FAKE + 8) == _lib.LCE_ERR_ALIGNMENT
    assert order_call(lib, y=FAKE + 4) == _lib.LCE_ERR_ALIGNMENT
    assert order_call(lib, order=FAKE + 2) == _lib.LCE_ERR_ALIGNMENT
    assert order_call(lib, mean=FAKE + 2) == _lib.LCE_ERR_ALIGNMENT
    assert order_call(lib, ws=FAKE + 16) == _lib.LCE_ERR_ALIGNMENT
    assert order_call(lib, wsb=16) == _lib.LCE_ERR_WORKSPACE


def test_sorted_backward_workspace_and_argument_checks(lib):
    for (N, H, V) in [(256, 64, 1000), (8192, 2304, 256128), (32768, 3584, 152064)]:
        for dt in (0, 1):
            plain = lib.lce_backward_workspace_bytes(N, H, V, dt)
            ws = lib.lce_backward_sorted_workspace_bytes(N, H, V, dt)
            # + one chunk (at most V rounded up to 256 rows) of bf16 W rows and
            # of fp32 dW rows, + O(N + V)
            v256 = -(-V // 256) * 256
            assert plain < ws <= plain + 6 * H * v256 + 4 * (N + V) + 4096
    assert lib.lce_backward_sorted_workspace_bytes(8, 12, 40, 0) == 0
    assert lib.lce_backward_sorted_workspace_bytes(8, 16, 40, 5) == 0
    o = opts()
    ok = ctypes.byref(o)
    assert sorted_bwd(lib, ok, H=12) == _lib.LCE_ERR_SHAPE
    assert sorted_bwd(lib, ok, order=0) == _lib.LCE_ERR_INVALID_ARG
    assert sorted_bwd(lib, ok, order=FAKE + 2) == _lib.LCE_ERR_ALIGNMENT
    assert sorted_bwd(lib, None) == _lib.LCE_ERR_INVALID_ARG
    assert sorted_bwd(lib, ok, dW=0) == _lib.LCE_ERR_INVALID_ARG
    assert sorted_bwd(lib, ok, dXt=4) == _lib.LCE_ERR_INVALID_ARG
    assert sorted_bwd(lib, ok, X=FAKE + 8) == _lib.LCE_ERR_ALIGNMENT
    both = opts(filter_eps=2.0 ** -12, label_smoothing=0.1)
    assert sorted_bwd(lib, ctypes.byref(both)) == _lib.LCE_ERR_INVALID_ARG
    # A workspace below what the sorted backward needs (its chunk buffers) is
    # refused before any launch.
    assert sorted_bwd(lib, ok, wsb=lib.lce_backward_sorted_workspace_bytes(4, 8, 5, 0) // 4) == \
        _lib.LCE_ERR_WORKSPACE


def test_forward_noalloc_host_checks(lib):
    """The no-allocation forward refuses bad arguments, and a shape whose
    workspace exceeds its fixed scratch, before any HIP call."""
    cap = lib.lce_forward_noalloc_max_bytes()
    assert cap == 64 << 20

    def na(X=FAKE, W=FAKE, y=FAKE, N=4, H=8, V=5, loss=FAKE, lse=FAKE, mean=FAKE, nv=FAKE):
        return lib.lce_forward_noalloc(X, W, y, N, H, V, -100, 0.0, loss, lse, mean, nv, None,
                                       None)

    assert na(H=12) == _lib.LCE_ERR_SHAPE
    assert na(X=0) == _lib.LCE_ERR_INVALID_ARG
    assert na(mean=0) == _lib.LCE_ERR_INVALID_ARG
    assert na(X=FAKE + 8) == _lib.LCE_ERR_ALIGNMENT
    big = 1 << 22
    assert lib.lce_forward_workspace_bytes(big, 8, 5) > cap
    assert na(N=big) == _lib.LCE_ERR_SCRATCH_LIMIT
    # The largest shapes of the benchmark workloads fit.
    for (N, H, V) in [(8192, 2304, 256128), (32768, 3584, 152064), (16384, 4096, 32000)]:
        assert lib.lce_forward_workspace_bytes(N, H, V) <= cap


def test_device_info_argument_checks(lib):
    """lce_device_info refuses NULL outputs before asking the runtime."""
    c = ctypes.c_int32(0)
    assert lib.lce_device_info(-1, None, ctypes.byref(c), None, 0) == _lib.LCE_ERR_INVALID_ARG
    assert lib.lce_device_info(-1, ctypes.byref(c), None, None, 0) == _lib.LCE_ERR_INVALID_ARG
