"""ctypes binding of liblce.so (argument marshalling only).

Every step of the computation runs in the HIP kernels behind the C ABI of
include/lce.h; this module only checks tensors, allocates outputs and the
workspace with torch, and passes raw device pointers and the current HIP
stream.  There is no fallback: if the library is not built, importing the
binding's entry points raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblce.so")

LCE_OK = 0
LCE_ERR_INVALID_ARG = 1
LCE_ERR_SHAPE = 2
LCE_ERR_ALIGNMENT = 3
LCE_ERR_WORKSPACE = 4
LCE_ERR_HIP = 5
LCE_ERR_SCRATCH_LIMIT = 6
LCE_F32 = 0
LCE_BF16 = 1
LCE_REDUCE_MEAN = 0
LCE_REDUCE_SUM = 1
LCE_REDUCE_NONE = 2
REDUCTIONS = {"mean": LCE_REDUCE_MEAN, "sum": LCE_REDUCE_SUM, "none": LCE_REDUCE_NONE}

# Every symbol include/lce.h declares.
EXPORTED = ("lce_forward_workspace_bytes", "lce_backward_workspace_bytes", "lce_forward",
            "lce_backward", "lce_options_default", "lce_forward_ex", "lce_backward_ex",
            "lce_shard_forward", "lce_shard_merge_workspace_bytes", "lce_shard_merge",
            "lce_shard_backward", "lce_fused_workspace_bytes", "lce_forward_backward",
            "lce_vocab_order_workspace_bytes", "lce_vocab_order",
            "lce_backward_sorted_workspace_bytes", "lce_backward_sorted",
            "lce_forward_noalloc_max_bytes", "lce_forward_noalloc", "lce_device_info",
            "lce_backward_plan", "lce_fused_plan",
            "lce_status_string",
            "lce_version", "lce_timing_enable", "lce_timing_reset", "lce_timing_read")


class Options(ctypes.Structure):
    """lce_options (include/lce.h)."""
    _fields_ = [("ignore_index", ctypes.c_int64), ("softcap", ctypes.c_float),
                ("logit_scale", ctypes.c_float), ("label_smoothing", ctypes.c_float),
                ("z_loss", ctypes.c_float), ("reduction", ctypes.c_int32),
                ("filter_eps", ctypes.c_float), ("precise", ctypes.c_int32)]


def make_options(ignore_index: int = -100, softcap: float = 0.0, logit_scale: float = 1.0,
                 label_smoothing: float = 0.0, z_loss: float = 0.0,
                 reduction: str = "mean", filter_eps: float = 0.0,
                 precise: bool = False) -> Options:
    if reduction not in REDUCTIONS:
        raise ValueError(f"reduction must be one of {sorted(REDUCTIONS)}, got {reduction!r}")
    return Options(int(ignore_index), float(softcap), float(logit_scale),
                   float(label_smoothing), float(z_loss), REDUCTIONS[reduction],
                   float(filter_eps), int(bool(precise)))


class KernelTiming(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int64),
                ("total_ms", ctypes.c_double)]

_lib = None


class LceError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: status {status} ({status_string(status)})")
        self.status = status


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load liblce.so and declare its signatures (raises if it is not built).
    The environment variable LCE_LIB selects another build of the library
    (the checking builds of build.py)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or os.environ.get("LCE_LIB") or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"liblce.so is not built ({p}); run "
                           "`python -m linear_cross_entropy_lse_amd.build`")
    lib = ctypes.CDLL(p)
    i64, vp, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    lib.lce_forward_workspace_bytes.argtypes = [i64, i64, i64]
    lib.lce_forward_workspace_bytes.restype = sz
    lib.lce_backward_workspace_bytes.argtypes = [i64, i64, i64, ctypes.c_int]
    lib.lce_backward_workspace_bytes.restype = sz
    lib.lce_forward.argtypes = [vp, vp, vp, i64, i64, i64, i64, ctypes.c_float,
                                vp, vp, vp, vp, vp, vp, sz, vp]
    lib.lce_forward.restype = ctypes.c_int
    lib.lce_backward.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_float,
                                 vp, ctypes.c_int, vp, ctypes.c_int, vp, sz, vp]
    lib.lce_backward.restype = ctypes.c_int
    opt_p = ctypes.POINTER(Options)
    lib.lce_options_default.argtypes = [opt_p]
    lib.lce_options_default.restype = None
    lib.lce_forward_ex.argtypes = [vp, vp, vp, i64, i64, i64, opt_p, vp, vp, vp, vp, vp, vp,
                                   sz, vp]
    lib.lce_forward_ex.restype = ctypes.c_int
    lib.lce_backward_ex.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, opt_p, vp, ctypes.c_int,
                                    vp, ctypes.c_int, vp, sz, vp]
    lib.lce_backward_ex.restype = ctypes.c_int
    lib.lce_shard_forward.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, opt_p, vp, vp, vp,
                                      vp, sz, vp]
    lib.lce_shard_forward.restype = ctypes.c_int
    lib.lce_shard_merge_workspace_bytes.argtypes = [i64]
    lib.lce_shard_merge_workspace_bytes.restype = sz
    lib.lce_shard_merge.argtypes = [vp, vp, vp, ctypes.c_int32, vp, i64, i64, opt_p, vp, vp, vp,
                                    vp, vp, vp, sz, vp]
    lib.lce_shard_merge.restype = ctypes.c_int
    lib.lce_shard_backward.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, opt_p, vp,
                                       ctypes.c_int, vp, ctypes.c_int, vp, sz, vp]
    lib.lce_shard_backward.restype = ctypes.c_int
    lib.lce_fused_workspace_bytes.argtypes = [i64, i64, i64, ctypes.c_int]
    lib.lce_fused_workspace_bytes.restype = sz
    lib.lce_forward_backward.argtypes = [vp, vp, vp, vp, i64, i64, i64, opt_p, vp, vp, vp, vp, vp,
                                         vp, ctypes.c_int, vp, ctypes.c_int, vp, sz, vp]
    lib.lce_forward_backward.restype = ctypes.c_int
    lib.lce_vocab_order_workspace_bytes.argtypes = [i64, i64, i64]
    lib.lce_vocab_order_workspace_bytes.restype = sz
    lib.lce_vocab_order.argtypes = [vp, vp, vp, i64, i64, i64, i64, vp, vp, vp, sz, vp]
    lib.lce_vocab_order.restype = ctypes.c_int
    lib.lce_backward_sorted_workspace_bytes.argtypes = [i64, i64, i64, ctypes.c_int]
    lib.lce_backward_sorted_workspace_bytes.restype = sz
    lib.lce_backward_sorted.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, opt_p, vp, vp,
                                        ctypes.c_int, vp, ctypes.c_int, vp, sz, vp]
    lib.lce_backward_sorted.restype = ctypes.c_int
    lib.lce_forward_noalloc_max_bytes.argtypes = []
    lib.lce_forward_noalloc_max_bytes.restype = sz
    lib.lce_forward_noalloc.argtypes = [vp, vp, vp, i64, i64, i64, i64, ctypes.c_float,
                                        vp, vp, vp, vp, vp, vp]
    lib.lce_forward_noalloc.restype = ctypes.c_int
    lib.lce_device_info.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_int32),
                                    ctypes.POINTER(ctypes.c_int32), ctypes.c_char_p,
                                    ctypes.c_int32]
    lib.lce_device_info.restype = ctypes.c_int
    lib.lce_backward_plan.argtypes = [i64, i64, i64, ctypes.c_int32, ctypes.POINTER(ctypes.c_int64),
                                      ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
    lib.lce_backward_plan.restype = ctypes.c_int
    lib.lce_fused_plan.argtypes = [i64, i64, i64, ctypes.POINTER(ctypes.c_int64),
                                   ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
    lib.lce_fused_plan.restype = ctypes.c_int
    lib.lce_status_string.argtypes = [ctypes.c_int]
    lib.lce_status_string.restype = ctypes.c_char_p
    lib.lce_version.argtypes = []
    lib.lce_version.restype = ctypes.c_int
    lib.lce_timing_enable.argtypes = [ctypes.c_int]
    lib.lce_timing_enable.restype = None
    lib.lce_timing_reset.argtypes = []
    lib.lce_timing_reset.restype = None
    lib.lce_timing_read.argtypes = [ctypes.POINTER(KernelTiming), ctypes.c_int]
    lib.lce_timing_read.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().lce_status_string(int(status)).decode()


def lce_version() -> int:
    return int(load().lce_version())


def lce_device_info(device: int = -1) -> dict:
    """Compute units, peak shader clock (kHz) and architecture of a device."""
    cus, clk = ctypes.c_int32(0), ctypes.c_int32(0)
    arch = ctypes.create_string_buffer(64)
    _check(load().lce_device_info(int(device), ctypes.byref(cus), ctypes.byref(clk), arch, 64),
           "lce_device_info")
    return {"cu_count": cus.value, "clock_khz": clk.value, "arch": arch.value.decode()}


def lce_backward_plan(N: int, H: int, V: int, precise: bool = False) -> dict:
    """The backward's chunking (include/lce.h): chunk_columns, n_chunks, dx_parts."""
    cols, nch, parts = ctypes.c_int64(0), ctypes.c_int32(0), ctypes.c_int32(0)
    _check(load().lce_backward_plan(int(N), int(H), int(V), 1 if precise else 0, ctypes.byref(cols),
                                    ctypes.byref(nch), ctypes.byref(parts)), "lce_backward_plan")
    return {"chunk_columns": cols.value, "n_chunks": nch.value, "dx_parts": parts.value}


def lce_fused_plan(N: int, H: int, V: int) -> dict:
    """The fused call's row chunking (include/lce.h): chunk_rows, n_chunks, dx_parts."""
    rows, nch, parts = ctypes.c_int64(0), ctypes.c_int32(0), ctypes.c_int32(0)
    _check(load().lce_fused_plan(int(N), int(H), int(V), ctypes.byref(rows), ctypes.byref(nch),
                                 ctypes.byref(parts)), "lce_fused_plan")
    return {"chunk_rows": rows.value, "n_chunks": nch.value, "dx_parts": parts.value}


def lce_timing_enable(enable: bool = True) -> None:
    load().lce_timing_enable(1 if enable else 0)


def lce_timing_reset() -> None:
    load().lce_timing_reset()


def lce_timing_read() -> dict:
    """{kernel name: (launches, total_ms)} since the last reset (waits for the
    recorded events)."""
    lib = load()
    n = lib.lce_timing_read(None, 0)
    if n < 0:
        raise RuntimeError("lce_timing_read: HIP event error")
    buf = (KernelTiming * max(n, 1))()
    n = lib.lce_timing_read(buf, n)
    if n < 0:
        raise RuntimeError("lce_timing_read: HIP event error")
    return {buf[i].name.decode(): (int(buf[i].launches), float(buf[i].total_ms))
            for i in range(n)}


def lce_forward_workspace_bytes(N: int, H: int, V: int) -> int:
    return int(load().lce_forward_workspace_bytes(N, H, V))


def lce_backward_workspace_bytes(N: int, H: int, V: int, dW_dtype=None) -> int:
    return int(load().lce_backward_workspace_bytes(N, H, V, _dtype_code(dW_dtype)))


def _dtype_code(dtype) -> int:
    import torch
    if dtype is None or dtype == torch.float32:
        return LCE_F32
    if dtype == torch.bfloat16:
        return LCE_BF16
    raise ValueError(f"gradient dtype must be float32 or bfloat16, got {dtype}")


def _check(status: int, where: str):
    if status != LCE_OK:
        raise LceError(status, where)


def _ptr(t) -> int:
    return int(t.data_ptr()) if t is not None and t.numel() > 0 else 0


def _prep(X, W, labels):
    import torch
    if not (X.is_cuda and W.is_cuda and labels.is_cuda):
        raise ValueError("X, W and labels must be device (HIP) tensors")
    if X.dtype != torch.bfloat16 or W.dtype != torch.bfloat16:
        raise ValueError("X and W must be bfloat16")
    if labels.dtype != torch.int64:
        raise ValueError("labels must be int64")
    if X.dim() != 2 or W.dim() != 2 or labels.dim() != 1:
        raise ValueError("expected X [N, H], W [V, H], labels [N]")
    if X.shape[1] != W.shape[1] or labels.shape[0] != X.shape[0]:
        raise ValueError(f"shape mismatch: X {tuple(X.shape)}, W {tuple(W.shape)}, "
                         f"labels {tuple(labels.shape)}")
    # Kernels address memory directly: non-contiguous views would be read wrong.
    return X.contiguous(), W.contiguous(), labels.contiguous()


def _stream(dev) -> int:
    import torch
    return int(torch.cuda.current_stream(dev).cuda_stream)


def lce_forward(X, W, labels, ignore_index: int = -100, softcap: float = 0.0,
                workspace=None):
    """Forward of the fused linear cross-entropy on the current HIP stream.

    Returns a dict of device tensors: loss [N] f32, lse [N] f32, mean [] f32,
    n_valid [] i32, bad_label [] i32.
    """
    import torch
    X, W, labels = _prep(X, W, labels)
    N, H = X.shape
    V = W.shape[0]
    dev = X.device
    loss = torch.empty(N, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    mean = torch.empty((), dtype=torch.float32, device=dev)
    n_valid = torch.empty((), dtype=torch.int32, device=dev)
    bad = torch.empty((), dtype=torch.int32, device=dev)
    need = lce_forward_workspace_bytes(N, H, V)
    if need == 0:
        _check(LCE_ERR_SHAPE, "lce_forward")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    st = load().lce_forward(_ptr(X), _ptr(W), _ptr(labels), N, H, V, int(ignore_index),
                            float(softcap), _ptr(loss), _ptr(lse), mean.data_ptr(),
                            n_valid.data_ptr(), bad.data_ptr(), _ptr(workspace),
                            workspace.numel(), _stream(dev))
    _check(st, "lce_forward")
    return {"loss": loss, "lse": lse, "mean": mean, "n_valid": n_valid, "bad_label": bad}


def lce_backward(X, W, labels, lse, dloss, ignore_index: int = -100, softcap: float = 0.0,
                 dX_dtype=None, dW_dtype=None, workspace=None):
    """Backward of the mean loss; `dloss` is a device scalar (or a float).
    Returns (dX [N, H], dW [V, H]) in the requested dtypes (float32 default)."""
    import torch
    X, W, labels = _prep(X, W, labels)
    N, H = X.shape
    V = W.shape[0]
    dev = X.device
    if not torch.is_tensor(dloss):
        dloss = torch.tensor(float(dloss), dtype=torch.float32, device=dev)
    dloss = dloss.to(device=dev, dtype=torch.float32).reshape(1).contiguous()
    lse = lse.to(device=dev, dtype=torch.float32).contiguous()
    if lse.shape != (N,):
        raise ValueError("lse must have shape [N]")
    dXc, dWc = _dtype_code(dX_dtype), _dtype_code(dW_dtype)
    dX = torch.empty(N, H, dtype=dX_dtype or torch.float32, device=dev)
    dW = torch.empty(V, H, dtype=dW_dtype or torch.float32, device=dev)
    need = lce_backward_workspace_bytes(N, H, V, dW_dtype)
    if need == 0:
        _check(LCE_ERR_SHAPE, "lce_backward")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    st = load().lce_backward(_ptr(X), _ptr(W), _ptr(labels), _ptr(lse), dloss.data_ptr(),
                             N, H, V, int(ignore_index), float(softcap), _ptr(dX), dXc,
                             dW.data_ptr(), dWc, _ptr(workspace), workspace.numel(),
                             _stream(dev))
    _check(st, "lce_backward")
    return dX, dW


def lce_forward_ex(X, W, labels, ignore_index: int = -100, softcap: float = 0.0,
                   logit_scale: float = 1.0, label_smoothing: float = 0.0, z_loss: float = 0.0,
                   reduction: str = "mean", workspace=None):
    """Forward with the loss variants of include/lce.h (logit scale, label
    smoothing, Z-loss, reduction).  Returns a dict of device tensors: loss [N],
    lse [N], reduced [] (mean or sum of the row losses), n_valid [], bad_label []."""
    import torch
    opt = make_options(ignore_index, softcap, logit_scale, label_smoothing, z_loss, reduction)
    X, W, labels = _prep(X, W, labels)
    N, H = X.shape
    V = W.shape[0]
    dev = X.device
    loss = torch.empty(N, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    reduced = torch.empty((), dtype=torch.float32, device=dev)
    n_valid = torch.empty((), dtype=torch.int32, device=dev)
    bad = torch.empty((), dtype=torch.int32, device=dev)
    need = lce_forward_workspace_bytes(N, H, V)
    if need == 0:
        _check(LCE_ERR_SHAPE, "lce_forward_ex")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    st = load().lce_forward_ex(_ptr(X), _ptr(W), _ptr(labels), N, H, V, ctypes.byref(opt),
                               _ptr(loss), _ptr(lse), reduced.data_ptr(), n_valid.data_ptr(),
                               bad.data_ptr(), _ptr(workspace), workspace.numel(), _stream(dev))
    _check(st, "lce_forward_ex")
    return {"loss": loss, "lse": lse, "reduced": reduced, "n_valid": n_valid, "bad_label": bad}


def lce_backward_ex(X, W, labels, lse, dloss, ignore_index: int = -100, softcap: float = 0.0,
                    logit_scale: float = 1.0, label_smoothing: float = 0.0, z_loss: float = 0.0,
                    reduction: str = "mean", dX_dtype=None, dW_dtype=None, workspace=None,
                    filter_eps: float = 0.0, precise: bool = False):
    """Backward with the loss variants.  `dloss`: a scalar (mean, sum) or an
    [N] tensor of per-row upstream gradients (none).  filter_eps > 0 turns on
    the (non-exact) gradient filter; precise=True carries the gradient chunk
    as two bf16 parts (twice the contraction work).  Returns (dX, dW)."""
    opt = make_options(ignore_index, softcap, logit_scale, label_smoothing, z_loss, reduction,
                       filter_eps, precise)
    return _backward_with_options(X, W, labels, lse, dloss, opt, reduction, dX_dtype, dW_dtype,
                                  workspace, None)


def lce_backward_sorted(X, W, labels, lse, dloss, order, ignore_index: int = -100,
                        softcap: float = 0.0, logit_scale: float = 1.0,
                        label_smoothing: float = 0.0, z_loss: float = 0.0,
                        reduction: str = "mean", dX_dtype=None, dW_dtype=None, workspace=None,
                        filter_eps: float = 0.0, precise: bool = False):
    """lce_backward_ex on the vocabulary reordered by `order` (an int32 device
    permutation of [0, V), e.g. from lce_vocab_order); dW rows come back in
    entry order.  Returns (dX, dW)."""
    import torch
    opt = make_options(ignore_index, softcap, logit_scale, label_smoothing, z_loss, reduction,
                       filter_eps, precise)
    if not (torch.is_tensor(order) and order.is_cuda and order.dtype == torch.int32
            and order.dim() == 1 and order.shape[0] == W.shape[0]):
        raise ValueError("order must be an int32 device tensor of shape [V]")
    return _backward_with_options(X, W, labels, lse, dloss, opt, reduction, dX_dtype, dW_dtype,
                                  workspace, order.contiguous())


def lce_vocab_order(X, W, labels, ignore_index: int = -100, workspace=None):
    """Average logit of every vocabulary entry over the rows with a target, and
    the entries by decreasing average (ties by index).  Returns (mean_logit [V]
    f32, order [V] i32), device tensors."""
    import torch
    X, W, labels = _prep(X, W, labels)
    N, H = X.shape
    V = W.shape[0]
    dev = X.device
    mean_logit = torch.empty(V, dtype=torch.float32, device=dev)
    order = torch.empty(V, dtype=torch.int32, device=dev)
    need = int(load().lce_vocab_order_workspace_bytes(N, H, V))
    if need == 0:
        _check(LCE_ERR_SHAPE, "lce_vocab_order")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    st = load().lce_vocab_order(_ptr(X), _ptr(W), _ptr(labels), N, H, V, int(ignore_index),
                                mean_logit.data_ptr(), order.data_ptr(), _ptr(workspace),
                                workspace.numel(), _stream(dev))
    _check(st, "lce_vocab_order")
    return mean_logit, order


def _backward_with_options(X, W, labels, lse, dloss, opt, reduction, dX_dtype, dW_dtype,
                           workspace, order):
    import torch
    where = "lce_backward_sorted" if order is not None else "lce_backward_ex"
    X, W, labels = _prep(X, W, labels)
    N, H = X.shape
    V = W.shape[0]
    dev = X.device
    n_d = N if reduction == "none" else 1
    if not torch.is_tensor(dloss):
        dloss = torch.full((n_d,), float(dloss), dtype=torch.float32, device=dev)
    dloss = dloss.to(device=dev, dtype=torch.float32).reshape(-1).contiguous()
    if dloss.numel() != n_d:
        raise ValueError(f"dloss must hold {n_d} value(s) for reduction {reduction!r}")
    if n_d == 0:
        dloss = torch.zeros(1, dtype=torch.float32, device=dev)
    lse = lse.to(device=dev, dtype=torch.float32).contiguous()
    if lse.shape != (N,):
        raise ValueError("lse must have shape [N]")
    dXc, dWc = _dtype_code(dX_dtype), _dtype_code(dW_dtype)
    dX = torch.empty(N, H, dtype=dX_dtype or torch.float32, device=dev)
    dW = torch.empty(V, H, dtype=dW_dtype or torch.float32, device=dev)
    if order is None:
        need = lce_backward_workspace_bytes(N, H, V, dW_dtype)
    else:
        need = int(load().lce_backward_sorted_workspace_bytes(N, H, V, dWc))
    if need == 0:
        _check(LCE_ERR_SHAPE, where)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if order is None:
        st = load().lce_backward_ex(_ptr(X), _ptr(W), _ptr(labels), _ptr(lse), dloss.data_ptr(),
                                    N, H, V, ctypes.byref(opt), _ptr(dX), dXc, dW.data_ptr(),
                                    dWc, _ptr(workspace), workspace.numel(), _stream(dev))
    else:
        st = load().lce_backward_sorted(_ptr(X), _ptr(W), _ptr(labels), _ptr(lse),
                                        dloss.data_ptr(), N, H, V, ctypes.byref(opt),
                                        order.data_ptr(), _ptr(dX), dXc, dW.data_ptr(), dWc,
                                        _ptr(workspace), workspace.numel(), _stream(dev))
    _check(st, where)
    return dX, dW



# --------------------------------------------------------------------------- #
# Vocabulary shards
# --------------------------------------------------------------------------- #
def lce_shard_forward(X, W_shard, labels, vocab_offset: int, vocab_total: int,
                      ignore_index: int = -100, softcap: float = 0.0, logit_scale: float = 1.0,
                      with_zsum: bool = False, workspace=None):
    """Per-row partials of the vocabulary shard W_shard = rows [vocab_offset,
    vocab_offset + V_shard) of a vocabulary of vocab_total rows.  Returns a
    dict of [N] device tensors: lse_part, target_part and (with_zsum) zsum_part."""
    import torch
    opt = make_options(ignore_index, softcap, logit_scale)
    X, W_shard, labels = _prep(X, W_shard, labels)
    N, H = X.shape
    Vs = W_shard.shape[0]
    dev = X.device
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    tgt = torch.empty(N, dtype=torch.float32, device=dev)
    zs = torch.empty(N, dtype=torch.float32, device=dev) if with_zsum else None
    need = lce_forward_workspace_bytes(N, H, Vs)
    if need == 0:
        _check(LCE_ERR_SHAPE, "lce_shard_forward")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    st = load().lce_shard_forward(_ptr(X), _ptr(W_shard), _ptr(labels), N, H, Vs,
                                  int(vocab_offset), int(vocab_total), ctypes.byref(opt),
                                  _ptr(lse), _ptr(tgt), _ptr(zs) if zs is not None else None,
                                  _ptr(workspace), workspace.numel(), _stream(dev))
    _check(st, "lce_shard_forward")
    out = {"lse_part": lse, "target_part": tgt}
    if zs is not None:
        out["zsum_part"] = zs
    return out


def lce_shard_merge(lse_parts, target_parts, labels, vocab_total: int, zsum_parts=None,
                    ignore_index: int = -100, label_smoothing: float = 0.0, z_loss: float = 0.0,
                    reduction: str = "mean"):
    """Merge [n_shards, N] shard partials (shard order along dim 0) into the
    loss.  Returns the dict of lce_forward_ex (loss, lse, reduced, n_valid,
    bad_label)."""
    import torch
    opt = make_options(ignore_index, 0.0, 1.0, label_smoothing, z_loss, reduction)
    dev = lse_parts.device
    lse_parts = lse_parts.to(torch.float32).contiguous()
    target_parts = target_parts.to(torch.float32).contiguous()
    if zsum_parts is not None:
        zsum_parts = zsum_parts.to(torch.float32).contiguous()
    labels = labels.to(device=dev, dtype=torch.int64).contiguous()
    g, N = lse_parts.shape
    if target_parts.shape != (g, N) or labels.shape != (N,) or \
            (zsum_parts is not None and zsum_parts.shape != (g, N)):
        raise ValueError("shard partials must be [n_shards, N] and labels [N]")
    loss = torch.empty(N, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    reduced = torch.empty((), dtype=torch.float32, device=dev)
    n_valid = torch.empty((), dtype=torch.int32, device=dev)
    bad = torch.empty((), dtype=torch.int32, device=dev)
    need = load().lce_shard_merge_workspace_bytes(N)
    if need == 0:
        _check(LCE_ERR_SHAPE, "lce_shard_merge")
    workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    st = load().lce_shard_merge(_ptr(lse_parts), _ptr(target_parts),
                                _ptr(zsum_parts) if zsum_parts is not None else None, g,
                                _ptr(labels), N, int(vocab_total), ctypes.byref(opt), _ptr(loss),
                                _ptr(lse), reduced.data_ptr(), n_valid.data_ptr(), bad.data_ptr(),
                                _ptr(workspace), workspace.numel(), _stream(dev))
    _check(st, "lce_shard_merge")
    return {"loss": loss, "lse": lse, "reduced": reduced, "n_valid": n_valid, "bad_label": bad}


def lce_shard_backward(X, W_shard, labels, lse, dloss, vocab_offset: int, vocab_total: int,
                       ignore_index: int = -100, softcap: float = 0.0, logit_scale: float = 1.0,
                       label_smoothing: float = 0.0, z_loss: float = 0.0,
                       reduction: str = "mean", dX_dtype=None, dW_dtype=None, workspace=None,
                       filter_eps: float = 0.0, precise: bool = False):
    """Backward of one vocabulary shard given the merged LSE.  Returns
    (dX share [N, H], dW rows of the shard [V_shard, H])."""
    import torch
    opt = make_options(ignore_index, softcap, logit_scale, label_smoothing, z_loss, reduction,
                       filter_eps, precise)
    X, W_shard, labels = _prep(X, W_shard, labels)
    N, H = X.shape
    Vs = W_shard.shape[0]
    dev = X.device
    n_d = N if reduction == "none" else 1
    if not torch.is_tensor(dloss):
        dloss = torch.full((n_d,), float(dloss), dtype=torch.float32, device=dev)
    dloss = dloss.to(device=dev, dtype=torch.float32).reshape(-1).contiguous()
    if dloss.numel() != n_d:
        raise ValueError(f"dloss must hold {n_d} value(s) for reduction {reduction!r}")
    if n_d == 0:
        dloss = torch.zeros(1, dtype=torch.float32, device=dev)
    lse = lse.to(device=dev, dtype=torch.float32).contiguous()
    if lse.shape != (N,):
        raise ValueError("lse must have shape [N]")
    dXc, dWc = _dtype_code(dX_dtype), _dtype_code(dW_dtype)
    dX = torch.empty(N, H, dtype=dX_dtype or torch.float32, device=dev)
    dW = torch.empty(Vs, H, dtype=dW_dtype or torch.float32, device=dev)
    need = lce_backward_workspace_bytes(N, H, Vs, dW_dtype)
    if need == 0:
        _check(LCE_ERR_SHAPE, "lce_shard_backward")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    st = load().lce_shard_backward(_ptr(X), _ptr(W_shard), _ptr(labels), _ptr(lse),
                                   dloss.data_ptr(), N, H, Vs, int(vocab_offset),
                                   int(vocab_total), ctypes.byref(opt), _ptr(dX), dXc,
                                   dW.data_ptr(), dWc, _ptr(workspace), workspace.numel(),
                                   _stream(dev))
    _check(st, "lce_shard_backward")
    return dX, dW


# --------------------------------------------------------------------------- #
# Forward and backward in one row-chunked pass
# --------------------------------------------------------------------------- #
def lce_fused_workspace_bytes(N: int, H: int, V: int, dW_dtype=None) -> int:
    return int(load().lce_fused_workspace_bytes(N, H, V, _dtype_code(dW_dtype)))


def lce_forward_backward(X, W, labels, dloss=1.0, ignore_index: int = -100, softcap: float = 0.0,
                         logit_scale: float = 1.0, label_smoothing: float = 0.0,
                         z_loss: float = 0.0, reduction: str = "mean", dX_dtype=None,
                         dW_dtype=None, workspace=None):
    """Forward and backward in one call, row chunk by row chunk (include/lce.h).
    `dloss` as in lce_backward_ex.  Returns (dict of lce_forward_ex, dX, dW)."""
    import torch
    opt = make_options(ignore_index, softcap, logit_scale, label_smoothing, z_loss, reduction)
    X, W, labels = _prep(X, W, labels)
    N, H = X.shape
    V = W.shape[0]
    dev = X.device
    n_d = N if reduction == "none" else 1
    if not torch.is_tensor(dloss):
        dloss = torch.full((n_d,), float(dloss), dtype=torch.float32, device=dev)
    dloss = dloss.to(device=dev, dtype=torch.float32).reshape(-1).contiguous()
    if dloss.numel() != n_d:
        raise ValueError(f"dloss must hold {n_d} value(s) for reduction {reduction!r}")
    if n_d == 0:
        dloss = torch.zeros(1, dtype=torch.float32, device=dev)
    loss = torch.empty(N, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    reduced = torch.empty((), dtype=torch.float32, device=dev)
    n_valid = torch.empty((), dtype=torch.int32, device=dev)
    bad = torch.empty((), dtype=torch.int32, device=dev)
    dXc, dWc = _dtype_code(dX_dtype), _dtype_code(dW_dtype)
    dX = torch.empty(N, H, dtype=dX_dtype or torch.float32, device=dev)
    dW = torch.empty(V, H, dtype=dW_dtype or torch.float32, device=dev)
    need = lce_fused_workspace_bytes(N, H, V, dW_dtype)
    if need == 0:
        _check(LCE_ERR_SHAPE, "lce_forward_backward")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    st = load().lce_forward_backward(_ptr(X), _ptr(W), _ptr(labels), dloss.data_ptr(), N, H, V,
                                     ctypes.byref(opt), _ptr(loss), _ptr(lse), reduced.data_ptr(),
                                     n_valid.data_ptr(), bad.data_ptr(), _ptr(dX), dXc,
                                     dW.data_ptr(), dWc, _ptr(workspace), workspace.numel(),
                                     _stream(dev))
    _check(st, "lce_forward_backward")
    return ({"loss": loss, "lse": lse, "reduced": reduced, "n_valid": n_valid, "bad_label": bad},
            dX, dW)
