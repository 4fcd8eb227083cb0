"""Fused LM-head linear + cross-entropy (linear-LSE) for AMD gfx950 (MI355X).

The computation lives in hand-written HIP kernels behind the C ABI of
`include/lce.h` (liblce.so, built in-tree by `linear_cross_entropy_lse_amd.build`).
This package is a thin binding with the same names, plus an autograd wrapper.
"""
from ._lib import (LCE_BF16, LCE_F32, LceError, lce_backward,  # noqa: F401
                   lce_backward_ex, lce_backward_plan, lce_backward_sorted, lce_backward_workspace_bytes,
                   lce_device_info,
                   lce_forward, lce_vocab_order,
                   lce_forward_backward, lce_forward_ex, lce_fused_plan, lce_fused_workspace_bytes,
                   lce_forward_workspace_bytes, lce_shard_backward, lce_shard_forward,
                   lce_shard_merge, lce_timing_enable, lce_timing_read, lce_timing_reset,
                   lce_version, load, make_options, status_string)
from .autograd import LinearCrossEntropy, linear_cross_entropy  # noqa: F401
