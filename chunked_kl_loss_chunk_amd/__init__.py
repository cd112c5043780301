"""Fused, chunked top-K KL distillation loss for AMD MI355X (gfx950).

The loss, its forward and its backward, and the offline teacher top-K cache
that feeds it, run in the HIP kernels of the in-tree
library ``libkdkl.so`` (C ABI: include/kd_fused_kl.h). This package only
marshals arguments; PyTorch provides device memory and streams.
"""
from ._build import LIB_PATH, build  # noqa: F401
from ._lib import KDError, lib, status_str  # noqa: F401
from .ops import (  # noqa: F401
    FusedTopKKL,
    cast_f32_to_bf16,
    check_inputs,
    fused_kl,
    kl_backward,
    kl_forward,
    kl_forward_backward,
    kl_forward_noalloc,
    scale_,
    teacher_topk,
    workspace_bytes,
)
