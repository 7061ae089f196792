"""Routed Mixture-of-Experts FFN layer for MI355X (gfx950).

The compute lives in libmoe_mi355x.so (hand-written HIP kernels behind a C
ABI, declared in include/moe_mi355x.h and include/moe_shared.h); this package is its ctypes binding
plus a small tensor-level helper.  PyTorch provides device memory and streams
only.
"""
from __future__ import annotations

from ._lib import (  # noqa: F401
    EXPORTED, LIB_PATH, MOE_BF16, MOE_ERR_HIP, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED,
    MOE_ERR_WORKSPACE, MOE_F32, MOE_OK, NOALLOC_SCRATCH_BYTES, MoeError, MoeShape, make_shape, moe_finalize,
    moe_finalize_shared, moe_forward, moe_forward_noalloc, moe_forward_shared, moe_get_shared_workspace_layout,
    moe_get_workspace_layout, moe_grouped_gemm_down, moe_grouped_gemm_w13_swiglu, moe_permute,
    moe_probe_mfma_bf16, moe_probe_read, moe_route, moe_shared_ffn, moe_shared_workspace_size,
    moe_workspace_size, status_string, y_nbytes,
)
from .layer import MoELayerBuffers, workspace_views  # noqa: F401
