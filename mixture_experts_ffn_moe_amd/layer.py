"""Tensor-level convenience over the C ABI: allocate a layer call's output and
workspace with torch and expose the workspace's intermediates as views."""
from __future__ import annotations

import torch

from ._lib import (MOE_BF16, moe_forward, moe_forward_shared, moe_get_shared_workspace_layout,
                   moe_get_workspace_layout, moe_shared_workspace_size, moe_workspace_size, y_nbytes)


def _dtype(shape) -> torch.dtype:
    return torch.bfloat16 if shape.dtype == MOE_BF16 else torch.float32


def workspace_views(shape, ws: torch.Tensor) -> dict:
    """Views of the intermediates moe_forward leaves in workspace `ws` (uint8)."""
    L = moe_get_workspace_layout(shape)
    T, E, k, H = shape.T, shape.E, shape.k, shape.H
    R = T * k
    I = shape.micro_count * shape.Im
    dt = _dtype(shape)
    es = 2 if dt == torch.bfloat16 else 4

    def view(name, n, elem, dtype, dims):
        off = L[name]
        return ws[off:off + n * elem].view(dtype).view(*dims)

    return {
        "logits": view("logits", T * E, 4, torch.float32, (T, E)),
        "ids": view("topk_ids", R, 4, torch.int32, (T, k)),
        "w": view("topk_w", R, 4, torch.float32, (T, k)),
        "counts": view("counts", E, 4, torch.int32, (E,)),
        "offsets": view("offsets", E + 1, 4, torch.int32, (E + 1,)),
        "perm": view("perm", R, 4, torch.int32, (R,)),
        "inv": view("inv", R, 4, torch.int32, (R,)),
        "h": view("h", R * I, es, dt, (R, I)),
        # raw bytes: block-scaled half in the bf16 layers, fp32 in the fp32 layer
        "y": ws[L["y"]:L["y"] + y_nbytes(shape, R)],
    }


class MoELayerBuffers:
    """Output and workspace of one layer shape, allocated once with torch.
    With shared_Im the workspace also holds the shared expert's regions and
    forward_shared runs the layer with its shared expert."""

    def __init__(self, shape, device="cuda", shared_Im=None):
        self.shape = shape
        self.shared_Im = shared_Im
        n = moe_workspace_size(shape) if shared_Im is None else moe_shared_workspace_size(shape, shared_Im)
        if n == 0:
            raise ValueError("shape (or shared_Im) outside the library's envelope")
        self.workspace = torch.empty(n, dtype=torch.uint8, device=device)
        self.out = torch.empty(shape.T, shape.H, dtype=_dtype(shape), device=device)

    def forward(self, x, wg, bias, w1, w2, stream=None) -> torch.Tensor:
        moe_forward(self.shape, x, wg, bias, w1, w2, self.out, self.workspace, stream)
        return self.out

    def forward_shared(self, x, wg, bias, w1, w2, w1s, w2s, stream=None) -> torch.Tensor:
        if self.shared_Im is None:
            raise ValueError("buffers were allocated without shared_Im")
        moe_forward_shared(self.shape, self.shared_Im, x, wg, bias, w1, w2, w1s, w2s, self.out,
                           self.workspace, stream)
        return self.out

    def views(self) -> dict:
        v = workspace_views(self.shape, self.workspace)
        if self.shared_Im is not None:
            Ls = moe_get_shared_workspace_layout(self.shape, self.shared_Im)
            dt = _dtype(self.shape)
            es = 2 if dt == torch.bfloat16 else 4
            T, H, Is = self.shape.T, self.shape.H, self.shared_Im
            v["hs"] = self.workspace[Ls["hs"]:Ls["hs"] + T * Is * es].view(dt).view(T, Is)
            v["ys"] = self.workspace[Ls["ys"]:Ls["ys"] + y_nbytes(self.shape, T)]
        return v
