"""ctypes binding of libmoe_mi355x.so: argument marshalling only.

Each function has the name of the C entry point it calls and takes torch
tensors, which supply device memory; the current torch stream is passed as
the HIP stream.  Every step of the layer runs in the library's HIP kernels:
if the library is missing this module raises on import instead of falling
back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_mi355x.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16 = 0, 1

EXPORTED = (
    "moe_status_string", "moe_workspace_size", "moe_get_workspace_layout", "moe_route",
    "moe_permute", "moe_grouped_gemm_w13_swiglu", "moe_grouped_gemm_down", "moe_finalize",
    "moe_forward", "moe_forward_noalloc",
    # shared expert (moe_shared.h)
    "moe_shared_workspace_size", "moe_get_shared_workspace_layout", "moe_shared_ffn",
    "moe_finalize_shared", "moe_forward_shared",
    # measurement probes (moe_probe.h)
    "moe_probe_mfma_bf16", "moe_probe_mfma_flops", "moe_probe_read",
)


class MoeError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {status_string(code)}")


class MoeShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("Im", ctypes.c_int32), ("micro_count", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("renormalize", ctypes.c_int32)]


class MoeWorkspaceLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("logits", "topk_ids", "topk_w", "counts", "offsets", "perm", "inv", "h", "y",
                 "scratch", "total")]


class MoeSharedLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("hs", "ys", "total")]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run python __graft_entry__.py build")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    S = ctypes.POINTER(MoeShape)
    i32 = ctypes.c_int32
    lib.moe_status_string.argtypes = [i32]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_workspace_size.argtypes = [S]
    lib.moe_workspace_size.restype = ctypes.c_size_t
    lib.moe_get_workspace_layout.argtypes = [S, ctypes.POINTER(MoeWorkspaceLayout)]
    lib.moe_get_workspace_layout.restype = i32
    lib.moe_route.argtypes = [S, P, P, P, P, P, P, P]
    lib.moe_route.restype = i32
    lib.moe_permute.argtypes = [S, P, P, P, P, P, P, P, P]
    lib.moe_permute.restype = i32
    lib.moe_grouped_gemm_w13_swiglu.argtypes = [S, P, P, P, P, P, P]
    lib.moe_grouped_gemm_w13_swiglu.restype = i32
    lib.moe_grouped_gemm_down.argtypes = [S, P, P, P, P, P]
    lib.moe_grouped_gemm_down.restype = i32
    lib.moe_finalize.argtypes = [S, P, P, P, P, P]
    lib.moe_finalize.restype = i32
    lib.moe_forward.argtypes = [S, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.moe_forward.restype = i32
    lib.moe_forward_noalloc.argtypes = [S, P, P, P, P, P, P, P]
    lib.moe_forward_noalloc.restype = i32
    lib.moe_shared_workspace_size.argtypes = [S, i32]
    lib.moe_shared_workspace_size.restype = ctypes.c_size_t
    lib.moe_get_shared_workspace_layout.argtypes = [S, i32, ctypes.POINTER(MoeSharedLayout)]
    lib.moe_get_shared_workspace_layout.restype = i32
    lib.moe_shared_ffn.argtypes = [S, i32, P, P, P, P, P, P]
    lib.moe_shared_ffn.restype = i32
    lib.moe_finalize_shared.argtypes = [S, P, P, P, P, P, P]
    lib.moe_finalize_shared.restype = i32
    lib.moe_forward_shared.argtypes = [S, i32, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.moe_forward_shared.restype = i32
    lib.moe_probe_mfma_bf16.argtypes = [i32, P, P]
    lib.moe_probe_mfma_bf16.restype = i32
    lib.moe_probe_mfma_flops.argtypes = [i32]
    lib.moe_probe_mfma_flops.restype = ctypes.c_double
    lib.moe_probe_read.argtypes = [P, ctypes.c_size_t, P, P]
    lib.moe_probe_read.restype = i32
    return lib


lib = _load()


def status_string(code: int) -> str:
    return lib.moe_status_string(code).decode()


def make_shape(T, H, E, k, Im, micro_count=1, dtype="bf16", renormalize=True) -> MoeShape:
    d = {"bf16": MOE_BF16, "f32": MOE_F32, MOE_BF16: MOE_BF16, MOE_F32: MOE_F32}[dtype]
    return MoeShape(T, H, E, k, Im, micro_count, d, int(bool(renormalize)))


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _layer_dtype(shape) -> torch.dtype:
    return torch.bfloat16 if shape.dtype == MOE_BF16 else torch.float32


def _arg(name: str, t, dtype: torch.dtype, numel: int, nullable: bool = False):
    """Check one tensor argument against the element type and element count
    the C entry point will read or write through its raw pointer (the library
    cannot check sizes itself), then return the pointer."""
    if t is None:
        if nullable:
            return None
        raise ValueError(f"{name}: a tensor is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor (got {t.device})")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.numel() != numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected {numel} for this shape")
    return _ptr(t)


Y_BLOCK = 256  # columns per exponent of a block-scaled half y (moe_mi355x.h)


def y_nbytes(shape, rows: int) -> int:
    """Bytes of a y buffer of `rows` rows: block-scaled half (fp16 values,
    then one int8 exponent per Y_BLOCK columns) in the bf16 layers, fp32 in
    the fp32 layer."""
    H = shape.H
    if shape.dtype == MOE_BF16:
        return rows * H * 2 + rows * (-(-H // Y_BLOCK))
    return rows * H * 4


def _arg_bytes(name: str, t, nbytes: int):
    """A contiguous GPU tensor of exactly nbytes bytes (any element type)."""
    if t is None:
        raise ValueError(f"{name}: a tensor is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor (got {t.device})")
    if t.numel() * t.element_size() != nbytes:
        raise ValueError(f"{name}: {t.numel() * t.element_size()} bytes, expected {nbytes} for this shape")
    return _ptr(t)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(code: int, where: str):
    if code != MOE_OK:
        raise MoeError(code, where)


def moe_workspace_size(shape: MoeShape) -> int:
    return int(lib.moe_workspace_size(ctypes.byref(shape)))


def moe_get_workspace_layout(shape: MoeShape) -> dict:
    L = MoeWorkspaceLayout()
    _check(lib.moe_get_workspace_layout(ctypes.byref(shape), ctypes.byref(L)), "moe_get_workspace_layout")
    return {n: int(getattr(L, n)) for n, _ in MoeWorkspaceLayout._fields_}


def moe_route(shape, x, wg, bias, logits, topk_ids, topk_w, stream=None):
    T, H, E, k = shape.T, shape.H, shape.E, shape.k
    dt = _layer_dtype(shape)
    _check(lib.moe_route(ctypes.byref(shape), _arg("x", x, dt, T * H), _arg("wg", wg, torch.float32, E * H),
                         _arg("gate_bias", bias, torch.float32, E, nullable=True),
                         _arg("logits", logits, torch.float32, T * E),
                         _arg("topk_ids", topk_ids, torch.int32, T * k),
                         _arg("topk_w", topk_w, torch.float32, T * k), _stream(stream)), "moe_route")


def moe_permute(shape, topk_ids, counts, offsets, perm, inv, x=None, permuted_x=None, stream=None):
    T, H, E, k = shape.T, shape.H, shape.E, shape.k
    R = T * k
    dt = _layer_dtype(shape)
    _check(lib.moe_permute(ctypes.byref(shape), _arg("topk_ids", topk_ids, torch.int32, R),
                           _arg("counts", counts, torch.int32, E), _arg("offsets", offsets, torch.int32, E + 1),
                           _arg("perm", perm, torch.int32, R), _arg("inv", inv, torch.int32, R),
                           _arg("x", x, dt, T * H, nullable=True),
                           _arg("permuted_x", permuted_x, dt, R * H, nullable=True), _stream(stream)),
           "moe_permute")


def moe_grouped_gemm_w13_swiglu(shape, x, perm, offsets, w1, h, stream=None):
    T, H, E, k, Im, mu = shape.T, shape.H, shape.E, shape.k, shape.Im, shape.micro_count
    R = T * k
    dt = _layer_dtype(shape)
    _check(lib.moe_grouped_gemm_w13_swiglu(ctypes.byref(shape), _arg("x", x, dt, T * H),
                                           _arg("perm", perm, torch.int32, R),
                                           _arg("offsets", offsets, torch.int32, E + 1),
                                           _arg("w1", w1, dt, mu * E * 2 * Im * H),
                                           _arg("h", h, dt, R * mu * Im), _stream(stream)),
           "moe_grouped_gemm_w13_swiglu")


def moe_grouped_gemm_down(shape, h, offsets, w2, y, stream=None):
    T, H, E, k, Im, mu = shape.T, shape.H, shape.E, shape.k, shape.Im, shape.micro_count
    R = T * k
    dt = _layer_dtype(shape)
    _check(lib.moe_grouped_gemm_down(ctypes.byref(shape), _arg("h", h, dt, R * mu * Im),
                                     _arg("offsets", offsets, torch.int32, E + 1),
                                     _arg("w2", w2, dt, mu * E * H * Im), _arg_bytes("y", y, y_nbytes(shape, R)),
                                     _stream(stream)), "moe_grouped_gemm_down")


def moe_finalize(shape, y, inv, topk_w, out, stream=None):
    T, H, k = shape.T, shape.H, shape.k
    R = T * k
    dt = _layer_dtype(shape)
    _check(lib.moe_finalize(ctypes.byref(shape), _arg_bytes("y", y, y_nbytes(shape, R)),
                            _arg("inv", inv, torch.int32, R),
                            _arg("topk_w", topk_w, torch.float32, R), _arg("out", out, dt, T * H),
                            _stream(stream)), "moe_finalize")


def _workspace(workspace):
    if workspace is None:
        raise ValueError("workspace: a tensor is required")
    if not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace: must be a contiguous GPU tensor")
    return _ptr(workspace), ctypes.c_size_t(workspace.numel() * workspace.element_size())


def moe_forward(shape, x, wg, bias, w1, w2, out, workspace, stream=None):
    T, H, E, Im, mu = shape.T, shape.H, shape.E, shape.Im, shape.micro_count
    dt = _layer_dtype(shape)
    ws, nbytes = _workspace(workspace)
    _check(lib.moe_forward(ctypes.byref(shape), _arg("x", x, dt, T * H), _arg("wg", wg, torch.float32, E * H),
                           _arg("gate_bias", bias, torch.float32, E, nullable=True),
                           _arg("w1", w1, dt, mu * E * 2 * Im * H), _arg("w2", w2, dt, mu * E * H * Im),
                           _arg("out", out, dt, T * H), ws, nbytes, _stream(stream)),
           "moe_forward")


NOALLOC_SCRATCH_BYTES = 16 << 20  # MOE_NOALLOC_SCRATCH_BYTES of moe_mi355x.h


def moe_forward_noalloc(shape, x, wg, bias, w1, w2, out, stream=None):
    """moe_forward on the library's static per-GPU scratch (no workspace)."""
    T, H, E, Im, mu = shape.T, shape.H, shape.E, shape.Im, shape.micro_count
    dt = _layer_dtype(shape)
    _check(lib.moe_forward_noalloc(ctypes.byref(shape), _arg("x", x, dt, T * H),
                                   _arg("wg", wg, torch.float32, E * H),
                                   _arg("gate_bias", bias, torch.float32, E, nullable=True),
                                   _arg("w1", w1, dt, mu * E * 2 * Im * H),
                                   _arg("w2", w2, dt, mu * E * H * Im),
                                   _arg("out", out, dt, T * H), _stream(stream)),
           "moe_forward_noalloc")


def moe_shared_workspace_size(shape: MoeShape, Is: int) -> int:
    return int(lib.moe_shared_workspace_size(ctypes.byref(shape), int(Is)))


def moe_get_shared_workspace_layout(shape: MoeShape, Is: int) -> dict:
    L = MoeSharedLayout()
    _check(lib.moe_get_shared_workspace_layout(ctypes.byref(shape), int(Is), ctypes.byref(L)),
           "moe_get_shared_workspace_layout")
    return {n: int(getattr(L, n)) for n, _ in MoeSharedLayout._fields_}


def moe_shared_ffn(shape, Is, x, w1s, w2s, hs, ys, stream=None):
    T, H = shape.T, shape.H
    dt = _layer_dtype(shape)
    _check(lib.moe_shared_ffn(ctypes.byref(shape), int(Is), _arg("x", x, dt, T * H),
                              _arg("w1s", w1s, dt, 2 * Is * H), _arg("w2s", w2s, dt, H * Is),
                              _arg("hs", hs, dt, T * Is), _arg_bytes("ys", ys, y_nbytes(shape, T)),
                              _stream(stream)),
           "moe_shared_ffn")


def moe_finalize_shared(shape, y, inv, topk_w, ys, out, stream=None):
    T, H, k = shape.T, shape.H, shape.k
    R = T * k
    dt = _layer_dtype(shape)
    _check(lib.moe_finalize_shared(ctypes.byref(shape), _arg_bytes("y", y, y_nbytes(shape, R)),
                                   _arg("inv", inv, torch.int32, R),
                                   _arg("topk_w", topk_w, torch.float32, R), _arg_bytes("ys", ys, y_nbytes(shape, T)),
                                   _arg("out", out, dt, T * H), _stream(stream)), "moe_finalize_shared")


def moe_forward_shared(shape, Is, x, wg, bias, w1, w2, w1s, w2s, out, workspace, stream=None):
    T, H, E, Im, mu = shape.T, shape.H, shape.E, shape.Im, shape.micro_count
    dt = _layer_dtype(shape)
    ws, nbytes = _workspace(workspace)
    _check(lib.moe_forward_shared(ctypes.byref(shape), int(Is), _arg("x", x, dt, T * H),
                                  _arg("wg", wg, torch.float32, E * H),
                                  _arg("gate_bias", bias, torch.float32, E, nullable=True),
                                  _arg("w1", w1, dt, mu * E * 2 * Im * H), _arg("w2", w2, dt, mu * E * H * Im),
                                  _arg("w1s", w1s, dt, 2 * Is * H), _arg("w2s", w2s, dt, H * Is),
                                  _arg("out", out, dt, T * H), ws, nbytes, _stream(stream)),
           "moe_forward_shared")


def moe_probe_mfma_bf16(iterations: int, sink, stream=None) -> float:
    """Enqueue the bf16 matrix-rate probe; returns the FLOPs it performs."""
    _check(lib.moe_probe_mfma_bf16(int(iterations), _arg("sink", sink, torch.float32, 1), _stream(stream)),
           "moe_probe_mfma_bf16")
    return float(lib.moe_probe_mfma_flops(int(iterations)))


def moe_probe_read(buf, sink, stream=None) -> int:
    """Enqueue the streaming-read probe over all of `buf`; returns its bytes."""
    if not isinstance(buf, torch.Tensor) or buf.device.type != "cuda":
        raise ValueError("buf: must be a GPU tensor")
    nbytes = buf.numel() * buf.element_size()
    _check(lib.moe_probe_read(_ptr(buf), ctypes.c_size_t(nbytes), _arg("sink", sink, torch.int32, 1),
                              _stream(stream)), "moe_probe_read")
    return nbytes
