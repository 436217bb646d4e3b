"""ctypes binding of libgsample's C ABI (include/gsample.h).

Argument marshalling only: shapes and pointers of torch tensors are passed to
the library; every step of the computation runs in the HIP kernels.  There is
no fallback: if libgsample.so is missing or the tensors are not on the GPU,
the call raises.
"""

from __future__ import annotations

import ctypes
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgsample.so")

GS_OK, GS_ERR_NULL, GS_ERR_SHAPE, GS_ERR_DTYPE, GS_ERR_ATTR, GS_ERR_TOO_LARGE, GS_ERR_HIP = range(7)
GS_F32, GS_F16, GS_BF16 = 0, 1, 2
MODES = {"linear": 0, "bilinear": 0, "nearest": 1, "cubic": 2, "bicubic": 2}
PADDINGS = {"zeros": 0, "border": 1, "reflection": 2}

# C entry points and their argument types (mirrors include/gsample.h)
_P = ctypes.c_void_p
_I = ctypes.c_int
_PI64 = ctypes.POINTER(ctypes.c_int64)
SIGNATURES = {
    "gs_abi_version": ([], _I),
    "gs_status_string": ([_I], ctypes.c_char_p),
    "gs_affine_grid": ([_P, _I, _PI64, _I, _I, _P, _P], _I),
    "gs_grid_sample_2d": ([_P, _I, _PI64, _P, _I, _PI64, _I, _I, _I, _P, _P], _I),
    "gs_grid_sample_3d": ([_P, _I, _PI64, _P, _I, _PI64, _I, _I, _I, _P, _P], _I),
    "gs_affine_grid_sample_fused": ([_P, _I, _P, _I, _PI64, _I, _PI64, _I, _I, _I, _P, _P], _I),
}

_lock = threading.Lock()
_lib = None


class GSError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().gs_status_string(status).decode()
        super().__init__("%s failed: %s (status %d)" % (where, msg, status))


def lib():
    """The loaded libgsample (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError("libgsample.so is not built (python -m "
                                  "spatial_transformer_grid_amd.build)")
            handle = ctypes.CDLL(LIB_PATH)
            for name, (args, res) in SIGNATURES.items():
                fn = getattr(handle, name)
                fn.argtypes = args
                fn.restype = res
            _lib = handle
        return _lib


def int64_array(values):
    vals = [int(v) for v in values]
    return (ctypes.c_int64 * max(1, len(vals)))(*vals)


def _torch():
    import torch

    return torch


def dtype_code(t) -> int:
    torch = _torch()
    codes = {torch.float32: GS_F32, torch.float16: GS_F16, torch.bfloat16: GS_BF16}
    if t.dtype not in codes:
        raise TypeError("unsupported element type %s" % t.dtype)
    return codes[t.dtype]


def _device_tensor(t, name):
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    return t.contiguous()


def _stream(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(status: int, where: str):
    if status != GS_OK:
        raise GSError(status, where)


def affine_grid(theta, size, align_corners: int = 0, out=None, stream=None):
    """AffineGrid(theta, size) -> grid on the GPU (gs_affine_grid)."""
    torch = _torch()
    theta = _device_tensor(theta, "theta")
    size = [int(s) for s in size]
    r = len(size) - 2
    if theta.dim() != 3 or theta.shape[0] != size[0] or theta.shape[1] != r or theta.shape[2] != r + 1:
        raise ValueError("theta %s does not match size %s" % (tuple(theta.shape), size))
    shape = (size[0], *size[2:], r)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=theta.device)
    elif tuple(out.shape) != shape or not out.is_contiguous() or out.dtype != torch.float32:
        raise ValueError("out must be a contiguous fp32 tensor of shape %s" % (shape,))
    st = lib().gs_affine_grid(ctypes.c_void_p(theta.data_ptr()), dtype_code(theta), int64_array(size),
                              len(size), int(align_corners), ctypes.c_void_p(out.data_ptr()),
                              _stream(stream, theta.device))
    _check(st, "gs_affine_grid")
    return out


def _out_tensor(out, shape, like):
    torch = _torch()
    if out is None:
        return torch.empty(shape, dtype=like.dtype, device=like.device)
    if tuple(out.shape) != tuple(shape) or out.dtype != like.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous %s tensor of shape %s" % (like.dtype, shape))
    return out


def grid_sample(X, grid, mode: str = "linear", padding_mode: str = "zeros",
                align_corners: int = 0, out=None, stream=None):
    """GridSample(X, grid) -> Y on the GPU (gs_grid_sample_2d / _3d)."""
    X = _device_tensor(X, "X")
    grid = _device_tensor(grid, "grid")
    r = X.dim() - 2
    if r not in (2, 3):
        raise ValueError("X must have 2 or 3 spatial dimensions")
    if grid.dim() != r + 2:
        raise ValueError("grid must have rank %d" % (r + 2))
    shape = (X.shape[0], X.shape[1], *grid.shape[1:-1])
    Y = _out_tensor(out, shape, X)
    fn = lib().gs_grid_sample_2d if r == 2 else lib().gs_grid_sample_3d
    st = fn(ctypes.c_void_p(X.data_ptr()), dtype_code(X), int64_array(X.shape),
            ctypes.c_void_p(grid.data_ptr()), dtype_code(grid), int64_array(grid.shape),
            MODES[mode], PADDINGS[padding_mode], int(align_corners),
            ctypes.c_void_p(Y.data_ptr()), _stream(stream, X.device))
    _check(st, "gs_grid_sample_%dd" % r)
    return Y


def affine_grid_sample_fused(theta, X, out_spatial, mode: str = "linear",
                             padding_mode: str = "zeros", align_corners: int = 0, out=None,
                             stream=None):
    """AffineGrid + GridSample in one pass, the grid never materialised."""
    theta = _device_tensor(theta, "theta")
    X = _device_tensor(X, "X")
    r = X.dim() - 2
    out_spatial = [int(s) for s in out_spatial]
    if len(out_spatial) != r:
        raise ValueError("out_spatial needs %d extents" % r)
    if tuple(theta.shape) != (X.shape[0], r, r + 1):
        raise ValueError("theta must have shape %s" % ((X.shape[0], r, r + 1),))
    shape = (X.shape[0], X.shape[1], *out_spatial)
    Y = _out_tensor(out, shape, X)
    st = lib().gs_affine_grid_sample_fused(
        ctypes.c_void_p(theta.data_ptr()), dtype_code(theta), ctypes.c_void_p(X.data_ptr()),
        dtype_code(X), int64_array(X.shape), X.dim(), int64_array(out_spatial),
        MODES[mode], PADDINGS[padding_mode], int(align_corners),
        ctypes.c_void_p(Y.data_ptr()), _stream(stream, X.device))
    _check(st, "gs_affine_grid_sample_fused")
    return Y
