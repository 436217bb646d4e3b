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

(GS_OK, GS_ERR_NULL, GS_ERR_SHAPE, GS_ERR_DTYPE, GS_ERR_ATTR, GS_ERR_LAYOUT, GS_ERR_TOO_LARGE,
 GS_ERR_HIP) = range(8)
(GS_F32, GS_F16, GS_BF16, GS_F64, GS_I8, GS_U8, GS_I16, GS_U16, GS_I32, GS_U32, GS_I64,
 GS_U64) = range(12)
MODES = {"linear": 0, "bilinear": 0, "nearest": 1, "cubic": 2, "bicubic": 2}
PADDINGS = {"zeros": 0, "border": 1, "reflection": 2}
RESIZE_MODES = {"nearest": 0, "linear": 1, "cubic": 2}
COORD_MODES = {"half_pixel": 0, "pytorch_half_pixel": 1, "align_corners": 2, "asymmetric": 3}
NEAREST_MODES = {"round_prefer_floor": 0, "round_prefer_ceil": 1, "floor": 2, "ceil": 3}
ASPECT_POLICIES = {"stretch": 0, "not_larger": 1, "not_smaller": 2}

# C entry points and their argument types (mirrors include/gsample.h)
_P = ctypes.c_void_p
_I = ctypes.c_int
_PI64 = ctypes.POINTER(ctypes.c_int64)
_PF32 = ctypes.POINTER(ctypes.c_float)
SIGNATURES = {
    "gs_abi_version": ([], _I),
    "gs_status_string": ([_I], ctypes.c_char_p),
    "gs_affine_grid": ([_P, _I, _PI64, _I, _I, _P, _P], _I),
    "gs_grid_sample_2d": ([_P, _I, _PI64, _P, _I, _PI64, _I, _I, _I, _P, _P], _I),
    "gs_grid_sample_3d": ([_P, _I, _PI64, _P, _I, _PI64, _I, _I, _I, _P, _P], _I),
    "gs_affine_grid_sample_fused": ([_P, _I, _P, _I, _PI64, _I, _PI64, _I, _I, _I, _P, _P], _I),
    "gs_grid_sample": ([_P, _I, _PI64, _I, _P, _I, _PI64, _I, _I, _I, _P, _P], _I),
    "gs_grid_sample_2d_ws": ([_P, _I, _PI64, _P, _I, _PI64, _I, _I, _I, _P, _P, ctypes.c_int64, _P],
                             _I),
    "gs_grid_sample_2d_workspace_size": ([_I, _PI64, _PI64, _PI64], _I),
    "gs_deform_conv": ([_P, _I, _PI64, _I, _P, _PI64, _P, _P, _P, _PI64, _PI64, _PI64, _I, _I,
                        _P, _P, ctypes.c_int64, _P], _I),
    "gs_deform_conv_workspace_size": ([_I, _PI64, _I, _PI64, _PI64, _PI64, _PI64, _I, _I, _PI64],
                                      _I),
    "gs_deform_conv_noalloc": ([_P, _I, _PI64, _I, _P, _PI64, _P, _P, _P, _PI64, _PI64, _PI64, _I,
                                _I, _P, _P], _I),
    "gs_resize_output_shape": ([_PI64, _I, _PI64, _I, _PF32, _PI64, _I, _PI64], _I),
    "gs_resize": ([_P, _I, _PI64, _I, _PI64, _PF32, _I, _I, _I, ctypes.c_float, _I, _P, _P], _I),
}

_lock = threading.Lock()
_lib = None


class GSError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().gs_status_string(status).decode()
        super().__init__("%s failed: %s (status %d)" % (where, msg, status))


def hip_runtimes_mapped():
    """Distinct HIP runtime files (libamdhip64) mapped into this process,
    read from /proc/self/maps (empty where that file does not exist)."""
    try:
        with open("/proc/self/maps") as f:
            lines = f.read().splitlines()
    except OSError:
        return []
    paths = set()
    for ln in lines:
        fields = ln.split(None, 5)  # the sixth field is the path, spaces included
        if len(fields) == 6 and "libamdhip64" in fields[5]:
            paths.add(fields[5].strip())
    return sorted(paths)


def lib():
    """The loaded libgsample (raises if it has not been built).

    torch is imported first so that its HIP runtime is the one the library
    binds to: both carry the soname libamdhip64.so.7, and whichever is loaded
    first satisfies the other's dependency.  Loaded the other way round, the
    process would hold two runtimes, and kernels registered with one cannot
    be launched on streams or memory of the other.
    """
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError("libgsample.so is not built (python -m "
                                  "spatial_transformer_grid_amd.build)")
            _torch()
            handle = ctypes.CDLL(LIB_PATH)
            runtimes = hip_runtimes_mapped()
            if len(runtimes) > 1:
                raise ImportError("more than one HIP runtime is loaded (%s); libgsample must "
                                  "share torch's" % ", ".join(runtimes))
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
    codes = {torch.float32: GS_F32, torch.float16: GS_F16, torch.bfloat16: GS_BF16,
             torch.float64: GS_F64, torch.int8: GS_I8, torch.uint8: GS_U8, torch.int16: GS_I16,
             torch.int32: GS_I32, torch.int64: GS_I64}
    for name, code in (("uint16", GS_U16), ("uint32", GS_U32), ("uint64", GS_U64)):
        if hasattr(torch, name):
            codes[getattr(torch, name)] = code
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
    """AffineGrid(theta, size) -> grid on the GPU (gs_affine_grid); the grid
    has theta's element type."""
    torch = _torch()
    theta = _device_tensor(theta, "theta")
    size = [int(s) for s in size]
    r = len(size) - 2
    if theta.dim() != 3 or theta.shape[0] != size[0] or theta.shape[1] != r or theta.shape[2] != r + 1:
        raise ValueError("theta %s does not match size %s" % (tuple(theta.shape), size))
    shape = (size[0], *size[2:], r)
    if out is None:
        out = torch.empty(shape, dtype=theta.dtype, device=theta.device)
    elif tuple(out.shape) != shape or not out.is_contiguous() or out.dtype != theta.dtype:
        raise ValueError("out must be a contiguous %s tensor of shape %s" % (theta.dtype, shape))
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


def grid_sample_2d_workspace_size(x_shape, grid_shape, dtype) -> int:
    """Bytes of workspace gs_grid_sample_2d_ws can use (0: none helps)."""
    need = ctypes.c_int64(0)
    _check(lib().gs_grid_sample_2d_workspace_size(dtype, int64_array(x_shape),
                                                  int64_array(grid_shape), ctypes.byref(need)),
           "gs_grid_sample_2d_workspace_size")
    return need.value


def grid_sample(X, grid, mode: str = "linear", padding_mode: str = "zeros",
                align_corners: int = 0, out=None, stream=None, workspace=None):
    """GridSample(X, grid) -> Y on the GPU: gs_grid_sample_2d / _3d for 2 and
    3 spatial dimensions, gs_grid_sample for 1 to 6.

    `workspace` (2-D only): a device tensor of scratch bytes, or "auto" for
    one of the size the library asks for from torch's allocator; with it the
    call is gs_grid_sample_2d_ws, which gathers from a channels-last copy of X
    when the grid scatters its locations (a random flow)."""
    X = _device_tensor(X, "X")
    grid = _device_tensor(grid, "grid")
    r = X.dim() - 2
    if grid.dim() != r + 2:
        raise ValueError("grid must have rank %d" % (r + 2))
    shape = (X.shape[0], X.shape[1], *grid.shape[1:-1])
    Y = _out_tensor(out, shape, X)
    args = (ctypes.c_void_p(X.data_ptr()), dtype_code(X), int64_array(X.shape))
    rest = (ctypes.c_void_p(grid.data_ptr()), dtype_code(grid), int64_array(grid.shape),
            MODES[mode], PADDINGS[padding_mode], int(align_corners),
            ctypes.c_void_p(Y.data_ptr()), _stream(stream, X.device))
    if r == 2 and workspace is not None:
        if isinstance(workspace, str):
            if workspace != "auto":
                raise ValueError('workspace must be a tensor or "auto"')
            need = grid_sample_2d_workspace_size(tuple(X.shape), tuple(grid.shape),
                                                 dtype_code(X))
            workspace = _torch().empty(need, dtype=_torch().uint8, device=X.device)
        ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace.numel() else None
        st = lib().gs_grid_sample_2d_ws(*args, *rest[:-1], ws_ptr,
                                        workspace.numel() * workspace.element_size(), rest[-1])
        _check(st, "gs_grid_sample_2d_ws")
        return Y
    if r in (2, 3):
        name = "gs_grid_sample_%dd" % r
        st = getattr(lib(), name)(*args, *rest)
    else:
        name = "gs_grid_sample"
        st = lib().gs_grid_sample(*args, X.dim(), *rest)
    _check(st, name)
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


def resize_output_shape(x_shape, scales=None, sizes=None, axes=None,
                        keep_aspect_ratio_policy: str = "stretch"):
    """Output extents of Resize from scales or sizes (gs_resize_output_shape)."""
    x_shape = [int(v) for v in x_shape]
    vals = scales if scales is not None else sizes
    if vals is None:
        raise ValueError("give scales or sizes")
    count = len(vals)
    ax = int64_array(axes) if axes is not None else None
    sc = (ctypes.c_float * max(1, count))(*[float(v) for v in scales]) if scales is not None else None
    sz = int64_array(sizes) if sizes is not None else None
    out = (ctypes.c_int64 * len(x_shape))()
    st = lib().gs_resize_output_shape(int64_array(x_shape), len(x_shape), ax, count, sc, sz,
                                      ASPECT_POLICIES[keep_aspect_ratio_policy], out)
    _check(st, "gs_resize_output_shape")
    return tuple(int(v) for v in out)


def resize(X, scales=None, sizes=None, axes=None, mode: str = "nearest",
           coordinate_transformation_mode: str = "half_pixel",
           nearest_mode: str = "round_prefer_floor", cubic_coeff_a: float = -0.75,
           exclude_outside: int = 0, keep_aspect_ratio_policy: str = "stretch", out=None,
           stream=None):
    """Resize(X, scales | sizes) -> Y on the GPU (gs_resize).

    Attribute names and defaults follow the Resize page (version 18); scales
    or sizes refer to `axes` (all axes when None)."""
    X = _device_tensor(X, "X")
    rank = X.dim()
    shape = resize_output_shape(X.shape, scales, sizes, axes, keep_aspect_ratio_policy)
    full = None
    if scales is not None:
        per_axis = [1.0] * rank
        for i, v in enumerate(scales):
            a = int(axes[i]) if axes is not None else i
            per_axis[a % rank] = float(v)
        full = (ctypes.c_float * rank)(*per_axis)
    Y = _out_tensor(out, shape, X)
    st = lib().gs_resize(ctypes.c_void_p(X.data_ptr()), dtype_code(X), int64_array(X.shape), rank,
                         int64_array(shape), full, RESIZE_MODES[mode],
                         COORD_MODES[coordinate_transformation_mode], NEAREST_MODES[nearest_mode],
                         float(cubic_coeff_a), int(exclude_outside),
                         ctypes.c_void_p(Y.data_ptr()), _stream(stream, X.device))
    _check(st, "gs_resize")
    return Y


def resize_to(X, y_shape, scales=None, mode: str = "nearest",
              coordinate_transformation_mode: str = "half_pixel",
              nearest_mode: str = "round_prefer_floor", cubic_coeff_a: float = -0.75,
              exclude_outside: int = 0, out=None, stream=None):
    """gs_resize with explicit output extents and per-axis scales (or None)."""
    X = _device_tensor(X, "X")
    rank = X.dim()
    y_shape = [int(v) for v in y_shape]
    full = (ctypes.c_float * rank)(*[float(v) for v in scales]) if scales is not None else None
    Y = _out_tensor(out, y_shape, X)
    st = lib().gs_resize(ctypes.c_void_p(X.data_ptr()), dtype_code(X), int64_array(X.shape), rank,
                         int64_array(y_shape), full, RESIZE_MODES[mode],
                         COORD_MODES[coordinate_transformation_mode], NEAREST_MODES[nearest_mode],
                         float(cubic_coeff_a), int(exclude_outside),
                         ctypes.c_void_p(Y.data_ptr()), _stream(stream, X.device))
    _check(st, "gs_resize")
    return Y


def deform_conv_output_shape(x_shape, w_shape, strides=None, pads=None, dilations=None):
    r = len(x_shape) - 2
    strides = [1] * r if strides is None else list(strides)
    dilations = [1] * r if dilations is None else list(dilations)
    pads = [0] * (2 * r) if pads is None else list(pads)
    out = [(x_shape[2 + a] + pads[a] + pads[r + a] - (dilations[a] * (w_shape[2 + a] - 1) + 1))
           // strides[a] + 1 for a in range(r)]
    return (x_shape[0], w_shape[0], *out)


def _deform_tensors(X, W, offset, B, mask, strides, pads, dilations, offset_group, out):
    """Checked device tensors of a DeformConv call and its output."""
    X = _device_tensor(X, "X")
    W = _device_tensor(W, "W")
    offset = _device_tensor(offset, "offset")
    B = _device_tensor(B, "B") if B is not None else None
    mask = _device_tensor(mask, "mask") if mask is not None else None
    for name, t in (("W", W), ("offset", offset), ("B", B), ("mask", mask)):
        if t is not None and t.dtype != X.dtype:
            raise TypeError("%s must have X's element type" % name)
    shape = deform_conv_output_shape(tuple(X.shape), tuple(W.shape), strides, pads, dilations)
    r = X.dim() - 2
    npos = 1
    for v in shape[2:]:
        npos *= v
    K = 1
    for v in W.shape[2:]:
        K *= v
    if tuple(offset.shape) != (X.shape[0], offset_group * K * r, *shape[2:]):
        raise ValueError("offset must have shape %s" % ((X.shape[0], offset_group * K * r,
                                                         *shape[2:]),))
    if mask is not None and tuple(mask.shape) != (X.shape[0], offset_group * K, *shape[2:]):
        raise ValueError("mask must have shape %s" % ((X.shape[0], offset_group * K,
                                                       *shape[2:]),))
    if B is not None and tuple(B.shape) != (W.shape[0],):
        raise ValueError("B must have shape (%d,)" % W.shape[0])
    return X, W, offset, B, mask, _out_tensor(out, shape, X)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _arr(v):
    return int64_array(v) if v is not None else None


def deform_conv(X, W, offset, B=None, mask=None, strides=None, pads=None, dilations=None,
                group: int = 1, offset_group: int = 1, out=None, stream=None, workspace=None):
    """DeformConv(X, W, offset, B, mask) -> Y on the GPU (gs_deform_conv).

    Attribute names follow the convolution operators (strides, pads as begins
    then ends, dilations, group, offset_group).  `workspace`: a device tensor
    of scratch bytes; None takes one of the size the library asks for from
    torch's allocator, and an empty tensor runs without one."""
    X, W, offset, B, mask, Y = _deform_tensors(X, W, offset, B, mask, strides, pads, dilations,
                                               offset_group, out)
    ptr, arr = _ptr, _arr
    need = ctypes.c_int64(0)
    _check(lib().gs_deform_conv_workspace_size(
        dtype_code(X), int64_array(X.shape), X.dim(), int64_array(W.shape), arr(strides),
        arr(pads), arr(dilations), int(group), int(offset_group), ctypes.byref(need)),
        "gs_deform_conv_workspace_size")
    if workspace is None and need.value > 0:
        workspace = _torch().empty(need.value, dtype=_torch().uint8, device=X.device)
    ws_ptr = ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().gs_deform_conv(ptr(X), dtype_code(X), int64_array(X.shape), X.dim(), ptr(W),
                              int64_array(W.shape), ptr(offset), ptr(B), ptr(mask), arr(strides),
                              arr(pads), arr(dilations), int(group), int(offset_group), ptr(Y),
                              ws_ptr, ws_bytes, _stream(stream, X.device))
    _check(st, "gs_deform_conv")
    return Y


def deform_conv_noalloc(X, W, offset, B=None, mask=None, strides=None, pads=None,
                        dilations=None, group: int = 1, offset_group: int = 1, out=None,
                        stream=None):
    """DeformConv through gs_deform_conv_noalloc: the library's own 64 MiB
    scratch array per GPU instead of a workspace (for callers that cannot
    allocate; pass `out` to allocate nothing here either).  Calls that may
    overlap on one GPU race on that array."""
    X, W, offset, B, mask, Y = _deform_tensors(X, W, offset, B, mask, strides, pads, dilations,
                                               offset_group, out)
    st = lib().gs_deform_conv_noalloc(_ptr(X), dtype_code(X), int64_array(X.shape), X.dim(),
                                      _ptr(W), int64_array(W.shape), _ptr(offset), _ptr(B),
                                      _ptr(mask), _arr(strides), _arr(pads), _arr(dilations),
                                      int(group), int(offset_group), _ptr(Y),
                                      _stream(stream, X.device))
    _check(st, "gs_deform_conv_noalloc")
    return Y


def deform_conv_workspace_size(X_shape, W_shape, dtype, strides=None, pads=None, dilations=None,
                               group: int = 1, offset_group: int = 1) -> int:
    """Bytes of workspace deform_conv uses (gs_deform_conv_workspace_size)."""
    arr = lambda v: int64_array(v) if v is not None else None
    need = ctypes.c_int64(0)
    _check(lib().gs_deform_conv_workspace_size(
        dtype, int64_array(X_shape), len(X_shape), int64_array(W_shape), arr(strides), arr(pads),
        arr(dilations), int(group), int(offset_group), ctypes.byref(need)),
        "gs_deform_conv_workspace_size")
    return need.value
