"""Plain CPU reference (oracle) for AffineGrid, GridSample, Resize and
DeformConv.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The GPU library and its Python
binding never import it, and it never imports them.

The arithmetic lives in ``oracle.c`` (AffineGrid, GridSample), ``resize.c``
(Resize) and ``deform_conv.c`` (DeformConv), plain scalar C built with gcc
``-O2 -ffp-contract=off``;
this module only builds them, loads them and marshals numpy arrays.
Attribute names and defaults follow the GridSample page (mode "linear",
padding_mode "zeros"; align_corners 0, the value every example that omits it
behaves as) and the Resize page.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_RESIZE_SRC = os.path.join(_HERE, "resize.c")
_DEFORM_SRC = os.path.join(_HERE, "deform_conv.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# the same sources built with -fopenmp: the output loops run on every host
# core (for timing the oracle and for large parity checks); values identical
_OMP_LIB = os.path.join(_HERE, "liboracle_omp.so")

MODES = {"linear": 0, "nearest": 1, "cubic": 2}
PADDINGS = {"zeros": 0, "border": 1, "reflection": 2}
RESIZE_MODES = {"nearest": 0, "linear": 1, "cubic": 2}
COORD_MODES = {"half_pixel": 0, "pytorch_half_pixel": 1, "align_corners": 2, "asymmetric": 3}
NEAREST_MODES = {"round_prefer_floor": 0, "round_prefer_ceil": 1, "floor": 2, "ceil": 3}
ASPECT_POLICIES = {"stretch": 0, "not_larger": 1, "not_smaller": 2}

_lock = threading.Lock()
_default = None
_parallel = None

# A handle from load_library() can be passed as `lib=` to run the same calls
# against another build of the oracle source (used by the mutation tests).


# ORACLE_LIB names another build of the oracle to load instead of
# liboracle.so, and ORACLE_EXTRA_CFLAGS adds compiler flags to every build
# made by build(): the sanitizer test uses both to run the pin batteries on an
# AddressSanitizer / UndefinedBehaviorSanitizer build.
_ENV_LIB = os.environ.get("ORACLE_LIB")


def build(force: bool = True, src: str = _SRC, out: str = _LIB,
          resize_src: str = _RESIZE_SRC, deform_src: str = _DEFORM_SRC,
          openmp: bool = False, extra_flags=()) -> str:
    """Compile oracle.c, resize.c and deform_conv.c (or other copies of them)
    into one shared library.  With the default arguments both the serial
    library and its OpenMP build are made."""
    if out == _LIB and not openmp and src == _SRC:
        build(force, src, _OMP_LIB, resize_src, deform_src, openmp=True)
    if not force and os.path.exists(out):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    env_flags = os.environ.get("ORACLE_EXTRA_CFLAGS", "").split()
    cmd = (["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
            "-Wall", "-Wextra"] + (["-fopenmp"] if openmp else []) + list(extra_flags) + env_flags
           + ["-o", tmp, src, resize_src, deform_src, "-lm"])
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _bind(path: str):
    lib = ctypes.CDLL(path)
    p_f32 = ctypes.POINTER(ctypes.c_float)
    p_f64 = ctypes.POINTER(ctypes.c_double)
    p_i64 = ctypes.POINTER(ctypes.c_int64)
    i64, c_int = ctypes.c_int64, ctypes.c_int
    lib.oracle_affine_grid.argtypes = [p_f32, c_int, i64, p_i64, c_int, p_f32]
    lib.oracle_affine_grid.restype = c_int
    lib.oracle_affine_grid_d.argtypes = [p_f64, c_int, i64, p_i64, c_int, p_f64]
    lib.oracle_affine_grid_d.restype = c_int
    lib.oracle_grid_sample.argtypes = [p_f32, c_int, i64, i64, p_i64, p_f32, p_i64,
                                       c_int, c_int, c_int, p_f64]
    lib.oracle_grid_sample.restype = c_int
    lib.oracle_grid_sample_points.argtypes = [p_f32, c_int, i64, i64, p_i64, p_f32, p_i64,
                                              c_int, c_int, c_int, p_i64, i64, p_f64]
    lib.oracle_grid_sample_points.restype = c_int
    lib.oracle_abi_version.restype = c_int
    lib.oracle_threads.restype = c_int
    lib.oracle_grid_sample_ex.argtypes = [p_f32, p_f64, c_int, i64, i64, p_i64, p_f32, p_f64,
                                          p_i64, c_int, c_int, c_int, p_f64]
    lib.oracle_grid_sample_ex.restype = c_int
    lib.oracle_grid_sample_points_ex.argtypes = [p_f32, p_f64, c_int, i64, i64, p_i64, p_f32,
                                                 p_f64, p_i64, c_int, c_int, c_int, p_i64, i64,
                                                 p_f64]
    lib.oracle_grid_sample_points_ex.restype = c_int
    lib.oracle_resize.argtypes = [p_f32, c_int, p_i64, p_i64, p_f32, c_int, c_int, c_int,
                                  ctypes.c_double, c_int, p_f64]
    lib.oracle_resize.restype = c_int
    lib.oracle_resize_output_shape.argtypes = [c_int, p_i64, c_int, p_i64, p_f32, p_i64, c_int,
                                               c_int, p_i64]
    lib.oracle_resize_output_shape.restype = c_int
    lib.oracle_resize_points.argtypes = [p_f32, c_int, p_i64, p_i64, p_f32, c_int, c_int, c_int,
                                         ctypes.c_double, c_int, p_i64, i64, p_f64]
    lib.oracle_resize_points.restype = c_int
    lib.oracle_deform_conv.argtypes = [p_f64, c_int, i64, i64, p_i64, p_f64, i64, p_i64, p_f64,
                                       p_f64, p_f64, p_i64, p_i64, p_i64, p_i64, i64, i64, c_int,
                                       p_f64]
    lib.oracle_deform_conv.restype = c_int
    lib.oracle_deform_conv_points.argtypes = lib.oracle_deform_conv.argtypes[:-1] + [p_i64, i64,
                                                                                   p_f64]
    lib.oracle_deform_conv_points.restype = c_int
    return lib


def _load():
    global _default
    with _lock:
        if _default is None:
            if _ENV_LIB:
                _default = _bind(_ENV_LIB)
            else:
                if not os.path.exists(_LIB):
                    build()
                _default = _bind(_LIB)
        return _default


def parallel():
    """Handle of the OpenMP build (same sources, same values, output loops on
    every core OpenMP is given); pass it as `lib=`."""
    global _parallel
    with _lock:
        if _parallel is None:
            if not os.path.exists(_OMP_LIB):
                build(force=True, out=_OMP_LIB, openmp=True)
            _parallel = _bind(_OMP_LIB)
        return _parallel


def threads(lib=None) -> int:
    """Threads the output loops of a build use (1 for the serial build)."""
    return int((lib or _load()).oracle_threads())


def load_library(path: str):
    """ctypes handle for an oracle library built from `path`."""
    return _bind(path)


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def affine_grid(theta: np.ndarray, size, align_corners: int = 0, lib=None) -> np.ndarray:
    """AffineGrid(theta, size) -> grid.

    theta: (N, r, r+1) fp32 (fp16 and bf16 theta are passed widened exactly;
    the caller rounds the fp32 grid to the half type) or float64 (then the
    steps run in float64 and the grid is float64).  size: (N, C, *spatial) as
    on the page (C unused).  Returns (N, *spatial, r).
    """
    lib = lib or _load()
    if np.asarray(theta).dtype == np.float64:
        return _affine_grid_d(np.ascontiguousarray(theta), size, align_corners, lib)
    theta = np.ascontiguousarray(theta, dtype=np.float32)
    size = [int(s) for s in size]
    n, r = theta.shape[0], theta.shape[1]
    if theta.shape != (n, r, r + 1) or len(size) != r + 2 or size[0] != n:
        raise ValueError("theta %s does not match size %s" % (theta.shape, size))
    spatial = np.asarray(size[2:], dtype=np.int64)
    out = np.empty((n, *size[2:], r), dtype=np.float32)
    rc = lib.oracle_affine_grid(_ptr(theta, ctypes.c_float), r, n, _ptr(spatial, ctypes.c_int64),
                                int(align_corners), _ptr(out, ctypes.c_float))
    if rc:
        raise ValueError("oracle_affine_grid rejected its arguments")
    return out


def _affine_grid_d(theta, size, align_corners, lib):
    size = [int(s) for s in size]
    n, r = theta.shape[0], theta.shape[1]
    if theta.shape != (n, r, r + 1) or len(size) != r + 2 or size[0] != n:
        raise ValueError("theta %s does not match size %s" % (theta.shape, size))
    spatial = np.asarray(size[2:], dtype=np.int64)
    out = np.empty((n, *size[2:], r), dtype=np.float64)
    rc = lib.oracle_affine_grid_d(_ptr(theta, ctypes.c_double), r, n,
                                  _ptr(spatial, ctypes.c_int64), int(align_corners),
                                  _ptr(out, ctypes.c_double))
    if rc:
        raise ValueError("oracle_affine_grid_d rejected its arguments")
    return out


def _check_sample_args(X, grid):
    """X as fp32 (fp32 and half inputs widened exactly) or float64 (double and
    integer inputs); the grid as fp32 (fp32, fp16) or float64 (double)."""
    X = np.asarray(X)
    grid = np.asarray(grid)
    if X.dtype in (np.float32, np.float16):
        X = np.ascontiguousarray(X, dtype=np.float32)
    else:
        X = np.ascontiguousarray(X, dtype=np.float64)
    if grid.dtype == np.float64:
        grid = np.ascontiguousarray(grid)
    elif grid.dtype in (np.float32, np.float16):
        grid = np.ascontiguousarray(grid, dtype=np.float32)
    else:
        raise TypeError("grid must be a float tensor, got %s" % grid.dtype)
    r = X.ndim - 2
    if r < 1 or grid.ndim != r + 2 or grid.shape[0] != X.shape[0] or grid.shape[-1] != r:
        raise ValueError("X %s and grid %s do not match" % (X.shape, grid.shape))
    return X, grid, r


def _xg_ptrs(X, grid):
    xf = _ptr(X, ctypes.c_float) if X.dtype == np.float32 else None
    xd = _ptr(X, ctypes.c_double) if X.dtype == np.float64 else None
    gf = _ptr(grid, ctypes.c_float) if grid.dtype == np.float32 else None
    gd = _ptr(grid, ctypes.c_double) if grid.dtype == np.float64 else None
    return xf, xd, gf, gd


def grid_sample(X: np.ndarray, grid: np.ndarray, mode: str = "linear",
                padding_mode: str = "zeros", align_corners: int = 0, lib=None) -> np.ndarray:
    """GridSample(X, grid) -> Y as float64 (unrounded).

    X: (N, C, *in_spatial), any rank r >= 1: fp32 (half inputs are passed
    widened exactly), float64, or an integer type (converted to float64).
    grid: (N, *out_spatial, r) fp32 or fp16 (coordinates in fp32) or float64
    (coordinates in float64).  Returns (N, C, *out_spatial) float64; integer
    outputs are to_integer() of it.
    """
    lib = lib or _load()
    X, grid, r = _check_sample_args(X, grid)
    n, c = X.shape[:2]
    in_sp = np.asarray(X.shape[2:], dtype=np.int64)
    out_sp = np.asarray(grid.shape[1:-1], dtype=np.int64)
    Y = np.empty((n, c, *grid.shape[1:-1]), dtype=np.float64)
    xf, xd, gf, gd = _xg_ptrs(X, grid)
    rc = lib.oracle_grid_sample_ex(xf, xd, r, n, c, _ptr(in_sp, ctypes.c_int64), gf, gd,
                                   _ptr(out_sp, ctypes.c_int64), MODES[mode],
                                   PADDINGS[padding_mode], int(align_corners),
                                   _ptr(Y, ctypes.c_double))
    if rc:
        raise ValueError("oracle_grid_sample rejected its arguments")
    return Y


def grid_sample_points(X: np.ndarray, grid: np.ndarray, flat_index: np.ndarray,
                       mode: str = "linear", padding_mode: str = "zeros",
                       align_corners: int = 0, lib=None) -> np.ndarray:
    """GridSample evaluated only at the listed flat indices of Y (float64)."""
    lib = lib or _load()
    X, grid, r = _check_sample_args(X, grid)
    n, c = X.shape[:2]
    in_sp = np.asarray(X.shape[2:], dtype=np.int64)
    out_sp = np.asarray(grid.shape[1:-1], dtype=np.int64)
    idx = np.ascontiguousarray(flat_index, dtype=np.int64)
    Y = np.empty(idx.shape[0], dtype=np.float64)
    xf, xd, gf, gd = _xg_ptrs(X, grid)
    rc = lib.oracle_grid_sample_points_ex(xf, xd, r, n, c, _ptr(in_sp, ctypes.c_int64), gf, gd,
                                          _ptr(out_sp, ctypes.c_int64), MODES[mode],
                                          PADDINGS[padding_mode], int(align_corners),
                                          _ptr(idx, ctypes.c_int64), idx.shape[0],
                                          _ptr(Y, ctypes.c_double))
    if rc:
        raise ValueError("oracle_grid_sample_points rejected its arguments")
    return Y


def _axes_list(rank, count, axes):
    if axes is None:
        if count != rank:
            raise ValueError("%d values for a tensor of rank %d and no axes" % (count, rank))
        return list(range(rank))
    return [int(a) for a in axes]


def resize_output_shape(in_shape, scales=None, sizes=None, axes=None,
                        keep_aspect_ratio_policy: str = "stretch", lib=None):
    """Output extents of Resize from scales or sizes (exactly one given)."""
    lib = lib or _load()
    if (scales is None) == (sizes is None):
        raise ValueError("give exactly one of scales and sizes")
    in_shape = np.asarray(in_shape, dtype=np.int64)
    rank = in_shape.shape[0]
    vals = scales if scales is not None else sizes
    ax = np.asarray(_axes_list(rank, len(vals), axes), dtype=np.int64)
    sc = np.asarray(scales if scales is not None else [0.0] * len(vals), dtype=np.float32)
    sz = np.asarray(sizes if sizes is not None else [0] * len(vals), dtype=np.int64)
    out = np.empty(rank, dtype=np.int64)
    rc = lib.oracle_resize_output_shape(rank, _ptr(in_shape, ctypes.c_int64), len(vals),
                                        _ptr(ax, ctypes.c_int64), _ptr(sc, ctypes.c_float),
                                        _ptr(sz, ctypes.c_int64), int(sizes is not None),
                                        ASPECT_POLICIES[keep_aspect_ratio_policy],
                                        _ptr(out, ctypes.c_int64))
    if rc:
        raise ValueError("oracle_resize_output_shape rejected its arguments")
    return tuple(int(v) for v in out)


def resize(X: np.ndarray, out_shape, scales=None, mode: str = "nearest",
           coordinate_transformation_mode: str = "half_pixel",
           nearest_mode: str = "round_prefer_floor", cubic_coeff_a: float = -0.75,
           exclude_outside: int = 0, lib=None) -> np.ndarray:
    """Resize(X) -> Y as float64 (unrounded).

    out_shape: extents of Y (one per axis of X).  scales: per-axis scale used
    by the coordinate transformation (one per axis), or None when the output
    came from sizes (then each axis uses output extent / input extent).
    Attribute names and defaults follow the Resize page (version 18).
    """
    lib = lib or _load()
    X = np.ascontiguousarray(X, dtype=np.float32)
    rank = X.ndim
    in_sp = np.asarray(X.shape, dtype=np.int64)
    out_sp = np.asarray([int(v) for v in out_shape], dtype=np.int64)
    if out_sp.shape[0] != rank:
        raise ValueError("out_shape %s does not match X %s" % (tuple(out_sp), X.shape))
    sc = None
    if scales is not None:
        sc = np.ascontiguousarray(scales, dtype=np.float32)
        if sc.shape != (rank,):
            raise ValueError("need one scale per axis")
    Y = np.empty(tuple(out_sp), dtype=np.float64)
    rc = lib.oracle_resize(_ptr(X, ctypes.c_float), rank, _ptr(in_sp, ctypes.c_int64),
                           _ptr(out_sp, ctypes.c_int64),
                           _ptr(sc, ctypes.c_float) if sc is not None else None,
                           RESIZE_MODES[mode], COORD_MODES[coordinate_transformation_mode],
                           NEAREST_MODES[nearest_mode], float(cubic_coeff_a),
                           int(exclude_outside), _ptr(Y, ctypes.c_double))
    if rc:
        raise ValueError("oracle_resize rejected its arguments")
    return Y


def resize_points(X: np.ndarray, out_shape, flat_index: np.ndarray, scales=None,
                  mode: str = "nearest", coordinate_transformation_mode: str = "half_pixel",
                  nearest_mode: str = "round_prefer_floor", cubic_coeff_a: float = -0.75,
                  exclude_outside: int = 0, lib=None) -> np.ndarray:
    """Resize evaluated only at the listed flat indices of Y (float64)."""
    lib = lib or _load()
    X = np.ascontiguousarray(X, dtype=np.float32)
    rank = X.ndim
    in_sp = np.asarray(X.shape, dtype=np.int64)
    out_sp = np.asarray([int(v) for v in out_shape], dtype=np.int64)
    sc = None if scales is None else np.ascontiguousarray(scales, dtype=np.float32)
    idx = np.ascontiguousarray(flat_index, dtype=np.int64)
    Y = np.empty(idx.shape[0], dtype=np.float64)
    rc = lib.oracle_resize_points(_ptr(X, ctypes.c_float), rank, _ptr(in_sp, ctypes.c_int64),
                                  _ptr(out_sp, ctypes.c_int64),
                                  _ptr(sc, ctypes.c_float) if sc is not None else None,
                                  RESIZE_MODES[mode], COORD_MODES[coordinate_transformation_mode],
                                  NEAREST_MODES[nearest_mode], float(cubic_coeff_a),
                                  int(exclude_outside), _ptr(idx, ctypes.c_int64), idx.shape[0],
                                  _ptr(Y, ctypes.c_double))
    if rc:
        raise ValueError("oracle_resize_points rejected its arguments")
    return Y


def to_integer(values: np.ndarray, dtype) -> np.ndarray:
    """The final cast of integer inputs (GridSample page, Outputs: integer
    inputs are interpolated in floating point and the result converted to
    the integer type).  Reading: truncation
    toward zero, as a C conversion does, saturated to the range of the type
    (cubic weights can overshoot it); a NaN becomes 0."""
    dtype = np.dtype(dtype)
    info = np.iinfo(dtype)
    v = np.nan_to_num(np.asarray(values, dtype=np.float64), nan=0.0)
    v = np.trunc(v)
    lo, hi = float(info.min), float(info.max)
    out = np.where(v <= lo, info.min, np.where(v >= hi, info.max, 0)).astype(dtype)
    inside = (v > lo) & (v < hi)
    out[inside] = v[inside].astype(dtype)
    return out


def deform_conv_output_shape(in_sp, ksz, strides, pads, dilations):
    """(in + pad_begin + pad_end - (dilation * (k - 1) + 1)) // stride + 1."""
    r = len(in_sp)
    return tuple((in_sp[a] + pads[a] + pads[r + a] - (dilations[a] * (ksz[a] - 1) + 1))
                 // strides[a] + 1 for a in range(r))


def deform_conv(X, W, offset, B=None, mask=None, strides=None, pads=None, dilations=None,
                group: int = 1, offset_group: int = 1, lib=None, flat_index=None) -> np.ndarray:
    """DeformConv(X, W, offset, B, mask) -> Y as float64 (unrounded).

    Arrays are fp32 (half data widened exactly: locations in fp32) or float64
    (locations in float64); attribute names and defaults follow the
    convolution operators (strides and dilations 1, pads 0, group and
    offset_group 1).  With flat_index, only those flat outputs of Y are
    computed (a 1-D array)."""
    lib = lib or _load()
    X = np.asarray(X)
    coord_f32 = 0 if X.dtype == np.float64 else 1
    X = np.ascontiguousarray(X, dtype=np.float64)
    W = np.ascontiguousarray(W, dtype=np.float64)
    offset = np.ascontiguousarray(offset, dtype=np.float64)
    n, c = X.shape[:2]
    r = X.ndim - 2
    in_sp = X.shape[2:]
    ksz = W.shape[2:]
    strides = [1] * r if strides is None else list(strides)
    dilations = [1] * r if dilations is None else list(dilations)
    pads = [0] * (2 * r) if pads is None else list(pads)
    out_sp = deform_conv_output_shape(in_sp, ksz, strides, pads, dilations)
    oc = W.shape[0]
    if flat_index is not None:
        idx = np.ascontiguousarray(flat_index, dtype=np.int64)
        Y = np.empty(idx.shape[0], dtype=np.float64)
    else:
        Y = np.empty((n, oc) + out_sp, dtype=np.float64)
    b = None if B is None else np.ascontiguousarray(B, dtype=np.float64)
    m = None if mask is None else np.ascontiguousarray(mask, dtype=np.float64)
    arr = lambda v: np.asarray(v, dtype=np.int64)
    in_a, k_a, o_a, s_a, p_a, d_a = (arr(in_sp), arr(ksz), arr(out_sp), arr(strides), arr(pads),
                                     arr(dilations))
    args = [_ptr(X, ctypes.c_double), r, n, c, _ptr(in_a, ctypes.c_int64),
            _ptr(W, ctypes.c_double), oc, _ptr(k_a, ctypes.c_int64), _ptr(offset, ctypes.c_double),
            _ptr(b, ctypes.c_double) if b is not None else None,
            _ptr(m, ctypes.c_double) if m is not None else None, _ptr(o_a, ctypes.c_int64),
            _ptr(s_a, ctypes.c_int64), _ptr(p_a, ctypes.c_int64), _ptr(d_a, ctypes.c_int64),
            int(group), int(offset_group), coord_f32]
    if flat_index is not None:
        rc = lib.oracle_deform_conv_points(*args, _ptr(idx, ctypes.c_int64), idx.shape[0],
                                           _ptr(Y, ctypes.c_double))
    else:
        rc = lib.oracle_deform_conv(*args, _ptr(Y, ctypes.c_double))
    if rc:
        raise ValueError("oracle_deform_conv rejected its arguments")
    return Y
