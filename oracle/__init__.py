"""Plain CPU reference (oracle) for AffineGrid and GridSample.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The GPU library and its Python
binding never import it, and it never imports them.

The arithmetic lives in ``oracle.c`` (plain scalar C, built with gcc
``-O2 -ffp-contract=off``); this module only builds it, loads it and marshals
numpy arrays.  Attribute names and defaults follow the GridSample page
(mode "linear", padding_mode "zeros"; align_corners 0, the value every example
that omits it behaves as).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

MODES = {"linear": 0, "nearest": 1, "cubic": 2}
PADDINGS = {"zeros": 0, "border": 1, "reflection": 2}

_lock = threading.Lock()
_default = None

# A handle from load_library() can be passed as `lib=` to run the same calls
# against another build of the oracle source (used by the mutation tests).


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile oracle.c (or another copy of it) into a shared library."""
    if not force and os.path.exists(out):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
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
    lib.oracle_grid_sample.argtypes = [p_f32, c_int, i64, i64, p_i64, p_f32, p_i64,
                                       c_int, c_int, c_int, p_f64]
    lib.oracle_grid_sample.restype = c_int
    lib.oracle_grid_sample_points.argtypes = [p_f32, c_int, i64, i64, p_i64, p_f32, p_i64,
                                              c_int, c_int, c_int, p_i64, i64, p_f64]
    lib.oracle_grid_sample_points.restype = c_int
    lib.oracle_abi_version.restype = c_int
    return lib


def _load():
    global _default
    with _lock:
        if _default is None:
            if not os.path.exists(_LIB):
                build()
            _default = _bind(_LIB)
        return _default


def load_library(path: str):
    """ctypes handle for an oracle library built from `path`."""
    return _bind(path)


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def affine_grid(theta: np.ndarray, size, align_corners: int = 0, lib=None) -> np.ndarray:
    """AffineGrid(theta, size) -> grid (fp32).

    theta: (N, r, r+1) fp32.  size: (N, C, *spatial) as on the page (C unused).
    Returns (N, *spatial, r) fp32.
    """
    lib = lib or _load()
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


def _check_sample_args(X, grid):
    X = np.ascontiguousarray(X, dtype=np.float32)
    grid = np.ascontiguousarray(grid, dtype=np.float32)
    r = X.ndim - 2
    if r < 1 or grid.ndim != r + 2 or grid.shape[0] != X.shape[0] or grid.shape[-1] != r:
        raise ValueError("X %s and grid %s do not match" % (X.shape, grid.shape))
    return X, grid, r


def grid_sample(X: np.ndarray, grid: np.ndarray, mode: str = "linear",
                padding_mode: str = "zeros", align_corners: int = 0, lib=None) -> np.ndarray:
    """GridSample(X, grid) -> Y as float64 (unrounded).

    X: (N, C, *in_spatial) fp32 (half inputs are passed widened exactly).
    grid: (N, *out_spatial, r) fp32.  Returns (N, C, *out_spatial) float64.
    """
    lib = lib or _load()
    X, grid, r = _check_sample_args(X, grid)
    n, c = X.shape[:2]
    in_sp = np.asarray(X.shape[2:], dtype=np.int64)
    out_sp = np.asarray(grid.shape[1:-1], dtype=np.int64)
    Y = np.empty((n, c, *grid.shape[1:-1]), dtype=np.float64)
    rc = lib.oracle_grid_sample(_ptr(X, ctypes.c_float), r, n, c, _ptr(in_sp, ctypes.c_int64),
                                _ptr(grid, ctypes.c_float), _ptr(out_sp, ctypes.c_int64),
                                MODES[mode], PADDINGS[padding_mode], int(align_corners),
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
    rc = lib.oracle_grid_sample_points(_ptr(X, ctypes.c_float), r, n, c,
                                       _ptr(in_sp, ctypes.c_int64), _ptr(grid, ctypes.c_float),
                                       _ptr(out_sp, ctypes.c_int64), MODES[mode],
                                       PADDINGS[padding_mode], int(align_corners),
                                       _ptr(idx, ctypes.c_int64), idx.shape[0],
                                       _ptr(Y, ctypes.c_double))
    if rc:
        raise ValueError("oracle_grid_sample_points rejected its arguments")
    return Y
