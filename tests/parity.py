"""Helpers shared by the GPU parity tests: tensor transfer and the tolerance
rules of each mode and element type.

Tolerances (stated for the sampler; the oracle is the float64 reference):
  fp32  nearest  bit-exact (same fp32 coordinate operations, same pixel)
        linear   max |gpu - oracle| <= 1e-5 * max|X|
        cubic    max |gpu - oracle| <= 1e-4 * max|X|
  fp16 / bf16    nearest bit-exact; linear and cubic within
                 2e-2 * max(|oracle|, 1e-3 * max|X|) per element, and within
                 one unit in the last place of the output type (plus the fp32
                 accumulation error 1e-5 * max|X|) of the oracle's value.
"""

from __future__ import annotations

import sys

import numpy as np

import workloads as W

TORCH_DTYPE = {}


def torch_mod():
    import torch

    if not TORCH_DTYPE:
        TORCH_DTYPE.update({"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16})
    return torch


def note(msg: str):
    """Print the case about to run on the GPU, flushed, so a failing run names it."""
    sys.stdout.write("[gpu] %s\n" % msg)
    sys.stdout.flush()


def to_gpu_f32(a: np.ndarray):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def x_to_gpu(X_f32: np.ndarray, kind: str):
    """Device copy of X in element type `kind`, plus the exact fp32 widening
    of what was uploaded (the oracle's input)."""
    torch = torch_mod()
    if kind == "f32":
        return to_gpu_f32(X_f32), np.ascontiguousarray(X_f32, dtype=np.float32)
    bits = W.to_half_bits(X_f32, kind)
    t = torch.from_numpy(bits.view(np.int16)).cuda().view(TORCH_DTYPE[kind])
    return t, W.half_bits_to_f32(bits, kind)


def from_gpu(Y) -> np.ndarray:
    torch = torch_mod()
    torch.cuda.synchronize()
    return Y.float().cpu().numpy().astype(np.float64)


def ulp(v: np.ndarray, kind: str) -> np.ndarray:
    a = np.abs(v)
    if kind == "f16":
        return np.spacing(a.astype(np.float16)).astype(np.float64)
    # bf16: 8 significant bits; subnormal spacing below 2^-126
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def round_to(v: np.ndarray, kind: str) -> np.ndarray:
    f = v.astype(np.float32)
    if kind == "f16":
        return f.astype(np.float16).astype(np.float64)
    return W.half_bits_to_f32(W.to_half_bits(f, "bf16"), "bf16").astype(np.float64)


def check(gpu: np.ndarray, ref: np.ndarray, mode: str, kind: str, xmax: float, what: str = ""):
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape, what)
    xmax = float(max(xmax, 1e-30))
    if mode == "nearest":
        bad = gpu != ref
        assert not bad.any(), "%s: %d nearest mismatches, first at %s" % (
            what, bad.sum(), np.argwhere(bad)[0])
        return
    err = np.abs(gpu - ref)
    if kind == "f32":
        tol = (1e-5 if mode == "linear" else 1e-4) * xmax
        assert err.max() <= tol, "%s: max err %.3g > %.3g at %s" % (
            what, err.max(), tol, np.unravel_index(err.argmax(), err.shape))
        return
    rel_tol = 2e-2 * np.maximum(np.abs(ref), 1e-3 * xmax)
    assert np.all(err <= rel_tol), "%s: half error beyond 2e-2 relative" % what
    tight = np.abs(gpu - round_to(ref, kind)) <= ulp(ref, kind) + 1e-5 * xmax
    assert tight.all(), "%s: %d half outputs more than 1 ulp from the rounded oracle" % (
        what, (~tight).sum())
