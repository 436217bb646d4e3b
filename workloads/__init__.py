"""Seeded synthetic inputs for the spatial-transformer sampler.

This module only draws random numbers and arranges them into arrays.  It holds
none of the sampler's arithmetic (no grid generator, no un-normalisation, no
padding, no interpolation), so the oracle and the GPU path can both be fed from
it without sharing any of the method.  The one place it touches coordinates is
the smooth-flow recipe, which lays its field over pixel-centre positions that it
computes for itself in float64 as part of the data, not as a step of the method.

Every generator returns host numpy arrays.  Half-precision tensors are returned
as ``uint16`` bit patterns together with a tag (``"f16"`` or ``"bf16"``), since
numpy has no bfloat16 type; :func:`half_bits_to_f32` widens them exactly.

The five named workloads mirror the shapes and value distributions of the
spatial-transformer use the GridSample page describes (an STN-style batch of
near-identity affine transforms, a random flow field, a volumetric transform
and a large smooth-flow half-precision batch).  The Resize workloads are
feature-map sized up- and downsampling batches.  The pages print no benchmark
and name no dataset; these synthetic inputs stand in for real images.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "rng",
    "uniform",
    "normal",
    "near_identity_theta",
    "random_theta",
    "uniform_grid",
    "smooth_flow_grid",
    "to_half_bits",
    "half_bits_to_f32",
    "make_inputs",
    "ResizeWorkload",
    "RESIZE_WORKLOADS",
    "make_resize_input",
    "TypeWorkload",
    "TYPE_WORKLOADS",
    "make_type_inputs",
    "smooth_warp_1d",
    "DeformWorkload",
    "DEFORM_WORKLOADS",
    "make_deform_inputs",
]


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def uniform(g: np.random.Generator, shape, lo: float, hi: float) -> np.ndarray:
    """fp32 samples of U(lo, hi)."""
    u = g.random(shape, dtype=np.float32)
    return (np.float32(lo) + np.float32(hi - lo) * u).astype(np.float32)


def normal(g: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    """fp32 samples of N(0, scale^2)."""
    z = g.standard_normal(shape, dtype=np.float32)
    return (np.float32(scale) * z).astype(np.float32)


def near_identity_theta(g: np.random.Generator, n: int, r: int, noise: float) -> np.ndarray:
    """(n, r, r+1) fp32 affine matrices [I | 0] + noise * N(0,1)."""
    eye = np.zeros((r, r + 1), dtype=np.float64)
    eye[:r, :r] = np.eye(r)
    z = g.standard_normal((n, r, r + 1))
    return (eye[None] + noise * z).astype(np.float32)


def random_theta(g: np.random.Generator, n: int, r: int) -> np.ndarray:
    """(n, r, r+1) fp32 affine matrices with N(0,1) entries."""
    return g.standard_normal((n, r, r + 1)).astype(np.float32)


def uniform_grid(g: np.random.Generator, n: int, out_spatial, lo: float, hi: float) -> np.ndarray:
    """i.i.d. U(lo, hi) sampling locations, shape (n, *out_spatial, r)."""
    r = len(out_spatial)
    return uniform(g, (n, *out_spatial, r), lo, hi)


def smooth_flow_grid(g: np.random.Generator, n: int, ho: int, wo: int,
                     n_waves: int = 4, amp: float = 0.05) -> np.ndarray:
    """(n, ho, wo, 2) fp32 field: pixel-centre positions plus a smooth flow.

    The positions are the centres of a wo x ho raster spread over [-1, 1]
    (the centre of column j is -1 + (2j+1)/wo).  For every sample and every
    component, the flow is a sum of ``n_waves`` sinusoids of amplitude ``amp``
    with random wave vectors u, v ~ U(-2, 2) and phases phi ~ U(0, 2*pi),
    evaluated at the same positions.  Computed in float64 and
    rounded once to fp32.
    """
    xs = -1.0 + (2.0 * np.arange(wo) + 1.0) / wo
    ys = -1.0 + (2.0 * np.arange(ho) + 1.0) / ho
    bx = np.broadcast_to(xs[None, :], (ho, wo))
    by = np.broadcast_to(ys[:, None], (ho, wo))
    out = np.empty((n, ho, wo, 2), dtype=np.float32)
    for b in range(n):
        for k, pos in enumerate((bx, by)):
            u = g.uniform(-2.0, 2.0, n_waves)
            v = g.uniform(-2.0, 2.0, n_waves)
            phi = g.uniform(0.0, 2.0 * math.pi, n_waves)
            flow = np.zeros((ho, wo))
            for j in range(n_waves):
                flow += amp * np.sin(2.0 * math.pi * (u[j] * bx + v[j] * by) + phi[j])
            out[b, :, :, k] = (pos + flow).astype(np.float32)
    return out


def to_half_bits(x: np.ndarray, kind: str) -> np.ndarray:
    """Round fp32 to fp16 or bf16 (round to nearest even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if kind == "f16":
        return x.astype(np.float16).view(np.uint16)
    if kind == "bf16":
        u = x.view(np.uint32).astype(np.uint64)
        bias = ((u >> 16) & 1) + 0x7FFF
        r = ((u + bias) >> 16).astype(np.uint16)
        nan = np.isnan(x)
        if nan.any():
            r[nan] = 0x7FC0
        return r
    raise ValueError(kind)


def half_bits_to_f32(h: np.ndarray, kind: str) -> np.ndarray:
    """Exact widening of fp16 / bf16 bit patterns to fp32."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    if kind == "f16":
        return h.view(np.float16).astype(np.float32)
    if kind == "bf16":
        return (h.astype(np.uint32) << 16).view(np.float32)
    raise ValueError(kind)


@dataclass(frozen=True)
class Workload:
    """One named input recipe (shapes, distributions, attributes)."""

    name: str
    seed: int
    rank: int                    # spatial rank r (2 or 3)
    x_shape: tuple               # (N, C, *in_spatial)
    out_spatial: tuple           # output spatial extents, outermost first
    mode: str                    # "linear" | "nearest" | "cubic"
    padding: str                 # "zeros" | "border" | "reflection"
    align_corners: int
    x_dist: str                  # "uniform" (U(-1,1)) | "normal" (N(0,1))
    grid_kind: str               # "affine_random" | "affine_near_identity" | "uniform" | "smooth_flow"
    grid_lo: float = -1.0        # for grid_kind == "uniform"
    grid_hi: float = 1.0
    dtypes: tuple = ("f32",)
    extra_modes: tuple = field(default_factory=tuple)   # (mode, padding) pairs also run

    @property
    def n(self) -> int:
        return self.x_shape[0]

    @property
    def c(self) -> int:
        return self.x_shape[1]

    @property
    def outputs(self) -> int:
        return int(self.n * self.c * np.prod(self.out_spatial))


WORKLOADS = {
    # Tiny 2D STN case: random affine matrices send much of the grid outside
    # [-1, 1]; input 16x16, output 5x6.
    "stn2d_tiny": Workload("stn2d_tiny", 1, 2, (2, 3, 16, 16), (5, 6), "linear", "zeros", 0,
                           "uniform", "affine_random"),
    # 2D STN batch: 64 images of 64 channels at 128x128, near-identity theta.
    "stn2d_batch": Workload("stn2d_batch", 2, 2, (64, 64, 128, 128), (128, 128), "linear", "zeros", 0,
                            "uniform", "affine_near_identity",
                            extra_modes=(("nearest", "border"),)),
    # 2D random flow: i.i.d. locations in U(-1.2, 1.2), bicubic + reflection.
    "flow2d_bicubic": Workload("flow2d_bicubic", 3, 2, (16, 128, 256, 256), (256, 256), "cubic",
                               "reflection", 1, "normal", "uniform", -1.2, 1.2),
    # 3D volumetric: 64^3 volumes, near-identity theta, trilinear + border.
    "vol3d": Workload("vol3d", 4, 3, (2, 16, 64, 64, 64), (64, 64, 64), "linear", "border", 0,
                      "normal", "affine_near_identity"),
    # Large half-precision batch with a smooth flow field.
    "flow2d_half": Workload("flow2d_half", 5, 2, (8, 256, 256, 256), (256, 256), "linear", "zeros", 0,
                            "uniform", "smooth_flow", dtypes=("bf16", "f16")),
}


def make_inputs(w: Workload, x_shape=None, out_spatial=None):
    """Draw one workload's inputs, optionally at reduced shapes.

    Draw order: theta (affine kinds) or grid (direct kinds) first, then X.
    Returns a dict with ``X`` (fp32), ``theta`` (or None) and ``grid`` (or None;
    for affine kinds the grid is produced by the grid generator under test).
    Half-precision workloads also carry ``X_bits[kind]`` and the exactly
    widened ``X_half_as_f32[kind]``.
    """
    x_shape = tuple(x_shape or w.x_shape)
    out_spatial = tuple(out_spatial or w.out_spatial)
    n = x_shape[0]
    r = len(out_spatial)
    g = rng(w.seed)
    theta = grid = None
    if w.grid_kind == "affine_random":
        theta = random_theta(g, n, r)
    elif w.grid_kind == "affine_near_identity":
        theta = near_identity_theta(g, n, r, 0.1)
    elif w.grid_kind == "uniform":
        grid = uniform_grid(g, n, out_spatial, w.grid_lo, w.grid_hi)
    elif w.grid_kind == "smooth_flow":
        grid = smooth_flow_grid(g, n, *out_spatial)
    else:
        raise ValueError(w.grid_kind)
    if w.x_dist == "uniform":
        X = uniform(g, x_shape, -1.0, 1.0)
    else:
        X = normal(g, x_shape)
    out = {"X": X, "theta": theta, "grid": grid, "x_shape": x_shape,
           "out_spatial": out_spatial, "X_bits": {}, "X_half_as_f32": {}}
    for kind in w.dtypes:
        if kind in ("f16", "bf16"):
            bits = to_half_bits(X, kind)
            out["X_bits"][kind] = bits
            out["X_half_as_f32"][kind] = half_bits_to_f32(bits, kind)
    return out


@dataclass(frozen=True)
class ResizeWorkload:
    """One named Resize input recipe: X ~ U(-1, 1) and per-axis scales of the
    resized trailing axes (the output extents follow from them)."""

    name: str
    seed: int
    x_shape: tuple
    scales: tuple                # one per trailing resized axis
    mode: str                    # "nearest" | "linear" | "cubic"
    coordinate_transformation_mode: str = "half_pixel"

    def full_scales(self):
        lead = len(self.x_shape) - len(self.scales)
        return [1.0] * lead + [float(v) for v in self.scales]


RESIZE_WORKLOADS = {
    # 2x upsampling of a batch of 64-channel 128x128 feature maps
    "resize2d_up2_linear": ResizeWorkload("resize2d_up2_linear", 21, (32, 64, 128, 128),
                                          (2.0, 2.0), "linear"),
    "resize2d_up2_nearest": ResizeWorkload("resize2d_up2_nearest", 22, (32, 64, 128, 128),
                                           (2.0, 2.0), "nearest"),
    "resize2d_up2_cubic": ResizeWorkload("resize2d_up2_cubic", 23, (32, 64, 128, 128),
                                         (2.0, 2.0), "cubic"),
    # 2x downsampling of 256x256 maps
    "resize2d_down2_linear": ResizeWorkload("resize2d_down2_linear", 24, (32, 64, 256, 256),
                                            (0.5, 0.5), "linear"),
    # 2x trilinear upsampling of 64^3 volumes
    "resize3d_up2_linear": ResizeWorkload("resize3d_up2_linear", 25, (2, 16, 64, 64, 64),
                                          (2.0, 2.0, 2.0), "linear"),
}


def make_resize_input(w: ResizeWorkload, x_shape=None) -> np.ndarray:
    """X of a Resize workload (optionally at a reduced shape), fp32 U(-1, 1)."""
    return uniform(rng(w.seed), tuple(x_shape or w.x_shape), -1.0, 1.0)


def smooth_warp_1d(g: np.random.Generator, n: int, wo: int, n_waves: int = 4,
                   amp: float = 0.01) -> np.ndarray:
    """(n, wo, 1) fp32 field: the pixel-centre positions of a wo-sample line
    over [-1, 1] plus a sum of ``n_waves`` sinusoids of amplitude ``amp`` with
    wave numbers u ~ U(-4, 4) and phases phi ~ U(0, 2*pi).  float64, rounded
    once to fp32."""
    xs = -1.0 + (2.0 * np.arange(wo) + 1.0) / wo
    out = np.empty((n, wo, 1), dtype=np.float32)
    for b in range(n):
        u = g.uniform(-4.0, 4.0, n_waves)
        phi = g.uniform(0.0, 2.0 * math.pi, n_waves)
        flow = np.zeros(wo)
        for j in range(n_waves):
            flow += amp * np.sin(2.0 * math.pi * u[j] * xs + phi[j])
        out[b, :, 0] = (xs + flow).astype(np.float32)
    return out


@dataclass(frozen=True)
class TypeWorkload:
    """A GridSample workload of another rank or element type."""

    name: str
    seed: int
    x_shape: tuple
    out_spatial: tuple
    mode: str
    padding: str
    align_corners: int
    x_kind: str                  # "uint8" | "f32" | "f64"
    grid_kind: str               # "affine_near_identity" | "smooth_warp_1d"
    precision: str = "f32"       # theta / grid element type: "f32" | "f64"

    @property
    def outputs(self) -> int:
        return int(self.x_shape[0] * self.x_shape[1] * np.prod(self.out_spatial))


TYPE_WORKLOADS = {
    # an STN batch of 8-bit RGB images warped by near-identity affine maps
    "stn2d_u8": TypeWorkload("stn2d_u8", 31, (64, 3, 512, 512), (512, 512), "linear", "zeros", 0,
                             "uint8", "affine_near_identity"),
    # 1-D resampling of long fp32 signals along smooth monotone warps
    "signal1d_f32": TypeWorkload("signal1d_f32", 32, (64, 128, 8192), (8192,), "linear", "zeros",
                                 0, "f32", "smooth_warp_1d"),
    # the volumetric transform in double precision (theta, grid and X)
    "vol3d_f64": TypeWorkload("vol3d_f64", 33, (2, 16, 64, 64, 64), (64, 64, 64), "linear",
                              "border", 0, "f64", "affine_near_identity", "f64"),
}


def make_type_inputs(w: TypeWorkload, x_shape=None, out_spatial=None):
    """Draw a TypeWorkload's inputs: theta (affine kinds, w.precision) or the
    grid, then X in its element type (uint8 uniform over 0..255, fp32
    U(-1, 1), double N(0, 1))."""
    x_shape = tuple(x_shape or w.x_shape)
    out_spatial = tuple(out_spatial or w.out_spatial)
    n = x_shape[0]
    r = len(out_spatial)
    g = rng(w.seed)
    theta = grid = None
    if w.grid_kind == "affine_near_identity":
        theta = near_identity_theta(g, n, r, 0.1)
        if w.precision == "f64":
            eye = np.zeros((r, r + 1))
            eye[:r, :r] = np.eye(r)
            theta = eye[None] + 0.1 * g.standard_normal((n, r, r + 1))
    elif w.grid_kind == "smooth_warp_1d":
        grid = smooth_warp_1d(g, n, out_spatial[0])
    else:
        raise ValueError(w.grid_kind)
    if w.x_kind == "uint8":
        X = g.integers(0, 256, x_shape, dtype=np.uint8)
    elif w.x_kind == "f64":
        X = g.standard_normal(x_shape)
    else:
        X = uniform(g, x_shape, -1.0, 1.0)
    return {"X": X, "theta": theta, "grid": grid, "x_shape": x_shape, "out_spatial": out_spatial}


@dataclass(frozen=True)
class DeformWorkload:
    """A DeformConv layer: X ~ U(-1, 1), W ~ U(-w, w) with w = 1/sqrt(fan-in),
    pixel offsets ~ N(0, offset_std^2), mask ~ U(0, 1), B ~ U(-0.1, 0.1)."""

    name: str
    seed: int
    x_shape: tuple               # (N, C, H, W)
    w_shape: tuple               # (oC, C / group, kH, kW)
    pads: tuple
    group: int = 1
    offset_group: int = 1
    offset_std: float = 1.0
    dtypes: tuple = ("bf16", "f32")

    def out_shape(self):
        n, _, h, w = self.x_shape
        oc, _, kh, kw = self.w_shape
        return (n, oc, h + self.pads[0] + self.pads[2] - kh + 1,
                w + self.pads[1] + self.pads[3] - kw + 1)

    @property
    def flops(self) -> int:
        n, oc, oh, ow = self.out_shape()
        k = self.w_shape[1] * self.w_shape[2] * self.w_shape[3]
        return 2 * n * oc * oh * ow * k


DEFORM_WORKLOADS = {
    # a modulated deformable 3x3 layer of a ResNet stage at 64x64 (DCNv2-style)
    "dcn2d_resnet": DeformWorkload("dcn2d_resnet", 41, (8, 256, 64, 64), (256, 256, 3, 3),
                                   (1, 1, 1, 1)),
}


def make_deform_inputs(w: DeformWorkload, x_shape=None, w_shape=None):
    """X, W, offset, mask, B of a DeformWorkload (fp32; optionally reduced)."""
    x_shape = tuple(x_shape or w.x_shape)
    w_shape = tuple(w_shape or w.w_shape)
    g = rng(w.seed)
    n, _, h, wd = x_shape
    kh, kw = w_shape[2:]
    oh = h + w.pads[0] + w.pads[2] - kh + 1
    ow = wd + w.pads[1] + w.pads[3] - kw + 1
    fan_in = w_shape[1] * kh * kw
    X = uniform(g, x_shape, -1.0, 1.0)
    Wt = uniform(g, w_shape, -1.0 / math.sqrt(fan_in), 1.0 / math.sqrt(fan_in))
    off = normal(g, (n, w.offset_group * kh * kw * 2, oh, ow), w.offset_std)
    mask = uniform(g, (n, w.offset_group * kh * kw, oh, ow), 0.0, 1.0)
    B = uniform(g, (w_shape[0],), -0.1, 0.1)
    return {"X": X, "W": Wt, "offset": off, "mask": mask, "B": B}
